"""Plain, slow, obviously correct CPU reference for the fused attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); the seeded input generators
in ``tiled_attention_10_amd.workloads`` are the only thing both sides use, and
they hold none of the method's arithmetic.

Sources (web pages; cited by title and section):

* [FA3-V3] "FlashAttention（V3）深度解析：从原理到工程实现-Hopper架构下的注意力机制优化革命"
  (dtcms.com): §2 defines attention, §4.2 the online-softmax merge rule,
  §4.3 block quantisation, §11 the PyTorch simulation (``standard_attention``,
  the consumer's online softmax and causal mask).
* [FA3-card] "FlashAttention-3——利用异步与低精度加速注意力机制" (knowledge card
  summarising the Together AI blog): "低精度优化：非相干处理" (random-sign
  Hadamard per head).
* [FA3-tile] "FlashAttention-3 进阶实录：Tile 级异步流水线与显存带宽榨取实战"
  (gsyq.cn): §四 keeps the softmax statistics in fp32.

Modules:

* ``attention``  -- fp64 definition of softmax(scale·QKᵀ + mask)·V, sampled
  rows, LSE, and the two-chunk merge rule (pinned by tests/test_oracle_attention.py).
* ``e4m3``       -- OCP FP8 E4M3FN decode table and round-to-nearest-even,
  saturating encoder (pinned against torch's float8_e4m3fn and brute force).
* ``hadamard``   -- Sylvester Hadamard matrix, fast Walsh–Hadamard transform,
  random-sign rotation (pinned by orthogonality and invariance tests).
* ``quant``      -- per-(batch, head, 64-row block) absmax scaling and e4m3
  codes, every decision taken on fp64 values by the definition: scale =
  fl32(absmax/448), code = e4m3(y/scale) (pinned by exact rational brute
  force over all codes and by orthogonal inputs that keep rows on the grid).
* ``rope``       -- rotary position embedding (half-split pairs, caller's cos/sin
  tables) ahead of the rotation and quantiser, in fp64: the fused prologue of
  [FA3-card] "低精度优化" (pinned by tests/test_oracle_rope.py: identity,
  norms, composition, complex form, relative position, planted sign error).
* ``decode``     -- one decode step over an FP8 block-quantised KV cache: the
  fp64 definition on the dequantised cache, per-sequence lengths, GQA
  (pinned by tests/test_oracle_decode.py: brute force, the causal prefill
  oracle's last row, torch float64 SDPA, block-boundary and planted mistakes).
* ``fp8_attention`` -- fp64 emulation of the fp8 attention path.  The pages
  give no worked FP8 result; it is pinned where nothing rounds (E4M3-exact
  codes, power-of-two block scales, probabilities that are E4M3 powers of
  two): there it must equal the plain definition (tests/test_oracle_fp8.py).
  Elsewhere it serves as a sanity bound, the criterion being RMSE against the
  exact fp64 result.
"""

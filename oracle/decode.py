"""Decode-step attention over an FP8 block-quantised KV cache (test infrastructure only; see oracle/__init__).

Setting.  In autoregressive generation each step adds one token per sequence,
whose query attends to the keys and values cached for that sequence so far.
[FA3-tile] opens with this setting at 128k to 1M tokens, where memory
bandwidth limits throughput (its §三 measures the bandwidth at 128k); [FA3-V3]
§5 notes FP8 KV caches among the deployment options, and §4.3 gives the
per-block scales.

Readings taken (the pages give no decode formula):

* The cache stores K and V as OCP E4M3FN codes [B, Nmax, Hkv, d] with one fp32
  scale per (batch, KV head, 64-row block) [B, Hkv, ceil(Nmax/64)], the layout
  ``quant.quantize`` produces.  The cached value of key j is
  decode(code_j) · scale[j // 64].
* The query of the step stays in its 16-bit storage type, q [B, Hq, d]; query
  head h reads KV head h // (Hq/Hkv).
* Sequence b has L_b = seqlens[b] valid cache rows, 1 <= L_b <= Nmax; rows past
  L_b are not part of the sequence.

The step is then attention (the definition of [FA3-V3] §2) of a single query
row against the dequantised cache, which this module writes out in fp64:

    s_j = scale · q·k_j  (j < L_b),   O = Σ_j softmax(s)_j · v_j,   LSE = log Σ_j e^(s_j).
"""
from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 64


def dequantize(codes, scales, block: int = BLOCK) -> np.ndarray:
    """codes uint8 [B, N, H, d], scales [B, H, ceil(N/block)] -> fp64 [B, N, H, d]:
    row j of head h is decode(code) · scales[b, h, j // block]."""
    codes = np.asarray(codes, dtype=np.uint8)
    B, N, H, d = codes.shape
    sc = np.asarray(scales, dtype=np.float64)
    assert sc.shape == (B, H, -(-N // block)), (sc.shape, codes.shape)
    per_row = np.repeat(sc, block, axis=2)[:, :, :N]           # [B, H, N]
    return e4m3.decode(codes) * per_row.transpose(0, 2, 1)[..., None]


def decode_attention(q, k_codes, k_scales, v_codes, v_scales, seqlens, scale=None,
                     return_lse: bool = False):
    """fp64 decode step.  q [B, Hq, d] (any float dtype, upcast exactly), cache as in
    the module docstring, seqlens [B] ints in [1, Nmax].  Returns O [B, Hq, d]
    (and LSE [B, Hq], natural log) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    K = dequantize(k_codes, k_scales)
    V = dequantize(v_codes, v_scales)
    B, Hq, d = q.shape
    _, Nmax, Hkv, _ = K.shape
    assert Hq % Hkv == 0 and V.shape == K.shape
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(seqlens[b])
        assert 1 <= L <= Nmax, L
        for h in range(Hq):
            kv = h // g
            s = scale * (K[b, :L, kv] @ q[b, h])        # [L]
            m = s.max()
            p = np.exp(s - m)
            z = p.sum()
            out[b, h] = (p @ V[b, :L, kv]) / z
            lse[b, h] = m + np.log(z)
    return (out, lse) if return_lse else out

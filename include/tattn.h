/*
 * tattn — tiled fused attention forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every tensor is a dense row-major
 * array laid out [B, N, H, d] (batch, sequence position, head, channel) in
 * device memory that the caller allocates and owns; the library allocates
 * nothing.  Its global state is a per-device cache of the compute-unit count
 * (written atomically) and, for attn_decode_fp8kv_noalloc only, a fixed device
 * array per GPU with its address (looked up under a lock), so calls from
 * several host threads are safe (except overlapping attn_decode_fp8kv_noalloc
 * calls on one GPU, which share that array).
 * Every call is asynchronous on ``stream`` (a hipStream_t; NULL means the
 * default stream) and returns before the GPU has finished.  The attention
 * kernels launch one workgroup per compute unit of the current device and each
 * workgroup walks a fixed share of the work; running them beside other kernels
 * on the same device is correct but may serialise part of the grid.  A call
 * only launches kernels on ``stream`` (no allocation, copy, memset or
 * synchronisation), so it can be recorded into a HIP graph by stream capture
 * (make one call on the device first: the first call per device queries the
 * compute-unit count and, for the allocation-free entry point, the scratch
 * address); the launch configuration depends on the sizes alone, so a captured call stays
 * valid for new contents of the same buffers (for the decode step, new sequence
 * lengths included).
 *
 * Return value: TATTN_OK (0) or one of the TATTN_ERR_* codes below.  Argument
 * checks run on the host before any HIP call, so a rejected call touches
 * neither the GPU nor the output buffers.  A HIP launch error is returned as
 * TATTN_ERR_HIP; a device fault after a successful launch surfaces at the
 * caller's next synchronisation.  tattn_last_error() gives a text detail of
 * the last failure on the calling thread.  No C++ exception crosses the ABI.
 *
 * Sources (web pages, cited by title and section):
 *   [FA3-V3]   "FlashAttention（V3）深度解析：从原理到工程实现" (dtcms.com)
 *   [FA3-card] "FlashAttention-3——利用异步与低精度加速注意力机制" (knowledge card
 *              summarising the Together AI blog post)
 *   [FA3-tile] "FlashAttention-3 进阶实录：Tile 级异步流水线与显存带宽榨取实战" (gsyq.cn)
 */
#ifndef TATTN_H
#define TATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum {
  TATTN_F16 = 1,  /* IEEE binary16 */
  TATTN_BF16 = 2  /* bfloat16 */
};

/* status codes */
enum {
  TATTN_OK = 0,
  TATTN_ERR_INVALID_ARG = 1, /* null pointer, size < 1, Hq % Hkv != 0, bad scale or flag */
  TATTN_ERR_UNSUPPORTED = 2, /* head dim not in {64, 128}, unknown dtype */
  TATTN_ERR_MISALIGNED = 3,  /* a tensor pointer is not 16-byte aligned (lse/scales: 4) */
  TATTN_ERR_HIP = 4          /* HIP runtime or launch error (see tattn_last_error) */
};

/*
 * attn_fwd — O = softmax(scale·Q·Kᵀ + mask)·V for 16-bit inputs.
 *
 * Defined by [FA3-V3] §2 (S = QKᵀ, P = softmax(S), O = PV; Q, K, V ∈ R^{N×d}
 * per head) with §11's 1/sqrt(d) scaling and causal mask (key j is visible to
 * query i iff j <= i).  Computed tile by tile with the online softmax of
 * [FA3-V3] §4.2 (running row max m and denominator z, merged as
 * m = max(m_a, m_b), z = z_a·e^(m_a−m) + z_b·e^(m_b−m)) with fp32 statistics
 * ([FA3-tile] §四), so the N×N score matrix never reaches memory.
 *
 *   q    [B, N, Hq,  d]  dtype           (read)
 *   k    [B, N, Hkv, d]  dtype           (read)
 *   v    [B, N, Hkv, d]  dtype           (read)
 *   o    [B, N, Hq,  d]  dtype           (written; must not alias q, k, v)
 *   lse  [B, Hq, N]      fp32 or NULL    (written if non-NULL: natural-log
 *                                         log-sum-exp of each row's scaled,
 *                                         masked scores)
 *   B, N, Hq, Hkv >= 1 with Hq % Hkv == 0; query head h reads key/value
 *   head h / (Hq/Hkv).  d ∈ {64, 128}.  Any N (a partial last tile is masked).
 *   64 key rows must span less than 4 GiB: Hkv·d·2·64 < 2^32 (Hkv·d·64 on
 *   the fp8 path), else TATTN_ERR_INVALID_ARG.
 *   softmax_scale: finite and > 0 (1/sqrt(d) for the standard definition).
 *   causal: 0 or 1.  dtype: TATTN_F16 or TATTN_BF16 (output in the same type).
 * Precision: the scores are the exact products of the 16-bit inputs summed in
 * fp32, times scale·log2(e) in fp32 (one fused multiply-add with the reference
 * max); each probability is rounded to dtype for P·V, and the denominator sums
 * the same rounded probabilities, so O is a weighted mean of V rows with fp32
 * accumulation, rounded once to dtype.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int N, int Hq, int Hkv, int d, float softmax_scale, int causal,
             int dtype, void* stream);

/*
 * attn_fwd_fp8 — the same operation on OCP FP8 E4M3FN codes with per-block
 * scales ([FA3-V3] §4.3: a scale factor per block of the quantised tensor).
 *
 * Each tensor x is represented by codes c (uint8, [B, N, H, d]) and fp32 scales
 * s ([B, H, ceil(N/64)]) with x[b, n, h, :] ≈ e4m3(c[b, n, h, :]) · s[b, h, n/64]
 * — the output of hadamard_rotate() with a non-NULL scales_out.  Q and K may
 * have been rotated with the same signs (the product Q·Kᵀ is unchanged by the
 * rotation); V must not be rotated.  Both products run on FP8 matrix cores with
 * fp32 accumulation; the scores' scales are applied in fp32; the probabilities
 * are rounded to E4M3 for the second product after multiplying them by
 * s_v(block) · 2^8 / max_blocks(s_v) (undone in fp32 in the epilogue), and
 * the softmax denominator sums those same rounded probabilities (mapped back
 * by the same factor), so O is a weighted mean with the weights that entered
 * the second product.
 *
 *   q8, k8, v8              codes as above (read); 16-byte aligned
 *   q_scale, k_scale, v_scale  fp32 [B, Hq|Hkv, ceil(N/64)], finite and > 0
 *   o                       [B, N, Hq, d] in out_dtype (TATTN_BF16 or TATTN_F16)
 *   lse                     as for attn_fwd, or NULL
 *   other arguments as for attn_fwd (d = 128 and N <= 262144 on this path:
 *   larger values return TATTN_ERR_UNSUPPORTED).
 */
int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                 const float* q_scale, const float* k_scale, const float* v_scale,
                 void* o, float* lse, int B, int N, int Hq, int Hkv, int d,
                 float softmax_scale, int causal, int out_dtype, void* stream);

/*
 * hadamard_rotate — random-sign Hadamard rotation of each head's rows,
 * optionally fused with FP8 block quantisation ([FA3-card] "低精度优化：
 * 非相干处理": each head's Q and K multiplied by a random orthogonal matrix made
 * of a Hadamard transform and random signs; [FA3-V3] §4.3: per-block scales).
 *
 * For every row r = x[b, n, h, :] of length d:
 *     y = H_d · (s ⊙ r) / sqrt(d)      if signs != NULL (Sylvester H_d, as one
 *                                      butterfly stage per channel-index bit in
 *                                      fp32, the kernel's order of the stages,
 *                                      then one fp32 multiply by fl32(1/sqrt(d)))
 *     y = r                            if signs == NULL
 * If scales_out == NULL, y is written to ``y`` in in_dtype (round to nearest
 * even).  Otherwise, per (b, h, block of 64 consecutive rows):
 *     scale = absmax(y) / 448            (IEEE fp32 division; 1 for an all-zero block)
 *     code  = E4M3FN(y · (448/absmax))   (one IEEE fp32 division per block, one
 *                                         fp32 multiply per element; nearest-even,
 *                                         saturating at ±448; y · 1 for a zero block)
 * and ``y`` receives uint8 codes [B, N, H, d], ``scales_out`` fp32
 * [B, H, ceil(N/64)].  With exact arithmetic this is the definition
 * scale = absmax/448, code = nearest E4M3 value of y/scale; the fp32 evaluation
 * can differ from it only where y/scale lies within its rounding error of an
 * E4M3 rounding boundary, and a 16-bit y only where y lies that close to a
 * 16-bit rounding boundary.
 *
 *   x          [B, N, H, d] in_dtype (TATTN_F16 or TATTN_BF16) (read)
 *   y          output as above; must not alias x
 *   signs      int8 [d] of +1/-1, or NULL
 *   d ∈ {64, 128}; B, N, H >= 1.
 */
int hadamard_rotate(const void* x, void* y, const int8_t* signs, float* scales_out,
                    int B, int N, int H, int d, int in_dtype, void* stream);

/*
 * rope_hadamard_rotate — hadamard_rotate() with a rotary position embedding
 * applied first, in the same pass over memory ([FA3-card] "低精度优化": the
 * Hadamard rotation is memory bound and can be fused with the rotary
 * embedding at no extra cost).  The pages do not define the embedding; it is
 * the standard rotation of channel pairs (i, i + d/2), i < d/2, of the row at
 * position n by the caller's angle θ[n, i]:
 *     r_i       = fl(fl(x_i · cos) − fl(x_{i+d/2} · sin))
 *     r_{i+d/2} = fl(fl(x_{i+d/2} · cos) + fl(x_i · sin))      (fp32, no fused ops)
 * and then exactly hadamard_rotate() on r (rotation if signs != NULL, FP8
 * block quantisation if scales_out != NULL, else output in in_dtype).
 *
 *   rope_cos, rope_sin   fp32 [N, d/2] (row n = position n), 16-byte aligned (read)
 *   other arguments as for hadamard_rotate.
 */
int rope_hadamard_rotate(const void* x, void* y, const float* rope_cos, const float* rope_sin,
                         const int8_t* signs, float* scales_out, int B, int N, int H, int d,
                         int in_dtype, void* stream);

/*
 * fp8_prologue — the whole FP8 prologue of one attention call in one launch
 * ([FA3-card] "低精度优化": incoherent processing of Q and K, fusable with the
 * rotary embedding; [FA3-V3] §4.3: block quantisation of Q, K and V):
 *     q8, q_scale = rope_hadamard_rotate(q) or hadamard_rotate(q) with signs, quantised
 *     k8, k_scale = the same for k, with the same signs and tables
 *     v8, v_scale = hadamard_rotate(v, signs = NULL), quantised (no rotation, no embedding)
 * Every output is bit for bit what those separate calls write; one launch
 * covers all three tensors, so the small K and V passes no longer pay their own
 * launch and ramp.  The results are the inputs of attn_fwd_fp8().
 *
 *   q          [B, N, Hq, d] in_dtype (read);  k, v  [B, N, Hkv, d] (read)
 *   signs      int8 [d] of +1/-1 for Q and K, or NULL (Q and K only quantised)
 *   rope_cos, rope_sin   fp32 [N, d/2], both or neither (NULL: no embedding)
 *   q8, k8, v8           uint8 E4M3FN codes, the layouts of q, k, v (written)
 *   q_scale    fp32 [B, Hq, ceil(N/64)];  k_scale, v_scale  [B, Hkv, ceil(N/64)] (written)
 *   d ∈ {64, 128}; Hq a multiple of Hkv; tensors and codes 16-byte aligned,
 *   scales 4-byte aligned, tables 16-byte aligned; outputs must not alias inputs.
 * Errors as for hadamard_rotate; one table without the other is TATTN_ERR_INVALID_ARG.
 */
int fp8_prologue(const void* q, const void* k, const void* v, const int8_t* signs,
                 const float* rope_cos, const float* rope_sin, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                 float* q_scale, float* k_scale, float* v_scale, int B, int N, int Hq, int Hkv, int d,
                 int in_dtype, void* stream);

/*
 * attn_decode_fp8kv — one decode step: each sequence's new query token attends
 * to the keys and values cached for that sequence so far, stored as FP8 with
 * per-block scales.
 *
 * The operation is [FA3-V3] §2's attention with a single query row per
 * (sequence, query head); the cache format is §4.3's block quantisation (the
 * layout hadamard_rotate() writes with signs = NULL and non-NULL scales_out).
 * [FA3-tile]'s opening discusses this autoregressive setting at 128k-1M
 * tokens, where memory bandwidth sets the speed; [FA3-V3] §5 lists FP8 KV
 * caches among the deployment options.  For sequence b with L = seqlens[b]
 * cached rows, query head h and KV head h / (Hq/Hkv):
 *     k_j = e4m3(k_cache[b, j, kv, :]) · k_scale[b, kv, j/64]   (j < L; same for v_j)
 *     s_j = softmax_scale · q[b, h, :]·k_j
 *     O[b, h, :] = Σ_j softmax(s)_j · v_j,   lse[b, h] = log Σ_j e^(s_j)
 * Computed in chunks of the sequence with the online-softmax merge of
 * [FA3-V3] §4.2 (m = max(m_a, m_b), z = z_a·e^(m_a−m) + z_b·e^(m_b−m)), fp32
 * statistics and accumulators; the products run on the matrix cores in the
 * query's 16-bit type (E4M3 values convert to it exactly) and the
 * probabilities are rounded to that type, times the V block scale over the
 * largest V block scale of the keys a wave covers, before the second product.
 *
 *   q            [B, Hq, d] dtype (read)
 *   k_cache      uint8 E4M3FN codes [B, Nmax, Hkv, d] (read; rows >= L unused)
 *   v_cache      likewise
 *   k_scale      fp32 [B, Hkv, ceil(Nmax/64)], finite and > 0 (read)
 *   v_scale      likewise
 *   seqlens      int32 [B] in DEVICE memory; values are clamped to [0, Nmax]
 *                (1 <= L <= Nmax is the meaningful range; L = 0 gives O = 0 and
 *                lse = -inf)
 *   o            [B, Hq, d] dtype (written)
 *   lse          fp32 [B, Hq] natural log, or NULL
 *   workspace    device scratch owned by the caller, at least
 *                attn_decode_fp8kv_workspace_size(B, Nmax, Hq, Hkv, d) bytes,
 *                16-byte aligned; overwritten by the call, so calls that overlap
 *                in time need separate workspaces
 *   B, Nmax, Hq, Hkv >= 1, Hq % Hkv == 0, Hkv <= 65536, d = 128,
 *   dtype TATTN_BF16 or TATTN_F16 (the type of q and o).
 * Errors: TATTN_ERR_INVALID_ARG also for a workspace smaller than required.
 */
int attn_decode_fp8kv(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* seqlens,
                      void* o, float* lse, void* workspace, size_t workspace_bytes,
                      int B, int Nmax, int Hq, int Hkv, int d, float softmax_scale,
                      int dtype, void* stream);

/* Workspace bytes attn_decode_fp8kv needs for these sizes (0 if they are invalid).
 * It depends on the sizes only (B·Hq·ceil(Nmax/chunk)·(d+2)·4 bytes, the chunk a
 * function of B, Nmax, Hq, Hkv). */
size_t attn_decode_fp8kv_workspace_size(int B, int Nmax, int Hq, int Hkv, int d);

/*
 * attn_decode_fp8kv_noalloc — attn_decode_fp8kv for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  It computes exactly what
 * attn_decode_fp8kv computes, with the same kernels, arguments (less the
 * workspace), checks and error codes, and allocates nothing: the chunk
 * partials go to a fixed scratch array of TATTN_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends.  Sizes whose
 * attn_decode_fp8kv_workspace_size() exceeds that return
 * TATTN_ERR_INVALID_ARG.  The first call on a device looks up that device's
 * address of the array (a failure returns TATTN_ERR_HIP).  Every call on one
 * GPU uses the same array: calls that overlap in time on one GPU (different
 * streams, or threads) race and must be serialised by the caller.  Nothing in
 * the array needs to start at zero; every value the step reads is written by
 * the same call first.
 */
#define TATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_decode_fp8kv_noalloc(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* seqlens,
                              void* o, float* lse, int B, int Nmax, int Hq, int Hkv, int d,
                              float softmax_scale, int dtype, void* stream);

/* Text for a status code (static storage). */
const char* tattn_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* tattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TATTN_H */

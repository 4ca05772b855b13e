// Decode step over an FP8 (E4M3FN) block-quantised KV cache for gfx950, head dim 128.
//
// One query token per sequence attends to the first L_b rows of its cached
// K and V ([FA3-V3] §2's definition with a single query row; §4.3's per-block
// scales).  The work is bound by HBM: every valid cache byte is read once.
//
// Split kernel — one workgroup per (sequence b, KV head, group of up to 16 of
// its query heads, chunk of the sequence).  The 4 waves take consecutive
// quarters of the chunk and run independently: each streams its keys 32 at a
// time through a private LDS ring filled by LDS-DMA (K and V rows of one step,
// 8 KB), so no barrier is needed inside the loop.  Long chunks use 4 stages (up
// to three steps per wave in flight) and one workgroup per CU; few or short
// workgroups use 2 stages and two workgroups per CU.  Per step, on 16x16x32 matrix-core products
// with the query heads as the N dimension:
//
//   Sᵀ = K·Qᵀ      A = 16 key rows x 32 channels (E4M3 codes converted exactly to
//                  the query's 16-bit type in registers), B = the query rows;
//                  K rows are taken in the order 8(r/4) + 4·blk + r%4, which makes
//                  the score accumulator the P operand of the second product.
//   scores         s = Sᵀ · scale·log2(e) · sk(block) in fp32; keys >= L_b masked.
//   softmax        online ([FA3-V3] §4.2) in base 2; the reference max of a head
//                  moves only when a score passes it by more than kSlack, so the
//                  cross-lane max is rare and P <= 2^kSlack.
//   Oᵀ += Vᵀ·Pᵀ    P̃ = round16(p · sv(block)/max sv): the V block scale is folded
//                  into the probabilities; A = Vᵀ from byte-transposing LDS reads
//                  (ds_read_b64_tr_b8), converted like K.  The denominator sums the
//                  same rounded P̃, mapped back by max sv/sv(block).
//
// The waves' partial results (m, z, O) are merged in LDS with the rule
// m = max(m_a, m_b), z = z_a·2^(m_a−m) + z_b·2^(m_b−m) (the same for O), and the
// workgroup writes one partial per query head to the caller's workspace — or,
// when one chunk covers Nmax, the final O and LSE, and the merge is not launched.
//
// Merge kernel — one workgroup per (b, query head): G groups of 128 threads (G = 8
// when there are few (b, head) merges, else 4) fold every G-th partial of the
// chunks that hold keys (ceil(L_b / chunk) of them) with the same rule, eight
// loads in flight per thread, then the G results are folded in LDS; it writes
// O = Σ/z in the query's type and the natural-log LSE.
#include <algorithm>

#include "tattn_device.hpp"
#include "tattn_pipeline.hpp"
#include "tattn_launch.hpp"
#include "tattn.h"

namespace tattn {
namespace {

constexpr int D = 128;
constexpr int NW = 4;                    // waves per workgroup
constexpr int kThreads = 64 * NW;
constexpr int KS = 32;                   // keys per step
constexpr int HALFB = KS * D;            // K (or V) bytes of one step: 4 KB
constexpr int STEPB = 2 * HALFB;         // one ring stage
constexpr int HG = 16;                   // query heads per workgroup
constexpr float kSlack = 8.f;            // log2 units
constexpr int kTargetItems = 1024;       // workgroups the chunk size aims for
constexpr int kMinItems = 256;           // ... but it is raised toward kLongChunk keys while
constexpr int kLongChunk = 4096;         // at least this many workgroups remain
constexpr int kMinChunk = 64 * NW;          // every wave starts on a scale block
constexpr int kMaxChunk = 64 * 64 * NW;     // a wave spans at most 64 blocks (one per lane)

// Physical 16-byte chunk of a 128-byte row = logical chunk ^ swz(row).  Both read
// shapes then hit 16 distinct 16-byte bank windows: the score reads (16 rows
// 8(r/4) + 4·blk + r%4, one chunk) and the transposing V reads (16 consecutive
// rows, one chunk).
__device__ inline int swz(int r) {
  const int x = (r >> 1) & 15;
  return (x & 1) | ((((x >> 1) ^ (x >> 3)) & 1) << 1) | (x & 4);
}

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-bit operand types with the exact E4M3 -> 16-bit conversion (every E4M3FN value
// is representable in bf16 and in fp16) and the 16x16x32 product.
struct DecBf16 : Bf16 {
  __device__ static inline vec8 from_e4m3(uint32_t w0, uint32_t w1) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true);
    return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                   __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ static inline f32x4_t mma(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

struct DecF16 : F16 {
  __device__ static inline vec8 from_e4m3(uint32_t w0, uint32_t w1) {
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, true);
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, false);
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, true);
    return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                   __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ static inline f32x4_t mma(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

struct DecParams {
  const uint16_t* q;      // [B, Hq, D]
  const uint8_t* k;       // [B, Nmax, Hkv, D] codes
  const uint8_t* v;
  const float* ksc;       // [B, Hkv, nblk]
  const float* vsc;
  const int* seqlens;     // [B]
  uint16_t* o;            // [B, Hq, D]
  float* lse;             // [B, Hq] or null
  float* ws_o;            // [B, Hq, nc, D] partial outputs (unnormalised)
  float* ws_ml;           // [B, Hq, nc, 2] partial (max in log2 units, denominator)
  int Nmax, Hq, Hkv, group, nhg, nblk, nc, chunk;
  float c;                // softmax scale · log2(e)
};

__device__ inline int seq_len(const DecParams& p, int b) {
  return min(max(p.seqlens[b], 0), p.Nmax);
}

// STAGES ring stages per wave (RINGB bytes), OCC workgroups per CU: 4 stages and one
// workgroup per CU stream long chunks best; 2 stages and two workgroups per CU let one
// workgroup's pipeline fill overlap another's streaming when workgroups are few or short.
template <typename T, int STAGES, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void attn_decode_split_kernel(DecParams p) {
  constexpr int RINGB = STAGES * STEPB;
  static_assert(RINGB >= 4 * (2 * HG + HG * D) + 256, "the ring holds a wave's merge block");
  __shared__ __attribute__((aligned(1024))) char smem[NW * RINGB];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ci = blockIdx.x, b = blockIdx.z;
  const int kvh = blockIdx.y / p.nhg, hg = blockIdx.y % p.nhg;
  const int L = seq_len(p, b);
  const int c0 = ci * p.chunk;
  if (c0 >= L) {                                 // no keys in this chunk (uniform)
    if (p.nc == 1) {                             // single-chunk plan: an empty sequence's output here
      const int h = threadIdx.x & 15, ch = 8 * (threadIdx.x >> 4), hh = hg * HG + h;
      if (hh < p.group) {
        const long long bh = (long long)b * p.Hq + kvh * p.group + hh;
        *(u32x4*)(p.o + bh * D + ch) = u32x4{0u, 0u, 0u, 0u};
        if (ch == 0 && p.lse != nullptr) p.lse[bh] = -INFINITY;
      }
    }
    return;
  }

  const int wlen = p.chunk / NW;
  const int kbeg = c0 + wave * wlen;
  const int kend = min(kbeg + wlen, L);
  const int nsteps = kend > kbeg ? (kend - kbeg + KS - 1) / KS : 0;

  const int li = lane & 15, lq = lane >> 4;
  const int hl = hg * HG + li;                   // head within the KV group
  const bool hvalid = hl < p.group;
  const int hq = kvh * p.group + (hvalid ? hl : 0);

  // Query fragments: lane holds channels 32·lq + 8·cb .. +7 of its head for product cb.
  typename T::vec8 qf[4];
  {
    const u32x4* src = (const u32x4*)(p.q + ((long long)b * p.Hq + hq) * D + 32 * lq);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const u32x4 w = hvalid ? src[cb] : u32x4{0, 0, 0, 0};
      qf[cb] = __builtin_bit_cast(typename T::vec8, w);
    }
  }
  // Block scales of the wave's keys, one block per lane (a wave spans at most 64 blocks).
  const long long sbase = ((long long)b * p.Hkv + kvh) * p.nblk + kbeg / 64;
  const int nbw = nsteps > 0 ? (kend - kbeg + 63) / 64 : 0;
  const float ks_l = lane < nbw ? p.ksc[sbase + lane] : 0.f;
  const float vs_l = lane < nbw ? p.vsc[sbase + lane] : 0.f;
  float vsmax = vs_l;
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) vsmax = fmaxf(vsmax, __shfl_xor(vsmax, off, 64));
  const float lvsmax = __log2f(vsmax);
  wait_vmcnt<0>();   // the loads above are complete before the asm loads are counted

  const long long rowstride = (long long)p.Hkv * D;
  const char* kg = (const char*)(p.k + ((long long)b * p.Nmax * p.Hkv + kvh) * D);
  const char* vg = (const char*)(p.v + ((long long)b * p.Nmax * p.Hkv + kvh) * D);
  const uint32_t ring = (uint32_t)(uintptr_t)lds + wave * RINGB;

  // LDS-DMA of one step: 4 + 4 loads of 1 KB (8 rows each).  Lane i fills physical
  // chunk i%8 of row 8·ii + i/8; rows at or past L repeat row L-1 (finite codes whose
  // probabilities are 0).
  auto issue = [&](int s) {
    const int key0 = kbeg + KS * s;
    const int lim = L - 1 - key0;
    const char* kb = kg + key0 * rowstride;
    const char* vb = vg + key0 * rowstride;
    const uint32_t dst = ring + (s % STAGES) * STEPB;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 8 * ii + (lane >> 3);
      const uint32_t off = (uint32_t)(min(r, lim) * rowstride + 16 * ((lane & 7) ^ swz(r)));
      lds_dma16(kb, off, dst + 1024 * ii);
      lds_dma16(vb, off, dst + HALFB + 1024 * ii);
    }
  };

  // Score reads: key row 8(li/4) + 4·blk + li%4, logical chunks 2·lq and 2·lq + 1.
  int koff[2][2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int r = 8 * (li >> 2) + 4 * blk + (li & 3);
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[blk][u] = r * D + 16 * ((2 * lq + u) ^ swz(r));
  }
  // Transposing V reads: source lane i = 2j + m of group lq gives row 8·lq + j, bytes
  // 16·cblk + 8m .. +7; output lane i then holds V[8·lq + 0..7][16·cblk + i].
  int voff[8];
  {
    const int r = 8 * lq + (li >> 1), m = li & 1;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) voff[cb] = HALFB + r * D + 16 * (cb ^ swz(r)) + 8 * m;
  }

  f32x4_t oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, z = 0.f;

  const int npro = min(STAGES - 1, nsteps);
  for (int s = 0; s < npro; ++s) issue(s);

  for (int j = 0; j < nsteps; ++j) {
    if (nsteps - j >= STAGES - 1)
      wait_vmcnt<8 * (STAGES - 2)>();
    else
      wait_vmcnt<0>();
    // This wave's reads of the stage reused below (step j-1) are complete.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (j + STAGES - 1 < nsteps) issue(j + STAGES - 1);

    const lds_char* st = lds + wave * RINGB + (j % STAGES) * STEPB;
    const int key0 = kbeg + KS * j;
    const int blk = j >> 1;
    const float ks_j = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ks_l), blk));
    const float vs_j = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vs_l), blk));

    // Sᵀ for keys 8·lq + 4·kb + e (kb = 0, 1; e = 0..3) of head li.
    f32x4_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 lo = *(const lds_u32x4*)(st + koff[kb][0]);
      const u32x4 hi = *(const lds_u32x4*)(st + koff[kb][1]);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = T::mma(T::from_e4m3(lo[0], lo[1]), qf[0], acc);
      acc = T::mma(T::from_e4m3(lo[2], lo[3]), qf[1], acc);
      acc = T::mma(T::from_e4m3(hi[0], hi[1]), qf[2], acc);
      acc = T::mma(T::from_e4m3(hi[2], hi[3]), qf[3], acc);
      sacc[kb] = acc;
    }
    const float cj = p.c * ks_j;
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = sacc[i >> 2][i & 3] * cj;
    if (key0 + KS > L) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (key0 + 8 * lq + i >= L) t[i] = -INFINITY;
    }
    float mx = t[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = __builtin_fmaxf(mx, t[i]);
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kSlack) != 0) {
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = __builtin_fmaxf(m_ref, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      z *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) oacc[i] *= alpha;
    }
    // p̃ = round16(2^(t - m) · sv/max sv); the denominator gets Σ p̃ · max sv/sv.
    const float lfv = __log2f(vs_j) - lvsmax;
    const float neg = lfv - m_ref;
    float pe[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pe[i] = fast_exp2(t[i] + neg);
    const typename T::vec8 pf = T::pack8(pe);
    z = fmaf(T::sum8(pf, 0.f), fast_exp2(-lfv), z);

#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(st + voff[cb]));
      oacc[cb] = T::mma(T::from_e4m3((uint32_t)w[0], (uint32_t)w[1]), pf, oacc[cb]);
    }
  }
  wait_vmcnt<0>();

  // Per head: the wave's denominator (sum over the four lane groups) and O·max sv.
  z += __shfl_xor(z, 16, 64);
  z += __shfl_xor(z, 32, 64);

  // Merge the four waves' partials in LDS (each wave writes into its own ring).  O is
  // kept as 16-byte units [channel block cb][lane group lq][head] (channels 16cb + 4lq
  // .. +3 of a head per unit), so that the 16 lanes of a store, and of a load below,
  // touch 16 distinct bank windows.
  float* mine = (float*)(smem + wave * RINGB);
  if (lq == 0) {
    mine[li] = m_ref;
    mine[HG + li] = z;
  }
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    f32x4_t w = oacc[cb] * vsmax;
    *(f32x4_t*)(mine + 2 * HG + 4 * ((4 * cb + lq) * HG + li)) = w;
  }
  __syncthreads();
  {
    // thread: head h, channels 8k .. 8k + 7 (units (cb, lq) = (k/2, 2(k%2)) and (k/2, 2(k%2) + 1))
    const int h = tid & 15, k = tid >> 4, ch = 8 * k;
    const int u0 = (4 * (k >> 1) + 2 * (k & 1)) * HG + h;
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = ((const float*)(smem + w * RINGB))[h];
      M = __builtin_fmaxf(M, mw[w]);
    }
    f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    float zt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* src = (const float*)(smem + w * RINGB);
      const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
      zt = fmaf(src[HG + h], f, zt);
      o0 += *(const f32x4_t*)(src + 2 * HG + 4 * u0) * f;
      o1 += *(const f32x4_t*)(src + 2 * HG + 4 * (u0 + HG)) * f;
    }
    const int hh = hg * HG + h;
    if (hh < p.group) {
      const long long bh = (long long)b * p.Hq + kvh * p.group + hh;
      if (p.nc == 1) {
        // The chunk is the whole sequence: this is the final result and no merge runs.
        const float den = zt > 0.f ? zt : 1.f;
        u32x4 w;
        w[0] = T::pack(o0[0] / den, o0[1] / den);
        w[1] = T::pack(o0[2] / den, o0[3] / den);
        w[2] = T::pack(o1[0] / den, o1[1] / den);
        w[3] = T::pack(o1[2] / den, o1[3] / den);
        *(u32x4*)(p.o + bh * D + ch) = w;
        if (k == 0 && p.lse != nullptr) p.lse[bh] = zt > 0.f ? (M + __log2f(zt)) * kLn2 : -INFINITY;
      } else {
        const long long row = bh * p.nc + ci;
        *(f32x4_t*)(p.ws_o + row * D + ch) = o0;
        *(f32x4_t*)(p.ws_o + row * D + ch + 4) = o1;
        if (k == 0) {
          p.ws_ml[2 * row] = M;
          p.ws_ml[2 * row + 1] = zt;
        }
      }
    }
  }
}

constexpr int kMergeBatch = 8;           // partials loaded before they are folded
constexpr int kWideMergeBelow = 256;     // fewer (b, head) merges than this: 8 groups each, else 4

// kMergeGroups groups of D threads fold chunk partials in parallel per (b, head).
template <typename T, int kMergeGroups>
__global__ __launch_bounds__(D * kMergeGroups) void attn_decode_merge_kernel(DecParams p) {
  __shared__ float red[kMergeGroups][D + 2];
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x % D, grp = threadIdx.x / D;
  const int L = seq_len(p, b);
  const int ncb = (L + p.chunk - 1) / p.chunk;
  const long long row0 = ((long long)b * p.Hq + hq) * p.nc;
  // Group grp folds partials grp, grp + G, grp + 2G, ...; the loads of a batch are
  // all issued before the first is used.
  float M = -INFINITY, Z = 0.f, O = 0.f;
  for (int i0 = grp; i0 < ncb; i0 += kMergeGroups * kMergeBatch) {
    float mi[kMergeBatch], zi[kMergeBatch], oi[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int i = min(i0 + u * kMergeGroups, ncb - 1);
      mi[u] = p.ws_ml[2 * (row0 + i)];
      zi[u] = p.ws_ml[2 * (row0 + i) + 1];
      oi[u] = p.ws_o[(row0 + i) * D + c];
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (i0 + u * kMergeGroups >= ncb) break;
      const float Mn = __builtin_fmaxf(M, mi[u]);
      const float a = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
      const float f = mi[u] == -INFINITY ? 0.f : fast_exp2(mi[u] - Mn);
      O = O * a + oi[u] * f;
      Z = Z * a + zi[u] * f;
      M = Mn;
    }
  }
  red[grp][c] = O;
  if (c == 0) {
    red[grp][D] = M;
    red[grp][D + 1] = Z;
  }
  __syncthreads();
  if (grp != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int g = 0; g < kMergeGroups; ++g) Mt = __builtin_fmaxf(Mt, red[g][D]);
  float Ot = 0.f, Zt = 0.f;
#pragma unroll
  for (int g = 0; g < kMergeGroups; ++g) {
    const float f = red[g][D] == -INFINITY ? 0.f : fast_exp2(red[g][D] - Mt);
    Ot = fmaf(red[g][c], f, Ot);
    Zt = fmaf(red[g][D + 1], f, Zt);
  }
  p.o[((long long)b * p.Hq + hq) * D + c] = T::from_f32(Zt > 0.f ? Ot / Zt : 0.f);
  if (c == 0 && p.lse != nullptr) p.lse[(long long)b * p.Hq + hq] = Zt > 0.f ? (Mt + __log2f(Zt)) * kLn2 : -INFINITY;
}

}  // namespace

DecodePlan plan_decode(int B, int Nmax, int Hq, int Hkv) {
  DecodePlan pl;
  const int group = Hq / Hkv;
  pl.nhg = (group + HG - 1) / HG;
  const long long pairs = (long long)B * Hkv * pl.nhg;
  // Aim for kTargetItems workgroups; when that makes chunks shorter than kLongChunk keys
  // (a few long sequences), lengthen them toward kLongChunk as long as kMinItems
  // workgroups remain: short workgroups spend much of their time filling the ring.
  const long long work = pairs * Nmax;
  long long chunk = (work + kTargetItems - 1) / kTargetItems;
  if (chunk < kLongChunk) chunk = std::max(chunk, std::min<long long>(kLongChunk, (work + kMinItems - 1) / kMinItems));
  chunk = (chunk + kMinChunk - 1) / kMinChunk * kMinChunk;
  chunk = chunk < kMinChunk ? kMinChunk : (chunk > kMaxChunk ? kMaxChunk : chunk);
  pl.chunk = (int)chunk;
  pl.nc = (Nmax + pl.chunk - 1) / pl.chunk;
  pl.ws_o_floats = (long long)B * Hq * pl.nc * D;
  pl.ws_bytes = (size_t)(pl.ws_o_floats + (long long)B * Hq * pl.nc * 2) * sizeof(float);
  return pl;
}

namespace {
template <typename T>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const DecodePlan pl = plan_decode(a.B, a.Nmax, a.Hq, a.Hkv);
  DecParams p;
  p.q = (const uint16_t*)a.q;
  p.k = a.k;
  p.v = a.v;
  p.ksc = a.k_scale;
  p.vsc = a.v_scale;
  p.seqlens = a.seqlens;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.ws_o = (float*)a.workspace;
  p.ws_ml = p.ws_o + pl.ws_o_floats;
  p.Nmax = a.Nmax;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.nhg = pl.nhg;
  p.nblk = (a.Nmax + 63) / 64;
  p.nc = pl.nc;
  p.chunk = pl.chunk;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  const dim3 grid((unsigned)pl.nc, (unsigned)(a.Hkv * pl.nhg), (unsigned)a.B);
  const long long wgs = (long long)pl.nc * a.Hkv * pl.nhg * a.B;
  if (pl.nc <= 2 || wgs <= 2LL * device_cu_count())   // short sequences, or few workgroups
    hipLaunchKernelGGL((attn_decode_split_kernel<T, 2, 2>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_decode_split_kernel<T, 4, 1>), grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nc == 1) return e;   // one chunk per sequence: the split kernel wrote O
  if ((long long)a.Hq * a.B < kWideMergeBelow)
    hipLaunchKernelGGL((attn_decode_merge_kernel<T, 8>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(D * 8), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_decode_merge_kernel<T, 4>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(D * 4), 0, stream, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == TATTN_BF16 ? launch_decode_t<DecBf16>(a, stream) : launch_decode_t<DecF16>(a, stream);
}

}  // namespace tattn

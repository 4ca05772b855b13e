// FP8 (OCP E4M3FN) attention forward for gfx950 (CDNA4), head dim 128.
//
// Same work decomposition, staging and ping-pong schedule as the 16-bit kernel
// (8 waves x 32 query rows, 64-key tiles, four-stage LDS-DMA rings for K and V,
// one barrier per tile), with both products on the fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales, fp32 accumulation):
//
//   Sᵀ = K8·Q8ᵀ     A = K rows (32 bytes per lane: two 16-byte LDS reads),
//                   B = Q8 rows held in VGPRs.
//   scores          s = Sᵀ · sq(row block) · sk(tile) · scale·log2(e): per-block
//                   scales ([FA3-V3] §4.3) applied in fp32; a 64-key tile is
//                   exactly one K/V scale block.
//   softmax         online, fp32 ([FA3-V3] §4.2); the running max is exact
//                   (rescale whenever a row max grows).
//   Oᵀ += V8ᵀ·P̃ᵀ    P̃ = e4m3(p · sv(tile)·2^8/max(sv)): the V block scale and a
//                   2^8 headroom are folded into the exponent bias, so p̃ <= 256
//                   and small probabilities keep E4M3's precision; the denominator
//                   accumulates the unrounded fp32 p.  A = Vᵀ gathered by
//                   byte-transposing LDS reads (ds_read_b64_tr_b8, 4 per MFMA).
// Epilogue: O = acc · max(sv)·2^-8 / z, rounded to the output type.
#include <type_traits>

#include "tattn_device.hpp"
#include "tattn_pipeline.hpp"
#include "tattn_launch.hpp"
#include "tattn.h"

namespace tattn {
namespace {

constexpr int NW = 8;
constexpr int kThreads = 64 * NW;
constexpr int BM = 32 * NW;
constexpr int BN = 64;                   // keys per tile = rows per scale block
constexpr int STAGES = 4;
constexpr int D = 128;
constexpr int ROWB = D;                  // bytes per fp8 row
constexpr int TILEB = BN * ROWB;         // 8 KB
constexpr int LDSB = 2 * STAGES * TILEB; // K ring + V ring
constexpr float kHeadroomLog2 = 8.0f;
constexpr int kMaxBlocks = 4096;         // scale blocks per head staged in LDS (N <= 262144)

// Physical 16-byte chunk = logical chunk ^ swz(row) (rows of 128 bytes).
__device__ inline int swz(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 3) << 1) | (x >> 2);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

__device__ inline f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // operand formats 0/0 = E4M3; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ inline i32x8 cat(i32x4 lo, i32x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* qsc;
  const float* ksc;
  const float* vsc;
  uint16_t* o;
  float* lse;
  int N, Hq, Hkv, group, nqt, nblk;
  float c;  // softmax scale · log2(e)
};

template <typename OutT, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_fp8_kernel(Fp8Params p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDSB];
  __shared__ float red[NW];
  __shared__ float sk_lds[kMaxBlocks], sv_lds[kMaxBlocks];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int Gn = gridDim.x;
  const int g = blockIdx.x;
  const int wi = (Gn % 8 == 0) ? (g % 8) * (Gn / 8) + g / 8 : g;
  int qt = wi % p.nqt;
  if (CAUSAL) qt = p.nqt - 1 - qt;
  const int rest = wi / p.nqt;
  const int hq = rest % p.Hq;
  const int b = rest / p.Hq;
  const int hkv = hq / p.group;
  const int N = p.N;

  const long long qstride = (long long)p.Hq * D;   // bytes between positions
  const long long kvrow = (long long)p.Hkv * D;
  const uint8_t* qb = p.q + ((long long)b * N * p.Hq + hq) * D;
  const char* kg = (const char*)(p.k + ((long long)b * N * p.Hkv + hkv) * D);
  const char* vg = (const char*)(p.v + ((long long)b * N * p.Hkv + hkv) * D);
  const float* ksc = p.ksc + ((long long)b * p.Hkv + hkv) * p.nblk;
  const float* vsc = p.vsc + ((long long)b * p.Hkv + hkv) * p.nblk;

  const int q0 = qt * BM;
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + l32;
  const int qr = min(qrow, N - 1);

  // Q fragments: lane holds Q8[qrow][64t + 32hh .. +31] for k-step t.
  i32x8 qf[2];
  {
    const uint8_t* src = qb + qr * qstride + 32 * hh;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      qf[t] = cat(*(const i32x4*)(src + 64 * t), *(const i32x4*)(src + 64 * t + 16));
  }
  const float sq = p.qsc[((long long)b * p.Hq + hq) * p.nblk + qr / BN];

  // Stage this head's K and V block scales in LDS (the loop then reads them with
  // LDS loads, which do not wait on the K/V prefetch) and take the largest V scale.
  float vmax = 0.f;
  for (int i = tid; i < p.nblk; i += kThreads) {
    const float sv = vsc[i];
    sk_lds[i] = ksc[i];
    sv_lds[i] = sv;
    vmax = fmaxf(vmax, sv);
  }
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
  if (lane == 0) red[wave] = vmax;
  __syncthreads();
  vmax = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) vmax = fmaxf(vmax, red[w]);

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;
  const int wend = (wq0 >= N) ? 0 : (CAUSAL ? min(kv_end, wq0 + 32) : kv_end);
  const int ntw = (wend + BN - 1) / BN;

  // LDS-DMA: one 1 KB load per wave per tile = rows 8·wave .. 8·wave+7.
  const int ld_row = 8 * wave + (lane >> 3);
  const int ld_col = 16 * ((lane & 7) ^ swz(ld_row));
  const uint32_t ld_off = (uint32_t)(ld_row * kvrow + ld_col);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  auto issue = [&](int ring, int stage, int t) {
    const int j0 = t * BN;
    const char* base = (ring ? vg : kg) + (long long)j0 * kvrow;
    uint32_t off = ld_off;
    if (j0 + BN > N) off = (uint32_t)((min(j0 + ld_row, N - 1) - j0) * kvrow + ld_col);   // rows past N repeat row N-1
    lds_dma16(base, off, lds_base + (ring * STAGES + stage) * TILEB + 1024 * wave);
  };

  // K reads: row kr = perm23(l32) (+32 per key block), 16-byte chunks 4t + 2hh + u.
  int koff[2][2];
  {
    const int kr = perm23(l32);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) koff[t][u] = kr * ROWB + 16 * ((4 * t + 2 * hh + u) ^ swz(kr));
  }
  // V byte-transposing reads: in each 16-lane group, source lane i = 2j + m supplies
  // V[16r + 8hh + j][dv0 + 8m .. +7] with dv0 = 32vq + 16(grp%2); output lane i then
  // holds V[16r + 8hh + 0..7][dv0 + i].
  int voff[D / 32];
  {
    const int grp = lane >> 4, i = lane & 15, j = i >> 1, m = i & 1;
    const int key = 8 * hh + j;                          // + 16r (swz depends on key % 16 only)
#pragma unroll
    for (int vq = 0; vq < D / 32; ++vq) {
      const int chunk = 2 * vq + (grp & 1);
      voff[vq] = STAGES * TILEB + key * ROWB + 16 * (chunk ^ swz(key)) + 8 * m;
    }
  }

  auto scores = [&](const int stage, f32x16 (&s)[2]) {
    const lds_char* ks = lds + stage * TILEB;
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const i32x8 a = cat(*(const lds_i32x4*)(ks + koff[t][0] + kq * 32 * ROWB),
                            *(const lds_i32x4*)(ks + koff[t][1] + kq * 32 * ROWB));
        s[kq] = mfma_fp8(a, qf[t], t == 0 ? f32x16{} : s[kq]);
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float cq = p.c * sq;
  const bool lead = wave < NW / 2;

#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t)
    if (t < nt) { issue(0, t, t); issue(1, t, t); }
  wait_vmcnt<0>();
  barrier();

  f32x16 scur[2];
  if (lead && ntw > 0) scores(0, scur);

  auto step = [&](auto stc, auto leadc, int j) {
    constexpr int st = decltype(stc)::value;
    constexpr int stn = (st + 1) % STAGES;
    constexpr bool is_lead = decltype(leadc)::value;
    if (j + 2 < nt) wait_vmcnt<2>();
    else wait_vmcnt<0>();
    barrier();
    if (j + 3 < nt) {
      issue(0, (st + 3) % STAGES, j + 3);
      issue(1, (st + 3) % STAGES, j + 3);
    }
    if (j >= ntw) return;

    i32x8 pf;
    auto softmax = [&]() {
      const int j0 = j * BN;
      const float cj = cq * sk_lds[j];
      const float bias = __log2f(sv_lds[j] / vmax) + kHeadroomLog2;
      if ((j0 + BN > N) || (CAUSAL && j0 + BN - 1 > wq0)) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * kq + 16 * (i >> 3) + 8 * hh + (i & 7);
            if (key >= N || (CAUSAL && key > qrow)) scur[kq][i] = -INFINITY;
          }
      }
      float mt = scur[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = __builtin_fmaxf(mt, scur[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = __builtin_fmaxf(mt, scur[1][i]);
      mt = __builtin_fmaxf(mt, xor32(mt));
      const float m_cand = mt * cj;
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run) != 0) {
        const float m_new = __builtin_fmaxf(m_run, m_cand);
        const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int vq = 0; vq < D / 32; ++vq)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[vq][i] *= alpha;
      }
      const float neg = bias - ((m_run == -INFINITY) ? 0.f : m_run);
      float pe[32];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int i = 0; i < 16; ++i) pe[16 * kq + i] = fast_exp2(fmaf(scur[kq][i], cj, neg));
      float ps[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i] = pe[2 * i] + pe[2 * i + 1];
#pragma unroll
      for (int w = 8; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) ps[i] = ps[i] + ps[i + w];
      l_run += ps[0] * fast_exp2(-bias);
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w], pe[4 * w + 1], 0, false);
        pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w + 2], pe[4 * w + 3], word, true);
      }
    };
    auto pv = [&]() {
      const lds_char* vs = lds + st * TILEB;   // voff carries the V ring base
#pragma unroll
      for (int vq = 0; vq < D / 32; ++vq) {
        const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq]));
        const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq] + 16 * ROWB));
        const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq] + 32 * ROWB));
        const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq] + 48 * ROWB));
        const i32x8 a = cat(__builtin_shufflevector(r0, r1, 0, 1, 2, 3), __builtin_shufflevector(r2, r3, 0, 1, 2, 3));
        oacc[vq] = mfma_fp8(a, pf, oacc[vq]);
      }
    };
    if constexpr (is_lead) {
      softmax();
      __builtin_amdgcn_sched_barrier(0);
      pv();
      __builtin_amdgcn_sched_barrier(0);
      scores(stn, scur);
    } else {
      scores(st, scur);
      __builtin_amdgcn_sched_barrier(0);
      softmax();
      __builtin_amdgcn_sched_barrier(0);
      pv();
    }
  };
  auto run = [&](auto leadc) {
    for (int j = 0; j < nt; j += STAGES) {
      step(std::integral_constant<int, 0>{}, leadc, j);
      if (j + 1 < nt) step(std::integral_constant<int, 1>{}, leadc, j + 1);
      if (j + 2 < nt) step(std::integral_constant<int, 2>{}, leadc, j + 2);
      if (j + 3 < nt) step(std::integral_constant<int, 3>{}, leadc, j + 3);
    }
  };
  if (lead) run(std::true_type{});
  else run(std::false_type{});

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? vmax * 0.00390625f / l_tot : 0.f;   // max(sv)·2^-8 / z
  // The rings are free once every wave has left the loop; each wave stages its rows in 8 KB.
  __syncthreads();
  store_rows<OutT>(lds + wave * 8192, oacc, inv, lane, p.o + ((long long)b * N * p.Hq + hq) * D + wq0 * qstride,
                   qstride, N - wq0);
  if (qrow < N && p.lse != nullptr && hh == 0)
    p.lse[((long long)b * p.Hq + hq) * N + qrow] =
        l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <typename OutT, bool CAUSAL>
hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
  Fp8Params p;
  p.q = (const uint8_t*)a.q;
  p.k = (const uint8_t*)a.k;
  p.v = (const uint8_t*)a.v;
  p.qsc = a.q_scale;
  p.ksc = a.k_scale;
  p.vsc = a.v_scale;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.nqt = (a.N + BM - 1) / BM;
  p.nblk = (a.N + BN - 1) / BN;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  const long long grid = (long long)p.nqt * a.Hq * a.B;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<OutT, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const AttnArgs& a, hipStream_t stream) {
  if (a.dtype == TATTN_BF16)
    return a.causal ? launch_one<Bf16, true>(a, stream) : launch_one<Bf16, false>(a, stream);
  return a.causal ? launch_one<F16, true>(a, stream) : launch_one<F16, false>(a, stream);
}

}  // namespace tattn

// Fused attention forward, fp16/bf16, for gfx950 (CDNA4).
//
// One workgroup = 4 waves = BM = 128 query rows of one (batch, head); each wave
// owns 32 rows.  The K/V sequence is walked in tiles of BN = 64 keys, staged
// global -> registers -> LDS in two buffers: tile j+1's loads are issued
// before tile j is computed and written to the other buffer afterwards, so one
// barrier per tile covers both the read-after-write and the write-after-read
// hazard ([FA3-tile] §二's double buffer, with both of its synchronisations).
//
// Per tile and wave, on the 32x32x16 matrix cores:
//   Sᵀ = K·Qᵀ   (A = K rows from LDS, B = the wave's Q rows held in VGPRs for
//                the whole loop).  The accumulator then holds, in lane l,
//                32 scores of query row l%32 -- the row statistics are lane-
//                local apart from one exchange with lane l^32.
//   online softmax in fp32 ([FA3-V3] §4.2): m' = max(m, rowmax), α = 2^(m−m'),
//                p = 2^(s·c − m') with c = scale·log2(e), z' = α·z + Σp.
//   Oᵀ += Vᵀ·Pᵀ (A = Vᵀ from LDS, B = P rounded to the input type).  The
//                score accumulator's register layout is exactly the B-operand
//                layout once Vᵀ's key positions are permuted (bits 2 and 3 of
//                the key index swapped), so P needs no shuffle ([FA3-V3] §7.4's
//                accumulator-to-operand problem, solved by operand order).
// The epilogue divides by z (deferred normalisation, [FA3-V3] §11) and writes
// O and optionally the log-sum-exp.
#include "tattn_device.hpp"
#include "tattn_launch.hpp"
#include "tattn.h"

namespace tattn {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 64;

template <int D>
struct Layout {
  static constexpr int KS = D + 8;    // K row stride in elements (16 B pad)
  static constexpr int VS = BN + 8;   // Vᵀ row stride in elements (16 B pad)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int KPT = D / 32;          // keys per thread in the V staging
  static constexpr int KGROUPS = BN / KPT;    // key groups per tile
  static constexpr int CHUNKS = D / 8;        // 16-byte chunks per row
};

// Position of key kk (0..63) inside a Vᵀ row: bits 2 and 3 swapped.
__device__ inline int vt_pos(int kk) { return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1); }

struct KernelParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N, Hq, Hkv, group, nqt;
  float c;  // scale · log2(e)
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd16_kernel(KernelParams p) {
  using L = Layout<D>;
  using vec8 = typename T::vec8;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // Work item: consecutive items go to one XCD (workgroups are dealt to the
  // 8 XCDs round-robin), ordered (batch, head, q tile) so that the heads of a
  // KV group and all q tiles of a head run close together and share L2.
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int wi = (G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
  int qt = wi % p.nqt;
  if (CAUSAL) qt = p.nqt - 1 - qt;   // longest rows first
  const int rest = wi / p.nqt;
  const int hq = rest % p.Hq;
  const int b = rest / p.Hq;
  const int hkv = hq / p.group;
  const int N = p.N;

  const long long qs = (long long)p.Hq * D;    // elements between positions
  const long long kvs = (long long)p.Hkv * D;
  const uint16_t* qb = p.q + ((long long)b * N * p.Hq + hq) * D;
  const uint16_t* kb = p.k + ((long long)b * N * p.Hkv + hkv) * D;
  const uint16_t* vb = p.v + ((long long)b * N * p.Hkv + hkv) * D;

  const int q0 = qt * BM;
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + l32;

  // Q fragments (B operand): lane holds Q[qrow][16t + 8hh .. +7].
  vec8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qrow < N) raw = *(const u32x4*)(qb + qrow * qs + 16 * t + 8 * hh);
    qf[t] = __builtin_bit_cast(vec8, raw);
  }

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  // Staging registers for one K tile and one V tile.
  u32x4 kst[D / 32], vst[L::KPT];
  const int vkg = tid % L::KGROUPS, vc = tid / L::KGROUPS;

  auto load_tile = [&](int j) {
    const int j0 = j * BN;
#pragma unroll
    for (int r = 0; r < D / 32; ++r) {
      const int ci = tid + kThreads * r;
      const int row = ci / L::CHUNKS, c = ci % L::CHUNKS;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (j0 + row < N) raw = *(const u32x4*)(kb + (j0 + row) * kvs + 8 * c);
      kst[r] = raw;
    }
#pragma unroll
    for (int e = 0; e < L::KPT; ++e) {
      const int key = j0 + vkg * L::KPT + e;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (key < N) raw = *(const u32x4*)(vb + key * kvs + 8 * vc);
      vst[e] = raw;
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * L::STAGE;
    uint16_t* vts = ks + L::K_ELEMS;
#pragma unroll
    for (int r = 0; r < D / 32; ++r) {
      const int ci = tid + kThreads * r;
      const int row = ci / L::CHUNKS, c = ci % L::CHUNKS;
      *(u32x4*)(ks + row * L::KS + 8 * c) = kst[r];
    }
    // Vᵀ: element x of this thread's 8 channels, for its KPT keys.
    const int pos = vt_pos(vkg * L::KPT);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      uint32_t w[L::KPT / 2];
#pragma unroll
      for (int e2 = 0; e2 < L::KPT / 2; ++e2) {
        const uint32_t a = vst[2 * e2][x / 2], c = vst[2 * e2 + 1][x / 2];
        w[e2] = (x & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      uint16_t* dst = vts + (8 * vc + x) * L::VS + pos;
      if constexpr (L::KPT == 4) {
        *(u32x2*)dst = u32x2{w[0], w[1]};
      } else {
        *(uint32_t*)dst = w[0];
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) load_tile(j + 1);
    const int j0 = j * BN;
    const uint16_t* ks = smem + (j & 1) * L::STAGE;
    const uint16_t* vts = ks + L::K_ELEMS;

    if (!(CAUSAL && j0 > wq0 + 31)) {   // wave-uniform: skip fully masked tiles
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const vec8 a = *(const vec8*)(ks + (32 * kq + l32) * L::KS + 16 * t + 8 * hh);
          sacc[kq] = T::mfma(a, qf[t], sacc[kq]);
        }
      }
      const bool need_mask = (j0 + BN > N) || (CAUSAL && j0 + BN - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * kq + 8 * (i / 4) + 4 * hh + (i % 4);
            if (key >= N || (CAUSAL && key > qrow)) sacc[kq][i] = -INFINITY;
          }
      }
      float mt = sacc[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sacc[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[1][i]);
      mt = fmaxf(mt, xor32(mt));
      const float m_new = fmaxf(m_run, mt * c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = fast_exp2(fmaf(sacc[kq][i], c, -m_use));
          sacc[kq][i] = pv;
          psum += pv;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int vq = 0; vq < D / 32; ++vq)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[vq][i] *= alpha;

#pragma unroll
      for (int s = 0; s < BN / 16; ++s) {
        u32x4 pw;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pw[e] = pack2<T>(sacc[s / 2][8 * (s % 2) + 2 * e], sacc[s / 2][8 * (s % 2) + 2 * e + 1]);
        const vec8 bfrag = __builtin_bit_cast(vec8, pw);
#pragma unroll
        for (int vq = 0; vq < D / 32; ++vq) {
          const vec8 a = *(const vec8*)(vts + (32 * vq + l32) * L::VS + 16 * s + 8 * hh);
          oacc[vq] = T::mfma(a, bfrag, oacc[vq]);
        }
      }
    }

    if (j + 1 < ntiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + xor32(l_run);
  if (qrow < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = p.o + ((long long)b * N * p.Hq + hq) * D + qrow * qs;
#pragma unroll
    for (int vq = 0; vq < D / 32; ++vq)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w;
        w[0] = pack2<T>(oacc[vq][4 * a + 0] * inv, oacc[vq][4 * a + 1] * inv);
        w[1] = pack2<T>(oacc[vq][4 * a + 2] * inv, oacc[vq][4 * a + 3] * inv);
        *(u32x2*)(orow + 32 * vq + 8 * a + 4 * hh) = w;
      }
    if (p.lse != nullptr && hh == 0)
      p.lse[((long long)b * p.Hq + hq) * N + qrow] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
  KernelParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.nqt = (a.N + BM - 1) / BM;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  const long long grid = (long long)p.nqt * a.Hq * a.B;
  hipLaunchKernelGGL((attn_fwd16_kernel<T, D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  if (a.d == 128) return a.causal ? launch_one<T, 128, true>(a, s) : launch_one<T, 128, false>(a, s);
  return a.causal ? launch_one<T, 64, true>(a, s) : launch_one<T, 64, false>(a, s);
}

}  // namespace

hipError_t launch_attn_fwd16(const AttnArgs& a, hipStream_t stream) {
  return a.dtype == TATTN_BF16 ? launch_t<Bf16>(a, stream) : launch_t<F16>(a, stream);
}

}  // namespace tattn

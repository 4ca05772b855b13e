// Fused attention forward, fp16/bf16, for gfx950 (CDNA4).
//
// Work decomposition.  One workgroup = 8 waves = BM = 256 query rows of one
// (batch, head); each wave owns 32 rows and keeps its Q rows in VGPRs for the
// whole sequence.  The K/V sequence is walked in tiles of BN = 64 keys.  Work
// items are ordered (batch, head, q tile) and dealt so that consecutive items
// land on one XCD, which keeps the heads of a KV group (and all q tiles of a
// head) on one L2.  Causal launches take the longest rows first.
//
// Staging ([FA3-tile] §二's double buffer, generalised to three stages).  K and
// V tiles go global -> LDS directly (16-byte LDS-DMA loads, no VGPR staging)
// into three-stage rings.  While tile j is consumed, the loads for K(j+3) and
// V(j+2) are in flight; one barrier per tile both publishes the finished loads
// (read after write) and retires the stages about to be overwritten (write
// after read).  LDS rows are unpadded and their 16-byte chunks are XOR-
// swizzled per row so that the K reads and the transposing V reads are free
// of bank conflicts.
//
// Per tile and wave, on the 32x32x16 matrix cores:
//   Sᵀ = K·Qᵀ   A = K rows from LDS (rows taken in an order that swaps bits 2
//                and 3 of the row index), B = Q.  Lane l then holds 32 scores
//                of query row l%32: row statistics are lane-local apart from
//                one exchange with lane l^32.
//   softmax     online, fp32 ([FA3-V3] §4.2): m' = max(m, rowmax), α = 2^(m−m'),
//                p = 2^(s·c − m') with c = scale·log2(e), z' = α·z + Σp.  The
//                reference max only moves when a row max grew by more than
//                kRescaleSlack, which skips the O rescale on almost every tile;
//                O/z is unchanged in exact arithmetic.
//   Oᵀ += Vᵀ·Pᵀ A = Vᵀ gathered by transposing LDS reads (ds_read_b64_tr_b16),
//                B = P rounded to the input type.  Thanks to the K row order
//                above, the score accumulator already is the B operand, so P
//                needs no shuffle ([FA3-V3] §7.4's accumulator-to-operand
//                problem, solved by operand order).
// The loop is software-pipelined ([FA3-V3] §7.3's intra-warpgroup overlap):
// tile j+1's score MFMAs are issued in the same basic block as tile j's
// exponentials and P·V MFMAs, so matrix-core and VALU work of one wave
// overlap; two waves per SIMD add overlap across waves.
// The epilogue divides by z (deferred normalisation, [FA3-V3] §11) and writes
// O and optionally the log-sum-exp.
#include "tattn_device.hpp"
#include "tattn_launch.hpp"
#include "tattn.h"

namespace tattn {
namespace {

constexpr int NW = 8;                // waves per workgroup
constexpr int kThreads = 64 * NW;
constexpr int BM = 32 * NW;          // query rows per workgroup
constexpr int BN = 64;               // keys per tile
constexpr int STAGES = 3;

#ifndef TATTN_RESCALE_SLACK
#define TATTN_RESCALE_SLACK 8.0f
#endif
constexpr float kRescaleSlack = TATTN_RESCALE_SLACK;

template <int D>
struct Geo {
  static constexpr int ROWB = 2 * D;                    // bytes per K/V row
  static constexpr int TILEB = BN * ROWB;               // bytes per tile
  static constexpr int LDSB = 2 * STAGES * TILEB;       // K ring + V ring
  static constexpr int LOADS = TILEB / (1024 * NW);     // 1 KB DMA loads per wave per tile
  static_assert(LOADS >= 1 && TILEB % (1024 * NW) == 0, "tile must split into 1 KB loads");
  // Physical 16-byte chunk = logical chunk ^ swz(row).
  __device__ static inline int swz(int r) {
    if constexpr (D == 128) {
      return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
    } else {
      const int x = (r >> 1) & 7;
      return ((x & 3) << 1) | (x >> 2);
    }
  }
};

// Row order of the score MFMA's A operand: bits 2 and 3 swapped.
__device__ inline int perm23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte LDS-DMA load per lane: lane i's 16 bytes from ``src`` land at LDS
// byte address ``lds_addr`` + 16·i.  Issued as inline assembly so that the
// compiler neither treats it as an aliasing LDS store (which would make it wait
// for the load before every later LDS read) nor counts it: the loop below waits
// for these loads explicitly with wait_vmcnt before each barrier.  M0 is only
// written here and consumed by the next instruction.
__device__ inline void lds_dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
               : "memory");
}

// Workgroup barrier without a memory fence: the LDS-DMA loads are published by
// the explicit wait_vmcnt before it; the asm also keeps the compiler from
// moving LDS accesses across it.
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

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
__global__ __launch_bounds__(kThreads, 2) void attn_fwd16_kernel(KernelParams p) {
  using G = Geo<D>;
  using vec8 = typename T::vec8;
  typedef __attribute__((address_space(3))) vec8 lds_vec8;
  constexpr int LOADS = G::LOADS;
  __shared__ __attribute__((aligned(1024))) char smem[G::LDSB];
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

  const long long qs = (long long)p.Hq * D;           // elements between positions
  const long long kvrow = (long long)p.Hkv * D * 2;   // bytes between key positions
  const uint16_t* qb = p.q + ((long long)b * N * p.Hq + hq) * D;
  const char* kg = (const char*)(p.k + ((long long)b * N * p.Hkv + hkv) * D);
  const char* vg = (const char*)(p.v + ((long long)b * N * p.Hkv + hkv) * D);

  const int q0 = qt * BM;
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + l32;

  // Q fragments (B operand of the score MFMA): lane holds Q[qrow][16t+8hh .. +7].
  vec8 qf[D / 16];
  {
    const uint16_t* qr = qb + (long long)min(qrow, N - 1) * qs + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = __builtin_bit_cast(vec8, *(const u32x4*)(qr + 16 * t));
  }

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;                    // tiles of the workgroup
  const int wend = (wq0 >= N) ? 0 : (CAUSAL ? min(kv_end, wq0 + 32) : kv_end);
  const int ntw = (wend + BN - 1) / BN;                     // tiles this wave computes

  // LDS-DMA geometry: load n of this wave covers tile bytes [1024(wave·LOADS+n), +1024);
  // lane writes 16 bytes at +16·lane, i.e. row r, physical chunk pc = logical chunk pc^swz(r).
  int ld_row[LOADS], ld_col[LOADS];
#pragma unroll
  for (int n = 0; n < LOADS; ++n) {
    const int o = 1024 * (wave * LOADS + n) + 16 * lane;
    const int r = o / G::ROWB, pc = (o % G::ROWB) / 16;
    ld_row[n] = r;
    ld_col[n] = 16 * (pc ^ G::swz(r));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  auto issue = [&](const char* gbase, int ring, int stage, int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int row = min(j0 + ld_row[n], N - 1);   // rows past N repeat row N-1 (their p is 0)
      lds_dma16(gbase + row * kvrow + ld_col[n],
                lds_base + (ring * STAGES + stage) * G::TILEB + 1024 * (wave * LOADS + n));
    }
  };

  // Per-lane LDS read offsets within a stage.
  //  K (score A operand): row kr = perm23(l32) (+32 per key block), chunk 2t+hh.
  int koff[D / 16];
  {
    const int kr = perm23(l32);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) koff[t] = kr * G::ROWB + 16 * ((2 * t + hh) ^ G::swz(kr));
  }
  //  V (transposing reads): in each 16-lane group, source lane i = 4e + m supplies
  //  V[key][dv .. dv+3] with key = 16s + 8hh + 4·half + e and dv = 32vq + 16(grp%2) + 4m;
  //  the group's output lane i then holds V[16s + 8hh + 4·half + 0..3][dv0 + i].
  int voff[2][D / 32];
  {
    const int grp = lane >> 4, i = lane & 15, e = i >> 2, m = i & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int vq = 0; vq < D / 32; ++vq) {
        const int key = 8 * hh + 4 * half + e;              // + 16s (swz depends on key % 16 only)
        const int dv = 32 * vq + 16 * (grp & 1) + 4 * m;
        voff[half][vq] = key * G::ROWB + 16 * ((dv >> 3) ^ G::swz(key)) + 8 * ((dv >> 2) & 1);
      }
  }

  auto scores = [&](int stage, f32x16 (&s)[2]) {
    const lds_char* ks = lds + stage * G::TILEB;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const vec8 a = *(const lds_vec8*)(ks + koff[t] + kq * 32 * G::ROWB);
        s[kq] = T::mfma(a, qf[t], s[kq]);
      }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

  // Prologue: K0, V0, K1, V1, K2 in flight, then S(0).
  issue(kg, 0, 0, 0);
  issue(vg, 1, 0, 0);
  if (nt > 1) { issue(kg, 0, 1, 1); issue(vg, 1, 1, 1); }
  if (nt > 2) issue(kg, 0, 2, 2);
  wait_vmcnt<0>();
  barrier();

  f32x16 scur[2];
  if (ntw > 0) scores(0, scur);

  int st0 = 0;   // stage of tile j
  for (int j = 0; j < nt; ++j) {
    const int st1 = (st0 == STAGES - 1) ? 0 : st0 + 1;   // stage of tile j+1
    const int st2 = (st1 == STAGES - 1) ? 0 : st1 + 1;   // stage of tile j+2 (held tile j-1)
    // Needed now: K(j+1), V(j).  Still allowed in flight: K(j+2), V(j+1) from the last
    // iteration.  The barrier also retires every wave's reads of K(j) and V(j-1), whose
    // stages are refilled next (at j = 0: the prologue's reads of K(0)).
    if (j + 2 < nt) wait_vmcnt<2 * LOADS>();
    else if (j + 1 < nt) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    barrier();
    if (j + 3 < nt) issue(kg, 0, st0, j + 3);   // K(j) was consumed in iteration j-1
    if (j + 2 < nt) issue(vg, 1, st2, j + 2);   // V(j-1) was consumed in iteration j-1

    if (j < ntw) {
      const int j0 = j * BN;
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
      const float m_cand = mt * c;
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kRescaleSlack) != 0) {
        const float m_new = __builtin_fmaxf(m_run, m_cand);
        const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int vq = 0; vq < D / 32; ++vq)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[vq][i] *= alpha;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;

      // Tile j+1's scores (its K stage is ready); overlaps the exponentials below.
      f32x16 snext[2];
      scores(st1, snext);

      float pe[32];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int i = 0; i < 16; ++i) pe[16 * kq + i] = fast_exp2(fmaf(scur[kq][i], c, neg_m));
      float ps[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i] = pe[2 * i] + pe[2 * i + 1];
#pragma unroll
      for (int w = 8; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) ps[i] = ps[i] + ps[i + w];
      l_run += ps[0];

      const lds_char* vs = lds + (STAGES + st0) * G::TILEB;
#pragma unroll
      for (int s = 0; s < BN / 16; ++s) {
        const vec8 bfrag = T::pack8(&pe[8 * s]);
#pragma unroll
        for (int vq = 0; vq < D / 32; ++vq) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vs + voff[0][vq] + 16 * s * G::ROWB));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vs + voff[1][vq] + 16 * s * G::ROWB));
          const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[vq] = T::mfma(a, bfrag, oacc[vq]);
        }
      }
      scur[0] = snext[0];
      scur[1] = snext[1];
    }
    st0 = st1;
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

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
//   softmax         online, fp32 ([FA3-V3] §4.2); the reference max moves when
//                   a row max passes it by more than kMaxSlack (log2 units), so
//                   p <= 2^kMaxSlack and P̃ stays inside E4M3's range.
//   Oᵀ += V8ᵀ·P̃ᵀ    P̃ = e4m3(p · sv(tile)·2^8/max(sv)): the V block scale and a
//                   2^8 headroom are folded into the exponent bias, so p̃ < 448
//                   and small probabilities keep E4M3's precision.  The denominator
//                   sums the same rounded P̃ with one more MFMA against an all-ones
//                   operand, which gives every lane its row's tile sum.  A = Vᵀ
//                   gathered by byte-transposing LDS reads (ds_read_b64_tr_b8, 4 per MFMA).
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
// How far a score may pass the reference max before it moves: with the 2^8
// headroom, p̃ <= 2^(8 + kMaxSlack) = 445.7 < 448, the largest E4M3 value.
constexpr float kMaxSlack = 0.8f;
constexpr int kMaxBlocks = 4096;         // scale blocks per head staged in LDS (N <= 262144)
#ifndef TATTN_FP8_READ_AHEAD
#define TATTN_FP8_READ_AHEAD 2
#endif
constexpr int kReadAhead = TATTN_FP8_READ_AHEAD;   // products between an LDS read and its use
// Of every 8 probabilities of a full tile, how many are computed on the ordinary
// VALU pipe (exp2_valu) instead of by v_exp_f32, so that the two pipes share the
// exponentials; tiles with masked keys use v_exp_f32 only.
#ifndef TATTN_FP8_EXP_VALU
#define TATTN_FP8_EXP_VALU 0
#endif
constexpr int kExpValu = TATTN_FP8_EXP_VALU;
static_assert(kExpValu >= 0 && kExpValu <= 8, "probabilities per 8 on the VALU");

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
  int nper;     // work items per (batch, head): q tiles, or causal pairs of q tiles
  int nitems;   // nper · Hq · B
  int remap;    // deal items so that each XCD gets a contiguous range (needs 8 | nitems, 8 | grid)
  float c;      // softmax scale · log2(e)
};

template <typename OutT, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_fp8_kernel(Fp8Params p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDSB];
  __shared__ float red[NW];
  __shared__ float sk_lds[kMaxBlocks], bias_lds[kMaxBlocks];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Persistent: one workgroup per CU walks its share of the items (the same
  // dealing as the 16-bit kernel: XCD-contiguous ranges, causal q tiles paired
  // nqt-1-r with r so that every item costs the same).
  for (int v = blockIdx.x; v < p.nitems; v += gridDim.x) {
  const int wi = p.remap ? (v % 8) * (p.nitems / 8) + v / 8 : v;
  const int r = wi % p.nper;
  const int rest = wi / p.nper;
  const int nsub = (CAUSAL && r != p.nqt - 1 - r) ? 2 : 1;
  for (int sub = 0; sub < nsub; ++sub) {
  const int qt = CAUSAL ? (sub == 0 ? p.nqt - 1 - r : r) : r;
  // Opaque per item: lane-derived offsets are recomputed for each item instead of
  // being hoisted out of the item loop and kept live through the tile loop.
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, hh = lane >> 5;
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

  // Stage this head's K block scales in LDS (the loop then reads them with LDS
  // loads, which do not wait on the K/V prefetch), take the largest V scale, and
  // stage each V block's exponent bias log2(sv/max sv) + 8.
  float vmax = 0.f;
  for (int i = tid; i < p.nblk; i += kThreads) {
    sk_lds[i] = ksc[i];
    vmax = fmaxf(vmax, vsc[i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
  if (lane == 0) red[wave] = vmax;
  __syncthreads();
  vmax = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) vmax = fmaxf(vmax, red[w]);
  for (int i = tid; i < p.nblk; i += kThreads) bias_lds[i] = __log2f(vsc[i] / vmax) + kHeadroomLog2;
  __syncthreads();

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;
  const int wend = (wq0 >= N) ? 0 : (CAUSAL ? min(kv_end, wq0 + 32) : kv_end);
  const int ntw = (wend + BN - 1) / BN;

  // LDS-DMA: one 1 KB load per wave per tile = rows 8·wave .. 8·wave+7.
  const int ld_row = 8 * wave + (lane >> 3);
  const int ld_col = 16 * ((lane & 7) ^ swz(ld_row));
  const uint32_t ld_off = (uint32_t)(ld_row * kvrow + ld_col);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  // Offsets for the last tile: rows past N repeat row N-1 (their probabilities are 0).
  const int jl = (nt - 1) * BN;
  const uint32_t ld_off_last = (uint32_t)((min(jl + ld_row, N - 1) - jl) * kvrow + ld_col);
  // Tile t of K (ring 0) or V (ring 1) into ring stage ``stage``.  Tiles past the end
  // repeat the last tile (into a stage nobody reads again), so every wave issues the
  // same loads in every step and every address stays inside K and V.
  auto issue = [&](int ring, int stage, int t) {
    t = min(t, nt - 1);
    const char* base = (ring ? vg : kg) + (long long)(t * BN) * kvrow;
    lds_dma16(base, t == nt - 1 ? ld_off_last : ld_off, lds_base + (ring * STAGES + stage) * TILEB + 1024 * wave);
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
    mma_read_order<4, 2, kReadAhead>();
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // Row sum of the last tile's P̃ (every element holds it) and its factor back to p
  // units; added to l_run at the start of the next softmax, once the MFMA is long done.
  f32x16 tsum = {};
  float tfac = 0.f;
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
  const float cq = p.c * sq;
  // Defined per item: left undefined, they would be carried from the last item.
  f32x16 scur[2] = {f32x16{}, f32x16{}};   // raw scores of the tile whose softmax comes next
  i32x8 pf = {};    // P̃ of the last softmax (operand of the next P·V)
  // The two wave groups sharing each SIMD alternate between exponentials and
  // matrix-core work ([FA3-V3] §7.3's ping-pong between warpgroups).  In step j:
  //   group 0: softmax(j)              | P·V(j), scores(j+1)   (scores(0) in the prologue)
  //   group 1: P·V(j-1), scores(j)     | softmax(j)            (P·V(last) after the loop)
  const bool lead = wave < NW / 2;

  auto pv = [&](const int vst) {
    const lds_char* vs = lds + vst * TILEB;   // voff carries the V ring base
#pragma unroll
    for (int vq = 0; vq < D / 32; ++vq) {
      const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq]));
      const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq] + 16 * ROWB));
      const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq] + 32 * ROWB));
      const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + voff[vq] + 48 * ROWB));
      const i32x8 a = cat(__builtin_shufflevector(r0, r1, 0, 1, 2, 3), __builtin_shufflevector(r2, r3, 0, 1, 2, 3));
      oacc[vq] = mfma_fp8(a, pf, oacc[vq]);
    }
    mma_read_order<D / 32, 4, kReadAhead>();
  };

  // Prologue: K tiles 0..2 and V tiles 0..1, then scores(0) for group 0.
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) {
    if (t < nt) issue(0, t, t);
    if (t < STAGES - 2 && t < nt) issue(1, t, t);
  }
  wait_vmcnt<0>();
  barrier();
  if (lead && ntw > 0) scores(0, scur);
  // Score scale and exponent bias of the tile whose softmax comes next, read from
  // LDS a phase ahead of their use (group 0 for tile j+1 during step j, group 1 for
  // tile j at the start of step j).
  float cj_next = 0.f, bias_next = 0.f;
  auto fetch_scales = [&](int t) {
    t = min(t, nt - 1);
    cj_next = cq * sk_lds[t];
    bias_next = bias_lds[t];
  };
  if (lead) fetch_scales(0);

  auto step = [&](auto stc, auto leadc, int j) {
    constexpr int st = decltype(stc)::value;
    constexpr int stn = (st + 1) % STAGES;
    constexpr int stp = (st + STAGES - 1) % STAGES;
    constexpr bool is_lead = decltype(leadc)::value;
    // Needed now: K(j+1) and V(j), issued two steps ago; K(j+2) and V(j+1) may be in
    // flight.  The barrier also retires every wave's reads of K(j-1) and V(j-2),
    // whose stages receive K(j+3) and V(j+2) in this step.
    wait_vmcnt<2>();
    barrier();
    // Loads go out at two points of each wave's schedule, which differ between the
    // groups, so that the loads of eight waves do not queue in the address unit together.
    auto load_k = [&]() { issue(0, (st + 3) % STAGES, j + 3); };
    auto load_v = [&]() { issue(1, (st + 2) % STAGES, j + 2); };

    auto softmax = [&]() {
      const int j0 = j * BN;
      const float cj = cj_next, bias = bias_next;
      const bool edge = (j0 + BN > N) || (CAUSAL && j0 + BN - 1 > wq0);
      if (edge) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * kq + 16 * (i >> 3) + 8 * hh + (i & 7);
            if (key >= N || (CAUSAL && key > qrow)) scur[kq][i] = -INFINITY;
          }
      }
      l_run = fmaf(tsum[0], tfac, l_run);   // the previous tile's sum, before any rescale
      float mt = max3f(scur[0][0], scur[0][1], scur[0][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mt = max3f(mt, scur[0][i], scur[0][i + 1]);
      mt = max3f(mt, scur[0][15], scur[1][0]);
#pragma unroll
      for (int i = 1; i < 16; i += 2) mt = max3f(mt, scur[1][i], scur[1][i + 1 < 16 ? i + 1 : i]);
      mt = max_xor32(mt);
      const float m_cand = mt * cj;
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kMaxSlack) != 0) {
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
      auto exps = [&](auto valu) {
        constexpr int kv = decltype(valu)::value;
        float pe[32];
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = fmaf(scur[kq][i], cj, neg);
            pe[16 * kq + i] = (i & 7) >= 8 - kv ? exp2_valu(x) : fast_exp2(x);
          }
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          // (the old-value operand is overwritten byte for byte; passing a source spares a move)
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w], pe[4 * w + 1], __builtin_bit_cast(int, pe[4 * w]), false);
          pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w + 2], pe[4 * w + 3], word, true);
        }
      };
      if (kExpValu == 0 || edge) exps(std::integral_constant<int, 0>{});
      else exps(std::integral_constant<int, kExpValu>{});
      // Row sum of this tile's P̃: ones(32x64) · P̃ᵀ puts it in every element of the lane.
      tsum = mfma_fp8(ones, pf, f32x16{});
      tfac = fast_exp2(-bias);
    };
    if constexpr (is_lead) {
      if (j >= ntw) {
        load_k();
        load_v();
        return;
      }
      softmax();
      __builtin_amdgcn_sched_barrier(0);
      fetch_scales(j + 1);
      load_k();
      pv(st);
      load_v();
      scores(stn, scur);   // also on the wave's last tile (unused there): no branch, no copies
    } else {
      const bool has_pv = j >= 1 && j - 1 < ntw, has_scores = j < ntw;
      fetch_scales(j);
      load_k();
      if (has_pv) pv(stp);
      load_v();
      scores(st, scur);   // also when unused, for the same reason
      if (!has_scores) return;
      __builtin_amdgcn_sched_barrier(0);
      softmax();
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
  if (lead) {
    run(std::true_type{});
  } else {
    run(std::false_type{});
    if (ntw == nt && nt > 0) pv((nt - 1) % STAGES);
  }
  wait_vmcnt<0>();   // the last steps' loads land in the rings reused below

  const float l_tot = fmaf(tsum[0], tfac, l_run);   // both lanes of a row hold the full row sum
  const float inv = l_tot > 0.f ? vmax * 0.00390625f / l_tot : 0.f;   // max(sv)·2^-8 / z
  // The rings are free once every wave has left the loop; each wave stages its rows in 8 KB.
  __syncthreads();
  store_rows<OutT>(lds + wave * 8192, oacc, inv, lane, p.o + ((long long)b * N * p.Hq + hq) * D + wq0 * qstride,
                   qstride, N - wq0);
  if (qrow < N && p.lse != nullptr && hh == 0)
    p.lse[((long long)b * p.Hq + hq) * N + qrow] =
        l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  // The next item's first loads and scale tables overwrite LDS that other waves
  // may still be reading.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  }
  }
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
  p.nper = CAUSAL ? (p.nqt + 1) / 2 : p.nqt;
  p.nitems = p.nper * a.Hq * a.B;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  const int grid = p.nitems < device_cu_count() ? p.nitems : device_cu_count();
  p.remap = (p.nitems % 8 == 0 && grid % 8 == 0) ? 1 : 0;
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

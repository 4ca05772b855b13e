// Fused attention forward, fp16/bf16, for gfx950 (CDNA4).
//
// Work decomposition.  A q tile = BM = 256 query rows of one (batch, head),
// processed by one workgroup of 8 waves; each wave owns 32 rows and keeps its Q
// rows in VGPRs for the whole sequence.  The K/V sequence is walked in tiles of
// BN = 64 keys.  The grid is persistent, one workgroup per CU (the 128 KB of LDS
// admit no second one), and each workgroup walks an equal share of the items:
// the hardware then dispatches only once, where handing out q tiles of unequal
// cost one by one left CUs idle between them.  Items are ordered (batch, head,
// q tile) and dealt so that each XCD takes one contiguous range, which keeps the
// heads of a KV group (and all q tiles of a head) on one L2.  A causal item is
// the pair of q tiles nqt-1-r and r (heavy first), which costs nqt + 1 tile
// rows whatever r is, so the static shares are balanced.
//
// Staging ([FA3-tile] §二's double buffer, generalised to four stages).  K and
// V tiles go global -> LDS directly (16-byte LDS-DMA loads, no VGPR staging)
// into four-stage rings; during step j the loads of K(j+3) and V(j+2) go out
// while K(j+1) and V(j) are consumed.  One barrier per tile both publishes the
// finished loads (read after write) and retires the stages about to be
// overwritten (write after read).  LDS rows are unpadded and their 16-byte
// chunks are XOR-swizzled per row so that the K reads and the transposing V
// reads are free of bank conflicts.
//
// Per tile and wave, on the 32x32x16 matrix cores:
//   Sᵀ = K·Qᵀ   A = K rows from LDS (rows taken in an order that swaps bits 2
//                and 3 of the row index), B = Q as given; the accumulator
//                starts from zero.  Lane l then holds 32 scores of query row
//                l%32: row statistics are lane-local apart from one exchange
//                with lane l^32.
//   softmax     online, fp32 ([FA3-V3] §4.2): p = 2^(c·s − m_ref) with
//                c = scale·log2(e) and m_ref the row's reference max in log2
//                units, one fused multiply-add and one v_exp per element,
//                z' = z + Σp.  (Folding c into Q, rounded to the input type,
//                and starting the accumulator from −m_ref would save the
//                multiply-add, but that rounding moves every score of a row
//                by up to u·scale·Σ|q_i k_i|, an error the method does not
//                have; it is kept only as a build-time variant.)  The
//                reference max is set on the first
//                tile and only moves (by δ, with O and z scaled by 2^−δ) when a
//                tile's probabilities would leave the 16-bit operand range,
//                which skips the row max and the O rescale on almost every tile;
//                O/z is unchanged in exact arithmetic.
//   Oᵀ += Vᵀ·Pᵀ A = Vᵀ gathered by transposing LDS reads (ds_read_b64_tr_b16),
//                B = P rounded to the input type.  Thanks to the K row order
//                above, the score accumulator already is the B operand, so P
//                needs no shuffle ([FA3-V3] §7.4's accumulator-to-operand
//                problem, solved by operand order).
// Scheduling ([FA3-V3] §7.3's ping-pong, between the two waves of each SIMD):
// a wave's VALU work does not overlap its own matrix-core work, so the two wave
// groups alternate, one running its exponentials while the other issues its
// products (see step() below).
// The epilogue divides by z (deferred normalisation, [FA3-V3] §11) and writes
// O and optionally the log-sum-exp.
#include <type_traits>

#include "tattn_device.hpp"
#include "tattn_pipeline.hpp"
#include "tattn_launch.hpp"
#include "tattn.h"

namespace tattn {
namespace {

constexpr int NW = 8;                // waves per workgroup
constexpr int kThreads = 64 * NW;
constexpr int BM = 32 * NW;          // query rows per workgroup
constexpr int BN = 64;               // keys per tile

// Schedule of the tile loop.  The library ships the default; the other settings
// build the variants the scheduling ablation compares (selected at build time):
//   STAGES       ring depth of the K and V rings (>= 3).  During step j the loads
//                of K(j + STAGES-1) and V(j + STAGES-2) go out while K(j), K(j+1),
//                V(j-1) and V(j) are read, so three stages is the least this
//                two-group schedule can run with (each step reads two K tiles).
//   READ_AHEAD   products between an LDS operand read and the product using it.
//   PINGPONG     two wave groups alternating exponentials and products (true), or
//                every wave on the same softmax -> P·V -> scores order (false).
//   SPLIT_LOADS  a step's tile loads issued at two points of each wave's schedule
//                (true), or all right after the barrier (false).
//   FOLD_SCALE   c = scale·log2(e) folded into Q and rounded to the input type, the
//                score products started from −m_ref, so a probability needs only
//                the v_exp (true), or Q kept as given and c·s − m_ref formed in
//                fp32 (false).  Not bit-identical to the shipped build.
#ifndef TATTN_STAGES
#define TATTN_STAGES 4
#endif
#ifndef TATTN_READ_AHEAD
#define TATTN_READ_AHEAD 2
#endif
#ifndef TATTN_PINGPONG
#define TATTN_PINGPONG 1
#endif
#ifndef TATTN_SPLIT_LOADS
#define TATTN_SPLIT_LOADS 1
#endif
#ifndef TATTN_FOLD_SCALE
#define TATTN_FOLD_SCALE 0
#endif
constexpr int STAGES = TATTN_STAGES;
constexpr int kReadAhead = TATTN_READ_AHEAD;
constexpr bool kPingPong = TATTN_PINGPONG != 0;
constexpr bool kSplitLoads = TATTN_SPLIT_LOADS != 0;
constexpr bool kFoldScale = TATTN_FOLD_SCALE != 0;
static_assert(STAGES >= 3 && STAGES <= 5, "ring depth");
constexpr int KDIST = STAGES - 1;    // K(j + KDIST) is loaded during step j
constexpr int VDIST = STAGES - 2;    // V(j + VDIST) likewise

// Calls f(integral_constant<int, I>) for I = 0 .. N-1.
template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Largest partial row sum of probabilities accepted before the reference max
// is moved: keeps every probability below the fp16 operand range.
constexpr float kOperandLimit = 32768.0f;

template <int D>
struct Geo {
  static constexpr int ROWB = 2 * D;                    // bytes per K/V row
  static constexpr int TILEB = BN * ROWB;               // bytes per tile
  static constexpr int LDSB = 2 * STAGES * TILEB;       // K ring + V ring
  static constexpr int LOADS = TILEB / (1024 * NW);     // 1 KB DMA loads per wave per tile
  static_assert(LOADS >= 1 && TILEB % (1024 * NW) == 0, "tile must split into 1 KB loads");
  // Physical 16-byte chunk = logical chunk ^ swz(row).  Conflict-free for both read kinds:
  // a 16-lane group of K reads (ds_read_b128, 16 distinct rows, one 16-byte chunk each) and
  // a 32-lane half-wave of V transposing reads (ds_read_b64_tr_b16, 4 consecutive keys x
  // 4 consecutive logical chunks starting at a multiple of 4) both land on 16 distinct
  // 16-byte bank windows.  Depends on row % 16 only.
  __device__ static inline int swz(int r) {
    if constexpr (D == 128) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
      return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    }
  }
};

struct KernelParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N, Hq, Hkv, group, nqt;
  int nper;     // work items per (batch, head): q tiles, or causal pairs of q tiles
  int nitems;   // nper · Hq · B
  int remap;    // deal items so that each XCD gets a contiguous range (needs 8 | nitems, 8 | grid)
  float c;      // scale · log2(e)
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Persistent: the grid holds one workgroup per CU and each walks its share of
  // the items; item v runs on XCD v % 8, and with ``remap`` the XCD's items form
  // one contiguous range of (batch, head), so a KV group stays in one L2.
  // Causal items pair q tile nqt-1-r with q tile r: every pair costs nqt + 1
  // units of 256 keys, so equal shares balance without a queue.
  for (int v = blockIdx.x; v < p.nitems; v += gridDim.x) {
  const int wi = p.remap ? (v % 8) * (p.nitems / 8) + v / 8 : v;
  const int r = wi % p.nper;
  const int rest = wi / p.nper;
  const int nsub = (CAUSAL && r != p.nqt - 1 - r) ? 2 : 1;
  for (int sub = 0; sub < nsub; ++sub) {
  const int qt = CAUSAL ? (sub == 0 ? p.nqt - 1 - r : r) : r;
  // The lane index comes from mbcnt, which needs no live register, and is opaque
  // per item: lane-derived offsets are recomputed for each item instead of being
  // hoisted out of the item loop and kept live through the tile loop.
  int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, hh = lane >> 5;
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

  // Q fragments (B operand of the score MFMA): lane holds Q[qrow][16t+8hh .. +7]
  // (folding the scale: c·Q rounded to the input type).
  vec8 qf[D / 16];
  {
    const uint16_t* qr = qb + (long long)min(qrow, N - 1) * qs + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const vec8 raw = __builtin_bit_cast(vec8, *(const u32x4*)(qr + 16 * t));
      if constexpr (kFoldScale) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)raw[e] * p.c;
        qf[t] = T::pack8(x);
      } else {
        qf[t] = raw;
      }
    }
  }
  const float c = p.c;

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
  // LDS address of this wave's first 1 KB load slot; the ring and stage offsets are
  // compile-time constants added to it, and it is opaque so that the compiler does
  // not keep one scalar register per (ring, stage, load) through the loop.
  uint32_t lds_wave = (uint32_t)(uintptr_t)lds + 1024 * (wave * LOADS);
  asm volatile("" : "+s"(lds_wave));
  uint32_t ld_off[LOADS];   // byte offset of this lane's 16 bytes within a tile (same for K and V)
#pragma unroll
  for (int n = 0; n < LOADS; ++n) ld_off[n] = (uint32_t)(ld_row[n] * kvrow + ld_col[n]);
  // Offsets for the last tile: rows past N repeat row N-1 (their probabilities are 0).
  uint32_t ld_off_last[LOADS];
  {
    const int jl = (nt - 1) * BN;
#pragma unroll
    for (int n = 0; n < LOADS; ++n)
      ld_off_last[n] = (uint32_t)((min(jl + ld_row[n], N - 1) - jl) * kvrow + ld_col[n]);
  }
  // Tile t of K (ring 0) or V (ring 1) into ring stage ``stage``.  Tiles past the
  // end repeat the last tile (into a stage nobody reads again), so every wave issues
  // the same loads in every step and every address stays inside K and V.
  auto issue = [&](int ring, int stage, int t) {
    t = min(t, nt - 1);
    const char* base = (ring ? vg : kg) + (long long)(t * BN) * kvrow;
    const bool last = t == nt - 1;
#pragma unroll
    for (int n = 0; n < LOADS; ++n)
      lds_dma16(base, last ? ld_off_last[n] : ld_off[n], lds_wave + (ring * STAGES + stage) * G::TILEB + 1024 * n);
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
        voff[half][vq] = STAGES * G::TILEB + key * G::ROWB + 16 * ((dv >> 3) ^ G::swz(key)) +
                         8 * ((dv >> 2) & 1);
      }
  }

  // Defined per item: left undefined, they would be carried from the last item.
  f32x16 scur[2] = {f32x16{}, f32x16{}};   // scores of the tile whose softmax comes next
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  // Reference max of the row (log2 units).  Folding the scale, its negation also
  // fills every element of ``negm``, the start value of the score products, so that
  // a score arrives as c·s − m_ref; otherwise the products start from zero.
  float m_ref = 0.f, l_run = 0.f;
  f32x16 negm = {};

  // Score product S^T = K·Q^T of one K stage into s[2] (keys 0..31 and 32..63).
  auto scores = [&](const int stage, f32x16 (&s)[2]) {
    const lds_char* ks = lds + stage * G::TILEB;
    if constexpr (kFoldScale) {
      s[0] = negm;
      s[1] = negm;
    } else {
      s[0] = f32x16{};
      s[1] = f32x16{};
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const vec8 a = *(const lds_vec8*)(ks + koff[t] + kq * 32 * G::ROWB);
        s[kq] = T::mfma(a, qf[t], s[kq]);
      }
  };

  // The two wave groups sharing each SIMD alternate between exponentials and
  // matrix-core work ([FA3-V3] §7.3's ping-pong between warpgroups).  In step j:
  //   group 0: softmax(j)              | P·V(j), scores(j+1)   (scores(0) in the prologue)
  //   group 1: P·V(j-1), scores(j)     | softmax(j)            (P·V(last) after the loop)
  // so each wave's softmax runs while the other wave of its SIMD issues both of
  // its products.  Step j reads K(j), K(j+1), V(j-1) and V(j).  Without the
  // ping-pong every wave runs group 0's order.
  const bool lead = !kPingPong || wave < NW / 2;
  vec8 pf[BN / 16] = {};   // probabilities of the last softmax (operand of the next P·V)

  // Prologue: K tiles 0 .. KDIST-1 and V tiles 0 .. VDIST-1, then scores(0) for group 0.
#pragma unroll
  for (int t = 0; t < KDIST; ++t) {
    if (t < nt) issue(0, t, t);
    if (t < VDIST && t < nt) issue(1, t, t);
  }
  wait_vmcnt<0>();
  barrier();

  // O^T += V^T·P^T for one V stage, with the probabilities in pf.
  auto pv = [&](const int vst) {
    const lds_char* vs = lds + vst * G::TILEB;   // voff carries the V ring base
#pragma unroll
    for (int s = 0; s < BN / 16; ++s) {
#pragma unroll
      for (int vq = 0; vq < D / 32; ++vq) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vs + voff[0][vq] + 16 * s * G::ROWB));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vs + voff[1][vq] + 16 * s * G::ROWB));
        const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[vq] = T::mfma(a, pf[s], oacc[vq]);
      }
    }
  };
  // Each matrix-core phase issues every LDS read kReadAhead products before the
  // product that consumes it.
  auto pv_only = [&](const int vst) {
    pv(vst);
    mma_read_order<BN / 16 * (D / 32), 2, kReadAhead>();
  };
  auto scores_only = [&](const int kst) {
    scores(kst, scur);
    mma_read_order<D / 8, 1, kReadAhead>();
  };

  if (lead && ntw > 0) scores_only(0);

  // One tile; ST = j % STAGES, so every LDS offset is a constant.
  auto step = [&](auto stc, auto leadc, int j) {
    constexpr int st = decltype(stc)::value;
    constexpr bool lead = decltype(leadc)::value;
    constexpr int stn = (st + 1) % STAGES;
    constexpr int stp = (st + STAGES - 1) % STAGES;
    // Needed now: K(j+1) and V(j), issued in step j+2-STAGES.  Allowed in flight: the
    // loads of the STAGES-3 steps since.  The barrier also retires every wave's reads
    // of K(j-1) and V(j-2), whose stages receive K(j+KDIST) and V(j+VDIST) in this step.
    wait_vmcnt<(STAGES - 3) * 2 * LOADS>();
    barrier();
    // The tile loads of a step go out at two points of each wave's schedule, which
    // differ between the groups: issued all at once, the loads of eight waves queue
    // in the address unit and stall the issuing waves.
    auto load_k = [&]() { issue(0, (st + KDIST) % STAGES, j + KDIST); };
    auto load_v = [&]() { issue(1, (st + VDIST) % STAGES, j + VDIST); };
    if constexpr (!kSplitLoads) {
      load_k();
      load_v();
    }
    auto load_k_split = [&]() { if constexpr (kSplitLoads) load_k(); };
    auto load_v_split = [&]() { if constexpr (kSplitLoads) load_v(); };

    // Online softmax of tile j ([FA3-V3] §4.2), fp32 statistics.  The row max is
    // only taken on the first tile and when the probabilities of a tile would no
    // longer fit the 16-bit operand range (partial row sum above 2^15, i.e. some
    // score grew more than 15 in log2 units past the reference max).  Between
    // those events the reference max stays put; O/z is the same in exact
    // arithmetic.  The denominator sums the rounded probabilities that enter P·V.
    // Folding the scale, ``shift`` (zero except right after the reference max
    // moved) is what the accumulators' start value lags behind m_ref.
    auto exps = [&](auto shifted, float shift) {
      float pe[32];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x;
          if constexpr (!kFoldScale) x = fmaf(scur[kq][i], c, -m_ref);
          else if constexpr (decltype(shifted)::value) x = scur[kq][i] - shift;
          else x = scur[kq][i];
          pe[16 * kq + i] = fast_exp2(x);
        }
#pragma unroll
      for (int s = 0; s < BN / 16; ++s) pf[s] = T::pack8(&pe[8 * s]);
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int s = 0; s < BN / 16; s += 2) {
        ps0 = T::sum8(pf[s], ps0);
        ps1 = T::sum8(pf[s + 1], ps1);
      }
      return ps0 + ps1;
    };
    // Moves the reference max to the row max of this tile and returns the shift.
    // On the first tile O and l are still zero and need no rescaling.
    auto rebase = [&](bool first) {
      float mt = scur[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = __builtin_fmaxf(mt, scur[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = __builtin_fmaxf(mt, scur[1][i]);
      mt = max_xor32(mt);
      // Folding the scale, mt is the tile's row max of c·s − m_ref, else of s.
      const float shift = (mt == -INFINITY) ? 0.f : (kFoldScale ? mt : mt * c - m_ref);
      m_ref += shift;
      if (!first) {
        const float alpha = fast_exp2(-shift);
        l_run *= alpha;
#pragma unroll
        for (int vq = 0; vq < D / 32; ++vq)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[vq][i] *= alpha;
      }
      if constexpr (kFoldScale) {
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -m_ref;
      }
      return shift;
    };
    auto softmax = [&]() {
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
      float psum;
      if (j == 0) psum = exps(std::true_type{}, rebase(true));
      else psum = exps(std::false_type{}, 0.f);
      if (__builtin_amdgcn_ballot_w64(!(psum <= kOperandLimit)) != 0)
        psum = exps(std::true_type{}, rebase(false));
      l_run += psum;
    };
    if constexpr (lead) {
      if (j >= ntw) {
        load_k_split();
        load_v_split();
        return;
      }
      softmax();
      __builtin_amdgcn_sched_barrier(0);
      load_k_split();
      pv_only(st);
      load_v_split();
      if (j + 1 < ntw) scores_only(stn);
    } else {
      const bool has_pv = j >= 1 && j - 1 < ntw, has_scores = j < ntw;
      load_k_split();
      if (has_pv) pv_only(stp);
      load_v_split();
      if (has_scores) scores_only(st);
      if (!has_scores) return;
      __builtin_amdgcn_sched_barrier(0);
      softmax();
    }
  };
  // Separate loops per group keep the two schedules' register lifetimes apart.
  auto run = [&](auto leadc) {
    for (int j = 0; j < nt; j += STAGES) {
      static_for<0, STAGES>([&](auto stc) {
        if (decltype(stc)::value == 0 || j + decltype(stc)::value < nt) step(stc, leadc, j + decltype(stc)::value);
      });
    }
  };
  if (lead) {
    run(std::true_type{});
  } else if constexpr (kPingPong) {
    run(std::false_type{});
    if (ntw == nt && nt > 0) pv_only((nt - 1) % STAGES);
  }
  wait_vmcnt<0>();   // the last steps' loads land in the rings reused below

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // The rings are free once every wave has left the loop; each wave stages its rows in 8 KB.
  __syncthreads();
  if constexpr (D == 128) {
    store_rows<T>(lds + wave * 8192, oacc, inv, lane, p.o + ((long long)b * N * p.Hq + hq) * D + wq0 * qs,
                  qs, N - wq0);
  } else if (qrow < N) {
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
  }
  if (qrow < N && p.lse != nullptr && hh == 0)
    p.lse[((long long)b * p.Hq + hq) * N + qrow] =
        l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  // The next item's first loads overwrite the staging blocks of other waves.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  }
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
  p.nper = CAUSAL ? (p.nqt + 1) / 2 : p.nqt;
  p.nitems = p.nper * a.Hq * a.B;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  const int grid = p.nitems < device_cu_count() ? p.nitems : device_cu_count();
  p.remap = (p.nitems % 8 == 0 && grid % 8 == 0) ? 1 : 0;
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

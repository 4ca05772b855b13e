// Random-sign Hadamard rotation with optional fused FP8 block quantisation,
// for gfx950.  Memory-bound: every element is read once and written once.
//
// One workgroup (4 waves) owns one (batch, head, block of 64 rows).  A row of
// d channels is spread over 4 neighbouring lanes, in 16-byte chunks of 8
// channels dealt round-robin: lane l of the quad holds chunks l, l+4, l+8, ...
// (channel 32v + 8l + e in its element 8v + e), so each 16-byte load of the
// quad reads 64 contiguous bytes of the row.  The Walsh–Hadamard transform is a
// product of one butterfly stage per channel-index bit, in any order: the
// stages over channel bits 0-2 and 5-6 (element distances 1, 2, 4, 8, 16) run
// inside a lane, and those over bits 3 and 4 (distances 8 and 16) pair lanes 1
// and 2 apart, exchanged with DPP quad permutes in the VALU rather than through
// LDS.  Each stage is one fp32 add or subtract per element, followed by one
// fp32 multiply by fl32(1/sqrt(d)), so the result is fully determined.
//
// Rotary embedding (optional, before everything else; [FA3-card] "低精度优化"
// names it as fusable with the rotation): the partner of channel i is i ± d/2,
// the top channel-index bit, which this layout keeps inside the lane, so the
// rotation costs two fp32 products and one add per element and no exchange.
//
// Quantisation ([FA3-V3] §4.3 per-block scales; the reading taken is
// symmetric absmax with no offset): the block's absmax is reduced across the
// workgroup, scale = absmax/448 and inv = 448/absmax are IEEE fp32 divisions,
// and each element becomes the E4M3FN code of fl32(y·inv), clamped to ±448
// and rounded to nearest even by the hardware conversion.
#include "tattn_device.hpp"
#include "tattn_launch.hpp"
#include "tattn.h"

#pragma clang fp contract(off)

namespace tattn {
namespace {

struct RotParams {
  const uint16_t* x;
  void* y;
  const int8_t* signs;
  float* scales;
  const float* rcos;
  const float* rsin;
  int N, H, nblk;
};

// Value of x in the lane whose index differs in bit ``ld`` (1 or 2) within its quad.
template <int LD>
__device__ inline float quad_xor(float x) {
  constexpr int ctrl = LD == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xF, 0xF, false));
}

// One (batch, head, 64-row block) of one tensor, block index ``bid`` in
// (batch, head, block) order, by the 256 threads of a workgroup; ``red`` is 4
// floats of LDS.
template <typename T, int D, bool ROT, bool QUANT, bool ROPE>
__device__ inline void rotate_block(const RotParams& p, int bid, float* red) {
  constexpr int CPL = D / 4;          // channels per lane
  constexpr int NV = CPL / 8;         // 16-byte chunks per lane: chunk 4v + li holds y[8v .. 8v+7]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 3;
  const int blk = bid % p.nblk;
  const int h = (bid / p.nblk) % p.H;
  const int b = bid / (p.nblk * p.H);
  const long long rs = (long long)p.H * D;     // elements between positions
  const long long base = ((long long)b * p.N * p.H + h) * D + 8 * li;
  const int row = blk * 64 + wave * 16 + (lane >> 2);
  const bool valid = row < p.N;
  // channel of element j: 32·(j/8) + 8·li + j%8

  float y[CPL];
  {
    u32x4 raw[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) raw[v] = valid ? *(const u32x4*)(p.x + base + row * rs + 32 * v) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const uint32_t w = raw[e / 8][(e % 8) / 2];
      y[e] = T::to_f32((e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffff));
    }
  }
  if (ROPE) {
    // elements j < CPL/2 hold channels of [0, d/2) and j + CPL/2 their partners i + d/2;
    // the table column of element j (and j + CPL/2) is 32·(j/8) + 8·li + j%8
    const long long t = (long long)min(row, p.N - 1) * (D / 2) + 8 * li;
    float c[CPL / 2], sn[CPL / 2];
#pragma unroll
    for (int v = 0; v < NV / 2; ++v)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 cv = *(const f32x4*)(p.rcos + t + 32 * v + 4 * hf);
        const f32x4 sv = *(const f32x4*)(p.rsin + t + 32 * v + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[8 * v + 4 * hf + e] = cv[e];
          sn[8 * v + 4 * hf + e] = sv[e];
        }
      }
#pragma unroll
    for (int j = 0; j < CPL / 2; ++j) {
      const float x0 = y[j], x1 = y[j + CPL / 2];
      y[j] = x0 * c[j] - x1 * sn[j];
      y[j + CPL / 2] = x1 * c[j] + x0 * sn[j];
    }
  }
  if (ROT) {
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      if (p.signs[32 * (e / 8) + 8 * li + (e % 8)] < 0) y[e] = -y[e];
#pragma unroll
    for (int hd = 1; hd < CPL; hd *= 2)
#pragma unroll
      for (int e = 0; e < CPL; ++e)
        if (!(e & hd)) {
          const float a = y[e], c = y[e + hd];
          y[e] = a + c;
          y[e + hd] = a - c;
        }
    {
      const bool upper = (li & 1) != 0;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const float other = quad_xor<1>(y[e]);
        y[e] = upper ? other - y[e] : y[e] + other;
      }
    }
    {
      const bool upper = (li & 2) != 0;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const float other = quad_xor<2>(y[e]);
        y[e] = upper ? other - y[e] : y[e] + other;
      }
    }
    const float inv_sqrt_d = (D == 128) ? 0.08838834764831845f : 0.125f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      y[e] = y[e] * inv_sqrt_d;
      // Keep the fp32 product: otherwise the multiply and the later 16-bit
      // conversion fuse into one singly-rounded mixed-precision FMA.
      __asm__ volatile("" : "+v"(y[e]));
    }
  }

  if constexpr (!QUANT) {
    if (valid) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack2<T>(y[8 * v + 2 * e], y[8 * v + 2 * e + 1]);
        *(u32x4*)((uint16_t*)p.y + base + row * rs + 32 * v) = w;
      }
    }
  } else {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) amax = fmaxf(amax, fabsf(y[e]));   // rows >= N hold zeros
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    if (tid == 0) p.scales[((long long)b * p.H + h) * p.nblk + blk] = scale;
    if (valid) {
      uint32_t w[CPL / 4];
#pragma unroll
      for (int q = 0; q < CPL / 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(y[4 * q + e] * inv, -448.0f), 448.0f);
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
        w[q] = (uint32_t)word;
      }
      // chunk 4v + li of the row: 8 code bytes at byte 8·(4v + li)
      uint8_t* dst = (uint8_t*)p.y + base + row * rs;
#pragma unroll
      for (int v = 0; v < NV; ++v) *(u32x2*)(dst + 32 * v) = u32x2{w[2 * v], w[2 * v + 1]};
    }
  }
}

template <typename T, int D, bool ROT, bool QUANT, bool ROPE>
__global__ __launch_bounds__(256) void hadamard_kernel(RotParams p) {
  __shared__ float red[4];
  rotate_block<T, D, ROT, QUANT, ROPE>(p, blockIdx.x, red);
}

// The FP8 prologue of one attention call in one launch: the first nq workgroups
// rotate (and embed, with ROPE) and quantise blocks of Q, the next nk those of K,
// the rest quantise blocks of V.  The tensor is uniform per workgroup, so the
// branch costs nothing; each block is computed exactly as hadamard_kernel would.
struct PrologueParams {
  RotParams q, k, v;
  int nq, nk;
};

template <typename T, int D, bool ROT, bool ROPE>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueParams p) {
  __shared__ float red[4];
  const int bid = blockIdx.x;
  if (bid < p.nq) rotate_block<T, D, ROT, true, ROPE>(p.q, bid, red);
  else if (bid < p.nq + p.nk) rotate_block<T, D, ROT, true, ROPE>(p.k, bid - p.nq, red);
  else rotate_block<T, D, false, true, false>(p.v, bid - p.nq - p.nk, red);
}

template <typename T, int D, bool ROPE>
hipError_t launch_dr(const RotParams& p, dim3 grid, bool rot, bool q, hipStream_t stream) {
  const dim3 block(256);
  if (rot && q) hipLaunchKernelGGL((hadamard_kernel<T, D, true, true, ROPE>), grid, block, 0, stream, p);
  else if (rot) hipLaunchKernelGGL((hadamard_kernel<T, D, true, false, ROPE>), grid, block, 0, stream, p);
  else if (q) hipLaunchKernelGGL((hadamard_kernel<T, D, false, true, ROPE>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((hadamard_kernel<T, D, false, false, ROPE>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const RotateArgs& a, hipStream_t stream) {
  RotParams p;
  p.x = (const uint16_t*)a.x;
  p.y = a.y;
  p.signs = a.signs;
  p.scales = a.scales;
  p.rcos = a.rope_cos;
  p.rsin = a.rope_sin;
  p.N = a.N;
  p.H = a.H;
  p.nblk = (a.N + 63) / 64;
  const dim3 grid((unsigned)((long long)p.nblk * a.H * a.B));
  const bool rot = a.signs != nullptr, q = a.scales != nullptr;
  if (a.rope_cos != nullptr) return launch_dr<T, D, true>(p, grid, rot, q, stream);
  return launch_dr<T, D, false>(p, grid, rot, q, stream);
}

template <typename T>
hipError_t launch_t(const RotateArgs& a, hipStream_t s) {
  return a.d == 128 ? launch_d<T, 128>(a, s) : launch_d<T, 64>(a, s);
}

RotParams rot_params(const void* x, void* y, const int8_t* signs, float* scales, const float* rcos,
                     const float* rsin, int N, int H) {
  RotParams r;
  r.x = (const uint16_t*)x;
  r.y = y;
  r.signs = signs;
  r.scales = scales;
  r.rcos = rcos;
  r.rsin = rsin;
  r.N = N;
  r.H = H;
  r.nblk = (N + 63) / 64;
  return r;
}

template <typename T, int D>
hipError_t launch_prologue_d(const PrologueArgs& a, hipStream_t stream) {
  PrologueParams p;
  p.q = rot_params(a.q, a.q8, a.signs, a.q_scale, a.rope_cos, a.rope_sin, a.N, a.Hq);
  p.k = rot_params(a.k, a.k8, a.signs, a.k_scale, a.rope_cos, a.rope_sin, a.N, a.Hkv);
  p.v = rot_params(a.v, a.v8, nullptr, a.v_scale, nullptr, nullptr, a.N, a.Hkv);
  const long long nblk = (a.N + 63) / 64;
  p.nq = (int)(nblk * a.Hq * a.B);
  p.nk = (int)(nblk * a.Hkv * a.B);
  const dim3 grid((unsigned)(p.nq + 2LL * p.nk)), block(256);
  const bool rot = a.signs != nullptr, rope = a.rope_cos != nullptr;
  if (rot && rope) hipLaunchKernelGGL((prologue_kernel<T, D, true, true>), grid, block, 0, stream, p);
  else if (rot) hipLaunchKernelGGL((prologue_kernel<T, D, true, false>), grid, block, 0, stream, p);
  else if (rope) hipLaunchKernelGGL((prologue_kernel<T, D, false, true>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((prologue_kernel<T, D, false, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_prologue_t(const PrologueArgs& a, hipStream_t s) {
  return a.d == 128 ? launch_prologue_d<T, 128>(a, s) : launch_prologue_d<T, 64>(a, s);
}

}  // namespace

hipError_t launch_hadamard_rotate(const RotateArgs& a, hipStream_t stream) {
  return a.dtype == TATTN_BF16 ? launch_t<Bf16>(a, stream) : launch_t<F16>(a, stream);
}

hipError_t launch_fp8_prologue(const PrologueArgs& a, hipStream_t stream) {
  return a.dtype == TATTN_BF16 ? launch_prologue_t<Bf16>(a, stream) : launch_prologue_t<F16>(a, stream);
}

}  // namespace tattn

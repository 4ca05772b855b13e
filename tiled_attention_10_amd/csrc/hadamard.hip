// Random-sign Hadamard rotation with optional fused FP8 block quantisation,
// for gfx950.  Memory-bound: every element is read once and written once.
//
// One workgroup (4 waves) owns one (batch, head, block of 64 rows).  A row of
// d channels is spread over d/8 lanes with 8 consecutive channels each, so a
// row is one fully coalesced 16-byte-per-lane load.  The Walsh–Hadamard
// butterflies with partner distance 1, 2, 4 run inside a lane; distances 8 ..
// d/2 pair lanes whose chunk indices differ in one bit.  Stages run in
// increasing distance with one fp32 add or subtract each, then one fp32
// multiply by fl32(1/sqrt(d)), so the result is fully determined.
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
  int N, H, nblk;
};

template <typename T, int D, bool ROT, bool QUANT>
__global__ __launch_bounds__(256) void hadamard_kernel(RotParams p) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPI = 64 / LPR;       // rows per wave per step
  constexpr int STEPS = 16 / RPI;     // each wave covers 16 rows
  __shared__ float red[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane % LPR, sub = lane / LPR;
  const int blk = blockIdx.x % p.nblk;
  const int h = (blockIdx.x / p.nblk) % p.H;
  const int b = blockIdx.x / (p.nblk * p.H);
  const long long rs = (long long)p.H * D;     // elements between positions
  const long long base = ((long long)b * p.N * p.H + h) * D + 8 * li;

  uint32_t flip[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) flip[e] = (ROT && p.signs[8 * li + e] < 0) ? 0x80000000u : 0u;

  float y[STEPS][8];
  int rows[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int row = blk * 64 + wave * 16 + s * RPI + sub;
    rows[s] = row;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (row < p.N) raw = *(const u32x4*)(p.x + base + row * rs);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = (e & 1) ? (uint16_t)(raw[e / 2] >> 16) : (uint16_t)(raw[e / 2] & 0xffff);
      y[s][e] = T::to_f32(bits);
    }
    if (ROT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[s][e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, y[s][e]) ^ flip[e]);
#pragma unroll
      for (int hd = 1; hd < 8; hd *= 2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!(e & hd)) {
            const float a = y[s][e], c = y[s][e + hd];
            y[s][e] = a + c;
            y[s][e + hd] = a - c;
          }
#pragma unroll
      for (int ld = 1; ld < LPR; ld *= 2) {
        const bool upper = (li & ld) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float other = __shfl_xor(y[s][e], ld, 64);
          y[s][e] = upper ? other - y[s][e] : y[s][e] + other;
        }
      }
      const float inv_sqrt_d = (D == 128) ? 0.08838834764831845f : 0.125f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[s][e] = y[s][e] * inv_sqrt_d;
        // Keep the fp32 product: otherwise the multiply and the later 16-bit
        // conversion fuse into one singly-rounded mixed-precision FMA.
        __asm__ volatile("" : "+v"(y[s][e]));
      }
    }
  }

  if constexpr (!QUANT) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (rows[s] >= p.N) continue;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack2<T>(y[s][2 * e], y[s][2 * e + 1]);
      *(u32x4*)((uint16_t*)p.y + base + rows[s] * rs) = w;
    }
  } else {
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[s][e]));  // rows >= N hold zeros
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    if (tid == 0) p.scales[((long long)b * p.H + h) * p.nblk + blk] = scale;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (rows[s] >= p.N) continue;
      u32x2 w;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(y[s][4 * half + e] * inv, -448.0f), 448.0f);
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
        w[half] = (uint32_t)word;
      }
      *(u32x2*)((uint8_t*)p.y + base + rows[s] * rs) = w;
    }
  }
}

template <typename T, int D>
hipError_t launch_d(const RotateArgs& a, hipStream_t stream) {
  RotParams p;
  p.x = (const uint16_t*)a.x;
  p.y = a.y;
  p.signs = a.signs;
  p.scales = a.scales;
  p.N = a.N;
  p.H = a.H;
  p.nblk = (a.N + 63) / 64;
  const dim3 grid((unsigned)((long long)p.nblk * a.H * a.B)), block(256);
  const bool rot = a.signs != nullptr, q = a.scales != nullptr;
  if (rot && q) hipLaunchKernelGGL((hadamard_kernel<T, D, true, true>), grid, block, 0, stream, p);
  else if (rot) hipLaunchKernelGGL((hadamard_kernel<T, D, true, false>), grid, block, 0, stream, p);
  else if (q) hipLaunchKernelGGL((hadamard_kernel<T, D, false, true>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((hadamard_kernel<T, D, false, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const RotateArgs& a, hipStream_t s) {
  return a.d == 128 ? launch_d<T, 128>(a, s) : launch_d<T, 64>(a, s);
}

}  // namespace

hipError_t launch_hadamard_rotate(const RotateArgs& a, hipStream_t stream) {
  return a.dtype == TATTN_BF16 ? launch_t<Bf16>(a, stream) : launch_t<F16>(a, stream);
}

}  // namespace tattn

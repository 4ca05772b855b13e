// Device-side helpers shared by the gfx950 kernels: vector types, matrix-core
// wrappers and small utilities.  CDNA4 only (wave64, MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element traits: storage as raw 16-bit words, 8-element vectors for
// the 32x32x16 matrix-core instructions.
struct Bf16 {
  typedef bf16x8 vec8;
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // round-to-nearest-even fp32 -> bf16 bits
  __device__ static inline uint16_t from_f32(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_f32(uint16_t x) {
    return (float)__builtin_bit_cast(__bf16, x);
  }
  // two fp32 -> one dword of bf16 (low half = a), one packed RNE conversion
  __device__ static inline uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
  __device__ static inline vec8 pack8(const float* x) {
    u32x4 w = {pack(x[0], x[1]), pack(x[2], x[3]), pack(x[4], x[5]), pack(x[6], x[7])};
    return __builtin_bit_cast(vec8, w);
  }
  // acc + sum of the 8 elements (four 2-element dot products with ones, fp32 accumulate)
  // (Pairs are taken with shufflevector: bit-casting single elements of a 4-dword
  // vector to bf16x2 was miscompiled into four uses of element 0.)
  __device__ static inline float sum8(vec8 v, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
    return acc;
  }
};

struct F16 {
  typedef f16x8 vec8;
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint16_t from_f32(float x) {
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_f32(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
  __device__ static inline uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
  __device__ static inline vec8 pack8(const float* x) {
    u32x4 w = {pack(x[0], x[1]), pack(x[2], x[3]), pack(x[4], x[5]), pack(x[6], x[7])};
    return __builtin_bit_cast(vec8, w);
  }
  __device__ static inline float sum8(vec8 v, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
    return acc;
  }
};

// Pack two fp32 values into one dword of 16-bit codes (low half = a).
template <typename T>
__device__ inline uint32_t pack2(float a, float b) {
  return T::pack(a, b);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x on the ordinary VALU pipe, for finite x: the split x = n + f with
// n = floor(x) and f = fract(x) in [0, 1) (Cody and Waite's range reduction),
// 2^f from the cubic 1 + f·(a1 + f·(a2 + f·a3)), and the result 2^n·P(f) by
// v_ldexp.  a1..a3 minimise the largest relative error of P(f)/2^f on [0, 1]
// under P(0) = 1 and P(1) = 2 (a linear program on a dense grid, see
// exp2_poly.py): 1.04e-4 evaluated in fp32.  The constraints make the result
// exact wherever x is an integer and continuous across integers.  A kernel
// evaluates part of its exponentials this way so that they run beside the
// v_exp_f32 of the others, which the transcendental unit issues at a fraction
// of the VALU rate.  Results below 2^-149 flush to zero and large x overflow to
// +inf, as for v_exp_f32; x = ±inf or NaN is not allowed.
constexpr float kExp2A1 = 0x1.640ea8p-1f;
constexpr float kExp2A2 = 0x1.cf7a66p-3f;
constexpr float kExp2A3 = 0x1.4095eap-4f;
__device__ inline float exp2_valu(float x) {
  const float f = __builtin_amdgcn_fractf(x);
  int n;   // floor(x) as an integer in one instruction (saturates for huge |x|)
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(n) : "v"(x));
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(kExp2A3, f, kExp2A2), f, kExp2A1), f, 1.0f);
  return __builtin_amdgcn_ldexpf(p, n);
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ inline float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(a, b, c) in one v_max3_f32.  (fmaxf would first quiet signalling NaNs
// with an extra v_max of each operand with itself; the scores this serves are
// matrix-core results or -inf, never signalling NaNs.)
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max(x, x of lane ^ 32) without an LDS round trip: v_permlane32_swap exchanges the
// upper half of one register with the lower half of the other, leaving the lower
// halves of x in both halves of ``lo`` and the upper halves in both halves of ``hi``.
// The nops cover the VALU-write / permlane-read and permlane-write / VALU-read
// hazards.  (The compiler builtin returns its first result for both outputs here.)
__device__ inline float max_xor32(float x) {
  float lo = x, hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
  return max3f(lo, hi, hi);
}

}  // namespace tattn

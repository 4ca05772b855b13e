// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tattn {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  // fp8 path only: per-(batch, head, 64-row block) scales
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int B, N, Hq, Hkv, d;
  float scale;   // softmax scale (> 0)
  int causal;
  int dtype;     // storage type of q/k/v (16-bit path) or of o (fp8 path)
};

struct RotateArgs {
  const void* x;
  void* y;
  const int8_t* signs;
  float* scales;
  const float* rope_cos;   // rotary tables [N, d/2] or NULL (no rotary embedding)
  const float* rope_sin;
  int B, N, H, d;
  int dtype;
};

// FP8 prologue of one attention call: Q and K rotated (and embedded) and quantised,
// V quantised, in one launch.
struct PrologueArgs {
  const void* q;            // [B, N, Hq, d] 16-bit
  const void* k;            // [B, N, Hkv, d]
  const void* v;
  const int8_t* signs;      // [d] or NULL (no rotation)
  const float* rope_cos;    // [N, d/2] or NULL (no rotary embedding)
  const float* rope_sin;
  uint8_t* q8;              // E4M3 codes, same layouts
  uint8_t* k8;
  uint8_t* v8;
  float* q_scale;           // [B, H, ceil(N/64)]
  float* k_scale;
  float* v_scale;
  int B, N, Hq, Hkv, d;
  int dtype;
};

// Decode step over an FP8 block-quantised KV cache.
struct DecodeArgs {
  const void* q;            // [B, Hq, d] 16-bit
  const uint8_t* k;         // [B, Nmax, Hkv, d] E4M3 codes
  const uint8_t* v;
  const float* k_scale;     // [B, Hkv, ceil(Nmax/64)]
  const float* v_scale;
  const int* seqlens;       // [B] device
  void* o;                  // [B, Hq, d] 16-bit
  float* lse;               // [B, Hq] or NULL
  void* workspace;          // plan_decode(...).ws_bytes bytes
  int B, Nmax, Hq, Hkv, d;
  float scale;
  int dtype;
};

// Chunking of the cached sequence into workgroups, and the workspace it needs
// (a function of the shapes only).
struct DecodePlan {
  int nhg;                  // groups of up to 16 query heads per KV head
  int chunk;                // keys per workgroup (multiple of 256)
  int nc;                   // chunks per sequence = ceil(Nmax / chunk)
  long long ws_o_floats;    // partial outputs [B, Hq, nc, d]; then [B, Hq, nc, 2] (max, denominator)
  size_t ws_bytes;
};
DecodePlan plan_decode(int B, int Nmax, int Hq, int Hkv);

// Compute units of the current device (cached per device); persistent grids hold
// one workgroup per CU.
int device_cu_count();

// Each returns hipSuccess or the launch error.
hipError_t launch_attn_fwd16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_fp8(const AttnArgs& a, hipStream_t stream);
hipError_t launch_hadamard_rotate(const RotateArgs& a, hipStream_t stream);
hipError_t launch_fp8_prologue(const PrologueArgs& a, hipStream_t stream);
hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace tattn

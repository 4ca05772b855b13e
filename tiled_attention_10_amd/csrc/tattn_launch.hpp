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

// Compute units of the current device (cached per device); persistent grids hold
// one workgroup per CU.
int device_cu_count();

// Each returns hipSuccess or the launch error.
hipError_t launch_attn_fwd16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_fp8(const AttnArgs& a, hipStream_t stream);
hipError_t launch_hadamard_rotate(const RotateArgs& a, hipStream_t stream);

}  // namespace tattn

// Shader-clock probe for the benchmark (not part of the attention library's ABI).
//
// One wave spins for a bounded wall time and reads the shader cycle counter
// (s_memtime) and the constant 100 MHz reference counter (s_memrealtime) at both
// ends; the ratio gives the clock the compute unit ran at meanwhile.  Launched on a
// second stream just before a series of attention launches, it samples the clock
// under that load.  The loop ends after ``ticks`` reference ticks or ``max_iter``
// iterations, whichever comes first, so every launch terminates.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long ticks, unsigned long long max_iter,
                                                         unsigned long long* out) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r1 = r0, c1 = c0;
  for (unsigned long long i = 0; i < max_iter && r1 - r0 < ticks; ++i) {
    __builtin_amdgcn_s_sleep(10);
    r1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x == 0) {
    out[0] = r1 - r0;
    out[1] = c1 - c0;
  }
}

extern "C" int tattn_clock_probe(unsigned long long ticks, unsigned long long max_iter, unsigned long long* out,
                                 void* stream) {
  if (!out || ticks == 0 || max_iter == 0) return 1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ticks, max_iter, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

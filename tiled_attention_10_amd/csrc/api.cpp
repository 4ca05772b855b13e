// C ABI of libtattn: argument validation, error reporting and dispatch to the
// gfx950 kernels.  All checks run on the host before any HIP call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "tattn.h"
#include "tattn_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Element counts must stay addressable with 64-bit offsets and the grid with
// 32-bit workgroup ids.
bool too_large(long long B, long long N, long long H, long long d) {
  const long long lim = (long long)1 << 40;
  return B > lim / N || B * N > lim / H || B * N * H > lim / d;
}

int check_shape(int B, int N, int Hq, int Hkv, int d) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1)
    return fail(TATTN_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d N=%d Hq=%d Hkv=%d)", B, N, Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(TATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (too_large(B, N, Hq, d > 0 ? d : 1))
    return fail(TATTN_ERR_INVALID_ARG, "tensor too large (B=%d N=%d H=%d d=%d)", B, N, Hq, d);
  const long long grid = (long long)((N + 127) / 128) * Hq * B;
  if (grid > 0x7fffffffLL) return fail(TATTN_ERR_INVALID_ARG, "too many query tiles");
  return TATTN_OK;
}

// The kernels address a 64-key K/V tile with a 32-bit byte offset per lane on top
// of a 64-bit tile base: 64 rows of Hkv heads must span less than 4 GiB.
int check_tile_span(int Hkv, int row_bytes) {
  if ((long long)Hkv * row_bytes * 64 >= (1LL << 32))
    return fail(TATTN_ERR_INVALID_ARG, "Hkv = %d: 64 key rows of all KV heads must span < 4 GiB", Hkv);
  return TATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TATTN_OK;
  return fail(TATTN_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

int rotate_common(const void* x, void* y, const float* rope_cos, const float* rope_sin, const int8_t* signs,
                  float* scales_out, int B, int N, int H, int d, int in_dtype, void* stream) {
  if (!x || !y) return fail(TATTN_ERR_INVALID_ARG, "null tensor pointer");
  if (int s = check_shape(B, N, H, H, d)) return s;
  if (d != 64 && d != 128) return fail(TATTN_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (in_dtype != TATTN_F16 && in_dtype != TATTN_BF16)
    return fail(TATTN_ERR_UNSUPPORTED, "in_dtype %d", in_dtype);
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(TATTN_ERR_MISALIGNED, "x, y must be 16-byte aligned");
  if (scales_out && !aligned(scales_out, 4)) return fail(TATTN_ERR_MISALIGNED, "scales_out must be 4-byte aligned");
  tattn::RotateArgs a{};
  a.x = x; a.y = y; a.signs = signs; a.scales = scales_out;
  a.rope_cos = rope_cos; a.rope_sin = rope_sin;
  a.B = B; a.N = N; a.H = H; a.d = d; a.dtype = in_dtype;
  return hip_status(tattn::launch_hadamard_rotate(a, (hipStream_t)stream), "rotation launch");
}

// Device scratch of attn_decode_fp8kv_noalloc, for callers that cannot allocate:
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address: the per-device address comes from
// hipGetSymbolAddress on the first call on each device.
constexpr size_t kNoAllocScratchBytes = TATTN_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

// This device's address of ``scratch`` (looked up once per device), or nullptr with
// the failure recorded in the last-error string.
void* noalloc_scratch() {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    fail(TATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fail(TATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

// Checks and launch of one decode step with the given workspace (validated
// here except for the workspace itself, which the callers check).
int decode_common(const void* q, const uint8_t* k_cache, const uint8_t* v_cache, const float* k_scale,
                  const float* v_scale, const int32_t* seqlens, void* o, float* lse, int B, int Nmax, int Hq,
                  int Hkv, int d, float softmax_scale, int dtype, tattn::DecodePlan* plan) {
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !seqlens || !o)
    return fail(TATTN_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || Nmax < 1 || Hq < 1 || Hkv < 1)
    return fail(TATTN_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d Nmax=%d Hq=%d Hkv=%d)", B, Nmax, Hq, Hkv);
  if (Hq % Hkv != 0) return fail(TATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (d != 128) return fail(TATTN_ERR_UNSUPPORTED, "head dim %d (the decode path supports 128)", d);
  if (dtype != TATTN_F16 && dtype != TATTN_BF16) return fail(TATTN_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (too_large(B, Nmax, Hq, d) || too_large(B, Nmax, Hkv, d) || Hkv > 65536 || B > 65535)
    return fail(TATTN_ERR_INVALID_ARG, "sizes too large (B=%d Nmax=%d Hq=%d Hkv=%d)", B, Nmax, Hq, Hkv);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(TATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
    return fail(TATTN_ERR_MISALIGNED, "q, caches and o must be 16-byte aligned");
  if (!aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(seqlens, 4) || (lse && !aligned(lse, 4)))
    return fail(TATTN_ERR_MISALIGNED, "scales, seqlens and lse must be 4-byte aligned");
  *plan = tattn::plan_decode(B, Nmax, Hq, Hkv);
  if ((long long)Hkv * plan->nhg > 65535) return fail(TATTN_ERR_INVALID_ARG, "too many head groups");
  return TATTN_OK;
}

int decode_launch(const void* q, const uint8_t* k_cache, const uint8_t* v_cache, const float* k_scale,
                  const float* v_scale, const int32_t* seqlens, void* o, float* lse, void* workspace, int B,
                  int Nmax, int Hq, int Hkv, int d, float softmax_scale, int dtype, void* stream) {
  tattn::DecodeArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.k_scale = k_scale; a.v_scale = v_scale;
  a.seqlens = seqlens; a.o = o; a.lse = lse; a.workspace = workspace;
  a.B = B; a.Nmax = Nmax; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.scale = softmax_scale; a.dtype = dtype;
  return hip_status(tattn::launch_attn_decode(a, (hipStream_t)stream), "attn_decode_fp8kv launch");
}

}  // namespace

namespace tattn {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace tattn

extern "C" {

const char* tattn_status_string(int status) {
  switch (status) {
    case TATTN_OK: return "ok";
    case TATTN_ERR_INVALID_ARG: return "invalid argument";
    case TATTN_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case TATTN_ERR_MISALIGNED: return "misaligned pointer";
    case TATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* tattn_last_error(void) { return g_last_error; }

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int N,
             int Hq, int Hkv, int d, float softmax_scale, int causal, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (!q || !k || !v || !o) return fail(TATTN_ERR_INVALID_ARG, "null tensor pointer");
  if (int s = check_shape(B, N, Hq, Hkv, d)) return s;
  if (d != 64 && d != 128) return fail(TATTN_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (dtype != TATTN_F16 && dtype != TATTN_BF16) return fail(TATTN_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (int s = check_tile_span(Hkv, 2 * d)) return s;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(TATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(TATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(TATTN_ERR_MISALIGNED, "q, k, v, o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(TATTN_ERR_MISALIGNED, "lse must be 4-byte aligned");
  tattn::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.N = N; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
  a.scale = softmax_scale; a.causal = causal; a.dtype = dtype;
  return hip_status(tattn::launch_attn_fwd16(a, (hipStream_t)stream), "attn_fwd launch");
}

int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                 const float* k_scale, const float* v_scale, void* o, float* lse, int B, int N,
                 int Hq, int Hkv, int d, float softmax_scale, int causal, int out_dtype,
                 void* stream) {
  g_last_error[0] = '\0';
  if (!q8 || !k8 || !v8 || !o || !q_scale || !k_scale || !v_scale)
    return fail(TATTN_ERR_INVALID_ARG, "null tensor pointer");
  if (int s = check_shape(B, N, Hq, Hkv, d)) return s;
  if (d != 128) return fail(TATTN_ERR_UNSUPPORTED, "head dim %d (fp8 path supports 128)", d);
  if (N > 262144) return fail(TATTN_ERR_UNSUPPORTED, "N = %d > 262144 on the fp8 path", N);
  if (int s = check_tile_span(Hkv, d)) return s;
  if (out_dtype != TATTN_F16 && out_dtype != TATTN_BF16)
    return fail(TATTN_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(TATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(TATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16))
    return fail(TATTN_ERR_MISALIGNED, "q8, k8, v8, o must be 16-byte aligned");
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) || (lse && !aligned(lse, 4)))
    return fail(TATTN_ERR_MISALIGNED, "scales and lse must be 4-byte aligned");
  tattn::AttnArgs a{};
  a.q = q8; a.k = k8; a.v = v8; a.o = o; a.lse = lse;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.B = B; a.N = N; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
  a.scale = softmax_scale; a.causal = causal; a.dtype = out_dtype;
  return hip_status(tattn::launch_attn_fwd_fp8(a, (hipStream_t)stream), "attn_fwd_fp8 launch");
}


int hadamard_rotate(const void* x, void* y, const int8_t* signs, float* scales_out, int B, int N,
                    int H, int d, int in_dtype, void* stream) {
  g_last_error[0] = '\0';
  return rotate_common(x, y, nullptr, nullptr, signs, scales_out, B, N, H, d, in_dtype, stream);
}

int rope_hadamard_rotate(const void* x, void* y, const float* rope_cos, const float* rope_sin,
                         const int8_t* signs, float* scales_out, int B, int N, int H, int d,
                         int in_dtype, void* stream) {
  g_last_error[0] = '\0';
  if (!rope_cos || !rope_sin) return fail(TATTN_ERR_INVALID_ARG, "null rotary table");
  if (!aligned(rope_cos, 16) || !aligned(rope_sin, 16))
    return fail(TATTN_ERR_MISALIGNED, "rotary tables must be 16-byte aligned");
  return rotate_common(x, y, rope_cos, rope_sin, signs, scales_out, B, N, H, d, in_dtype, stream);
}

int fp8_prologue(const void* q, const void* k, const void* v, const int8_t* signs, const float* rope_cos,
                 const float* rope_sin, uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_scale, float* k_scale,
                 float* v_scale, int B, int N, int Hq, int Hkv, int d, int in_dtype, void* stream) {
  g_last_error[0] = '\0';
  if (!q || !k || !v || !q8 || !k8 || !v8) return fail(TATTN_ERR_INVALID_ARG, "null tensor pointer");
  if (!q_scale || !k_scale || !v_scale) return fail(TATTN_ERR_INVALID_ARG, "null scale pointer");
  if (!rope_cos != !rope_sin) return fail(TATTN_ERR_INVALID_ARG, "give both rotary tables or neither");
  if (int s = check_shape(B, N, Hq, Hkv, d)) return s;
  if (d != 64 && d != 128) return fail(TATTN_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (in_dtype != TATTN_F16 && in_dtype != TATTN_BF16)
    return fail(TATTN_ERR_UNSUPPORTED, "in_dtype %d", in_dtype);
  if ((long long)((N + 63) / 64) * (Hq + 2LL * Hkv) * B > 0x7fffffffLL)
    return fail(TATTN_ERR_INVALID_ARG, "too many row blocks");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q8, 16) || !aligned(k8, 16) ||
      !aligned(v8, 16))
    return fail(TATTN_ERR_MISALIGNED, "tensors and codes must be 16-byte aligned");
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return fail(TATTN_ERR_MISALIGNED, "scales must be 4-byte aligned");
  if (rope_cos && (!aligned(rope_cos, 16) || !aligned(rope_sin, 16)))
    return fail(TATTN_ERR_MISALIGNED, "rotary tables must be 16-byte aligned");
  tattn::PrologueArgs a{};
  a.q = q; a.k = k; a.v = v; a.signs = signs; a.rope_cos = rope_cos; a.rope_sin = rope_sin;
  a.q8 = q8; a.k8 = k8; a.v8 = v8; a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.B = B; a.N = N; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.dtype = in_dtype;
  return hip_status(tattn::launch_fp8_prologue(a, (hipStream_t)stream), "fp8 prologue launch");
}

size_t attn_decode_fp8kv_workspace_size(int B, int Nmax, int Hq, int Hkv, int d) {
  if (B < 1 || Nmax < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || d != 128) return 0;
  if (too_large(B, Nmax, Hq, d) || too_large(B, Nmax, Hkv, d)) return 0;
  return tattn::plan_decode(B, Nmax, Hq, Hkv).ws_bytes;
}

int attn_decode_fp8kv(const void* q, const uint8_t* k_cache, const uint8_t* v_cache, const float* k_scale,
                      const float* v_scale, const int32_t* seqlens, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, int B, int Nmax, int Hq, int Hkv, int d, float softmax_scale,
                      int dtype, void* stream) {
  g_last_error[0] = '\0';
  tattn::DecodePlan pl{};
  if (int s = decode_common(q, k_cache, v_cache, k_scale, v_scale, seqlens, o, lse, B, Nmax, Hq, Hkv, d,
                            softmax_scale, dtype, &pl))
    return s;
  if (!workspace) return fail(TATTN_ERR_INVALID_ARG, "null workspace");
  if (!aligned(workspace, 16)) return fail(TATTN_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (workspace_bytes < pl.ws_bytes)
    return fail(TATTN_ERR_INVALID_ARG, "workspace of %zu bytes < %zu required", workspace_bytes, pl.ws_bytes);
  return decode_launch(q, k_cache, v_cache, k_scale, v_scale, seqlens, o, lse, workspace, B, Nmax, Hq, Hkv, d,
                       softmax_scale, dtype, stream);
}

int attn_decode_fp8kv_noalloc(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* seqlens, void* o,
                              float* lse, int B, int Nmax, int Hq, int Hkv, int d, float softmax_scale,
                              int dtype, void* stream) {
  g_last_error[0] = '\0';
  tattn::DecodePlan pl{};
  if (int s = decode_common(q, k_cache, v_cache, k_scale, v_scale, seqlens, o, lse, B, Nmax, Hq, Hkv, d,
                            softmax_scale, dtype, &pl))
    return s;
  if (pl.ws_bytes > kNoAllocScratchBytes)
    return fail(TATTN_ERR_INVALID_ARG, "these sizes need %zu bytes of decode scratch; the fixed scratch holds %zu",
                pl.ws_bytes, kNoAllocScratchBytes);
  void* ws = noalloc_scratch();
  if (ws == nullptr) return TATTN_ERR_HIP;
  return decode_launch(q, k_cache, v_cache, k_scale, v_scale, seqlens, o, lse, ws, B, Nmax, Hq, Hkv, d,
                       softmax_scale, dtype, stream);
}

}  // extern "C"

// Pipeline helpers shared by the attention kernels: LDS-DMA loads, fence-free
// barrier, explicit vector-memory waits and the key-row order of the score MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tattn {

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
// for the load before every later LDS read) nor counts it: the kernels wait for
// these loads explicitly with wait_vmcnt before each barrier.  M0 is only
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

}  // namespace tattn

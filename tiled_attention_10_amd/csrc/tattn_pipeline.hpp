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

// One 16-byte LDS-DMA load per lane: lane i's 16 bytes from ``base`` +
// ``offset`` (wave-uniform base, 32-bit per-lane byte offset) land at LDS byte
// address ``lds_addr`` + 16·i.  Issued as inline assembly so that the compiler
// neither treats it as an aliasing LDS store (which would make it wait for the
// load before every later LDS read) nor counts it: the kernels wait for these
// loads explicitly with wait_vmcnt before each barrier.  M0 is only written here
// and consumed by the next instruction.
__device__ inline void lds_dma16(const void* base, uint32_t offset, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(offset), "s"(base)
               : "memory");
}

// Workgroup barrier without a memory fence: the LDS-DMA loads are published by
// the explicit wait_vmcnt before it; the asm also keeps the compiler from
// moving LDS accesses across it.
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Epilogue store of one wave's 32 x 128 output rows.  The Oᵀ accumulator gives
// each lane one row and 4-element runs of channels, which would make every store
// instruction touch 32 rows with 16 bytes each; instead the wave stages its rows
// in an 8 KB LDS block (16-byte chunk c of row r kept at chunk c ^ (r % 16), so
// both the 8-byte writes and the 16-byte reads are free of bank conflicts) and
// writes them back 16 bytes per lane, four whole 256-byte rows per instruction.
//   oacc[vq][4a + e] = O[row l%32][32vq + 8a + 4(l/32) + e] (already normalised
//   by ``inv``); ``out`` points at row 0 of the wave, rows ``rowstride`` elements
//   apart; only rows < ``nvalid`` are written.
template <typename T, typename F32x16>
__device__ inline void store_rows(__attribute__((address_space(3))) char* stage, const F32x16 (&oacc)[4],
                                  float inv, int lane, uint16_t* out, long long rowstride, int nvalid) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int vq = 0; vq < 4; ++vq)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int u = 8 * vq + 2 * a + hh;        // 8-byte unit within the row
      const int c = u >> 1;
      u32x2_t w;
      w[0] = T::pack(oacc[vq][4 * a + 0] * inv, oacc[vq][4 * a + 1] * inv);
      w[1] = T::pack(oacc[vq][4 * a + 2] * inv, oacc[vq][4 * a + 3] * inv);
      *(__attribute__((address_space(3))) u32x2_t*)(stage + r * 256 + 16 * (c ^ (r & 15)) + 8 * (u & 1)) = w;
    }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = 64 * i + lane, row = idx >> 4, c = idx & 15;
    const u32x4_t v = *(__attribute__((address_space(3))) u32x4_t*)(stage + row * 256 + 16 * (c ^ (row & 15)));
    if (row < nvalid) *(u32x4_t*)(out + row * rowstride + 8 * c) = v;
  }
}

// Scheduling order of a stream of N matrix-core products that each consume R LDS
// reads: the reads of the first A products, then each product followed by the
// reads of the product A places later, so every read is issued A products ahead
// of its use.  (Masks: 0x100 LDS read, 0x008 MFMA.)
template <int N, int R, int A, int I = 0>
__device__ inline void mma_read_order() {
  constexpr int AA = A < N ? A : N;
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, R * AA, 0);
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I + AA < N) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    mma_read_order<N, R, A, I + 1>();
  }
}

}  // namespace tattn

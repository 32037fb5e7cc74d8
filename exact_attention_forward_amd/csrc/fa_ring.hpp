// Helpers for streaming tiles of 128-byte rows from global memory into LDS
// with direct global-to-LDS loads (global_load_lds_*), shared by the hd-64
// kernels.  The loads are issued as inline assembly, so the compiler neither
// tracks nor waits for them: a kernel waits with wait_vm() and makes the data
// visible to the other waves with a barrier.  On this architecture the vector
// memory counter also counts stores and decrements in issue order, so a wait
// for a copy also waits for every load and store issued before it.
#pragma once
#include <hip/hip_runtime.h>

namespace fa {

// Granule slot of column granule c in LDS row r of a 128-byte-row tile:
// c ^ swz128(r).  Rows 0..7 map to 0, 2, 4, 6, 1, 3, 5, 7: eight consecutive
// rows reading one granule hit eight slots, and four consecutive rows reading
// two adjacent granules (the transposing reads) hit eight slots too.
__device__ __forceinline__ int swz128(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

typedef __attribute__((address_space(3))) void lds_void_t;

// A pointer that is equal across the wave, moved to scalar registers (for
// the scalar base operand of the copies above).
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const unsigned long long v = (unsigned long long)(uintptr_t)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (P*)(uintptr_t)(((unsigned long long)hi << 32) | lo);
}

// One 16-byte global-to-LDS copy per lane: lane i writes LDS bytes
// [dst + 16 i, dst + 16 i + 16), dst uniform across the wave.  Issued as
// inline assembly so that the compiler does not track it (it would drain every
// outstanding copy before LDS reads it cannot prove disjoint from them);
// callers wait for completion explicitly.
__device__ __forceinline__ void lds_copy16(const void* src, unsigned dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory", "m0");
}
// The same copy from a wave-uniform base address plus a per-lane 32-bit byte
// offset (no per-lane 64-bit address arithmetic).  base and dst must be equal
// across the wave; the read-first-lane moves cost nothing when the compiler
// already holds them in scalar registers.
__device__ __forceinline__ void lds_copy16(const void* base, unsigned off, unsigned dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(__builtin_amdgcn_readfirstlane(dst))
               : "memory", "m0");
}

// One 4-byte global-to-LDS copy per lane: lane i writes LDS bytes
// [dst + 4 i, dst + 4 i + 4).
__device__ __forceinline__ void lds_copy4(const void* base, unsigned off, unsigned dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(__builtin_amdgcn_readfirstlane(dst))
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) (the other counters unconstrained) for the counts the
// kernels use: multiples of 4 or 5 up to 15; anything else waits for all.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

}  // namespace fa

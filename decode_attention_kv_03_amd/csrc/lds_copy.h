// Direct global -> LDS copies (gfx950 global_load_lds_dwordx4) shared by the
// bf16/fp8 decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvattn {

// 16-byte global -> LDS copy of every lane: lane i's bytes land at
// lds_base + 16 * i (lds_base is wave-uniform, taken through M0).  The
// non-temporal hint marks the cache stream as read-once.  Issued as inline
// assembly so the compiler does not treat every later LDS read as a possible
// alias of the copy; M0 is written here and nowhere else in these kernels.
// The copies are counted by vmcnt; callers wait for them explicitly.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// The same copy addressed as a wave-uniform 64-bit base plus a per-lane
// 32-bit byte offset, so the per-tile address arithmetic is scalar.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// Wait until at most `N` of this wave's copies are outstanding, then
// synchronise the workgroup (LDS reads of every wave complete first).
template <int N>
__device__ __forceinline__ void wait_copies_and_sync() {
  static_assert(N == 0 || N == 8 || N == 16, "copy counts come in tiles of 8");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace kvattn

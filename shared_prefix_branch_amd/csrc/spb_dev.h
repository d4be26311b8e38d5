// spb_dev.h -- device helpers shared by the attention and lm-head kernels
// (gfx950): asynchronous global -> LDS copies and the waits that order them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spb {

// Asynchronous copy of 16 bytes per lane from global memory into LDS: lane i
// writes lds + 16 i (lds: a wave-uniform LDS byte address).  Issued from
// inline assembly so that the compiler does not wait on it before unrelated
// LDS reads; callers order it with explicit vmcnt waits and barriers.  m0
// (the LDS address operand) is saved and restored around the copy.
__device__ inline void dma16(const void *base, uint32_t voff, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}

// The same for 4 bytes per lane: lane i writes lds + 4 i.
__device__ inline void dma4(const void *base, uint32_t voff, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// vmcnt(0) issued through the compiler's own builtin, so its wait-count
// tracking knows that every load it issued so far has landed.  The copies
// above are invisible to that tracking; without this, a register loaded
// before a copy loop is waited for at its first use inside the loop, with an
// s_waitcnt vmcnt(0) that runs on every trip and so also waits for the
// copies of later stages.  (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15.)
__device__ inline void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Barrier for an LDS hand-off that leaves outstanding global loads in flight.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS byte address of a shared-memory object, uniform over the wave.
template <typename T>
__device__ inline uint32_t lds_addr(T *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)p);
}

}  // namespace spb

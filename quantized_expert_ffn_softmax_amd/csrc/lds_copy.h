// Global-to-LDS copies (gfx950 LDS DMA) that the kernels wait for themselves.
//
// A copy moves 16 (or 4) bytes per lane from a per-lane global address to LDS
// byte lds + 16 l (or + 4 l) of lane l, with no register result.  They are
// written as assembly so that the compiler's wait insertion neither counts
// them nor treats every later LDS read as possibly overlapping them (it would
// wait for every load in flight); a kernel that issues them waits with an
// explicit s_waitcnt vmcnt before the barrier that publishes the data.  M0
// (the LDS base, uniform across the wave) is saved and restored around each.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ inline uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)(p);
}

__device__ inline void lds_copy16(const void *src, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
      : "memory");
}

__device__ inline void lds_copy4(const void *src, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
      : "memory");
}

// The same with a wave-uniform 64-bit base and a per-lane 32-bit byte offset
// (the address is base + off): one VGPR per copy address instead of two.
// (readfirstlane returns int: each half goes through uint32_t so that the low
// half is zero-extended, never sign-extended into the high one)
__device__ inline uint64_t uniform_base(const void *base) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

__device__ inline void lds_copy16_off(uint64_t base, uint32_t off, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
      : "memory");
}

__device__ inline void lds_copy4_off(uint64_t base, uint32_t off, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base)
      : "memory");
}

}  // namespace moe

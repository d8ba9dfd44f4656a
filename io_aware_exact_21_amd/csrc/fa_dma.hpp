// Direct global -> LDS copies and LDS addressing shared by the streaming kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace dma {

typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ const lds_u8* lds_ptr(unsigned a) { return (const lds_u8*)(uintptr_t)a; }

// Wave-level copies: lane i's 16 (copy16) or 4 (copy4) bytes at base + voff_i land at
// LDS byte lds + 16 i (4 i); base is wave-uniform in SGPRs. The LDS destination travels
// in m0, which the asm saves to a scratch SGPR first and restores after issuing the copy
// (the instruction reads m0 when it issues), so m0 is unchanged for any code around it.
// Issued as inline assembly so the compiler does not order later LDS reads of other ring
// stages behind it; completion is tracked with wait_vmcnt plus a barrier.
__device__ __forceinline__ void copy16(const void* base, unsigned voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(m)
      : "memory");
}
__device__ __forceinline__ void copy4(const void* base, unsigned voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(m)
      : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace dma
}  // namespace fa

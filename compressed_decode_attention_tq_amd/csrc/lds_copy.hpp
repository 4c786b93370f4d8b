// Direct global-to-LDS copies and counted waits on them (gfx950), shared by the
// kernels that stream tiles through an LDS ring.
#pragma once

#include <hip/hip_runtime.h>

namespace tq {

typedef __attribute__((address_space(3))) unsigned char lds_byte;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// One 16-byte copy per active lane from global memory into LDS at dst + 16*lane
// (inline asm so the compiler's waits do not drain on it; awaited with
// wait_vmcnt).  dst is wave-uniform.  M0 is set inside the same asm statement
// that uses it; the compiler warns that it treats M0 as reserved, and the
// kernels that use this copy use M0 nowhere else (checked in the generated
// code), so nothing else depends on its value.
__device__ __forceinline__ void copy_to_lds(const void* src, void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<unsigned long>((lds_byte*)dst)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
               : "memory", "m0");
}

}  // namespace tq

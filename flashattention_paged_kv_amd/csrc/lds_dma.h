// Direct global -> LDS loads (gfx950 global_load_lds_*) shared by the extend
// kernels, which stage K/V tiles through LDS.
#pragma once

#include "device_common.h"

namespace pkv {

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(lds_char*)(const_cast<char*>(p));
}

// Global -> LDS loads.  Written as inline assembly so the compiler neither
// counts them nor orders LDS reads of other stages behind them; the kernel
// waits for them explicitly (wait_vmem<N>) before publishing a stage.  Each
// 64-lane instruction writes consecutive LDS bytes from `lds` (M0), lane i at
// lds + i * size.  M0 is used by nothing else in the kernels that use them.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 15, "vmcnt wait depth");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace pkv

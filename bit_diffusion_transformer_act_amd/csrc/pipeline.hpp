// LDS-DMA pipeline helpers shared by the GEMM kernels.
#pragma once

#include "common.hpp"

namespace svdq {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS-DMA loads: lane l's bytes land at lds_base + l * size. The LDS base is
// wave-uniform (M0); the instruction has no destination register. Completion
// is tracked with vmcnt by the caller (waitvm) before the barrier that
// publishes the data.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base)
               : "memory", "m0");
}
// Same, with a wave-uniform 64-bit base (SGPRs) and a per-lane 32-bit offset.
__device__ __forceinline__ void dma16_so(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_so(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_base)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void waitvm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// vmcnt <= N and every LDS access of this wave completed
template <int N>
__device__ __forceinline__ void waitvm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

// Code rows are 64 bytes (one K step of 128 codes); their four 16-byte chunks
// are XOR-swizzled so that 16 consecutive rows read at one chunk index touch 16
// distinct 16-byte bank slots.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

}  // namespace svdq

// LDS DMA (global_load_lds_dwordx4 / _dword) and the waits around it,
// shared by the kernels that stage K/V rows in LDS rings.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace pkv {
namespace dev {

// Every LDS access of this wave has completed, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most n of this wave's vector-memory instructions are in
// flight (the instruction takes an immediate; n is uniform, n < 32).
template <int N>
__device__ __forceinline__ void wait_vm_imm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int... Ns>
__device__ __forceinline__ void wait_vm_sel(int n, std::integer_sequence<int, Ns...>) {
  ((n == Ns ? (wait_vm_imm<Ns>(), 0) : 0), ...);
}
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 32) n = 0;                             // stricter than needed, never looser
  wait_vm_sel(n, std::make_integer_sequence<int, 32>{});
}

// s_waitcnt immediate with vmcnt = 0 and the other counters at their
// maximum (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

// LDS DMA, 16 (or 4) bytes per lane to LDS m0 + 16 (or 4) * lane.  The
// address is either a per-lane 64-bit pointer or a wave-uniform 64-bit base
// plus a per-lane 32-bit offset (the block's address formed on the scalar
// unit).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m0), "v"(src) : "memory", "m0");
}

}  // namespace dev
}  // namespace pkv

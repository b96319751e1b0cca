// LDS-DMA and synchronisation helpers shared by the bf16-MFMA GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {
namespace gemm {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

// LDS-DMA loads: lane l's bytes land at lds + 16 l (dwordx4) or in the dword slot
// lds + 4 l, zero-extended (dword / ushort / ubyte).  `base` is wave-uniform (SGPRs),
// `voff` the lane's 32-bit byte offset.  M0 holds the LDS base; s_nop covers the
// M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ushort %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma1(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// gfx9 s_waitcnt immediate that waits for vmcnt <= n and lgkmcnt == 0 (expcnt untouched).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// Workgroup barrier for the stage hand-off; the caller has already waited for its
// own LDS writes and LDS-DMA loads.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Tile index of block b under the XCD-aware order (b runs on XCD b % 8).
__device__ __forceinline__ int tile_of_block(int b, int nblk) {
  const int per = nblk >> 3, rem = nblk & 7;
  const int x = b & 7, local = b >> 3;
  const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + local;
}

}  // namespace gemm
}  // namespace aq

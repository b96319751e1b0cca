// Device-side helpers shared by the gfx950 kernels of libaq.
//
// Everything here is written for CDNA4 (gfx950): 64-lane wavefronts, bf16
// MFMA, DPP / ds_swizzle cross-lane moves.  No other target is supported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Pack the upper halves of two fp32 values whose low 16 bits are zero (exact bf16 values).
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Byte i of w as an fp32 integer (a single v_cvt_f32_ubyte<i>).
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t w) { return (float)((w >> (8 * I)) & 0xFFu); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// ---- cross-lane reductions inside one 64-lane wave -----------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
// Sum of a wave's 64 lanes into lane 63 with DPP (quad permutations, row mirrors,
// row_bcast:15 / row_bcast:31); the other lanes hold partial sums.
__device__ __forceinline__ float dpp_sum_to_lane63(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return v;
}
// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int W>
__device__ __forceinline__ float segment_sum(float v) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
template <int W>
__device__ __forceinline__ float segment_min(float v) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, kWave));
  return v;
}
template <int W>
__device__ __forceinline__ float segment_max(float v) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

}  // namespace aq

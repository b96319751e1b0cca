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

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
// Byte i of w as an fp32 integer (a single v_cvt_f32_ubyte<i>).
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t w) { return (float)((w >> (8 * I)) & 0xFFu); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

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

// ---- group-wise asymmetric INT4 parameters --------------------------------
// S = fl32(fl32(max - min) / 15); z = clamp(rne(fl32(-min / S)), 0, 15); a constant
// group (S == 0) stores S = 0, z = 0 and codes 0.  All divisions are IEEE
// correctly rounded (the library is compiled without fast-math, without
// contraction, and with fp32 denormals preserved).
struct GroupQ {
  float S;
  float zf;   // zero point as an exact float in 0..15 (0..255 for 8-bit codes)
  float inv;  // correctly rounded 1/S (or 0 for a constant group)
};

// Asymmetric min-max parameters for the unsigned range 0 .. QM (15: INT4, 255: INT8):
// S = fl32(fl32(max - min) / QM), z = clamp(rne(fl32(-min / S)), 0, QM).
template <int QM>
__device__ __forceinline__ GroupQ group_params_q(float mn, float mx) {
  GroupQ g;
  float r = mx - mn;
  float s = r / (float)QM;
  if (s == 0.0f) {
    g.S = 0.0f; g.zf = 0.0f; g.inv = 0.0f;
    return g;
  }
  float z = __builtin_rintf((-mn) / s);
  z = fminf(fmaxf(z, 0.0f), (float)QM);
  g.S = s; g.zf = z; g.inv = 1.0f / s;
  return g;
}
__device__ __forceinline__ GroupQ group_params(float mn, float mx) { return group_params_q<15>(mn, mx); }

// q = clamp(rne(fl32(v / S)) + z, 0, QM).
// Fast path: t = v * (1/S) differs from fl32(v / S) by at most one ulp-scale
// error, so rne(t) equals rne(fl32(v / S)) unless t lies within a few ulps of a
// rounding boundary (a half-integer); only then is the true division done.
template <int QM>
__device__ __forceinline__ uint32_t group_code_q(float v, const GroupQ& g) {
  if (g.S == 0.0f) return 0u;
  float t = v * g.inv;
  float fr = t - __builtin_floorf(t);
  // |t - fl32(v/S)| <= 1.5 * 2^-23 |t|; t - floor(t) adds at most 2^-24 when -1 < t < 0.
  float slack = fabsf(t) * 4.8e-7f + 1.2e-7f;
  if (!(fabsf(fr - 0.5f) > slack)) t = v / g.S;   // also taken when 1/S overflowed (NaN)
  float q = __builtin_rintf(t) + g.zf;
  q = fminf(fmaxf(q, 0.0f), (float)QM);
  return (uint32_t)q;
}
__device__ __forceinline__ uint32_t group_code(float v, const GroupQ& g) { return group_code_q<15>(v, g); }

}  // namespace aq

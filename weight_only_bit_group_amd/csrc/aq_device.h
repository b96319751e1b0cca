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

// (hi:lo) >> S as one v_lshrrev_b64: the low dword is lo >> S with hi's low S bits above
// bit 31 - S.  The INT4 decodes keep only bits 0-3 and 16-19 of each shifted dword
// (S <= 12), so one 64-bit shift serves two code dwords; written out because the
// compiler splits a 64-bit shift of a dword pair into v_alignbit_b32 + v_lshrrev_b32.
template <int S>
__device__ __forceinline__ uint64_t shr64(uint64_t v) {
  uint64_t t;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(t) : "i"(S), "v"(v));
  return t;
}
// The shifted copies >> 0, 4, 8, 12 of the code dword pair (hi:lo), as dwords
// sh[s][h] (h = 0: lo's, h = 1: hi's).
__device__ __forceinline__ void nibble_shifts(uint32_t lo, uint32_t hi, uint32_t (&sh)[4][2]) {
  const uint64_t pr = ((uint64_t)hi << 32) | lo;
  const uint64_t t1 = shr64<4>(pr), t2 = shr64<8>(pr), t3 = shr64<12>(pr);
  sh[0][0] = lo; sh[0][1] = hi;
  sh[1][0] = (uint32_t)t1; sh[1][1] = (uint32_t)(t1 >> 32);
  sh[2][0] = (uint32_t)t2; sh[2][1] = (uint32_t)(t2 >> 32);
  sh[3][0] = (uint32_t)t3; sh[3][1] = (uint32_t)(t3 >> 32);
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
// Totals of V per-lane values over a wave's 64 lanes (V a power of two): the values
// are halved across lanes 32 apart (v_permlane32_swap), then 16 apart
// (v_permlane16_swap), and each remaining value is summed inside its 16-lane row with
// DPP (quad permutations, row rotations by 4 and 8).  Afterwards every lane of 16-lane
// row rho holds in a[j], j < wave_sums_out<V>, the total of value
// wave_sums_index<V>(j, rho); the lanes where wave_sums_owner<V> is true hold each total
// once.  Every value takes the same addition tree, so its total does not depend on its
// index.  Against one DPP chain per value into lane 63 this is V / 2 + V / 4 swaps and
// 4 V / 4 row steps instead of 6 V dependent DPP steps.
template <int V>
constexpr int wave_sums_out = V >= 4 ? V / 4 : 1;
template <int V>
__host__ __device__ constexpr int wave_sums_index(int j, int rho) {
  return V >= 4 ? j + (rho & 1) * (V / 4) + (rho >> 1) * (V / 2) : V == 2 ? (rho >> 1) : 0;
}
template <int V>
__device__ __forceinline__ bool wave_sums_owner(int lane) {
  return (lane & 15) == 0 && (V >= 4 || (V == 2 ? (lane & 16) == 0 : lane == 0));
}
// lanes 0-31: a[l] + a[l + 32]; lanes 32-63: b[l - 32] + b[l]
__device__ __forceinline__ float permlane32_add(float a, float b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// 16-lane rows 0 and 2: a[l] + a[l + 16]; rows 1 and 3: b[l - 16] + b[l]
__device__ __forceinline__ float permlane16_add(float a, float b) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int V>
__device__ __forceinline__ void wave_sums(float (&a)[V]) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two");
  constexpr int H = V >= 2 ? V / 2 : 1, Q = wave_sums_out<V>;
#pragma unroll
  for (int j = 0; j < H; ++j) a[j] = permlane32_add(a[j], a[V >= 2 ? j + H : 0]);
#pragma unroll
  for (int j = 0; j < Q; ++j) a[j] = permlane16_add(a[j], a[H >= 2 ? j + Q : 0]);
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    a[j] = dpp_add<0xB1>(a[j]);    // quad_perm [1, 0, 3, 2]
    a[j] = dpp_add<0x4E>(a[j]);    // quad_perm [2, 3, 0, 1]
    a[j] = dpp_add<0x124>(a[j]);   // row_ror:4
    a[j] = dpp_add<0x128>(a[j]);   // row_ror:8
  }
}
// Smallest power of two >= n (n >= 1).
__host__ __device__ constexpr int pow2_ceil(int n) { return n <= 1 ? 1 : 2 * pow2_ceil((n + 1) / 2); }

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

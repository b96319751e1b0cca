// Group-wise asymmetric INT4 quantization and nibble packing (gfx950).
//
// What it computes ("Quantization：模型量化", xingyuwang.me, section 2, asymmetric
// quantization with clipping to the integer range; section 3, per-group
// granularity; "Lance-Quant", zingnex.cn, grid-search / grouped INT4 packing
// section): for every group of g consecutive input channels of a weight row,
//   v = w * s_k  (fp32, only when an AWQ channel scale is given)
//   S = fl32(fl32(max v - min v) / 15),  z = clamp(rne(fl32(-min v / S)), 0, 15)
//   q = clamp(rne(fl32(v / S)) + z, 0, 15)
// with two codes per byte (even k in the low nibble).
//
// Symmetric variant (same page, section 2: a symmetric integer range with zero at
// integer zero, q = round(x / s), x_hat = q s, clipped to the range): per group
//   S = fl32(max |v| / 7),  q = clamp(rne(fl32(v / S)), -7, 7)
// stored as the code q + 8 with a zero point of 8, so the decode (code - z) S of
// the asymmetric format applies unchanged; an all-zero group stores S = 0, codes 8.
//
// 8-bit variant: the asymmetric formulas with the range 0 .. 255 and one code byte
// per weight (codes [N, K]).
//
// Mapping: W[N, K] row-major is a flat run of N*K/g groups of g contiguous
// elements.  Each lane owns 8 consecutive elements (one 16-byte bf16 load or two
// 16-byte fp32 loads), so a group spans g/8 lanes and its min/max is a
// g/8-lane butterfly; a wave covers 512 elements.  Stores are 4 bytes of codes
// per lane (256 contiguous bytes per wave), one fp32 S and one u8 z per group.
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

namespace {

// The codes of one lane's eight values, each equal to group_code_q: the reciprocal
// fast path for all eight, and the true division only in a branch taken when a value
// of the lane lies within the tie slack of a half-integer (rare).  Written per
// element, the compiler turns that branch into a division computed for every value
// and a select.
template <int QM>
__device__ __forceinline__ void group_codes8(const float (&v)[8], const GroupQ& g, uint32_t (&q)[8]) {
  float t[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t[i] = v[i] * g.inv;
    const float fr = t[i] - __builtin_floorf(t[i]);
    near |= !(fabsf(fr - 0.5f) > fabsf(t[i]) * 4.8e-7f + 1.2e-7f);
  }
  if (__builtin_expect(near, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float fr = t[i] - __builtin_floorf(t[i]);
      if (!(fabsf(fr - 0.5f) > fabsf(t[i]) * 4.8e-7f + 1.2e-7f)) t[i] = v[i] / g.S;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = fminf(fmaxf(__builtin_rintf(t[i]) + g.zf, 0.0f), (float)QM);
    q[i] = g.S == 0.0f ? 0u : (uint32_t)c;
  }
}

}  // namespace

// MODE: 0 asymmetric INT4, 1 symmetric INT4, 2 asymmetric INT8.
template <int G, bool BF16, bool SCALED, int MODE>
__global__ __launch_bounds__(256) void quant_pack_kernel(const void* __restrict__ W,
                                                         const float* __restrict__ chan_scale,
                                                         uint8_t* __restrict__ packed,
                                                         float* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros,
                                                         int64_t total, int64_t K) {
  constexpr int LPG = G / 8;  // lanes per group
  const int64_t lane_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = lane_id * 8;
  const bool live = e0 < total;
  const int64_t e = live ? e0 : 0;

  float v[8];
  if (BF16) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + e);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  if (SCALED) {
    const int64_t k0 = e % K;
    const float4* sp = reinterpret_cast<const float4*>(chan_scale + k0);
    const float4 a = sp[0], b = sp[1];
    v[0] = v[0] * a.x; v[1] = v[1] * a.y; v[2] = v[2] * a.z; v[3] = v[3] * a.w;
    v[4] = v[4] * b.x; v[5] = v[5] * b.y; v[6] = v[6] * b.z; v[7] = v[7] * b.w;
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  mn = segment_min<LPG>(mn);
  mx = segment_max<LPG>(mx);
  constexpr bool SYM = MODE == 1;
  constexpr int QM = MODE == 2 ? 255 : 15;
  GroupQ g;
  if constexpr (SYM) {
    g.S = fmaxf(-mn, mx) / 7.0f;   // max |v| / 7 (fmaxf(-min, max) is max |v| exactly)
    g.zf = 8.0f;
    g.inv = g.S == 0.0f ? 0.0f : 1.0f / g.S;
  } else {
    g = group_params_q<QM>(mn, mx);
  }

  uint32_t q[8];
  group_codes8<QM>(v, g, q);
  if constexpr (MODE == 2) {
    uint32_t b[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i >> 2] |= q[i] << (8 * (i & 3));
    if (!live) return;
    *reinterpret_cast<uint2*>(packed + e) = uint2{b[0], b[1]};
  } else {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // |v / S| <= 7 (1 + 2^-23), so rne(v / S) + 8 stays in 1 .. 15 and the 0 .. 15
      // clamp of the code is the -7 .. 7 clamp of the symmetric code
      const uint32_t c = (SYM && g.S == 0.0f) ? 8u : q[i];
      word |= c << (4 * i);
    }
    if (!live) return;
    *reinterpret_cast<uint32_t*>(packed + e / 2) = word;
  }
  if ((threadIdx.x % LPG) == 0) {
    const int64_t grp = e / G;
    scales[grp] = g.S;
    zeros[grp] = (uint8_t)g.zf;
  }
}

// AWQ search: the error matrix E = Q(W s) / s - W of one candidate scale, written
// as two bf16 planes E_hi = bf16(e), E_lo = bf16(e - E_hi) ([N, K] each, E_lo
// after E_hi).  Same lane mapping and the same (bit-exact) group parameters and
// codes as the packing kernel; the dequantized value (q - z) * S is divided by
// s_k and the original weight subtracted in fp32.
template <int G, bool BF16>
__global__ __launch_bounds__(256) void quant_error_kernel(const void* __restrict__ W,
                                                          const float* __restrict__ chan_scale,
                                                          uint16_t* __restrict__ E, int64_t total, int64_t K) {
  constexpr int LPG = G / 8;
  const int64_t lane_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = lane_id * 8;
  const bool live = e0 < total;
  const int64_t e = live ? e0 : 0;
  float w[8], v[8], s[8];
  if (BF16) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[2 * i] = bf16_lo(x[i]); w[2 * i + 1] = bf16_hi(x[i]); }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + e);
    const float4 a = p[0], b = p[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  {
    const float4* sp = reinterpret_cast<const float4*>(chan_scale + (e % K));
    const float4 a = sp[0], b = sp[1];
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w; s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
  }
  float mn, mx;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = w[i] * s[i];
    mn = i ? fminf(mn, v[i]) : v[i];
    mx = i ? fmaxf(mx, v[i]) : v[i];
  }
  mn = segment_min<LPG>(mn);
  mx = segment_max<LPG>(mx);
  const GroupQ g = group_params(mn, mx);
  uint32_t qc[8];
  group_codes8<15>(v, g, qc);
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h16[2], l16[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 2 * i + h;
      const float q = (float)qc[j];
      const float what = (q - g.zf) * g.S;
      const float err = what / s[j] - w[j];
      h16[h] = f32_to_bf16_rne(err);
      l16[h] = f32_to_bf16_rne(err - __uint_as_float(h16[h] << 16));
    }
    hi[i] = h16[0] | (h16[1] << 16);
    lo[i] = l16[0] | (l16[1] << 16);
  }
  if (!live) return;
  *reinterpret_cast<u32x4*>(E + e) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<u32x4*>(E + total + e) = u32x4{lo[0], lo[1], lo[2], lo[3]};
}

hipError_t launch_quant_error(const void* W, bool w_bf16, const float* chan_scale, uint16_t* E, int64_t N,
                              int64_t K, int group, hipStream_t stream) {
  const int64_t total = N * K;
  const dim3 block(256), grid((unsigned)((total / 8 + 255) / 256));
#define AQ_QE(GG)                                                                                               \
  if (w_bf16) hipLaunchKernelGGL((quant_error_kernel<GG, true>), grid, block, 0, stream, W, chan_scale, E, total, K); \
  else hipLaunchKernelGGL((quant_error_kernel<GG, false>), grid, block, 0, stream, W, chan_scale, E, total, K);
  switch (group) {
    case 32: AQ_QE(32) break;
    case 64: AQ_QE(64) break;
    case 128: AQ_QE(128) break;
    default: return hipErrorInvalidValue;
  }
#undef AQ_QE
  return hipGetLastError();
}

template <int G, int MODE>
static hipError_t launch_g(const void* W, bool bf16, const float* s, uint8_t* packed, float* scales,
                           uint8_t* zeros, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t total = N * K;
  const int64_t lanes = total / 8;
  const dim3 block(256);
  const dim3 grid((unsigned)((lanes + 255) / 256));
  if (bf16) {
    if (s) hipLaunchKernelGGL((quant_pack_kernel<G, true, true, MODE>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
    else hipLaunchKernelGGL((quant_pack_kernel<G, true, false, MODE>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
  } else {
    if (s) hipLaunchKernelGGL((quant_pack_kernel<G, false, true, MODE>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
    else hipLaunchKernelGGL((quant_pack_kernel<G, false, false, MODE>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(const void* W, bool w_bf16, const float* chan_scale, uint8_t* packed, float* scales,
                              uint8_t* zeros, int64_t N, int64_t K, int group, hipStream_t stream) {
  switch (group) {
    case 32: return launch_g<32, MODE>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, stream);
    case 64: return launch_g<64, MODE>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, stream);
    case 128: return launch_g<128, MODE>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_pack(const void* W, bool w_bf16, const float* chan_scale, uint8_t* packed,
                             float* scales, uint8_t* zeros, int64_t N, int64_t K, int group, bool sym,
                             hipStream_t stream) {
  if (sym) return launch_mode<1>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, group, stream);
  return launch_mode<0>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, group, stream);
}

hipError_t launch_quant_pack8(const void* W, bool w_bf16, const float* chan_scale, uint8_t* codes, float* scales,
                              uint8_t* zeros, int64_t N, int64_t K, int group, hipStream_t stream) {
  return launch_mode<2>(W, w_bf16, chan_scale, codes, scales, zeros, N, K, group, stream);
}

}  // namespace aq

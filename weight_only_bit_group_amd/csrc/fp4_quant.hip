// FP4 encoder (gfx950): W -> E2M1 codes, an E4M3 scale per 16-element block and an
// fp32 tensor scale.
//
// Format ("Lance-Quant", zingnex.cn, grid-search / grouping section: NVFP4 packs
// E2M1 codes with an FP8 E4M3 scale per 16-element block from the same
// calibration; "Quantization：模型量化", xingyuwang.me, section 12: E4M3 is
// 1 sign + 4 exponent + 3 mantissa bits).  The encoder's choices are the ones the
// decode path is tested with:
//   ts   = fl32(amax |W| / 2688)   (2688 = 6 * 448: the largest E2M1 magnitude
//          times the largest E4M3 value); ts = 1 when W is all zero
//   b    = E4M3 of fl32(amax_block / fl32(6 ts)), round to nearest, ties to the
//          even code, saturating at 448 (0 for an all-zero block)
//   code = nearest E2M1 magnitude of fl32(|w| / fl32(e4m3(b) ts)), ties to the
//          even code, saturating at 6; sign bit 3 set for negative non-zero codes
// Layout as the decode path: codes [N, K/2] with even k in the low nibble, block
// scales [N, K/16].
//
// Kernels: a grid-stride max of |w| into per-block partials, a one-block finish
// that forms ts (max is order-free, so the result is deterministic), and the
// encoder, one thread per 16-element block (64 or 32 contiguous bytes in, 8 bytes
// of codes and one scale byte out).  Every quotient is the correctly rounded fp32
// quotient (IEEE divisions, or a reciprocal with an fma correction that equals
// them), and the library is built without contraction, as the formulas above
// require.
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

namespace {

constexpr int kAmaxThreads = 256;

// 16 consecutive elements starting at element e (16 * 4 or 16 * 2 bytes, 16-byte aligned).
template <bool BF16>
__device__ __forceinline__ void load16(const void* W, int64_t e, float (&v)[16]) {
  if constexpr (BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + e);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = p[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * h + 2 * i] = bf16_lo(w[i]);
        v[8 * h + 2 * i + 1] = bf16_hi(w[i]);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + e);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 a = p[h];
      v[4 * h] = a.x; v[4 * h + 1] = a.y; v[4 * h + 2] = a.z; v[4 * h + 3] = a.w;
    }
  }
}

__device__ __forceinline__ float block_max(float m) {
  __shared__ float red[kAmaxThreads / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kAmaxThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void fp4_amax_partial_kernel(const void* __restrict__ W, int64_t nblk16,
                                                                          float* __restrict__ partial) {
  float m = 0.0f;
  for (int64_t b = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; b < nblk16;
       b += (int64_t)gridDim.x * kAmaxThreads) {
    float v[16];
    load16<BF16>(W, b * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = block_max(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kAmaxThreads) void fp4_amax_finish_kernel(const float* __restrict__ partial, int n,
                                                                         float* __restrict__ ts) {
  float m = 0.0f;
  int i = threadIdx.x;
  for (; i + 7 * kAmaxThreads < n; i += 8 * kAmaxThreads) {   // eight loads in flight
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[i + u * kAmaxThreads];
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, v[u]);
  }
  for (; i < n; i += kAmaxThreads) m = fmaxf(m, partial[i]);
  m = block_max(m);
  if (threadIdx.x == 0) {
    const float t = m / 2688.0f;
    ts[0] = t == 0.0f ? 1.0f : t;
  }
}

// E4M3 byte (non-negative, finite t): nearest value, ties to the even code,
// saturating at 448 (0x7E).  Normal range: round the fp32 significand to 3 bits
// (the carry moves into the exponent by itself); below 2^-6 the codes are the
// multiples of 2^-9, so the code is rne(t * 512) (exact scaling).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
  if (t >= 448.0f) return 0x7Eu;
  if (t < 0.015625f) return (uint32_t)__builtin_rintf(t * 512.0f);
  const uint32_t u = __builtin_bit_cast(uint32_t, t);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;   // exponent : 3 mantissa bits
  return r - ((127u - 7u) << 3);
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return (float)m * 0.001953125f;                      // m * 2^-9
  return __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
}

// Nearest E2M1 magnitude code of r >= 0 over {0, .5, 1, 1.5, 2, 3, 4, 6}; exact
// midpoints go to the even code, values past 6 saturate to code 7.  Below 1 the grid
// is the multiples of 0.5, so the code is rne(2 r) (the low bits of 2 r + 1.5 * 2^23,
// one fma, exact); from 1 up the grid is the fp32 binades rounded to one mantissa
// bit (1, 1.5 | 2, 3 | 4, 6 | 8 ..), so the code is the exponent : mantissa-bit pair
// of r rounded to nearest even on its bit pattern, minus the pair of 1.0 (254) plus
// 2, capped at 7.
__device__ __forceinline__ uint32_t e2m1_code(float r) {
  const uint32_t lo = __float_as_uint(__builtin_fmaf(r, 2.0f, 12582912.0f)) & 7u;
  const uint32_t u = __float_as_uint(r);
  const uint32_t hi = min(((u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22) - 252u, 7u);
  return r < 1.0f ? lo : hi;
}

template <bool BF16>
__global__ __launch_bounds__(256) void fp4_encode_kernel(const void* __restrict__ W, int64_t nblk16,
                                                           const float* __restrict__ ts_ptr,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ bscale) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk16) return;
  float v[16];
  load16<BF16>(W, b * 16, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float ts = ts_ptr[0];
  const float six_ts = 6.0f * ts;
  const uint32_t sb = e4m3_rne_sat(amax / six_ts);
  const float scale = e4m3_value(sb) * ts;
  // r = fl32(|w| / scale) without a division per value: with inv = fl32(1 / scale),
  // q0 = fl32(|w| inv) is within an ulp of the quotient, the remainder |w| - q0 scale
  // is exact under fma, and fl32(q0 + rem inv) is the correctly rounded quotient
  // (Markstein's theorem; it needs no underflow or overflow, which a scale in
  // [2^-90, 2^90] guarantees wherever the quotient is near a code boundary).  Other
  // scales take the divisions; a zero scale (all-zero block) gives codes 0.
  uint32_t mag[16];
  if (scale >= 0x1p-90f && scale <= 0x1p90f) {
    const float inv = 1.0f / scale;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = fabsf(v[i]);
      const float q0 = a * inv;
      const float rem = __builtin_fmaf(-q0, scale, a);
      mag[i] = e2m1_code(__builtin_fmaf(rem, inv, q0));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) mag[i] = scale == 0.0f ? 0u : e2m1_code(fabsf(v[i]) / scale);
  }
  // codes with the sign (bit 3) of the negative values whose magnitude code is not 0:
  // (m + 7) & 8 is 8 exactly for m = 1 .. 7, and no nibble of m + 0x77777777 carries
  uint32_t word[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t m = 0, sgn = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m |= mag[8 * h + i] << (4 * i);
      sgn |= (__float_as_uint(v[8 * h + i]) >> 31) << (4 * i + 3);
    }
    word[h] = m | (sgn & (m + 0x77777777u));
  }
  *reinterpret_cast<uint2*>(codes + b * 8) = uint2{word[0], word[1]};
  bscale[b] = (uint8_t)sb;
}

// Partials of the |w| maximum: enough blocks to cover the device, capped.
int amax_blocks(int64_t nblk16) {
  const int64_t want = (nblk16 + kAmaxThreads * 8 - 1) / (kAmaxThreads * 8);
  return (int)(want < 1 ? 1 : (want > 2048 ? 2048 : want));
}

}  // namespace

size_t fp4_quantize_workspace_bytes(int64_t N, int64_t K) {
  return (size_t)amax_blocks(N * (K / 16)) * sizeof(float);
}

hipError_t launch_fp4_quantize(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* codes, uint8_t* bscale,
                               float* ts, float* partial, hipStream_t stream) {
  const int64_t nblk16 = N * (K / 16);
  const int pb = amax_blocks(nblk16);
  if (w_bf16) {
    hipLaunchKernelGGL((fp4_amax_partial_kernel<true>), dim3(pb), dim3(kAmaxThreads), 0, stream, W, nblk16, partial);
  } else {
    hipLaunchKernelGGL((fp4_amax_partial_kernel<false>), dim3(pb), dim3(kAmaxThreads), 0, stream, W, nblk16, partial);
  }
  hipLaunchKernelGGL(fp4_amax_finish_kernel, dim3(1), dim3(kAmaxThreads), 0, stream, partial, pb, ts);
  if (nblk16 > 0) {
    const unsigned grid = (unsigned)((nblk16 + 255) / 256);
    if (w_bf16) {
      hipLaunchKernelGGL((fp4_encode_kernel<true>), dim3(grid), dim3(256), 0, stream, W, nblk16, ts, codes, bscale);
    } else {
      hipLaunchKernelGGL((fp4_encode_kernel<false>), dim3(grid), dim3(256), 0, stream, W, nblk16, ts, codes, bscale);
    }
  }
  return hipGetLastError();
}

}  // namespace aq

// W4A16 decode GEMV (M = 1..16 activation rows), gfx950, VALU only.
//
// What it computes: Y[m, n] = sum_g S[n, g] * sum_{k in g} X[m, k] * (q[n, k] - z[n, g]),
// the quantized linear's forward with the weight dequantized in registers
// ("模型量化指南", blog.yoooo.fun, common conventions: the quantized layer
// dequantizes in memory and equals the original layer with W replaced by its
// dequantized value; "Quantization：模型量化", xingyuwang.me, section 13: read
// the compressed weights, dequantize inside the kernel, then contract; decode is
// memory-bound, so fewer weight bytes read means a faster step).
//
// Design (HBM-bound at M = 1): one wavefront owns R output rows.  A row of
// packed codes is K/2 bytes; lane l reads the 16-byte chunks c = l, l + 64, ...
// (32 codes each, always inside one group since g >= 32), so every load
// instruction of the wave covers 1 KiB of one row with 128-bit accesses.  The
// R rows' chunks, their S and z are issued before any arithmetic.
//
// Exact integer dequantization: for a code dword d (8 nibbles),
//   ((d >> 4s) & 0x000F000F) | 0x43004300
// is a pair of bf16 values (128 + q_{s}, 128 + q_{s+4}) -- exact, one op per two
// weights -- and v_dot2_f32_bf16 accumulates x * (128 + q) in fp32.  The chunk
// sum is corrected by -(128 + z) * sum(x) before the fp32 group scale is applied,
// so Y never goes through a rounded bf16 weight.  The activations are permuted
// once per chunk into the matching (k, k + 4) pairs and reused for all R rows.
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

template <int M, int R>
__global__ __launch_bounds__(256) void w4a16_gemv_kernel(const uint16_t* __restrict__ X,
                                                          const uint8_t* __restrict__ P,
                                                          const float* __restrict__ S,
                                                          const uint8_t* __restrict__ Z,
                                                          float* __restrict__ Y,
                                                          int N, int K, int gshift) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = wave * R;
  if (n0 >= N) return;  // uniform per wave
  const int kbytes = K >> 1;
  const int nchunk = K >> 5;
  const int ngroups = K >> gshift;

  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  for (int c = lane; c < nchunk; c += 64) {
    u32x4 code[R];
    float sc[R], zc[R];
    const int grp = (c << 5) >> gshift;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(n0 + r, N - 1);
      code[r] = *reinterpret_cast<const u32x4*>(P + (int64_t)row * kbytes + (c << 4));
      sc[r] = S[(int64_t)row * ngroups + grp];
      zc[r] = 128.0f + (float)Z[(int64_t)row * ngroups + grp];
    }
    uint32_t deq[R][16];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          deq[r][4 * i + s] = ((code[r][i] >> (4 * s)) & 0x000F000Fu) | 0x43004300u;

#pragma unroll
    for (int m = 0; m < M; ++m) {
      const u32x4* xp4 = reinterpret_cast<const u32x4*>(X + (int64_t)m * K + (c << 5));
      uint32_t xw[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 t = xp4[i];
        xw[4 * i] = t[0]; xw[4 * i + 1] = t[1]; xw[4 * i + 2] = t[2]; xw[4 * i + 3] = t[3];
      }
      uint32_t xp[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xp[4 * i + 0] = __builtin_amdgcn_perm(xw[4 * i + 2], xw[4 * i + 0], 0x05040100u);
        xp[4 * i + 1] = __builtin_amdgcn_perm(xw[4 * i + 2], xw[4 * i + 0], 0x07060302u);
        xp[4 * i + 2] = __builtin_amdgcn_perm(xw[4 * i + 3], xw[4 * i + 1], 0x05040100u);
        xp[4 * i + 3] = __builtin_amdgcn_perm(xw[4 * i + 3], xw[4 * i + 1], 0x07060302u);
      }
      float xs = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) xs = dot2_bf16(xw[j], 0x3F803F80u, xs);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) d = dot2_bf16(deq[r][j], xp[j], d);
        acc[m][r] = __builtin_fmaf(sc[r], __builtin_fmaf(-zc[r], xs, d), acc[m][r]);
      }
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = wave_sum(acc[m][r]);
      if (lane == 0 && n0 + r < N) Y[(int64_t)m * N + n0 + r] = v;
    }
}

template <int M>
static hipError_t launch_m(const uint16_t* X, const uint8_t* P, const float* S, const uint8_t* Z, float* Y,
                           int N, int K, int gshift, hipStream_t stream) {
  // Rows per wave: enough waves to keep every CU's memory pipeline full.
  int R = 1;
  if (N >= 8192) R = 4;
  else if (N >= 4096) R = 2;
  const int waves = (N + R - 1) / R;
  const dim3 grid((waves + 3) / 4), block(256);
  if (R == 4) hipLaunchKernelGGL((w4a16_gemv_kernel<M, 4>), grid, block, 0, stream, X, P, S, Z, Y, N, K, gshift);
  else if (R == 2) hipLaunchKernelGGL((w4a16_gemv_kernel<M, 2>), grid, block, 0, stream, X, P, S, Z, Y, N, K, gshift);
  else hipLaunchKernelGGL((w4a16_gemv_kernel<M, 1>), grid, block, 0, stream, X, P, S, Z, Y, N, K, gshift);
  return hipGetLastError();
}

hipError_t launch_w4a16_gemv(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                             const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  switch (M) {
#define AQ_CASE(mm) case mm: return launch_m<mm>(X, P, S, Z, Y, N, K, gshift, stream);
    AQ_CASE(1) AQ_CASE(2) AQ_CASE(3) AQ_CASE(4) AQ_CASE(5) AQ_CASE(6) AQ_CASE(7) AQ_CASE(8)
    AQ_CASE(9) AQ_CASE(10) AQ_CASE(11) AQ_CASE(12) AQ_CASE(13) AQ_CASE(14) AQ_CASE(15) AQ_CASE(16)
#undef AQ_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aq

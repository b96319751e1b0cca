// W8A16 decode GEMV (M = 1..16 activation rows), gfx950, VALU only.
//
// What it computes: Y[m, n] = sum_g S[n, g] * sum_{k in g} X[m, k] * (q[n, k] - z[n, g])
// with one 8-bit code byte per weight (the 8-bit member of the mixed 4/8-bit
// policy: "模型量化指南", blog.yoooo.fun, "混合精度（按层 4/8-bit）" keeps key layers
// at 8 bits; the quantized layer dequantizes in memory, same page, "共同约定").
//
// Design (HBM-bound at M = 1, one byte per weight):
//  * One wavefront owns R output rows; lane l reads the 16-byte chunks c = l, l + 64,
//    ... of a row (16 codes each, inside one group since g >= 32), each load
//    instruction of the wave covering 1 KiB of one row; all code / S / z loads of a
//    batch of chunks are issued before any is used.
//  * The lane's 16 activations of a chunk are read from global memory (the same
//    activation rows are shared by every wave and stay in the L2) and widened to
//    fp32; each code byte becomes an fp32 integer (v_cvt_f32_ubyte), and x * q is
//    exact in fp32 (8 x 8 significant bits).  The chunk sum is corrected by
//    -z * sum(x) before the fp32 group step S is applied.  For up to six chunk rows
//    (M x CPL <= 6) a batch's activations are requested before its weights: loads
//    return in order, so activations requested after the weights would wait for the
//    HBM stream.
//  * Each row's 64 lane partials are reduced with DPP; lane 63 writes the result.
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

namespace {

template <int M, int R, int CPL>
__global__ __launch_bounds__(256) void w8a16_gemv_kernel(const uint16_t* __restrict__ X, const uint8_t* C,
                                                          const float* S, const uint8_t* Z, float* __restrict__ Y,
                                                          int N, int K, int gshift) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = wave * R;
  if (n0 >= N) return;   // uniform per wave; no block-level synchronisation follows
  const int nchunk = K >> 4;
  const int ngroups = K >> gshift;
  const int nbatch = (nchunk + 64 * CPL - 1) / (64 * CPL);

  u32x4 code[R][CPL];
  float sc[R][CPL];
  uint32_t zb[R][CPL];
  auto issue = [&](int b) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(lane + 64 * (b * CPL + j), nchunk - 1);
      const int grp = (c << 4) >> gshift;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(n0 + r, N - 1);
        code[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(C + (int64_t)row * K + (c << 4)));
        sc[r][j] = S[(int64_t)row * ngroups + grp];
        zb[r][j] = Z[(int64_t)row * ngroups + grp];
      }
    }
  };

  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  constexpr bool PX = M * CPL <= 6;   // activations of a batch requested ahead of its weights
  for (int b = 0; b < nbatch; ++b) {
    u32x4 xr[PX ? M : 1][PX ? CPL : 1][2];
    if constexpr (PX) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = min(lane + 64 * (b * CPL + j), nchunk - 1);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4* xs16 = reinterpret_cast<const u32x4*>(X + (int64_t)m * K + (c << 4));
          xr[m][j][0] = xs16[0];
          xr[m][j][1] = xs16[1];
        }
      }
      asm volatile("" ::: "memory");
    }
    issue(b);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * (b * CPL + j);
      if (c >= nchunk) break;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4* xs16 = reinterpret_cast<const u32x4*>(X + (int64_t)m * K + (c << 4));
        const u32x4 xa = PX ? xr[PX ? m : 0][PX ? j : 0][0] : xs16[0];
        const u32x4 xb = PX ? xr[PX ? m : 0][PX ? j : 0][1] : xs16[1];
        float x[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf16_lo(xa[i]);
          x[2 * i + 1] = bf16_hi(xa[i]);
          x[8 + 2 * i] = bf16_lo(xb[i]);
          x[8 + 2 * i + 1] = bf16_hi(xb[i]);
        }
        float xsum0 = 0.0f, xsum1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          xsum0 += x[i];
          xsum1 += x[i + 1];
        }
        const float xsum = xsum0 + xsum1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = code[r][j][i];
            d0 = __builtin_fmaf(x[4 * i], ubyte_f32<0>(w), d0);
            d1 = __builtin_fmaf(x[4 * i + 1], ubyte_f32<1>(w), d1);
            d0 = __builtin_fmaf(x[4 * i + 2], ubyte_f32<2>(w), d0);
            d1 = __builtin_fmaf(x[4 * i + 3], ubyte_f32<3>(w), d1);
          }
          const float zf = (float)zb[r][j];
          acc[m][r] = __builtin_fmaf(sc[r][j], __builtin_fmaf(-zf, xsum, d0 + d1), acc[m][r]);
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = dpp_sum_to_lane63(acc[m][r]);
      if (lane == 63 && n0 + r < N) Y[(int64_t)m * N + n0 + r] = v;
    }
}

template <int M, int R, int CPL>
hipError_t launch_cfg8(const uint16_t* X, const uint8_t* C, const float* S, const uint8_t* Z, float* Y, int N, int K,
                       int gshift, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  hipLaunchKernelGGL((w8a16_gemv_kernel<M, R, CPL>), dim3((waves + 3) / 4), dim3(256), 0, stream, X, C, S, Z, Y, N,
                     K, gshift);
  return hipGetLastError();
}

// Rows of up to 2048 codes: four rows per wave; over a wide N (>= 8192) one chunk per
// lane and row in flight (measured on [11008, 2048]: 6.1 us at M = 1 against 6.5 with
// two chunks, 7.2 with two rows and two chunks), over a narrower N two, so the fewer
// waves each request a whole 2048-code row at once ([2048, 2048] 4.1 -> 3.7 us,
// [4096, 2048] 4.6 -> 4.2 us); longer rows one row per wave with six chunks per lane in
// flight (the best of 1-4 rows on [2048, 11008]).
template <int M>
hipError_t launch_m8(const uint16_t* X, const uint8_t* C, const float* S, const uint8_t* Z, float* Y, int N, int K,
                     int gshift, hipStream_t stream) {
  static_assert(M >= 1 && M <= 3, "the VALU W8A16 GEMV serves 1 .. 3 activation rows");
  if ((K >> 4) <= 128) {
    if (N >= 8192) return launch_cfg8<M, 4, 1>(X, C, S, Z, Y, N, K, gshift, stream);
    return launch_cfg8<M, 4, 2>(X, C, S, Z, Y, N, K, gshift, stream);
  }
  return launch_cfg8<M, 1, 6>(X, C, S, Z, Y, N, K, gshift, stream);
}

}  // namespace

// M = 1 .. 3 (more rows take the matrix-core kernel)
hipError_t launch_w8a16_gemv_valu(const uint16_t* X, int M, int K, const uint8_t* C, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  switch (M) {
#define AQ_CASE(mm) case mm: return launch_m8<mm>(X, C, S, Z, Y, N, K, gshift, stream);
    AQ_CASE(1) AQ_CASE(2) AQ_CASE(3)
#undef AQ_CASE
    default: return hipErrorInvalidValue;
  }
}

// The VALU kernel up to 3 activation rows, the matrix-core kernel from 4 (measured on
// [11008, 2048]: 7.7 against 8.6 us at M = 3, 9.8 against 8.9 at M = 4, 32 against 11
// at M = 16; on [2048, 11008] 15.4 against 14.2 us at M = 4).
hipError_t launch_w8a16_gemv(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z,
                             int N, int group, float* Y, hipStream_t stream) {
  if (M >= 4) return launch_w8a16_gemv_mfma(X, M, K, C, S, Z, N, group, Y, stream);
  return launch_w8a16_gemv_valu(X, M, K, C, S, Z, N, group, Y, stream);
}

}  // namespace aq

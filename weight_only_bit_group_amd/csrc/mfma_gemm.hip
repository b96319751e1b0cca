// bf16-MFMA GEMMs of libaq (gfx950): the W4A16 prefill GEMM, the FP4 decode GEMM
// and the AWQ search's error GEMM with a sum-of-squares epilogue.
//
// All three contract a bf16 activation matrix X[M, K] (K contiguous) with a
// weight-side operand B[N, K] whose rows are produced on the fly in LDS:
//
//   INT4  B = (q - z) exactly, as bf16 integers -15..15, with the fp32 group step
//         S[n, g] applied to a per-group partial accumulator once per group
//         ("Quantization：模型量化", xingyuwang.me, sections 2-4: asymmetric
//         group-wise weights, W4A16; section 13: dequantization fused into the
//         matrix computation).  A bf16-rounded (q - z) * S would cost ~2e-3 mean
//         absolute error on these shapes; the exact integer operand keeps the
//         output within fp32 accumulation error.
//   FP4   B = e2m1(code) * e4m3(block scale) exactly (at most 6 significant bits,
//         always representable in bf16); the fp32 tensor scale multiplies the
//         result ("Lance-Quant", zingnex.cn: E2M1 codes with an E4M3 scale per
//         16-element block).
//   SPLIT B = E_hi + E_lo, the search's error matrix as two bf16 planes (E_hi the
//         nearest bf16, E_lo the nearest bf16 of the remainder, ~16 significant
//         bits in all); both planes are multiplied into the same accumulator and
//         the epilogue returns, per block, the fp64 sum of squares of its outputs
//         (the MSE numerator).
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid, each wave a WM x WN tile made
// of 32 x 32 blocks of v_mfma_f32_32x32x16_bf16.  K advances in 32-wide slabs
// through double-buffered LDS (one barrier per slab).  A lane of a 32x32x16 MFMA
// holds row (lane % 32) and k = 8 (lane / 32) .. +7 of each operand, and its 16
// results are column (lane % 32), rows 8 (v / 4) + 4 (lane / 32) + v % 4; so a
// lane's results share one weight row n and need one S per block per group.
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

enum BKind { B_INT4 = 0, B_SPLIT = 1, B_FP4 = 2 };

struct GemmArgs {
  const uint16_t* X;
  int M, N, K;
  // INT4
  const uint8_t* P;
  const float* S;
  const uint8_t* Z;
  // SPLIT: the two bf16 planes of E
  const uint16_t* B;
  const uint16_t* B2;
  // FP4
  const uint8_t* codes;
  const uint8_t* bscale;
  float ts;
  // outputs
  float* Y;           // [M, N] fp32 (INT4, FP4)
  double* partial;    // [gridDim.x * gridDim.y] fp64 sums of squares (SPLIT)
};

constexpr int KS = 32;         // k per LDS slab
constexpr int LDS_STRIDE = KS + 8;  // bf16 elements per LDS row (16-byte pad against bank conflicts)

template <int BK, int WM, int WN, int G>
__global__ __launch_bounds__(256) void mfma_gemm_kernel(GemmArgs a) {
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int SLABS_PER_GROUP = (BK == B_INT4) ? G / KS : 1;
  constexpr int A_LOADS = BM * KS / 8 / 256;  // 16-byte loads per thread per slab
  static_assert(BN == 128, "B loader assumes 2 threads per weight row");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDS_STRIDE];
  constexpr int PLANES = (BK == B_SPLIT) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][PLANES][BN][LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int M = a.M, N = a.N, K = a.K;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int nslab = K / KS;

  // ---- global -> register staging ------------------------------------------
  u32x4 areg[A_LOADS];
  const int a_part = tid & 3;  // 16-byte quarter of a 64-byte slab row
  auto load_a = [&](int slab) {
#pragma unroll
    for (int u = 0; u < A_LOADS; ++u) {
      const int r = (tid >> 2) + 64 * u;
      const int row = min(m0 + r, M - 1);
      areg[u] = *reinterpret_cast<const u32x4*>(a.X + (int64_t)row * K + slab * KS + a_part * 8);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int u = 0; u < A_LOADS; ++u) {
      const int r = (tid >> 2) + 64 * u;
      *reinterpret_cast<u32x4*>(&As[buf][r][a_part * 8]) = areg[u];
    }
  };

  const int b_row = tid >> 1;            // weight row within the block tile
  const int b_half = tid & 1;            // k half of the slab: 16 values
  const int b_n = min(n0 + b_row, N - 1);
  uint2 breg_i4;                         // INT4: 16 codes
  float bz = 0.0f;                       // INT4: zero point of the group
  u32x4 breg_bf[2][2];                   // SPLIT: 16 values of each plane
  uint2 breg_f4;                         // FP4: 16 codes
  float bsc = 0.0f;                      // FP4: decoded E4M3 block scale
  auto load_b = [&](int slab) {
    const int k0 = slab * KS + b_half * 16;
    if constexpr (BK == B_INT4) {
      breg_i4 = *reinterpret_cast<const uint2*>(a.P + (int64_t)b_n * (K >> 1) + (k0 >> 1));
      bz = (float)a.Z[(int64_t)b_n * (K / G) + k0 / G];
    } else if constexpr (BK == B_SPLIT) {
      const u32x4* p = reinterpret_cast<const u32x4*>(a.B + (int64_t)b_n * K + k0);
      const u32x4* q = reinterpret_cast<const u32x4*>(a.B2 + (int64_t)b_n * K + k0);
      breg_bf[0][0] = p[0];
      breg_bf[0][1] = p[1];
      breg_bf[1][0] = q[0];
      breg_bf[1][1] = q[1];
    } else {
      breg_f4 = *reinterpret_cast<const uint2*>(a.codes + (int64_t)b_n * (K >> 1) + (k0 >> 1));
      bsc = __builtin_amdgcn_cvt_f32_fp8((int)a.bscale[(int64_t)b_n * (K >> 4) + (k0 >> 4)], 0);
    }
  };
  auto store_b = [&](int buf) {
    if constexpr (BK == B_SPLIT) {
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        u32x4* dst = reinterpret_cast<u32x4*>(&Bs[buf][pl][b_row][b_half * 16]);
        dst[0] = breg_bf[pl][0];
        dst[1] = breg_bf[pl][1];
      }
      return;
    }
    uint32_t w[8];
    if constexpr (BK == B_INT4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t byte = ((i < 4 ? breg_i4.x : breg_i4.y) >> (8 * (i & 3))) & 0xFFu;
        const float lo = (float)(byte & 0xFu) - bz;
        const float hi = (float)(byte >> 4) - bz;
        w[i] = pack_bf16_exact(lo, hi);
      }
    } else if constexpr (BK == B_FP4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t src = (i < 4 ? breg_f4.x : breg_f4.y);
        uint32_t e2;
        switch (i & 3) {
          case 0: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 0)); break;
          case 1: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 1)); break;
          case 2: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 2)); break;
          default: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 3)); break;
        }
        w[i] = pack_bf16_exact(bf16_lo(e2) * bsc, bf16_hi(e2) * bsc);
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(&Bs[buf][0][b_row][b_half * 16]);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  };

  // ---- accumulators ----------------------------------------------------------
  f32x16 acc[MI][NJ];   // running output (INT4: sum over finished groups)
  f32x16 part[MI][NJ];  // INT4: the current group's partial sum
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) { acc[i][j][v] = 0.0f; part[i][j][v] = 0.0f; }

  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  const int ngroups = K / G;
  int ncol[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) ncol[j] = min(n0 + wn * WN + 32 * j + lrow, N - 1);

  auto mma_slab = [&](int buf, bool first_in_group) {
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
      bf16x8 af[MI], bfr[NJ], bf2[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm * WM + 32 * i + lrow][kk * 16 + lk]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][0][wn * WN + 32 * j + lrow][kk * 16 + lk]);
      if constexpr (BK == B_SPLIT) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bf2[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][1][wn * WN + 32 * j + lrow][kk * 16 + lk]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if constexpr (BK == B_INT4) {
            if (first_in_group && kk == 0) {
              const f32x16 zero = {};
              part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], zero, 0, 0, 0);
            } else {
              part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], part[i][j], 0, 0, 0);
            }
          } else if constexpr (BK == B_SPLIT) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf2[j], acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          }
        }
    }
  };

  // ---- main loop -------------------------------------------------------------
  load_a(0);
  load_b(0);
  store_a(0);
  store_b(0);
  __syncthreads();
  float gscale[NJ];
  for (int g = 0; g < (BK == B_INT4 ? ngroups : 1); ++g) {
    if constexpr (BK == B_INT4) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) gscale[j] = a.S[(int64_t)ncol[j] * ngroups + g];
    }
    const int s_begin = (BK == B_INT4) ? g * SLABS_PER_GROUP : 0;
    const int s_end = (BK == B_INT4) ? s_begin + SLABS_PER_GROUP : nslab;
    for (int s = s_begin; s < s_end; ++s) {
      const int buf = s & 1;
      const bool more = s + 1 < nslab;
      if (more) { load_a(s + 1); load_b(s + 1); }
      mma_slab(buf, s == s_begin);
      if (more) { store_a(buf ^ 1); store_b(buf ^ 1); }
      __syncthreads();
    }
    if constexpr (BK == B_INT4) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(gscale[j], part[i][j][v], acc[i][j][v]);
    }
  }

  // ---- epilogue --------------------------------------------------------------
  if constexpr (BK == B_SPLIT) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * WN + 32 * j + lrow;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * WM + 32 * i + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const double d = (double)acc[i][j][v];
          if (m < M && n < N) ss = __builtin_fma(d, d, ss);
        }
      }
    ss = wave_sum(ss);
    __shared__ double wsum[4];
    if (lane == 0) wsum[wid] = ss;
    __syncthreads();
    if (tid == 0) a.partial[blockIdx.y * gridDim.x + blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * WN + 32 * j + lrow;
        if (n >= N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * WM + 32 * i + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          if (m < M) {
            const float y = (BK == B_FP4) ? acc[i][j][v] * a.ts : acc[i][j][v];
            a.Y[(int64_t)m * N + n] = y;
          }
        }
      }
  }
}

template <int BK, int G>
static hipError_t launch_tiles(const GemmArgs& a, hipStream_t stream) {
  const dim3 block(256);
  if (a.M >= 2048) {
    const dim3 grid((a.N + 127) / 128, (a.M + 255) / 256);
    hipLaunchKernelGGL((mfma_gemm_kernel<BK, 128, 64, G>), grid, block, 0, stream, a);
  } else {
    const dim3 grid((a.N + 127) / 128, (a.M + 127) / 128);
    hipLaunchKernelGGL((mfma_gemm_kernel<BK, 64, 64, G>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                             const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.P = P; a.S = S; a.Z = Z; a.Y = Y;
  switch (group) {
    case 32: return launch_tiles<B_INT4, 32>(a, stream);
    case 64: return launch_tiles<B_INT4, 64>(a, stream);
    case 128: return launch_tiles<B_INT4, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fp4_gemm(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale,
                           float ts, int N, float* Y, hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.codes = codes; a.bscale = bscale; a.ts = ts; a.Y = Y;
  return launch_tiles<B_FP4, 32>(a, stream);
}

int sumsq_gemm_blocks(int M, int N) {
  if (M >= 2048) return ((N + 127) / 128) * ((M + 255) / 256);
  return ((N + 127) / 128) * ((M + 127) / 128);
}

hipError_t launch_sumsq_gemm(const uint16_t* X, int M, int K, const uint16_t* E, int N, double* partial,
                             hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.B = E; a.B2 = E + (size_t)N * K; a.partial = partial;
  return launch_tiles<B_SPLIT, 32>(a, stream);
}

}  // namespace aq

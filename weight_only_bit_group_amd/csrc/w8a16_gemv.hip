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
//  * The activation rows are staged once per block in LDS by LDS-DMA, ahead of the
//    first weight batch, when they fit 64 KiB, or 152 KiB for rows longer than 2048
//    codes whose blocks still fit one round (else each lane reads its chunk's 16
//    activations from global memory, where they stay in the L2); a lane's 16
//    activations are widened to fp32; each code byte becomes an fp32 integer
//    (v_cvt_f32_ubyte), and x * q is exact in fp32 (8 x 8 significant bits).  The
//    chunk sum is corrected by -z * sum(x) before the fp32 group step S is applied.
//    Without staging, for up to six chunk rows (M x CPL <= 6) a batch's activations
//    are requested before its weights: loads return in order, so activations
//    requested after the weights would wait for the HBM stream.
//  * The M x R sets of 64 lane partials are reduced together (permlane swaps, then DPP
//    inside 16-lane rows); one lane per total writes it.
#include <atomic>

#include "aq_device.h"
#include "aq_kernels.h"
#include "gemm_lds.h"

namespace aq {

namespace {

// LDS_X: X [M][K] staged once per block in LDS by LDS-DMA (M * K * 2 bytes, in whole
// 1 KiB pieces), requested ahead of the first weight batch
template <int M, int R, int CPL, bool LDS_X>
__global__ __launch_bounds__(256) void w8a16_gemv_kernel(const uint16_t* __restrict__ X, const uint8_t* C,
                                                          const float* S, const uint8_t* Z, float* __restrict__ Y,
                                                          int N, int K, int gshift) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = wave * R;
  if constexpr (!LDS_X) {
    if (n0 >= N) return;   // uniform per wave; no block-level synchronisation follows
  }
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

  if constexpr (LDS_X) {
    // the block's activations by LDS-DMA (no registers, no VALU), then the first weight
    // batch; the DMA loads are not in the compiler's count, so wait for every load of
    // this wave (the first batch is needed next anyway) before the barrier
    const int xbytes = M * K * 2;
    const int pieces = (xbytes + 1023) >> 10;
    const int wu = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const uint32_t lbase = gemm::lds_addr(xl);
    for (int pc = wu; pc < pieces; pc += 4)
      gemm::dma16(X, (uint32_t)min(pc * 1024 + 16 * lane, xbytes - 16),
                  __builtin_amdgcn_readfirstlane(lbase + (uint32_t)pc * 1024u));
    asm volatile("" ::: "memory");
    issue(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(gemm::vmcnt_lgkm0_imm(0));
    __builtin_amdgcn_s_barrier();
    if (n0 >= N) return;   // uniform per wave, after the block barrier
  }

  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  constexpr bool PX = !LDS_X && M * CPL <= 6;   // activations of a batch requested ahead of its weights
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
    if (!LDS_X || b > 0) issue(b);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * (b * CPL + j);
      if (c >= nchunk) break;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4* xs16 = LDS_X ? reinterpret_cast<const u32x4*>(xl) + ((m * K + (c << 4)) >> 3)
                                  : reinterpret_cast<const u32x4*>(X + (int64_t)m * K + (c << 4));
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

  // all M x R totals at once (permlane swaps, then DPP inside 16-lane rows)
  constexpr int V = pow2_ceil(M * R);
  float t[V];
#pragma unroll
  for (int i = 0; i < V; ++i) t[i] = i < M * R ? acc[i / R][i % R] : 0.0f;
  wave_sums<V>(t);
  if (wave_sums_owner<V>(lane)) {
#pragma unroll
    for (int j = 0; j < wave_sums_out<V>; ++j) {
      const int i = wave_sums_index<V>(j, lane >> 4);
      if (i < M * R && n0 + i % R < N) Y[(int64_t)(i / R) * N + n0 + i % R] = t[j];
    }
  }
}

template <int M, int R, int CPL>
hipError_t launch_cfg8(const uint16_t* X, const uint8_t* C, const float* S, const uint8_t* Z, float* Y, int N, int K,
                       int gshift, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  // activations in LDS when they fit 64 KiB (whole 1 KiB pieces: the DMA writes a partial
  // last piece's padding too)
  const size_t lds = ((size_t)M * K * 2 + 1023) / 1024 * 1024;
  if (lds <= 64 * 1024) {
    hipLaunchKernelGGL((w8a16_gemv_kernel<M, R, CPL, true>), dim3((waves + 3) / 4), dim3(256), lds, stream, X, C, S,
                       Z, Y, N, K, gshift);
  } else {
    hipLaunchKernelGGL((w8a16_gemv_kernel<M, R, CPL, false>), dim3((waves + 3) / 4), dim3(256), 0, stream, X, C, S,
                       Z, Y, N, K, gshift);
  }
  return hipGetLastError();
}

// Rows of up to 2048 codes: over a wide N (>= 8192) four rows per wave and one chunk per
// lane and row in flight (graph-replayed on [11008, 2048]: 6.27 us at M = 1 against 6.55
// with two rows and two chunks, 7.1 with one row); below, each wave requests whole
// 2048-code rows at once (two chunks per lane) and fewer rows per wave give the narrower
// outputs more waves to share the memory latency: two rows from N = 4096 ([4096, 2048]
// M = 1 4.21 us), one row below ([2048, 2048] M = 1 3.75 -> 3.19 us, M = 3 4.99 -> 3.81
// against four rows; [256, 2048] M = 1 3.24 -> 2.46, M = 3 4.49 -> 3.00); longer rows
// one row per wave with six chunks per lane in flight (the best of 1-4 rows on
// [2048, 11008]).
// Long rows with the activations staged beyond 64 KiB of LDS: the dynamic-LDS limit of
// the instance raised to kLdsLong8 once per device.
constexpr int kLdsLong8 = 152 * 1024;
constexpr int kLdsPerCu8 = 160 * 1024;

template <int M, int R, int CPL>
hipError_t launch_long8(const uint16_t* X, const uint8_t* C, const float* S, const uint8_t* Z, float* Y, int N, int K,
                        int gshift, size_t lds, hipStream_t stream) {
  static std::atomic<uint64_t> done{0};   // bit d: the limit is raised on device d
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (!(done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(w8a16_gemv_kernel<M, R, CPL, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLong8);
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int waves = (N + R - 1) / R;
  hipLaunchKernelGGL((w8a16_gemv_kernel<M, R, CPL, true>), dim3((waves + 3) / 4), dim3(256), lds, stream, X, C, S, Z,
                     Y, N, K, gshift);
  return hipGetLastError();
}

template <int M>
hipError_t launch_m8(const uint16_t* X, const uint8_t* C, const float* S, const uint8_t* Z, float* Y, int N, int K,
                     int gshift, hipStream_t stream) {
  static_assert(M >= 1 && M <= 3, "the VALU W8A16 GEMV serves 1 .. 3 activation rows");
  if ((K >> 4) > 128) {
    // Long rows: the activations staged in LDS up to kLdsLong8 when the blocks fit one
    // round on the device; two rows per wave and four chunks per lane from N = 4096, one
    // row and six chunks below (graph-replayed: [4096, 14336] M = 1 15.0 -> 13.6 us,
    // M = 2 21.7 -> 16.9; [2048, 11008] M = 3 12.9 -> 11.8; staged launches that need two
    // rounds of blocks were slower: [4096, 14336] M = 3 25.5 -> 27.6 .. 38.6)
    const size_t lds = ((size_t)M * K * 2 + 1023) / 1024 * 1024;
    if (lds <= (size_t)kLdsLong8) {
      const int64_t slots = (int64_t)device_cu_count() * (int64_t)(kLdsPerCu8 / lds);
      if (N >= 4096 && ((int64_t)(N + 1) / 2 + 3) / 4 <= slots)
        return launch_long8<M, 2, 4>(X, C, S, Z, Y, N, K, gshift, lds, stream);
      if (((int64_t)N + 3) / 4 <= slots) return launch_long8<M, 1, 6>(X, C, S, Z, Y, N, K, gshift, lds, stream);
    }
  }
  if ((K >> 4) <= 128) {
    if (N >= 8192) return launch_cfg8<M, 4, 1>(X, C, S, Z, Y, N, K, gshift, stream);
    if (N >= 4096) return launch_cfg8<M, 2, 2>(X, C, S, Z, Y, N, K, gshift, stream);
    return launch_cfg8<M, 1, 2>(X, C, S, Z, Y, N, K, gshift, stream);
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

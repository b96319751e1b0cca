// FP4 decode GEMV (M = 1..16), gfx950, VALU only.
//
// What it computes: Y[m, n] = ts * sum_k X[m, k] * e2m1(c[n, k]) * e4m3(b[n, k / 16])
// for E2M1 codes with one E4M3 scale per 16-element block and an fp32 tensor
// scale ("Lance-Quant", zingnex.cn, grid-search / grouped packing section: E2M1
// codes plus an FP8 E4M3 scale for every 16-element block; "Quantization：模型量化",
// xingyuwang.me, section 12: E4M3 = 1 + 4 + 3 bits).
//
// Design: as the INT4 GEMV -- one wave per R output rows, lane l reading the
// 16-byte code chunks c = l, l + 64, ... (32 codes = two scale blocks), CPL of them
// requested at once.  gfx950's
// v_cvt_scalef32_pk_bf16_fp4 (unit scale) turns one code byte into the exact bf16
// pair (k, k + 1), which lines up with the activation pairs as loaded, so
// v_dot2_f32_bf16 accumulates each 16-block and the fp32 block scale multiplies
// the block sum once.  At one or two activation rows that fit 64 KiB the block stages
// them once in LDS by LDS-DMA (fp4_gemv_lds_kernel); otherwise, for M <= 4, a chunk's
// activations are requested before its codes and scales: loads return in order, so
// activations requested after the weights would wait for the HBM stream.
#include "aq_device.h"
#include "aq_kernels.h"
#include "gemm_lds.h"

namespace aq {

__device__ __forceinline__ uint32_t fp4_pair(uint32_t src, int sel) {
  switch (sel) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, 1.0f, 3));
  }
}

template <int M, int R, int CPL>
__global__ __launch_bounds__(256) void fp4_gemv_kernel(const uint16_t* __restrict__ X,
                                                        const uint8_t* __restrict__ C,
                                                        const uint8_t* __restrict__ B,
                                                        float ts, float* __restrict__ Y, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = wave * R;
  if (n0 >= N) return;
  const int kbytes = K >> 1;
  const int nblk = K >> 4;
  const int nchunk = K >> 5;

  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  constexpr bool PX = M <= 4;   // activations requested ahead of the weights
  // CPL chunks per lane in flight: chunks c0, c0 + 64, ..., all requested before any is used
  for (int c0 = lane; c0 < nchunk; c0 += 64 * CPL) {
    int cc[CPL];
    bool ok[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      ok[u] = c0 + 64 * u < nchunk;
      cc[u] = min(c0 + 64 * u, nchunk - 1);   // in-bounds address for a lane past the row's end
    }
    u32x4 xr[CPL][PX ? M : 1][4];
    if constexpr (PX) {
#pragma unroll
      for (int u = 0; u < CPL; ++u)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xr[u][m][i] = reinterpret_cast<const u32x4*>(X + (int64_t)m * K + (cc[u] << 5))[i];
      asm volatile("" ::: "memory");
    }
    u32x4 code[CPL][R];
    uint32_t two[CPL][R];
#pragma unroll
    for (int u = 0; u < CPL; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(n0 + r, N - 1);
        code[u][r] = *reinterpret_cast<const u32x4*>(C + (int64_t)row * kbytes + (cc[u] << 4));
        two[u][r] = *reinterpret_cast<const uint16_t*>(B + (int64_t)row * nblk + (cc[u] << 1));
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      if (!ok[u]) continue;
      uint32_t deq[R][16];
      float bs[R][2];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bs[r][0] = __builtin_amdgcn_cvt_f32_fp8((int)two[u][r], 0);
        bs[r][1] = __builtin_amdgcn_cvt_f32_fp8((int)two[u][r], 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int s = 0; s < 4; ++s) deq[r][4 * i + s] = fp4_pair(code[u][r][i], s);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4* xp4 = reinterpret_cast<const u32x4*>(X + (int64_t)m * K + (cc[u] << 5));
        uint32_t xw[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 t = PX ? xr[u][PX ? m : 0][i] : xp4[i];
          xw[4 * i] = t[0]; xw[4 * i + 1] = t[1]; xw[4 * i + 2] = t[2]; xw[4 * i + 3] = t[3];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) d0 = dot2_bf16(deq[r][j], xw[j], d0);
#pragma unroll
          for (int j = 8; j < 16; ++j) d1 = dot2_bf16(deq[r][j], xw[j], d1);
          acc[m][r] = __builtin_fmaf(bs[r][1], d1, __builtin_fmaf(bs[r][0], d0, acc[m][r]));
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
      if (i < M * R && n0 + i % R < N) Y[(int64_t)(i / R) * N + n0 + i % R] = t[j] * ts;
    }
  }
}

// M <= 2 with the activations in LDS (M * K * 2 bytes <= 64 KiB): each block stages
// X once, by LDS-DMA ahead of the first weight batch, so the activation bytes cross the
// memory pipeline once per block of four waves instead of once per wave; each wave
// then reads its chunks' activations from LDS.
constexpr int kFp4LdsBytes = 64 * 1024;

template <int M, int R, int CPL>
// (no __restrict__ on the inputs: with it the compiler may treat their loads as freely
// movable and sink the first weight batch below the staging barrier)
__global__ __launch_bounds__(256) void fp4_gemv_lds_kernel(const uint16_t* X, const uint8_t* C, const uint8_t* B,
                                                            float ts, float* __restrict__ Y, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xl[];   // X [M][K] bf16, as loaded
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = wave * R;
  const int kbytes = K >> 1;
  const int nblk = K >> 4;
  const int nchunk = K >> 5;
  const int nbatch = (nchunk + 64 * CPL - 1) / (64 * CPL);

  u32x4 code[CPL][R];
  uint32_t two[CPL][R];
  auto issue = [&](int b) {
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = min(lane + 64 * (b * CPL + u), nchunk - 1);   // in-bounds address past the row's end
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(n0 + r, N - 1);
        code[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(C + (int64_t)row * kbytes + (c << 4)));
        two[u][r] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(B + (int64_t)row * nblk + (c << 1)));
      }
    }
  };

  // X -> LDS by LDS-DMA (no registers, no VALU), requested before the first weight
  // batch: 1 KiB pieces over the block's waves, lane l's 16 bytes at the piece's start
  // + 16 l (a partial last piece reads its last 16 bytes again into the LDS padding)
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
  // the LDS-DMA loads are not in the compiler's count: wait for every load of this wave
  // (the first weight batch too -- its products need it next anyway), then the barrier
  // publishes every wave's X pieces
  __builtin_amdgcn_s_waitcnt(gemm::vmcnt_lgkm0_imm(0));
  __builtin_amdgcn_s_barrier();
  if (n0 >= N) return;   // uniform per wave, after the block barrier

  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  for (int b = 0; b < nbatch; ++b) {
    if (b > 0) issue(b);
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = lane + 64 * (b * CPL + u);
      if (c >= nchunk) break;
      uint32_t deq[R][16];
      float bs[R][2];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bs[r][0] = __builtin_amdgcn_cvt_f32_fp8((int)two[u][r], 0);
        bs[r][1] = __builtin_amdgcn_cvt_f32_fp8((int)two[u][r], 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) deq[r][4 * i + q] = fp4_pair(code[u][r][i], q);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4* src = reinterpret_cast<const u32x4*>(xl) + (m * (K >> 3)) + 4 * c;   // the chunk's 32 activations
        uint32_t xw[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 t = src[i];
          xw[4 * i] = t[0]; xw[4 * i + 1] = t[1]; xw[4 * i + 2] = t[2]; xw[4 * i + 3] = t[3];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) d0 = dot2_bf16(deq[r][j], xw[j], d0);
#pragma unroll
          for (int j = 8; j < 16; ++j) d1 = dot2_bf16(deq[r][j], xw[j], d1);
          acc[m][r] = __builtin_fmaf(bs[r][1], d1, __builtin_fmaf(bs[r][0], d0, acc[m][r]));
        }
      }
    }
  }

  constexpr int V = pow2_ceil(M * R);
  float t[V];
#pragma unroll
  for (int i = 0; i < V; ++i) t[i] = i < M * R ? acc[i / R][i % R] : 0.0f;
  wave_sums<V>(t);
  if (wave_sums_owner<V>(lane)) {
#pragma unroll
    for (int j = 0; j < wave_sums_out<V>; ++j) {
      const int i = wave_sums_index<V>(j, lane >> 4);
      if (i < M * R && n0 + i % R < N) Y[(int64_t)(i / R) * N + n0 + i % R] = t[j] * ts;
    }
  }
}

template <int M, int R, int CPL>
static hipError_t launch_cfg(const uint16_t* X, const uint8_t* C, const uint8_t* B, float ts, float* Y, int N,
                             int K, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  // whole 1 KiB pieces: the LDS-DMA writes a partial last piece's padding too
  const size_t lds = ((size_t)M * K * 2 + 1023) / 1024 * 1024;
  if constexpr (M <= 2) {
    if (lds <= (size_t)kFp4LdsBytes) {
      hipLaunchKernelGGL((fp4_gemv_lds_kernel<M, R, CPL>), dim3((waves + 3) / 4), dim3(256), lds, stream, X, C, B, ts,
                         Y, N, K);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fp4_gemv_kernel<M, R, CPL>), dim3((waves + 3) / 4), dim3(256), 0, stream, X, C, B, ts, Y, N,
                     K);
  return hipGetLastError();
}

// Rows per wave by N (more rows per wave over a wide N); for one activation row, two
// chunks per lane in flight, four over rows of more than 128 chunks (K > 4096), so a
// wave's row is requested in one or two round trips (measured at M = 1: [4096, 14336]
// 14.3 -> 9.9 us, [14336, 4096] 9.05 -> 8.9 us; at M = 2 the extra registers cost more
// than they gain, so one chunk).
template <int M>
static hipError_t launch_m(const uint16_t* X, const uint8_t* C, const uint8_t* B, float ts, float* Y, int N,
                           int K, hipStream_t stream) {
  const int nchunk = K >> 5;
  // rows of more than 8192 codes (K > 8192): eight chunks per lane, the whole row of a
  // 14336-code row in one round trip ([4096, 14336] with the activations in LDS:
  // 9.47 -> 9.17 us against four)
  const int cpl = M == 1 ? (nchunk > 256 ? 8 : nchunk > 128 ? 4 : 2) : 1;
  if constexpr (M == 1) {
    // one row over a wide N with rows of more than 2048 codes: two rows per wave, so twice
    // the waves share the memory latency ([14336, 4096] 8.9 -> 8.66 us; at K = 2048 four
    // rows per wave stay faster)
    if (N >= 8192 && nchunk > 64) {
      if (cpl == 8) return launch_cfg<M, 2, 8>(X, C, B, ts, Y, N, K, stream);
      if (cpl == 4) return launch_cfg<M, 2, 4>(X, C, B, ts, Y, N, K, stream);
      return launch_cfg<M, 2, 2>(X, C, B, ts, Y, N, K, stream);
    }
  }
  if (N >= 8192) {
    if constexpr (M == 1) {
      if (cpl == 4) return launch_cfg<M, 4, 4>(X, C, B, ts, Y, N, K, stream);
      if (cpl == 2) return launch_cfg<M, 4, 2>(X, C, B, ts, Y, N, K, stream);
    }
    return launch_cfg<M, 4, 1>(X, C, B, ts, Y, N, K, stream);
  }
  if (N >= 4096) {
    if constexpr (M == 1) {
      if (cpl == 8) return launch_cfg<M, 2, 8>(X, C, B, ts, Y, N, K, stream);
      if (cpl == 4) return launch_cfg<M, 2, 4>(X, C, B, ts, Y, N, K, stream);
      if (cpl == 2) return launch_cfg<M, 2, 2>(X, C, B, ts, Y, N, K, stream);
    }
    return launch_cfg<M, 2, 1>(X, C, B, ts, Y, N, K, stream);
  }
  if constexpr (M == 1) {
    if (cpl == 8) return launch_cfg<M, 1, 8>(X, C, B, ts, Y, N, K, stream);
    if (cpl == 4) return launch_cfg<M, 1, 4>(X, C, B, ts, Y, N, K, stream);
    if (cpl == 2) return launch_cfg<M, 1, 2>(X, C, B, ts, Y, N, K, stream);
  }
  return launch_cfg<M, 1, 1>(X, C, B, ts, Y, N, K, stream);
}

hipError_t launch_fp4_gemv_valu(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale,
                                float ts, int N, float* Y, hipStream_t stream) {
  switch (M) {
#define AQ_CASE(mm) case mm: return launch_m<mm>(X, codes, bscale, ts, Y, N, K, stream);
    AQ_CASE(1) AQ_CASE(2) AQ_CASE(3) AQ_CASE(4) AQ_CASE(5) AQ_CASE(6) AQ_CASE(7) AQ_CASE(8)
    AQ_CASE(9) AQ_CASE(10) AQ_CASE(11) AQ_CASE(12) AQ_CASE(13) AQ_CASE(14) AQ_CASE(15) AQ_CASE(16)
#undef AQ_CASE
    default: return hipErrorInvalidValue;
  }
}

// The VALU kernel up to 2 activation rows, the matrix-core kernel from 3 when K % 64 == 0
// (measured at M = 3: 8.2 against 7.2 us on [11008, 2048], 7.4 against 6.7 on
// [4096, 4096], 4.5 against 4.6 on [2048, 2048]; at M = 16 on [14336, 4096], 62 against
// 23 us).  Rows with K % 64 != 0 take the VALU kernel at any M.
hipError_t launch_fp4_gemv(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale,
                           float ts, int N, float* Y, hipStream_t stream) {
  if (M >= 3 && K % 64 == 0) return launch_fp4_gemv_mfma(X, M, K, codes, bscale, ts, N, Y, stream);
  return launch_fp4_gemv_valu(X, M, K, codes, bscale, ts, N, Y, stream);
}

}  // namespace aq

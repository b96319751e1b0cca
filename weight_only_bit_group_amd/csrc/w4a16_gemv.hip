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
// Design (HBM-bound at M = 1):
//  * One wavefront owns R output rows.  A row of packed codes is K/2 bytes; lane l
//    reads the 16-byte chunks c = l, l + 64, ... (32 codes each, always inside one
//    group since g >= 32), so each load instruction of the wave covers 1 KiB of one
//    row with 128-bit accesses.  All code / S / z loads of a batch of chunks are
//    issued before anything waits on them (and are pinned there: the compiler may
//    otherwise sink them below the block barrier, which serialises the X staging
//    latency with the weight stream).
//  * X is staged once per block in LDS, already permuted into the (k, k + 4)
//    bf16 pairs the dequantized codes come out in, plus the sum of every 8
//    activations; a raw s_barrier waits only for LDS.  The first activation units
//    are requested before the weights (loads return in order, so L2-resident
//    activations requested behind the HBM weight stream would wait for it).  The
//    staging takes up to 64 KiB of LDS, up to 152 KiB for rows longer than 4096 codes
//    at two or more activation rows when the blocks still fit one round; otherwise each
//    lane reads its activation chunk straight from global memory.
//  * Exact integer dequantization: for a code dword d (8 nibbles)
//      v_and_or_b32(d >> 4s, 0x000F000F, 0x43004300)
//    is the bf16 pair (128 + q_s, 128 + q_{s+4}) (the shifts one v_lshrrev_b64 per
//    dword pair); v_dot2_f32_bf16 accumulates
//    x * (128 + q) in fp32 and the chunk sum is corrected by -(128 + z) * sum(x)
//    before the fp32 group step S is applied -- no rounded bf16 weight is formed.
//  * The wave's M x R sets of 64 lane partials are reduced together: halved across
//    lanes 32 and 16 apart with v_permlane32_swap / v_permlane16_swap, then summed in
//    16-lane rows with DPP; one lane per total writes it.
#include <atomic>

#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

namespace {

constexpr int kLdsBytes = 64 * 1024;
// staged activations of long rows at M >= 2 (the dynamic-LDS limit raised per instance)
constexpr int kLdsLongBytes = 152 * 1024;
constexpr int kLdsPerCu = 160 * 1024;

// (k, k+4) pairing of one 8-activation dword quad: xw = 4 dwords of natural bf16 pairs.
__device__ __forceinline__ u32x4 permute_pairs(const u32x4 t) {
  u32x4 p;
  p[0] = __builtin_amdgcn_perm(t[2], t[0], 0x05040100u);
  p[1] = __builtin_amdgcn_perm(t[2], t[0], 0x07060302u);
  p[2] = __builtin_amdgcn_perm(t[3], t[1], 0x05040100u);
  p[3] = __builtin_amdgcn_perm(t[3], t[1], 0x07060302u);
  return p;
}

__device__ __forceinline__ float sum8(const u32x4 t) {
  float s = dot2_bf16(t[0], 0x3F803F80u, 0.0f);
  s = dot2_bf16(t[1], 0x3F803F80u, s);
  s = dot2_bf16(t[2], 0x3F803F80u, s);
  return dot2_bf16(t[3], 0x3F803F80u, s);
}

// sum_k x_k * (128 + q_k) over one 32-code chunk; xp = the chunk's 16 permuted pairs.
// The shifted code copies come from one 64-bit shift per dword pair (3 instead of 6
// shifts per pair; [11008, 2048] M = 1: 4.34 -> 4.27 us).
__device__ __forceinline__ float chunk_dot(const u32x4 code, const uint32_t* xp, uint32_t mask, uint32_t magic) {
  float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i += 2) {
    uint32_t sh[4][2];
    nibble_shifts(code[i], code[i + 1], sh);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w = (sh[s][h] & mask) | magic;
        if (s & 1) d1 = dot2_bf16(w, xp[4 * (i + h) + s], d1);
        else d0 = dot2_bf16(w, xp[4 * (i + h) + s], d0);
      }
  }
  return d0 + d1;
}

// LDS_X: X [M, K] staged in LDS as permuted pairs (M * K / 2 dwords) + 8-sums (M * K / 8 floats).
// CPL: 16-byte code chunks per lane loaded per batch (all issued before use).
// KF: the row length when fixed at compile time (0: K as passed).
// WPB: waves per block (the activation staging is shared by the block's waves).
template <int M, int R, int CPL, bool LDS_X, int KF, int WPB = 4>
__global__ __launch_bounds__(64 * WPB) void w4a16_gemv_kernel(const uint16_t* X, const uint8_t* P, const float* S,
                                                          const uint8_t* Z, float* __restrict__ Y, int N, int gshift,
                                                          int k_arg) {
  // (N and gshift adjacent: the compiler fetches them with the pointers, in one scalar
  // load batch before the first weight load, instead of a second round trip)
  const int K = KF ? KF : k_arg;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & 63;
  constexpr int NT = 64 * WPB;   // threads per block
  const int wave = blockIdx.x * WPB + (threadIdx.x >> 6);
  const int n0 = wave * R;
  const int kbytes = K >> 1;
  const int nchunk = K >> 5;
  const int ngroups = K >> gshift;
  const int nbatch = (nchunk + 64 * CPL - 1) / (64 * CPL);
  uint32_t* xpl = lds;                                    // [M][K/2] permuted pairs
  float* xsl = reinterpret_cast<float*>(lds + M * (K >> 1));  // [M][K/8] 8-sums

  u32x4 code[R][CPL];
  float sc[R][CPL];
  uint32_t zb[R][CPL];
  auto issue = [&](int b) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(lane + 64 * (b * CPL + j), nchunk - 1);
      const int grp = (c << 5) >> gshift;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(n0 + r, N - 1);
        code[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(P + (int64_t)row * kbytes + (c << 4)));
        sc[r][j] = S[(int64_t)row * ngroups + grp];
        zb[r][j] = Z[(int64_t)row * ngroups + grp];
      }
    }
  };

  // X staging: up to XU 16-byte units per thread requested together, then converted
  // (one activation round trip per XU units instead of one per unit); XU follows the
  // units a thread has (M * K / 8 over the block's threads), so short single rows keep the
  // plain one-unit loop.  The first XU units are requested before the weight batch:
  // loads return in order, so activations requested after the weights would wait for
  // the HBM stream; requested first, they come back from the L2 while the weights are
  // still in flight, and the LDS staging overlaps the weight latency.
  constexpr int XU = M * CPL < 6 ? M * CPL : 6;
  const int n8 = M * (K >> 3);
  u32x4 t0[XU];
  // unit u of this thread exists (always, when the row length is fixed and the units
  // fill whole rounds of the block: the loads then issue unconditionally, ahead of the rest)
  auto xunit_ok = [&](int u) { return (KF && NT * (u + 1) <= n8) || (int)threadIdx.x + NT * u < n8; };
  if constexpr (LDS_X) {
#pragma unroll
    for (int u = 0; u < XU; ++u)
      if (xunit_ok(u)) t0[u] = reinterpret_cast<const u32x4*>(X)[threadIdx.x + NT * u];
  }
  asm volatile("" ::: "memory");
  issue(0);
  asm volatile("" ::: "memory");  // keep the first weight batch ahead of the X staging
  if constexpr (LDS_X) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int i = (int)threadIdx.x + NT * u;
      if (xunit_ok(u)) {
        reinterpret_cast<u32x4*>(xpl)[i] = permute_pairs(t0[u]);
        xsl[i] = sum8(t0[u]);
      }
    }
    for (int i0 = threadIdx.x + NT * XU; i0 < n8; i0 += NT * XU) {
      u32x4 t[XU];
#pragma unroll
      for (int u = 0; u < XU; ++u)
        if (i0 + NT * u < n8) t[u] = reinterpret_cast<const u32x4*>(X)[i0 + NT * u];
#pragma unroll
      for (int u = 0; u < XU; ++u)
        if (i0 + NT * u < n8) {
          reinterpret_cast<u32x4*>(xpl)[i0 + NT * u] = permute_pairs(t[u]);
          xsl[i0 + NT * u] = sum8(t[u]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are complete
    __builtin_amdgcn_s_barrier();
  }
  if (n0 >= N) return;  // uniform per wave, after the block barrier

  uint32_t mask, magic;
  asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(mask));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic));

  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  for (int b = 0; b < nbatch; ++b) {
    if (b > 0) issue(b);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * (b * CPL + j);
      if (c >= nchunk) break;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        uint32_t xp[16];
        float xs;
        if constexpr (LDS_X) {
          const u32x4* src = reinterpret_cast<const u32x4*>(xpl + m * (K >> 1)) + 4 * c;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 t = src[i];
            xp[4 * i] = t[0]; xp[4 * i + 1] = t[1]; xp[4 * i + 2] = t[2]; xp[4 * i + 3] = t[3];
          }
          const float4 p = reinterpret_cast<const float4*>(xsl + m * (K >> 3))[c];
          xs = (p.x + p.y) + (p.z + p.w);
        } else {
          const u32x4* src = reinterpret_cast<const u32x4*>(X + (int64_t)m * K + (c << 5));
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 t = src[i];
            const u32x4 q = permute_pairs(t);
            xp[4 * i] = q[0]; xp[4 * i + 1] = q[1]; xp[4 * i + 2] = q[2]; xp[4 * i + 3] = q[3];
            p[i] = sum8(t);
          }
          xs = (p[0] + p[1]) + (p[2] + p[3]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float d = chunk_dot(code[r][j], xp, mask, magic);
          const float zc = 128.0f + (float)zb[r][j];
          acc[m][r] = __builtin_fmaf(sc[r][j], __builtin_fmaf(-zc, xs, d), acc[m][r]);
        }
      }
    }
  }

  // all M x R totals at once (permlane swaps, then DPP inside 16-lane rows): a DPP
  // chain per total into one lane was ~0.3 us of the [11008, 2048] M = 1 launch
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

template <int M, int R, int CPL, bool LDS_X, int KF = 0, int WPB = 4>
hipError_t launch_cfg(const uint16_t* X, const uint8_t* P, const float* S, const uint8_t* Z, float* Y, int N, int K,
                      int gshift, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const size_t lds = LDS_X ? (size_t)M * (K >> 1) * 4 + (size_t)M * (K >> 3) * 4 : 0;
  hipLaunchKernelGGL((w4a16_gemv_kernel<M, R, CPL, LDS_X, KF, WPB>), dim3((waves + WPB - 1) / WPB), dim3(64 * WPB), lds,
                     stream, X, P, S, Z, Y, N, gshift, K);
  return hipGetLastError();
}

// Raise the dynamic-LDS limit of one kernel instance to kLdsLongBytes, once per device.
template <int M, int R, int CPL>
hipError_t long_lds_limit() {
  static std::atomic<uint64_t> done{0};   // bit d: set for device d
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(w4a16_gemv_kernel<M, R, CPL, true, 0>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLongBytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int M>
hipError_t launch_m(const uint16_t* X, const uint8_t* P, const float* S, const uint8_t* Z, float* Y, int N, int K,
                    int gshift, hipStream_t stream) {
  static_assert(M >= 1 && M <= 4, "the VALU GEMV serves 1 .. 4 activation rows");
  const size_t lds = (size_t)M * (K >> 1) * 4 + (size_t)M * (K >> 3) * 4;
  const bool lds_x = lds <= (size_t)kLdsBytes;
  constexpr int R = 2;
  const int nchunk = K >> 5;
  if constexpr (M >= 2) {
    // rows of more than 4096 codes at two or more activation rows: the activations staged
    // in LDS beyond 64 KiB (up to kLdsLongBytes), two rows per wave, six chunks per lane,
    // when the blocks still fit one round on the device (graph-replayed on [2048, 11008]:
    // M = 2 8.2 -> 7.3 us, M = 4 11.8 -> 10.0 against the previous launches; every wave
    // read its activation chunks from L2 before, ~90 MB at M = 4; [4096, 14336] M = 2
    // 15.4 -> 13.5 us, at M = 3, 4 two rounds of blocks would be slower)
    if (nchunk > 128 && lds <= (size_t)kLdsLongBytes) {
      const int64_t blocks = ((int64_t)(N + 1) / 2 + 3) / 4;
      if (blocks <= (int64_t)device_cu_count() * (int64_t)(kLdsPerCu / lds)) {
        const hipError_t e = long_lds_limit<M, 2, 6>();
        if (e != hipSuccess) return e;
        return launch_cfg<M, 2, 6, true>(X, P, S, Z, Y, N, K, gshift, stream);
      }
    }
  }
  if (lds_x) {
    if (nchunk <= 64) {
      // one or two rows over a wide N (e.g. the MLP projections): four rows per wave, so
      // half as many blocks stage the activations (M = 1: 4.5 -> 4.35 us on [11008, 2048];
      // M = 2: 5.45 -> 5.26 us; from M = 3 two rows per wave stay faster)
      // (K = 2048, the hidden size of the q / k / v / gate / up projections, has a
      // compile-time instance: loops and bounds fold away)
      if (M <= 2 && N >= 8192) {
        if (K == 2048) return launch_cfg<M, 4, 1, true, 2048>(X, P, S, Z, Y, N, K, gshift, stream);
        return launch_cfg<M, 4, 1, true>(X, P, S, Z, Y, N, K, gshift, stream);
      }
      // narrow outputs (e.g. the k / v projections): one row per wave, twice the waves
      // sharing the memory latency ([256, 2048] graph-replayed: M = 1 2.17 -> 2.09 us,
      // M = 4 2.74 -> 2.44; from N = 2048 two rows per wave stay faster)
      if (N <= 512) {
        if (K == 2048) return launch_cfg<M, 1, 1, true, 2048>(X, P, S, Z, Y, N, K, gshift, stream);
        return launch_cfg<M, 1, 1, true>(X, P, S, Z, Y, N, K, gshift, stream);
      }
      return launch_cfg<M, R, 1, true>(X, P, S, Z, Y, N, K, gshift, stream);
    }
    // long rows (K > 4096, e.g. a down projection): one row per wave and up to six
    // chunks per lane in flight, so the whole row is requested at once and twice as
    // many waves share the HBM latency; rows of more than 12288 codes at one activation
    // row in blocks of eight waves, so each staging of the activation row serves twice
    // the waves (graph-replayed M = 1: [4096, 14336] 10.24 -> 9.50 us, [8192, 14336]
    // 17.1 -> 16.5; at K = 11008 equal, at K = 8192 slower)
    if (nchunk > 128) {
      if (M == 1 && nchunk > 384) return launch_cfg<M, 1, 6, true, 0, 8>(X, P, S, Z, Y, N, K, gshift, stream);
      return launch_cfg<M, 1, 6, true>(X, P, S, Z, Y, N, K, gshift, stream);
    }
    return launch_cfg<M, R, 2, true>(X, P, S, Z, Y, N, K, gshift, stream);
  }
  if (nchunk <= 64) return launch_cfg<M, R, 1, false>(X, P, S, Z, Y, N, K, gshift, stream);
  return launch_cfg<M, R, 2, false>(X, P, S, Z, Y, N, K, gshift, stream);
}

}  // namespace

// M = 1 .. 4 (more rows take the matrix-core kernel)
hipError_t launch_w4a16_gemv_valu(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  switch (M) {
#define AQ_CASE(mm) case mm: return launch_m<mm>(X, P, S, Z, Y, N, K, gshift, stream);
    AQ_CASE(1) AQ_CASE(2) AQ_CASE(3) AQ_CASE(4)
#undef AQ_CASE
    default: return hipErrorInvalidValue;
  }
}

// The VALU kernel up to 4 activation rows, the matrix-core kernels from 5 (measured on
// the gate [11008, 2048], down [2048, 11008], q [2048, 2048] and [4096, 4096] shapes:
// the VALU kernel's time grows with M; at M = 4 it is 7.1 against 7.3 us on gate and
// 10.5 against 12.6 on down for the chunked matrix-core kernel, at M = 5 10.9 against
// 7.7 on gate, 17.0 against 12.6 on down and 4.1 against 4.2 on q; at M = 16 45 against
// 10 us on gate).  Where the LDS-staged matrix-core kernel applies (K = 2048, N >= 8192)
// it takes M = 4 as well: 6.6 against 7.3 us on gate.
hipError_t launch_w4a16_gemv(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                             const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  if (M >= 5 || (M == 4 && w4a16_lds_decode(M, N, K)))
    return launch_w4a16_gemv_mfma(X, M, K, P, S, Z, N, group, Y, stream);
  return launch_w4a16_gemv_valu(X, M, K, P, S, Z, N, group, Y, stream);
}

}  // namespace aq

// Decode products for small batches (up to 16 activation rows) on the matrix cores,
// gfx950: W4A16, W8A16 and FP4 weights.
//
// What they compute: the same products as the VALU decode kernels --
//   INT4 / INT8  Y[m, n] = sum_g S[n, g] * sum_{k in g} X[m, k] * (q[n, k] - z[n, g])
//                ("Quantization：模型量化", xingyuwang.me, sections 4 and 13: W4A16,
//                the compressed weights are read, dequantized inside the kernel and
//                contracted; "模型量化指南", blog.yoooo.fun, mixed 4/8-bit: 8-bit
//                codes for the layers kept at higher precision)
//   FP4          Y[m, n] = ts * sum_k X[m, k] * e2m1(c[n, k]) * e4m3(b[n, k / 16])
//                ("Lance-Quant", zingnex.cn: E2M1 codes with an E4M3 scale per
//                16-element block and an fp32 tensor scale).
// On the VALU every activation row re-does the products with the dequantized
// weights, so the VALU kernels are bound by arithmetic from a few rows up; here one
// v_mfma_f32_16x16x32_bf16 multiplies 16 activation rows (rows past M are zero)
// with 16 weight rows over 32 k.
//
// Layout of one MFMA (16 x 16 x 32): lane l holds A row (l % 16) and B column
// (l % 16), each at the eight k slots 8 (l / 16) .. +7, and the results of rows
// 4 (l / 16) .. +3 of column l % 16.  A = X, B = the weights (column n = weight
// row n), so a lane's four results share one weight row and one group step.
//  * k assignment: within a group of G consecutive k (the quantization group; for
//    FP4 a span of 64 k), lane group h = l / 16 takes the G / 4 consecutive k from
//    G g + (G / 4) h, so the G / 32 MFMA steps of a group stay inside it and each
//    group's partial is rescaled once by its fp32 step; for FP4 a lane's 16 k are
//    one scale block.
//  * Weights enter the MFMA exactly in bf16.  INT4: (code >> 4 s) & 0x000F000F |
//    0x43004300 is the exact bf16 pair (128 + q_s, 128 + q_{s+4}) (two VALU ops per
//    pair), the activation operand is permuted into the same (k, k + 4) pairs, and a
//    second MFMA against the constant -(128 + z) removes the offset, every product and
//    partial sum an exact integer times x.  INT8: the integers q - z (|q - z| <= 255,
//    at most 8 significant bits); FP4: e2m1 * e4m3 (at most 6); both in natural k
//    order, with the activation operand as loaded.
//  * Block: 16 weight rows, 4, 8 or 16 waves.  Per chunk of 2048 or 4096 k the
//    block loads the rows' codes and scales with contiguous 16-byte loads (whole
//    cache lines per instruction) into LDS, where each lane reads its operands in the
//    MFMA layout (rows padded by 32 bytes so the 16 rows of one read fall on
//    different banks); the chunk's groups are split over the waves, whose partial
//    results are added in LDS in a fixed order at the end (deterministic).  The next chunk's weights are in
//    flight while one is used; each wave's activation operands are requested
//    before the weights (loads return in order, so L2-resident activations
//    requested after the weights would wait for them).
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

namespace {

enum WFormat { WF_INT4 = 0, WF_INT8 = 1, WF_FP4 = 2 };

// (k, k + 4) pairing of 8 activations (four dwords of natural bf16 pairs).
__device__ __forceinline__ u32x4 pair_k_k4(const u32x4 t) {
  u32x4 p;
  p[0] = __builtin_amdgcn_perm(t[2], t[0], 0x05040100u);
  p[1] = __builtin_amdgcn_perm(t[2], t[0], 0x07060302u);
  p[2] = __builtin_amdgcn_perm(t[3], t[1], 0x05040100u);
  p[3] = __builtin_amdgcn_perm(t[3], t[1], 0x07060302u);
  return p;
}

// n dwords from LDS (n = 1, 2, 4 or 8; 16-byte aligned for n >= 4)
template <int NW>
__device__ __forceinline__ void lds_dwords(const uint8_t* p, uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * q);
      w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
    }
  }
}

template <int WF, int G, int NWV, int KC>
__global__ __launch_bounds__(64 * NWV) void decode_mfma_kernel(const uint16_t* __restrict__ X, int M,
                                                           const uint8_t* __restrict__ C,
                                                           const float* __restrict__ S,
                                                           const uint8_t* __restrict__ Z, float ts,
                                                           float* __restrict__ Y, int N, int K) {
  constexpr bool INT8 = WF == WF_INT8, FP4 = WF == WF_FP4;
  constexpr int CB = INT8 ? KC : KC / 2;   // code bytes per row and full chunk
  constexpr int CROW = CB + 32;            // LDS bytes per row of codes
  constexpr int TPR = 4 * NWV;             // loading threads per weight row (64 NWV threads, 16 rows)
  constexpr int NL = CB / (16 * TPR);      // 16-byte code loads per thread and chunk
  constexpr int NJ = G / 32;               // MFMA steps per group
  constexpr int NW = INT8 ? 2 * NJ : NJ;   // code dwords per lane and group
  constexpr int GPC = KC / G;              // groups per full chunk
  constexpr int GPW = GPC / NWV;           // groups per wave and full chunk
  constexpr int SZS = GPC + 1;             // INT4 / INT8: float2 per row of steps / zero points (+1: banks)
  constexpr int BSS = KC / 16 + 4;         // FP4: bytes per row of block scales
  constexpr int SZL = FP4 ? 1 : (GPC + TPR - 1) / TPR;   // INT4 / INT8 step / zero-point loads per thread
  constexpr int BPT = (KC / 16) / TPR;     // FP4: block-scale bytes per thread and full chunk (ushort loads)
  __shared__ __attribute__((aligned(16))) uint8_t cs[16 * CROW];
  __shared__ float2 sz[FP4 ? 1 : 16 * SZS];
  __shared__ uint8_t bsl[FP4 ? 16 * BSS : 4];
  __shared__ f32x4 part[NWV - 1][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int r16 = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int ngroups = K / G;
  const int64_t rowbytes = INT8 ? (int64_t)K : (int64_t)(K >> 1);
  const bool xrow = r16 < M;               // activation rows past M are zero
  const uint16_t* xp = X + (int64_t)min(r16, M - 1) * K + (G / 4) * h;

  // weight loads of one chunk: thread t takes row t / TPR; its TPR lanes cover 16 TPR
  // contiguous bytes of the row per load; INT4 / INT8 steps and zero points: groups
  // (t % TPR) + TPR i; FP4 block scales: BPT bytes from (t % TPR) BPT, as ushorts
  const int lrow = tid / TPR, lcol = tid % TPR;
  const int nl = min(n0 + lrow, N - 1);
  const uint8_t* pl = C + (int64_t)nl * rowbytes + 16 * lcol;
  struct WLoad {
    u32x4 c[NL];
    float s[SZL];
    uint32_t z[SZL];
    uint32_t b[FP4 ? BPT / 2 : 1];
  };
  auto cbytes = [&](int kc) { return INT8 ? kc : (kc >> 1); };
  auto load_w = [&](WLoad& w, int c0, int kc) {
    const int cb = cbytes(kc), coff = INT8 ? c0 : (c0 >> 1);
#pragma unroll
    for (int i = 0; i < NL; ++i)
      w.c[i] = (16 * TPR * i + 16 * lcol < cb) ? *reinterpret_cast<const u32x4*>(pl + coff + 16 * TPR * i)
                                               : u32x4{0u, 0u, 0u, 0u};
    if constexpr (FP4) {
      const int nb = kc >> 4;   // block scales in the chunk
      const uint8_t* bp = Z + (int64_t)nl * (K >> 4) + (c0 >> 4);
#pragma unroll
      for (int i = 0; i < BPT / 2; ++i) {
        const int bb = min(BPT * lcol + 2 * i, nb - 2);
        w.b[i] = *reinterpret_cast<const uint16_t*>(bp + bb);
      }
    } else {
      const int g0 = c0 / G, gc = kc / G;
#pragma unroll
      for (int i = 0; i < SZL; ++i) {
        const int gg = g0 + min(lcol + TPR * i, gc - 1);
        w.s[i] = S[(int64_t)nl * ngroups + gg];
        w.z[i] = Z[(int64_t)nl * ngroups + gg];
      }
    }
  };
  auto store_w = [&](const WLoad& w, int kc) {
    const int cb = cbytes(kc);
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (16 * TPR * i + 16 * lcol < cb)
        *reinterpret_cast<u32x4*>(&cs[lrow * CROW + 16 * TPR * i + 16 * lcol]) = w.c[i];
    if constexpr (FP4) {
      const int nb = kc >> 4;
#pragma unroll
      for (int i = 0; i < BPT / 2; ++i)
        if (BPT * lcol + 2 * i < nb)
          *reinterpret_cast<uint16_t*>(&bsl[lrow * BSS + BPT * lcol + 2 * i]) = (uint16_t)w.b[i];
    } else {
      const int gc = kc / G;
#pragma unroll
      for (int i = 0; i < SZL; ++i) {
        const int g = lcol + TPR * i;
        if (g < gc) sz[lrow * SZS + g] = make_float2(w.s[i], (float)w.z[i]);
      }
    }
  };

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  u32x4 xa[GPW][NJ];
  auto load_x = [&](int c0, int kc) {
    const int gc = kc / G, per = (gc + NWV - 1) / NWV, ga = wid * per;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = min(ga + i, gc - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        xa[i][j] = xrow ? *reinterpret_cast<const u32x4*>(xp + c0 + (int64_t)g * G + 8 * j) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // one chunk: its weights (loaded into w) go to LDS, w is reloaded with the next
  // chunk, and the wave's groups of the chunk are multiplied
  auto chunk = [&](WLoad& w, int c0) {
    const int kc = min(KC, K - c0);
    const int gc = kc / G, per = (gc + NWV - 1) / NWV, ga = wid * per, gb = min(gc, ga + per);
    __syncthreads();                 // the previous chunk's weights are no longer read
    store_w(w, kc);
    __syncthreads();
    if (c0 + KC < K) load_w(w, c0 + KC, min(KC, K - c0 - KC));   // next chunk's weights, in flight meanwhile
    // group g of the chunk, with the activation registers xa[i]
    auto group = [&](int i, int g) {
        uint32_t wc[NW];
        lds_dwords<NW>(&cs[r16 * CROW + g * (INT8 ? G : G / 2) + (INT8 ? G / 4 : G / 8) * h], wc);
        float sc = 1.0f, zf = 0.0f;
        if constexpr (FP4) {
          sc = __builtin_amdgcn_cvt_f32_fp8((int)bsl[r16 * BSS + 4 * g + h], 0);   // the lane's 16-k block
        } else {
          const float2 s_z = sz[r16 * SZS + g];
          sc = s_z.x;
          zf = s_z.y;
        }
        f32x4 tmp = {0.0f, 0.0f, 0.0f, 0.0f};
        // INT4: the bf16 pairs (128 + q_s, 128 + q_{s+4}) straight from the code dword,
        // the activations in the same (k, k + 4) pair order, and a second MFMA with the
        // constant -(128 + z) subtracting the offset (exact integers, see the header)
        const uint32_t zb16 = __float_as_uint(-(128.0f + zf)) >> 16;
        const u32x4 bz = {zb16 | (zb16 << 16), zb16 | (zb16 << 16), zb16 | (zb16 << 16), zb16 | (zb16 << 16)};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          u32x4 b;
          if constexpr (WF == WF_INT4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) b[q] = ((wc[j] >> (4 * q)) & 0x000F000Fu) | 0x43004300u;
            const u32x4 xk = pair_k_k4(xa[i][j]);
            tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xk), __builtin_bit_cast(bf16x8, b),
                                                           tmp, 0, 0, 0);
            tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xk),
                                                           __builtin_bit_cast(bf16x8, bz), tmp, 0, 0, 0);
            continue;
          } else if constexpr (INT8) {
            const uint32_t w0 = wc[2 * j], w1 = wc[2 * j + 1];
            b[0] = pack_bf16_exact(ubyte_f32<0>(w0) - zf, ubyte_f32<1>(w0) - zf);
            b[1] = pack_bf16_exact(ubyte_f32<2>(w0) - zf, ubyte_f32<3>(w0) - zf);
            b[2] = pack_bf16_exact(ubyte_f32<0>(w1) - zf, ubyte_f32<1>(w1) - zf);
            b[3] = pack_bf16_exact(ubyte_f32<2>(w1) - zf, ubyte_f32<3>(w1) - zf);
          } else {
            // unit-scale E2M1 -> bf16 pairs (k, k + 1), then the exact product with the block scale
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              uint32_t e2;
              switch (p) {
                case 0: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wc[j], 1.0f, 0)); break;
                case 1: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wc[j], 1.0f, 1)); break;
                case 2: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wc[j], 1.0f, 2)); break;
                default: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wc[j], 1.0f, 3)); break;
              }
              b[p] = pack_bf16_exact(bf16_lo(e2) * sc, bf16_hi(e2) * sc);
            }
          }
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][j]),
                                                         __builtin_bit_cast(bf16x8, b), tmp, 0, 0, 0);
        }
        if constexpr (FP4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += tmp[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(sc, tmp[e], acc[e]);
        }
    };
    if (gb - ga == GPW) {
      // a full share (every wave of a full chunk): straight-line code, so the LDS reads
      // and dequantization of the next groups can be scheduled under this group's MFMAs
#pragma unroll
      for (int i = 0; i < GPW; ++i) group(i, ga + i);
    } else {
#pragma unroll
      for (int i = 0; i < GPW; ++i)
        if (ga + i < gb) group(i, ga + i);   // uniform
    }
    if (c0 + KC < K) load_x(c0 + KC, min(KC, K - c0 - KC));
  };
  WLoad wl;
  load_x(0, min(KC, K));
  asm volatile("" ::: "memory");
  load_w(wl, 0, min(KC, K));
  for (int c0 = 0; c0 < K; c0 += KC) chunk(wl, c0);

  // the waves' partial results added in a fixed order: ((w0 + w1) + w2) + ...
  if (wid > 0) part[wid - 1][lane] = acc;
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int w = 0; w < NWV - 1; ++w) {
      const f32x4 p = part[w][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += p[e];
    }
    if (n0 + r16 < N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * h + e;
        if (m < M) Y[(int64_t)m * N + n0 + r16] = FP4 ? acc[e] * ts : acc[e];
      }
    }
  }
}

template <int WF, int G, int NWV, int KC>
hipError_t launch_cfg(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z, float ts,
                      int N, float* Y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 15) / 16)), block(64 * NWV);
  hipLaunchKernelGGL((decode_mfma_kernel<WF, G, NWV, KC>), grid, block, 0, stream, X, M, C, S, Z, ts, Y, N, K);
  return hipGetLastError();
}

// Waves per block and chunk length (measured on gfx950, M = 4 .. 16):
//  * rows longer than 2048 k: 16 waves over chunks of 4096 k -- a block's weights take
//    half as many serial round trips to memory, and the extra waves share the
//    dequantization (2048 x 11008 INT4: 13 us against 21 us with 4 waves and 2048 k);
//  * shorter rows (one chunk): 8 waves over 2048 k -- the smaller LDS footprint keeps
//    several blocks per compute unit; INT4 with many blocks (N >= 8192) is a little
//    faster with 4 waves.
template <int WF, int G>
hipError_t launch_group(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z,
                        float ts, int N, float* Y, hipStream_t stream) {
  if (K > 2048) return launch_cfg<WF, G, 16, 4096>(X, M, K, C, S, Z, ts, N, Y, stream);
  if (WF == WF_INT4 && N >= 8192) return launch_cfg<WF, G, 4, 2048>(X, M, K, C, S, Z, ts, N, Y, stream);
  return launch_cfg<WF, G, 8, 2048>(X, M, K, C, S, Z, ts, N, Y, stream);
}

template <int WF>
hipError_t launch_format(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z,
                         float ts, int N, int group, float* Y, hipStream_t stream) {
  switch (group) {
    case 32: return launch_group<WF, 32>(X, M, K, C, S, Z, ts, N, Y, stream);
    case 64: return launch_group<WF, 64>(X, M, K, C, S, Z, ts, N, Y, stream);
    case 128: return launch_group<WF, 128>(X, M, K, C, S, Z, ts, N, Y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_w4a16_gemv_mfma(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  return launch_format<WF_INT4>(X, M, K, P, S, Z, 1.0f, N, group, Y, stream);
}

hipError_t launch_w8a16_gemv_mfma(const uint16_t* X, int M, int K, const uint8_t* C, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  return launch_format<WF_INT8>(X, M, K, C, S, Z, 1.0f, N, group, Y, stream);
}

// FP4: K % 64 == 0 (groups of 64 k, each lane's 16 k one scale block)
hipError_t launch_fp4_gemv_mfma(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale,
                                float ts, int N, float* Y, hipStream_t stream) {
  return launch_group<WF_FP4, 64>(X, M, K, codes, nullptr, bscale, ts, N, Y, stream);
}

}  // namespace aq

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
//  * Two kernels.  The chunked one: a block of 16 weight rows, 4, 8 or 16 waves; per
//    chunk of 2048 or 4096 k the block loads the rows' codes and scales with
//    contiguous 16-byte loads (whole cache lines per instruction) into LDS, where each
//    lane reads its operands in the MFMA layout (rows padded by 32 bytes so the 16
//    rows of one read fall on different banks); the chunk's groups are split over the
//    waves, whose partial results are added in LDS in a fixed order at the end
//    (deterministic).  The next chunk's weights are in flight while one is used; each
//    wave loads the activation operands of its groups (rows below M only) straight in
//    the MFMA layout, requested before the weights (loads return in order, so
//    L2-resident activations requested after the weights would wait for them).  The
//    LDS-staged one (rows of at most 2048 k, many rows, larger batches) is described
//    at its definition: 48 or 64 weight rows per block and the activations staged once
//    per block.
#include <atomic>

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

// INT4: the bf16 pair (-(128 + z), -(128 + z)) of a zero point (exact: 128 + z <= 143).
__device__ __forceinline__ uint32_t offset_pair(float zf) {
  const uint32_t zb16 = __float_as_uint(-(128.0f + zf)) >> 16;
  return zb16 | (zb16 << 16);
}

// The products of one group for a lane: wc = its code dwords, xk = its activation
// operands per 32-k MFMA step (INT4: already in (k, k + 4) pair order), sc / zf = the
// group step and zero point (FP4: the lane's block scale), zp = offset_pair(zf) (INT4).
// Returns the unscaled partial (INT4 / INT8) or the block-scaled one (FP4).
template <int WF, int G>
__device__ __forceinline__ f32x4 group_product(const uint32_t* wc, const u32x4* xk, float sc, float zf, uint32_t zp) {
  constexpr int NJ = G / 32;
  f32x4 tmp = {0.0f, 0.0f, 0.0f, 0.0f};
  // INT4: the bf16 pairs (128 + q_s, 128 + q_{s+4}) straight from the code dword, the
  // activations in the same (k, k + 4) pair order, and a second MFMA with the constant
  // -(128 + z) subtracting the offset (exact integers, see the header)
  const u32x4 bz = {zp, zp, zp, zp};
  // the mask in an SGPR and the magic in a VGPR, both opaque to the optimizer, so each
  // pair is one v_and_or_b32 (with the constants visible it emits and + or; gfx9 VOP3
  // takes no literal operand)
  uint32_t mask = 0, magic = 0;
  if constexpr (WF == WF_INT4) {
    asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic));
  }
  // INT4: the shifted code copies of dword pairs from one 64-bit shift each
  uint32_t sh[NJ >= 2 ? NJ / 2 : 1][4][2];
  if constexpr (WF == WF_INT4 && NJ >= 2) {
#pragma unroll
    for (int j = 0; j < NJ; j += 2) nibble_shifts(wc[j], wc[j + 1], sh[j / 2]);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    u32x4 b;
    if constexpr (WF == WF_INT4) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        b[q] = ((NJ >= 2 ? sh[j / 2][q][j & 1] : wc[j] >> (4 * q)) & mask) | magic;
      tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xk[j]), __builtin_bit_cast(bf16x8, b),
                                                     tmp, 0, 0, 0);
      tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xk[j]), __builtin_bit_cast(bf16x8, bz),
                                                     tmp, 0, 0, 0);
      continue;
    } else if constexpr (WF == WF_INT8) {
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
    tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xk[j]), __builtin_bit_cast(bf16x8, b),
                                                   tmp, 0, 0, 0);
  }
  return tmp;
}

// acc += S * partial (INT4 / INT8), acc += partial (FP4: the block scale is in the weights)
template <int WF>
__device__ __forceinline__ void accumulate_group(f32x4& acc, const f32x4 tmp, float sc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = WF == WF_FP4 ? acc[e] + tmp[e] : __builtin_fmaf(sc, tmp[e], acc[e]);
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
        u32x4 xk[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) xk[j] = WF == WF_INT4 ? pair_k_k4(xa[i][j]) : xa[i][j];
        accumulate_group<WF>(acc, group_product<WF, G>(wc, xk, sc, zf, offset_pair(zf)), sc);
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

// floor(u / d) for 0 <= u < 2^22, 1 <= d < 2^22, with rd = fl32(1 / d): the fp32
// product is within 0.5 of u / d, so one correction each way gives the exact quotient
// (the integer division would cost ~25 VALU instructions per index before the loads
// that need it can issue).
__device__ __forceinline__ int div_small(int u, int d, float rd) {
  int q = (int)((float)u * rd);
  q -= (q * d > u) ? 1 : 0;
  q += ((q + 1) * d <= u) ? 1 : 0;
  return q;
}

// ---- rows of at most 2048 k: activations staged once per block in LDS ------------
// The block covers RG x 16 weight rows with 4 RG waves: wave (rg, kq) multiplies row
// group rg (16 rows) over the kq-th quarter of the groups, and the four quarters are
// added in LDS in a fixed order.  Everything the block reads is requested at once, the
// weight codes first: codes, steps and zero points (or block scales) as contiguous
// 16-byte / element loads; the activation rows (rows past M zero) as contiguous 16-byte
// loads, stored in LDS already in the MFMA operand order (INT4: (k, k + 4) pairs), so
// every block reads each activation byte once, with whole cache lines per load.
// Loading the activations per wave in the MFMA layout instead (16 rows x 16 bytes per
// instruction, every block all of X) costs ~3 us of the 9.8 us the [11008, 2048] M = 16
// product took that way; 48 rows per block keep the grid to one round of blocks.
// Dynamic LDS: X [16][2 K + 16], codes [16 RG][K / 2 (INT8: K) + 32], steps and zero
// points [16 RG][K / G + 1] float2 (INT4: the step and the bf16 offset pair of the zero
// point; FP4: block scales [16 RG][K / 16 + 4] bytes),
// partials [3][RG][64] f32x4.
constexpr int kLdsKMax = 2048;
constexpr size_t kLdsLimit = 160 * 1024;   // LDS of one gfx950 compute unit
// smallest batch for which the LDS-staged kernel runs (below it the chunked kernel,
// which loads only the M activation rows, reads less): at K = 2048 (the compile-time
// instance) from 4 rows, at other K from 12
constexpr int kLdsMinMFixed = 4;
constexpr int kLdsMinM = 12;

template <int WF>
__host__ __device__ constexpr int lds_code_bytes(int K) { return WF == WF_INT8 ? K : K / 2; }

template <int WF, int G>
constexpr size_t decode_lds_bytes(int RG, int K) {
  const size_t rows = 16 * (size_t)RG;
  const size_t aux = WF == WF_FP4 ? rows * (size_t)(K / 16 + 4) : rows * (size_t)(K / G + 1) * 8;
  return 16 * (size_t)(2 * K + 16) + rows * (size_t)(lds_code_bytes<WF>(K) + 32) + aux + 3 * (size_t)RG * 64 * 16;
}

// KF: the row length when fixed at compile time (0: K as passed)
template <int WF, int G, int RG, int KF>
__global__ __launch_bounds__(256 * RG) void decode_lds_kernel(const uint16_t* __restrict__ X, int M,
                                                             const uint8_t* __restrict__ C,
                                                             const float* __restrict__ S,
                                                             const uint8_t* __restrict__ Z, float ts,
                                                             float* __restrict__ Y, int N, int k_arg) {
  const int K = KF ? KF : k_arg;
  constexpr bool INT8 = WF == WF_INT8, FP4 = WF == WF_FP4;
  constexpr int NT = 256 * RG, ROWS = 16 * RG;
  constexpr int NJ = G / 32;                       // MFMA steps per group
  constexpr int NW = INT8 ? 2 * NJ : NJ;           // code dwords per lane and group
  // per-thread load slots, sized for K = kLdsKMax
  constexpr int CU = (ROWS * lds_code_bytes<WF>(kLdsKMax) / 16 + NT - 1) / NT;
  constexpr int XU = (16 * kLdsKMax / 8 + NT - 1) / NT;
  constexpr int AU = FP4 ? (ROWS * kLdsKMax / 32 + NT - 1) / NT      // block-scale ushorts
                         : (ROWS * (kLdsKMax / G) + NT - 1) / NT;    // steps / zero points
  constexpr int GQ = (kLdsKMax / G + 3) / 4;       // most groups per quarter
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int cbk = lds_code_bytes<WF>(K), upr = cbk >> 4;   // code bytes / 16-byte units per row
  const int crow = cbk + 32, xrow = 2 * K + 16;
  const int ng = K / G, szs = ng + 1, bss = K / 16 + 4;
  const int xpr = K >> 3, bpr = K >> 5;   // 16-byte activation units / block-scale ushorts per row
  const float rupr = 1.0f / (float)upr, rng = 1.0f / (float)ng, rxpr = 1.0f / (float)xpr, rbpr = 1.0f / (float)bpr;
  // u / d: folded into shifts when K is a compile-time constant, else from the reciprocal
  auto quo = [&](int u, int d, float rd) -> int { return KF ? (int)((unsigned)u / (unsigned)d) : div_small(u, d, rd); };
  uint8_t* xs = dyn;
  uint8_t* cs = xs + 16 * xrow;
  float2* sz = reinterpret_cast<float2*>(cs + ROWS * crow);
  uint8_t* bsl = reinterpret_cast<uint8_t*>(sz + (FP4 ? 0 : ROWS * szs));
  f32x4* part = reinterpret_cast<f32x4*>(bsl + (FP4 ? ROWS * bss : 0));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int r16 = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * ROWS;
  const int nrows = min(ROWS, N - n0);
  const uint32_t rowbytes = (uint32_t)cbk;

  // ---- loads (all in flight together; rows past N clamped to the last row) ----
  const int cunits = ROWS * upr;
  // loads address a uniform block base plus a 32-bit lane offset (the block's rows span
  // less than 2^32 bytes)
  const uint8_t* cblk = C + (int64_t)n0 * rowbytes;
  u32x4 cw[CU];
#pragma unroll
  for (int i = 0; i < CU; ++i) {
    const int u = min(tid + NT * i, cunits - 1);
    const int q = quo(u, upr, rupr), r = min(q, nrows - 1);
    cw[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(cblk + ((uint32_t)r * rowbytes + 16u * (uint32_t)(u - q * upr))));
  }
  float av[FP4 ? 1 : AU];
  uint32_t zv[AU];
  if constexpr (FP4) {
    const int aunits = ROWS * bpr;
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int e = min(tid + NT * i, aunits - 1);
      const int q = quo(e, bpr, rbpr), r = min(q, nrows - 1);
      zv[i] = *reinterpret_cast<const uint16_t*>(Z + (int64_t)n0 * (K >> 4) +
                                                 ((uint32_t)r * (uint32_t)(K >> 4) + 2u * (uint32_t)(e - q * bpr)));
    }
  } else {
    const int aunits = ROWS * ng;
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int e = min(tid + NT * i, aunits - 1);
      const int q = quo(e, ng, rng), r = min(q, nrows - 1), g = e - q * ng;
      const uint32_t off = (uint32_t)r * (uint32_t)ng + (uint32_t)g;
      av[i] = (S + (int64_t)n0 * ng)[off];
      zv[i] = (Z + (int64_t)n0 * ng)[off];
    }
  }
  const int xunits = 16 * xpr;
  u32x4 xv[XU];
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int u = min(tid + NT * i, xunits - 1);
    const int r = quo(u, xpr, rxpr);
    xv[i] = r < M ? *reinterpret_cast<const u32x4*>(X + ((uint32_t)r * (uint32_t)K + 8u * (uint32_t)(u - r * xpr)))
                  : u32x4{0u, 0u, 0u, 0u};
  }
  // ---- to LDS ----
#pragma unroll
  for (int i = 0; i < CU; ++i) {
    const int u = tid + NT * i;
    if (u < cunits) {
      const int q = quo(u, upr, rupr);
      *reinterpret_cast<u32x4*>(&cs[q * crow + 16 * (u - q * upr)]) = cw[i];
    }
  }
  if constexpr (FP4) {
    const int aunits = ROWS * bpr;
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int e = tid + NT * i;
      if (e < aunits) {
        const int r = quo(e, bpr, rbpr);
        *reinterpret_cast<uint16_t*>(&bsl[r * bss + 2 * (e - r * bpr)]) = (uint16_t)zv[i];
      }
    }
  } else {
    const int aunits = ROWS * ng;
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int e = tid + NT * i;
      if (e < aunits) {
        const int r = quo(e, ng, rng);
        // INT4: the offset pair of the zero point, formed once per row and group
        const float zslot = WF == WF_INT4 ? __uint_as_float(offset_pair((float)zv[i])) : (float)zv[i];
        sz[r * szs + (e - r * ng)] = make_float2(av[i], zslot);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int u = tid + NT * i;
    if (u < xunits) {
      const int r = quo(u, xpr, rxpr);
      *reinterpret_cast<u32x4*>(&xs[r * xrow + 16 * (u - r * xpr)]) = WF == WF_INT4 ? pair_k_k4(xv[i]) : xv[i];
    }
  }
  __syncthreads();

  // ---- products: wave (rg, kq), groups [kq per, min(ng, (kq + 1) per)) ----
  const int rg = wid >> 2, kq = wid & 3;
  const int row = 16 * rg + r16;
  const int per = (ng + 3) >> 2, ga = kq * per, gb = min(ng, ga + per);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto group = [&](int g) {
    uint32_t wc[NW];
    lds_dwords<NW>(&cs[row * crow + g * (INT8 ? G : G / 2) + (INT8 ? G / 4 : G / 8) * h], wc);
    float sc = 1.0f, zf = 0.0f;
    uint32_t zp = 0;
    if constexpr (FP4) {
      sc = __builtin_amdgcn_cvt_f32_fp8((int)bsl[row * bss + 4 * g + h], 0);   // the lane's 16-k block
    } else {
      const float2 s_z = sz[row * szs + g];
      sc = s_z.x;
      if constexpr (WF == WF_INT4) zp = __float_as_uint(s_z.y);
      else zf = s_z.y;
    }
    u32x4 xk[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      xk[j] = *reinterpret_cast<const u32x4*>(&xs[r16 * xrow + 2 * (g * G + (G / 4) * h + 8 * j)]);
    accumulate_group<WF>(acc, group_product<WF, G>(wc, xk, sc, zf, zp), sc);
  };
  if (gb - ga == GQ) {
    // a full quarter (K = 2048): straight-line code, so the LDS reads and dequantization
    // of the next groups can be scheduled under this group's MFMAs
#pragma unroll
    for (int i = 0; i < GQ; ++i) group(ga + i);
  } else {
#pragma unroll
    for (int i = 0; i < GQ; ++i)
      if (ga + i < gb) group(ga + i);   // uniform
  }
  // quarters added in a fixed order: ((q0 + q1) + q2) + q3
  if (kq > 0) part[((kq - 1) * RG + rg) * 64 + lane] = acc;
  __syncthreads();
  if (kq == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const f32x4 p = part[(w * RG + rg) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += p[e];
    }
    const int n = n0 + row;
    if (n < N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * h + e;
        if (m < M) Y[(int64_t)m * N + n] = FP4 ? acc[e] * ts : acc[e];
      }
    }
  }
}

// Raise the dynamic-LDS limit of one kernel instance once per device.
template <int WF, int G, int RG, int KF>
hipError_t lds_limit() {
  static std::atomic<uint64_t> done{0};   // bit d: set for device d
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_lds_kernel<WF, G, RG, KF>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int WF, int G, int RG, int KF>
hipError_t launch_lds_k(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z, float ts,
                        int N, float* Y, hipStream_t stream) {
  const size_t bytes = decode_lds_bytes<WF, G>(RG, K);
  hipError_t e = lds_limit<WF, G, RG, KF>();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_lds_kernel<WF, G, RG, KF>), dim3((unsigned)((N + 16 * RG - 1) / (16 * RG))),
                     dim3(256 * RG), bytes, stream, X, M, C, S, Z, ts, Y, N, K);
  return hipGetLastError();
}

// K = 2048 (the hidden size of the models served here) has its own instance, with the
// index arithmetic folded at compile time
template <int WF, int G, int RG>
hipError_t launch_lds(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z, float ts,
                      int N, float* Y, hipStream_t stream) {
  if (K == kLdsKMax) return launch_lds_k<WF, G, RG, kLdsKMax>(X, M, K, C, S, Z, ts, N, Y, stream);
  return launch_lds_k<WF, G, RG, 0>(X, M, K, C, S, Z, ts, N, Y, stream);
}

template <int WF, int G, int NWV, int KC>
hipError_t launch_cfg(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z, float ts,
                      int N, float* Y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 15) / 16)), block(64 * NWV);
  hipLaunchKernelGGL((decode_mfma_kernel<WF, G, NWV, KC>), grid, block, 0, stream, X, M, C, S, Z, ts, Y, N, K);
  return hipGetLastError();
}

// Kernel choice (measured on gfx950, g = 64, microseconds per launch, the chunked kernel
// with its best wave count against the LDS-staged one):
//  * N >= 8192 and K <= 2048: the LDS-staged kernel, 48 rows per block, 64 once 48
//    would need more blocks than CUs -- INT4 [11008, 2048]: M = 16 9.9 -> 7.4, M = 8
//    7.9 -> 6.9, M = 5 7.4 -> 6.8; [16384, 2048] M = 16 12.1 -> 8.5; FP4 [11008, 2048]
//    M = 16 9.7 -> 8.0, M = 4 7.4 -> 7.3.  At other K (no compile-time instance) it
//    wins from M = 12 ([8192, 1024] INT4 M = 16 6.6 -> 5.8, M = 8 5.4 against 5.6);
//    INT8 (twice the code bytes, 32 rows per block) does not win at these sizes;
//  * fewer rows (N < 8192: too few blocks of 48 rows) and shorter rows: the chunked
//    kernel with 8 waves over 2048 k (INT4 with N >= 8192: 4 waves);
//  * rows longer than 2048 k: 16 waves over chunks of 4096 k -- a block's weights take
//    half as many serial round trips to memory, and the extra waves share the
//    dequantization (2048 x 11008 INT4: 13 us against 21 us with 4 waves and 2048 k).
template <int WF, int G>
hipError_t launch_group(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z,
                        float ts, int N, float* Y, hipStream_t stream) {
  if constexpr (WF != WF_INT8) {
    static_assert(decode_lds_bytes<WF, G>(3, kLdsKMax) <= kLdsLimit, "48 rows fit the LDS at K = 2048");
    if (K <= kLdsKMax && N >= 8192 && M >= (K == kLdsKMax ? kLdsMinMFixed : kLdsMinM)) {
      // one round of blocks: 64 rows per block once 48 would need more blocks than CUs
      if (N > 48 * device_cu_count() && decode_lds_bytes<WF, G>(4, K) <= kLdsLimit)
        return launch_lds<WF, G, 4>(X, M, K, C, S, Z, ts, N, Y, stream);
      return launch_lds<WF, G, 3>(X, M, K, C, S, Z, ts, N, Y, stream);
    }
  }
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

bool w4a16_lds_decode(int M, int N, int K) { return K == kLdsKMax && N >= 8192 && M >= kLdsMinMFixed; }

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

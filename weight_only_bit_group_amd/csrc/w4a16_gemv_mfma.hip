// W4A16 decode product for small batches (up to 16 activation rows) on the matrix
// cores, gfx950.
//
// What it computes: the same Y[m, n] = sum_g S[n, g] * sum_{k in g} X[m, k] *
// (q[n, k] - z[n, g]) as the VALU GEMV ("Quantization：模型量化", xingyuwang.me,
// sections 4 and 13: W4A16, the compressed weights are read, dequantized inside
// the kernel and contracted).  On the VALU every activation row re-does the
// products with the dequantized weights, so the VALU GEMV is bound by arithmetic
// from a few rows up; here one v_mfma_f32_16x16x32_bf16 multiplies 16 activation
// rows (rows past M are zero) with 16 weight rows over 32 k.
//
// Layout of one MFMA (16 x 16 x 32): lane l holds A row (l % 16) and B column
// (l % 16), each at the eight k slots 8 (l / 16) .. +7, and the results of rows
// 4 (l / 16) .. +3 of column l % 16.  A = X, B = the weights (column n = weight
// row n), so a lane's four results share one weight row and one group step.
//  * k assignment: within quantization group G (g consecutive k), lane group
//    h = l / 16 takes the g / 4 consecutive k from g G + (g / 4) h, so the g / 32
//    MFMA steps of a group stay inside it and each group's partial is rescaled
//    once by its fp32 step.
//  * Weights enter the MFMA as the exact bf16 integers q - z (|q - z| <= 15), in
//    natural k order, so the activation operand is 8 consecutive bf16 of X loaded
//    as they are; no rounded weight is formed.
//  * Block: 16 weight rows.  Per chunk of 2048 k the block loads the rows' packed
//    codes (16 KiB), steps and zero points with contiguous 16-byte loads (whole
//    cache lines per instruction) into LDS, where each lane reads its operands in
//    the MFMA layout (rows padded so the 16 rows of one read hit different banks);
//    the chunk's groups are split over the 4 waves, whose partial results are added
//    in LDS in a fixed order at the end (deterministic).  The next chunk's weights
//    are in flight while one is used; each wave's activation
//    operands are requested before the weights (loads return in order, so
//    L2-resident activations requested after the weights would wait for them).
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

namespace {

constexpr int KC = 2048;              // k per chunk
constexpr int CROW = KC / 2 + 32;     // LDS bytes per weight row of codes (32 bytes of padding)

template <int G>
__global__ __launch_bounds__(256) void w4a16_gemv_mfma_kernel(const uint16_t* __restrict__ X, int M,
                                                               const uint8_t* __restrict__ P,
                                                               const float* __restrict__ S,
                                                               const uint8_t* __restrict__ Z, float* __restrict__ Y,
                                                               int N, int K) {
  constexpr int NJ = G / 32;          // MFMA steps per group
  constexpr int GPC = KC / G;         // groups per full chunk
  constexpr int GPW = GPC / 4;        // groups per wave and full chunk
  constexpr int SZS = GPC + 1;        // float2 per row of steps / zero points (+1: rows on different banks)
  __shared__ __attribute__((aligned(16))) uint8_t cs[16 * CROW];
  __shared__ float2 sz[16 * SZS];
  __shared__ f32x4 part[3][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int r16 = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int ngroups = K / G;
  const bool xrow = r16 < M;          // activation rows past M are zero
  const uint16_t* xp = X + (int64_t)min(r16, M - 1) * K + (G / 4) * h;

  // weight loads of one chunk: thread t takes row t / 16; its 16 lanes cover 256
  // contiguous bytes of the row per load (4 loads per full chunk); steps and zero
  // points: thread t takes row t / 16, groups (t % 16) + 16 i
  const int lrow = tid >> 4, lcol = tid & 15;
  const int nl = min(n0 + lrow, N - 1);
  const uint8_t* pl = P + (int64_t)nl * (K >> 1) + 16 * lcol;
  constexpr int SZL = (GPC + 15) / 16;  // step / zero-point loads per thread and chunk
  struct WLoad {
    u32x4 c[4];
    float s[SZL];
    uint32_t z[SZL];
  };
  auto load_w = [&](WLoad& w, int c0, int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w.c[i] = (256 * i + 16 * lcol < (kc >> 1)) ? *reinterpret_cast<const u32x4*>(pl + (c0 >> 1) + 256 * i)
                                                 : u32x4{0u, 0u, 0u, 0u};
    const int g0 = c0 / G, gc = kc / G;
#pragma unroll
    for (int i = 0; i < SZL; ++i) {
      const int gg = g0 + min(lcol + 16 * i, gc - 1);
      w.s[i] = S[(int64_t)nl * ngroups + gg];
      w.z[i] = Z[(int64_t)nl * ngroups + gg];
    }
  };
  auto store_w = [&](const WLoad& w, int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (256 * i + 16 * lcol < (kc >> 1)) *reinterpret_cast<u32x4*>(&cs[lrow * CROW + 256 * i + 16 * lcol]) = w.c[i];
    const int gc = kc / G;
#pragma unroll
    for (int i = 0; i < SZL; ++i) {
      const int g = lcol + 16 * i;
      if (g < gc) sz[lrow * SZS + g] = make_float2(w.s[i], (float)w.z[i]);
    }
  };

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  u32x4 xa[GPW][NJ];
  auto load_x = [&](int c0, int kc) {
    const int gc = kc / G, per = (gc + 3) / 4, ga = wid * per;
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
    const int gc = kc / G, per = (gc + 3) / 4, ga = wid * per, gb = min(gc, ga + per);
    __syncthreads();                 // the previous chunk's weights are no longer read
    store_w(w, kc);
    __syncthreads();
    if (c0 + KC < K) load_w(w, c0 + KC, min(KC, K - c0 - KC));
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = ga + i;
      if (g < gb) {   // uniform
        const float2 s_z = sz[r16 * SZS + g];
        const uint8_t* cp = &cs[r16 * CROW + g * (G / 2) + (G / 8) * h];
        uint32_t wc[NJ];
        if constexpr (NJ == 1) {
          wc[0] = *reinterpret_cast<const uint32_t*>(cp);
        } else if constexpr (NJ == 2) {
          const uint2 v = *reinterpret_cast<const uint2*>(cp);
          wc[0] = v.x; wc[1] = v.y;
        } else {
          const u32x4 v = *reinterpret_cast<const u32x4*>(cp);
          wc[0] = v[0]; wc[1] = v[1]; wc[2] = v[2]; wc[3] = v[3];
        }
        f32x4 tmp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          // codes k = 0 .. 7 of this step: even k in the low nibbles, odd k in the high ones
          const uint32_t lo = wc[j] & 0x0F0F0F0Fu, hi = (wc[j] >> 4) & 0x0F0F0F0Fu;
          const float zf = s_z.y;
          u32x4 b;
          b[0] = pack_bf16_exact(ubyte_f32<0>(lo) - zf, ubyte_f32<0>(hi) - zf);
          b[1] = pack_bf16_exact(ubyte_f32<1>(lo) - zf, ubyte_f32<1>(hi) - zf);
          b[2] = pack_bf16_exact(ubyte_f32<2>(lo) - zf, ubyte_f32<2>(hi) - zf);
          b[3] = pack_bf16_exact(ubyte_f32<3>(lo) - zf, ubyte_f32<3>(hi) - zf);
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][j]),
                                                         __builtin_bit_cast(bf16x8, b), tmp, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(s_z.x, tmp[e], acc[e]);
      }
    }
    if (c0 + KC < K) load_x(c0 + KC, min(KC, K - c0 - KC));
  };
  WLoad wl;
  load_x(0, min(KC, K));
  asm volatile("" ::: "memory");
  load_w(wl, 0, min(KC, K));
  for (int c0 = 0; c0 < K; c0 += KC) chunk(wl, c0);

  // the four partial results added in a fixed order: ((w0 + w1) + w2) + w3
  if (wid > 0) part[wid - 1][lane] = acc;
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const f32x4 p = part[w][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += p[e];
    }
    if (n0 + r16 < N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * h + e;
        if (m < M) Y[(int64_t)m * N + n0 + r16] = acc[e];
      }
    }
  }
}

}  // namespace

hipError_t launch_w4a16_gemv_mfma(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 15) / 16)), block(256);
  switch (group) {
    case 32: hipLaunchKernelGGL(w4a16_gemv_mfma_kernel<32>, grid, block, 0, stream, X, M, P, S, Z, Y, N, K); break;
    case 64: hipLaunchKernelGGL(w4a16_gemv_mfma_kernel<64>, grid, block, 0, stream, X, M, P, S, Z, Y, N, K); break;
    case 128: hipLaunchKernelGGL(w4a16_gemv_mfma_kernel<128>, grid, block, 0, stream, X, M, P, S, Z, Y, N, K); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace aq

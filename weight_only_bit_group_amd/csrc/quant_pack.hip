// Group-wise asymmetric INT4 quantization and nibble packing (gfx950).
//
// What it computes ("Quantization：模型量化", xingyuwang.me, section 2, asymmetric
// quantization with clipping to the integer range; section 3, per-group
// granularity; "Lance-Quant", zingnex.cn, grid-search / grouped INT4 packing
// section): for every group of g consecutive input channels of a weight row,
//   v = w * s_k  (fp32, only when an AWQ channel scale is given)
//   S = fl32(fl32(max v - min v) / 15),  z = clamp(rne(fl32(-min v / S)), 0, 15)
//   q = clamp(rne(fl32(v / S)) + z, 0, 15)
// with two codes per byte (even k in the low nibble).
//
// Symmetric variant (same page, section 2: a symmetric integer range with zero at
// integer zero, q = round(x / s), x_hat = q s, clipped to the range): per group
//   S = fl32(max |v| / 7),  q = clamp(rne(fl32(v / S)), -7, 7)
// stored as the code q + 8 with a zero point of 8, so the decode (code - z) S of
// the asymmetric format applies unchanged; an all-zero group stores S = 0, codes 8.
//
// 8-bit variant: the asymmetric formulas with the range 0 .. 255 and one code byte
// per weight (codes [N, K]).
//
// Mapping: W[N, K] row-major is a flat run of N*K/g groups of g contiguous
// elements.  Each lane owns U units of 8 consecutive elements (one 16-byte bf16 load
// or two 16-byte fp32 loads per unit), so a group spans g/(8U) lanes and its min/max
// is a g/(8U)-lane butterfly.  Stores are 4U bytes of codes per lane (8U for 8-bit
// codes, contiguous across the wave), one fp32 S and one u8 z per group.
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

namespace {

constexpr float kRound = 12582912.0f;   // 1.5 * 2^23

// A group's parameters as the codes use them:
//   S = fl32(fl32(max - min) / QM) (symmetric: fl32(max |v| / 7)),
//   z = clamp(rne(fl32(-min / S)), 0, QM) (symmetric: 8),
// all-zero range: S = 0, z = 0 (symmetric 8), codes z.
struct PackQ {
  float S;
  float zf;    // zero point, an exact float
  float inv;   // 1/S within 1 ulp (v_rcp_f32); 0 when S = 0
  float thr;   // tie threshold of the group's values (see near_tie)
  float kz;    // kRound + zf (exact)
};

// Whether t = v * inv may round differently from fl32(v / S): t is within 2 ulp of the
// quotient (inv within 1 ulp of 1/S, the product rounded), so only t within about 4 ulp
// of a half-integer can; with d = t - rne(t) (exact for |t| < 2^22) that is
// |d| >= 0.5 - (4.8e-7 |t| + 1.2e-7).  The threshold is taken once per group, at its
// largest |t| (so no smaller than any value's own slack); NaN (from a non-finite inv)
// counts as near.
__device__ __forceinline__ float tie_threshold(float tmax) { return __builtin_fmaf(tmax, -4.8e-7f, 0.5f - 1.2e-7f); }
__device__ __forceinline__ bool near_tie(float d, float thr) { return !(fabsf(d) < thr); }

// fl32(r / Q) for a constant Q: with y = fl32(1 / Q), q0 = fl32(r y) is within an ulp of
// r / Q, and fl32(q0 + (r - q0 Q) y), the remainder exact under fma, is the correctly
// rounded quotient (Markstein's theorem; it needs no underflow, hence the division
// below 2^-100).
template <int Q>
__device__ __forceinline__ float div_const(float r) {
  constexpr float y = 1.0f / (float)Q;
  if (__builtin_expect(!(r >= 0x1p-100f), 0)) return r / (float)Q;
  const float q0 = r * y;
  return __builtin_fmaf(__builtin_fmaf(-q0, (float)Q, r), y, q0);
}

// Parameters of a group with minimum mn and maximum mx.  MODE: 0 asymmetric INT4,
// 1 symmetric INT4, 2 asymmetric INT8.  z = rne(fl32(-mn / S)) is taken from
// -mn * inv (sum with kRound, as for the codes) unless that is near a tie.
template <int MODE>
__device__ __forceinline__ PackQ pack_params(float mn, float mx) {
  constexpr int QM = MODE == 2 ? 255 : 15;
  const float amax = fmaxf(-mn, mx);   // max |v|
  PackQ g;
  g.S = MODE == 1 ? div_const<7>(amax) : div_const<QM>(mx - mn);
  g.inv = g.S == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(g.S);
  g.thr = tie_threshold(amax * g.inv);
  if constexpr (MODE == 1) {
    g.zf = 8.0f;
  } else {
    const float tz = -mn * g.inv;
    float z = (tz + kRound) - kRound;
    if (__builtin_expect(near_tie(tz - z, g.thr), 0)) z = __builtin_rintf(-mn / g.S);
    g.zf = g.S == 0.0f ? 0.0f : fminf(fmaxf(z, 0.0f), (float)QM);
  }
  g.kz = kRound + g.zf;
  return g;
}

// The codes of one lane's eight values, q = clamp(rne(fl32(v / S)) + z, 0, QM), each
// returned as the bits of the float kRound + q (q in the low byte, the bits above it
// constant).  rne comes from adding 1.5 * 2^23: the sum's unit in the last place is 1
// while |t| < 2^22, and the constant is even, so halfway cases go to the even integer
// as rne does.  Away from ties rne(t) + z = rne(t + z), so the sum is taken with
// kRound + z at once; a tie is always near (|d| = 1/2) and is redone in the branch,
// rounded before z is added.  For larger |t| the sum is not rne(t), but then rne(t) + z
// lies far outside 0 .. QM and the clamp (one v_med3 on kRound + 0 .. QM) gives the same
// code.  t = v * inv for all eight, the true division only in a branch taken when a
// value of the lane is near a tie (rare); written per element, the compiler would
// compute the division for every value and select.  A constant group (S = 0) has
// inv = 0, so t = 0 and the code is z (inputs are finite).
template <int QM>
__device__ __forceinline__ void group_codes8(const float (&v)[8], const PackQ& g, uint32_t (&q)[8]) {
  float t[8], r[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t[i] = v[i] * g.inv;
    r[i] = t[i] + g.kz;
    near |= near_tie(t[i] - (r[i] - g.kz), g.thr);
  }
  if (__builtin_expect(near, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (near_tie(t[i] - (r[i] - g.kz), g.thr)) r[i] = (v[i] / g.S + kRound) + g.zf;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    q[i] = __float_as_uint(__builtin_amdgcn_fmed3f(r[i], kRound, kRound + (float)QM));
}

// Low bytes of four code words (as returned by group_codes8) as the bytes of one dword.
__device__ __forceinline__ uint32_t bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);   // a.b0, b.b0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);   // c.b0, d.b0, 0, 0
  return lo | (hi << 16);
}
// Eight 4-bit codes (even index in the low nibble of each byte) as one dword.
__device__ __forceinline__ uint32_t nibbles8(const uint32_t (&q)[8]) {
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = q[2 * j] | (q[2 * j + 1] << 4);   // low byte: q0 | q1 << 4
  return bytes4(p[0], p[1], p[2], p[3]);
}

}  // namespace

// 8-element units per lane: two for the packing kernels (16 elements, two loads in
// flight per lane, the group's parameters and lane reductions shared by twice the
// elements: 17.4 -> 13.0 us on [11008, 2048] bf16), one for the error kernel (its
// per-element division and bf16 splits make it slower with two: 30.6 against 32.4 us)
constexpr int kPackU = 2;
constexpr int kErrorU = 1;

// Column of flat element e of a row-major [N, K] matrix: a 32-bit remainder while the
// matrix has fewer than 2^32 elements (a uniform branch), else the 64-bit one.
__device__ __forceinline__ int64_t column_of(int64_t e, int64_t K, int64_t total) {
  if (total <= 0xFFFFFFFFll) return (int64_t)((uint32_t)e % (uint32_t)K);
  return e % K;
}

// One lane's U units of 8 consecutive elements as fp32 (times the channel scale
// when one is given).
template <int U, bool BF16, bool SCALED>
__device__ __forceinline__ void load_units(const void* W, const float* chan_scale, int64_t e, int64_t K,
                                           int64_t total, float (&v)[U][8]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (BF16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + e + 8 * u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[u][2 * i] = bf16_lo(w[i]);
        v[u][2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + e + 8 * u);
      const float4 a = p[0], b = p[1];
      v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
      v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
    }
  }
  if (SCALED) {
    const int64_t k0 = column_of(e, K, total);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float4* sp = reinterpret_cast<const float4*>(chan_scale + k0 + 8 * u);
      const float4 a = sp[0], b = sp[1];
      v[u][0] = v[u][0] * a.x; v[u][1] = v[u][1] * a.y; v[u][2] = v[u][2] * a.z; v[u][3] = v[u][3] * a.w;
      v[u][4] = v[u][4] * b.x; v[u][5] = v[u][5] * b.y; v[u][6] = v[u][6] * b.z; v[u][7] = v[u][7] * b.w;
    }
  }
}

// MODE: 0 asymmetric INT4, 1 symmetric INT4, 2 asymmetric INT8.
template <int G, bool BF16, bool SCALED, int MODE, int U>
__global__ __launch_bounds__(256) void quant_pack_kernel(const void* __restrict__ W,
                                                         const float* __restrict__ chan_scale,
                                                         uint8_t* __restrict__ packed,
                                                         float* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros,
                                                         int64_t total, int64_t K) {
  constexpr int EPL = 8 * U;     // elements per lane
  constexpr int LPG = G / EPL;   // lanes per group
  static_assert(LPG >= 1, "a lane's elements lie in one group");
  const int64_t lane_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = lane_id * EPL;
  const bool live = e0 < total;   // total is a multiple of G, so a live lane's EPL elements all exist
  const int64_t e = live ? e0 : 0;

  float v[U][8];
  load_units<U, BF16, SCALED>(W, chan_scale, e, K, total, v);
  float mn = v[0][0], mx = v[0][0];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn = fminf(mn, v[u][i]);
      mx = fmaxf(mx, v[u][i]);
    }
  mn = segment_min<LPG>(mn);
  mx = segment_max<LPG>(mx);
  constexpr int QM = MODE == 2 ? 255 : 15;
  const PackQ g = pack_params<MODE>(mn, mx);

  // symmetric: |v / S| <= 7 (1 + 2^-23), so rne(v / S) + 8 stays in 1 .. 15 and the
  // 0 .. 15 clamp of the code is the -7 .. 7 clamp of the symmetric code; an all-zero
  // group (S = 0, 1/S = 0) gets code 8
  uint32_t out[MODE == 2 ? 2 * U : U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t q[8];
    group_codes8<QM>(v[u], g, q);
    if constexpr (MODE == 2) {
      out[2 * u] = bytes4(q[0], q[1], q[2], q[3]);
      out[2 * u + 1] = bytes4(q[4], q[5], q[6], q[7]);
    } else {
      out[u] = nibbles8(q);
    }
  }
  if (!live) return;
  constexpr int OUT_BYTES = MODE == 2 ? 8 * U : 4 * U;   // code bytes per lane
  uint8_t* dst = packed + (MODE == 2 ? e : e / 2);
  if constexpr (OUT_BYTES == 4) {
    *reinterpret_cast<uint32_t*>(dst) = out[0];
  } else if constexpr (OUT_BYTES == 8) {
    *reinterpret_cast<uint2*>(dst) = uint2{out[0], out[1]};
  } else {
#pragma unroll
    for (int i = 0; i < OUT_BYTES / 16; ++i)
      *reinterpret_cast<u32x4*>(dst + 16 * i) = u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
  }
  if ((threadIdx.x % LPG) == 0) {
    const int64_t grp = e / G;
    scales[grp] = g.S;
    zeros[grp] = (uint8_t)g.zf;
  }
}

// AWQ search: the error matrix E = Q(W s) / s - W of one candidate scale, written
// as two bf16 planes E_hi = bf16(e), E_lo = bf16(e - E_hi) ([N, K] each, E_lo
// after E_hi).  Same lane mapping and the same (bit-exact) group parameters and
// codes as the packing kernel; the dequantized value (q - z) * S is multiplied by
// fl32(1 / s_k) (chan_rcp, from the host) and the original weight subtracted in
// fp32 -- within 1.5 ulp of the fp32 quotient, far below the 16 bits the two bf16
// planes keep, and without a per-element IEEE division.
template <int G, bool BF16, int U>
__global__ __launch_bounds__(256) void quant_error_kernel(const void* __restrict__ W,
                                                          const float* __restrict__ chan_scale,
                                                          const float* __restrict__ chan_rcp,
                                                          uint16_t* __restrict__ E, int64_t total, int64_t K) {
  constexpr int EPL = 8 * U;
  constexpr int LPG = G / EPL;
  static_assert(LPG >= 1, "a lane's elements lie in one group");
  const int64_t lane_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = lane_id * EPL;
  const bool live = e0 < total;
  const int64_t e = live ? e0 : 0;
  float w[U][8], v[U][8];
  load_units<U, BF16, false>(W, nullptr, e, K, total, w);
  const int64_t k0 = column_of(e, K, total);
  float mn = 0.0f, mx = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float4* sp = reinterpret_cast<const float4*>(chan_scale + k0 + 8 * u);
    const float4 a = sp[0], b = sp[1];
    const float s[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[u][i] = w[u][i] * s[i];
      mn = (u || i) ? fminf(mn, v[u][i]) : v[u][i];
      mx = (u || i) ? fmaxf(mx, v[u][i]) : v[u][i];
    }
  }
  mn = segment_min<LPG>(mn);
  mx = segment_max<LPG>(mx);
  const PackQ g = pack_params<0>(mn, mx);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t qc[8];
    group_codes8<15>(v[u], g, qc);
    const float4* rp = reinterpret_cast<const float4*>(chan_rcp + k0 + 8 * u);
    const float4 a = rp[0], b = rp[1];
    const float r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    // E_hi = bf16(err), E_lo = bf16(err - E_hi), round to nearest even, two values per
    // v_cvt_pk_bf16_f32 (equal to the bitwise rounding for every non-NaN fp32)
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float err[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * i + h;
        const float what = (__uint_as_float(qc[j]) - g.kz) * g.S;   // (q - z) S, q - z exact
        err[h] = what * r[j] - w[u][j];                               // (q - z) S / s_k - w
      }
      const bf16x2 eh = {(__bf16)err[0], (__bf16)err[1]};
      hi[i] = __builtin_bit_cast(uint32_t, eh);
      const bf16x2 el = {(__bf16)(err[0] - bf16_lo(hi[i])), (__bf16)(err[1] - bf16_hi(hi[i]))};
      lo[i] = __builtin_bit_cast(uint32_t, el);
    }
    if (live) {
      *reinterpret_cast<u32x4*>(E + e + 8 * u) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<u32x4*>(E + total + e + 8 * u) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
}

hipError_t launch_quant_error(const void* W, bool w_bf16, const float* chan_scale, const float* chan_rcp, uint16_t* E,
                              int64_t N, int64_t K, int group, hipStream_t stream) {
  const int64_t total = N * K;
  const dim3 block(256), grid((unsigned)((total / (8 * kErrorU) + 255) / 256));
#define AQ_QE(GG)                                                                                               \
  if (w_bf16)                                                                                                   \
    hipLaunchKernelGGL((quant_error_kernel<GG, true, kErrorU>), grid, block, 0, stream, W, chan_scale, chan_rcp, E,    \
                       total, K);                                                                                 \
  else                                                                                                          \
    hipLaunchKernelGGL((quant_error_kernel<GG, false, kErrorU>), grid, block, 0, stream, W, chan_scale, chan_rcp, E,   \
                       total, K);
  switch (group) {
    case 32: AQ_QE(32) break;
    case 64: AQ_QE(64) break;
    case 128: AQ_QE(128) break;
    default: return hipErrorInvalidValue;
  }
#undef AQ_QE
  return hipGetLastError();
}

template <int G, int MODE>
static hipError_t launch_g(const void* W, bool bf16, const float* s, uint8_t* packed, float* scales,
                           uint8_t* zeros, int64_t N, int64_t K, hipStream_t stream) {
  constexpr int U = kPackU;
  const int64_t total = N * K;
  const int64_t lanes = total / (8 * U);
  const dim3 block(256);
  const dim3 grid((unsigned)((lanes + 255) / 256));
  if (bf16) {
    if (s) hipLaunchKernelGGL((quant_pack_kernel<G, true, true, MODE, U>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
    else hipLaunchKernelGGL((quant_pack_kernel<G, true, false, MODE, U>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
  } else {
    if (s) hipLaunchKernelGGL((quant_pack_kernel<G, false, true, MODE, U>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
    else hipLaunchKernelGGL((quant_pack_kernel<G, false, false, MODE, U>), grid, block, 0, stream, W, s, packed, scales, zeros, total, K);
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(const void* W, bool w_bf16, const float* chan_scale, uint8_t* packed, float* scales,
                              uint8_t* zeros, int64_t N, int64_t K, int group, hipStream_t stream) {
  switch (group) {
    case 32: return launch_g<32, MODE>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, stream);
    case 64: return launch_g<64, MODE>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, stream);
    case 128: return launch_g<128, MODE>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_pack(const void* W, bool w_bf16, const float* chan_scale, uint8_t* packed,
                             float* scales, uint8_t* zeros, int64_t N, int64_t K, int group, bool sym,
                             hipStream_t stream) {
  if (sym) return launch_mode<1>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, group, stream);
  return launch_mode<0>(W, w_bf16, chan_scale, packed, scales, zeros, N, K, group, stream);
}

hipError_t launch_quant_pack8(const void* W, bool w_bf16, const float* chan_scale, uint8_t* codes, float* scales,
                              uint8_t* zeros, int64_t N, int64_t K, int group, hipStream_t stream) {
  return launch_mode<2>(W, w_bf16, chan_scale, codes, scales, zeros, N, K, group, stream);
}

}  // namespace aq

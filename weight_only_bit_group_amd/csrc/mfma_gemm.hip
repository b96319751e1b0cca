// bf16-MFMA GEMMs of libaq (gfx950): the W4A16 prefill GEMM, the FP4 decode GEMM
// and the AWQ search's error GEMM with a sum-of-squares epilogue.
//
// All three contract a bf16 activation matrix X[M, K] (K contiguous) with a
// weight-side operand B[N, K] produced in LDS:
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
// Block: 2 * WGM waves (WGM = 4 for large M: 512 threads, a 256 x 128 tile), the
// waves in a WGM x 2 grid of 64 x 64 wave tiles, each four 32x32 output blocks of
// v_mfma_f32_32x32x16_bf16.  K advances in stages of 64 (one INT4 group at
// g = 64), one workgroup barrier per stage.
//
//   * Every global -> LDS transfer is an LDS-DMA load (global_load_lds_*): the
//     activation rows (and the SPLIT planes) as 16-byte units straight into their
//     swizzled LDS tile, the packed codes of the weight tile, and the per-row
//     group steps, zero points or block scales (one dword slot per row).  No
//     registers, no VALU.  They are issued from inline asm: with the compiler's
//     own intrinsic it cannot tell which LDS bytes a load in flight writes and
//     waits for every outstanding load before any LDS read, which would cost the
//     prefetch depth.  The kernel counts them itself (loads complete in order):
//     at the end of stage s each wave waits until only the loads it issued in
//     stage s are outstanding, then the barrier publishes everything older.
//   * Prefetch distances: activations 2 stages (ring of 3 LDS tiles), codes and
//     per-row scalars 3 stages (rings of 3 and 4), so each load has about two
//     stages of MFMA work to land.  SPLIT (no dequantization, twice the MFMAs per
//     stage) prefetches activations and planes 1 stage ahead (rings of 2).
//   * INT4 / FP4 weights are dequantized one stage ahead from the LDS codes into
//     a bf16 LDS tile (two buffers), once per block: each weight row feeds BM
//     activation rows.
//   * LDS rows are 128 bytes (64 bf16, 8 units of 16 bytes) with unit u of row r
//     stored at u ^ (r & 7): the 8 rows read by each 8-lane phase of a
//     ds_read_b128 hit 8 different bank groups.
//   * Block order is XCD-aware: block b runs on XCD b % 8; each XCD gets a
//     contiguous range of a grouped tile order (a few row tiles, all column
//     tiles), so the blocks it runs together share their activation and weight
//     tiles in its L2.
//   * INT4: the MFMAs of one group run block by block into a temporary that is
//     rescaled by S[n, g] straight into the VGPR-resident output (one v_fma per
//     output element per group), software-pipelined one block behind the MFMAs.
//     A group wider than a stage (g = 128) is rescaled once per stage with the
//     same S.
// A lane of a 32x32x16 MFMA holds row (lane % 32) and k = 8 (lane / 32) .. +7 of
// each operand; its 16 results are column (lane % 32), rows
// 8 (i / 4) + 4 (lane / 32) + (i % 4), so they share one weight row n and need
// one S per block per group.
#include <type_traits>

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
  double* partial;    // [number of blocks] fp64 sums of squares (SPLIT)
};

namespace {

constexpr int KS = 64;            // k per stage
constexpr int BN = 128;           // block tile columns (weight rows)
constexpr int ROW_UNITS = KS / 8;  // 16-byte units per LDS row

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int unit) { return row * ROW_UNITS + (unit ^ (row & 7)); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

// LDS-DMA loads: lane l's bytes land at lds + 16 l (dwordx4) or in the dword slot
// lds + 4 l, zero-extended (dword / ushort / ubyte).  `base` is wave-uniform (SGPRs),
// `voff` the lane's 32-bit byte offset.  M0 holds the LDS base; s_nop covers the
// M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ushort %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma1(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// gfx9 s_waitcnt immediate that waits for vmcnt <= n and lgkmcnt == 0 (expcnt untouched).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// Workgroup barrier for the stage hand-off; the caller has already waited for its
// own LDS writes and LDS-DMA loads.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Tile index of block b under the XCD-aware order (b runs on XCD b % 8).
__device__ __forceinline__ int tile_of_block(int b, int nblk) {
  const int per = nblk >> 3, rem = nblk & 7;
  const int x = b & 7, local = b >> 3;
  const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + local;
}

template <int BK, int G, bool TAIL, int WGM>
__global__ __launch_bounds__(128 * WGM, 1) void gemm_kernel(GemmArgs a) {
  constexpr int NW = 2 * WGM, NT = 64 * NW;
  constexpr int BM = 64 * WGM;
  constexpr bool DEQ = BK != B_SPLIT;
  constexpr int NA = DEQ ? 3 : 2;                   // activation ring
  constexpr int PD = NA - 1;                        // activation prefetch distance
  constexpr int CD = 3;                             // code / per-row scalar prefetch distance
  constexpr int A_DMA = BM / 8 / NW;                // activation loads per wave per stage (8 rows each)
  constexpr int B_DMA = DEQ ? 0 : 2 * (BN / 8) / NW;  // SPLIT plane loads per wave per stage
  // code + per-row scalar loads per stage: 4 code loads (1 KB each) and the scalars
  // (INT4: steps and zero points, two 64-row halves per group, one or two groups per
  // stage, the zero-point loads repeated at g = 32 so every wave issues the same
  // number; FP4: two ushorts of block scales per row)
  constexpr int NAUX = (BK == B_INT4 && G == 32) ? 12 : 4;
  constexpr int JOBS = DEQ ? 4 + NAUX : 0;
  constexpr int JPW = JOBS / NW;
  static_assert(!DEQ || JOBS % NW == 0, "scalar loads must split evenly over the waves");

  __shared__ __attribute__((aligned(16))) uint16_t As[NA][BM * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][DEQ ? 1 : 2][BN * KS];
  __shared__ __attribute__((aligned(16))) uint8_t Cs[DEQ ? 3 : 1][BN * KS / 2];
  // per-row scalars: [slot][INT4: 0 = S bits, 1 = zero point | FP4: 0][group in stage or FP4 half][row]
  __shared__ __attribute__((aligned(16))) uint32_t AX[DEQ ? 4 : 1][2][2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 1, wn = wid & 1;
  const int M = a.M, N = a.N, K = a.K;
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = (M + BM - 1) / BM;
  // XCD-contiguous linear index, then groups of GM row tiles walked column by column:
  // the blocks an XCD runs at once cover GM row tiles x (blocks / GM) column tiles,
  // so their activation and weight tiles stay in that XCD's L2.
  const int t = tile_of_block(blockIdx.x, tiles_m * tiles_n);
  const int GM = max(1, (tiles_m + 7) / 8);
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int within = t - group * GM * tiles_n;
  const int m0 = (first_m + within % gm) * BM;
  const int n0 = (within / gm) * BN;
  const int nfull = K / KS;                    // full 64-wide stages; TAIL adds one 32-wide stage
  const int nstage = nfull + (TAIL ? 1 : 0);
  const int ngroups = K / G;

  // ---- LDS-DMA loads --------------------------------------------------------
  // Tile rows: load j of wave w covers rows R0 = (j NW + w) 8 .. + 8; lane l lands at
  // LDS unit (R0 + l / 8, l % 8) and fetches global unit (l % 8) ^ (l / 8), which is
  // the swizzle since R0 is a multiple of 8.  Offsets are 32-bit (M K, N K < 2^30).
  // In the 32-wide tail stage the upper four units are folded back onto the lower
  // four (loaded, never multiplied), so no load runs past a row.
  const int lrow8 = lane >> 3;
  const int gunit = (lane & 7) ^ lrow8;
  const uint32_t tail_fold = (TAIL && gunit >= 4) ? 64u : 0u;
  uint32_t aoff[A_DMA];
#pragma unroll
  for (int j = 0; j < A_DMA; ++j) {
    const int row = (j * NW + wid) * 8 + lrow8;
    aoff[j] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)K * 2u + (uint32_t)gunit * 16u;
  }
  auto issue_a = [&](int s, int slot) {
    const char* base = reinterpret_cast<const char*>(a.X) + (size_t)s * (KS * 2);
    const uint32_t fold = (TAIL && s == nfull) ? tail_fold : 0u;
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) dma16(base, aoff[j] - fold, lds_addr(&As[slot][(j * NW + wid) * 8 * KS]));
  };
  auto issue_planes = [&](int s, int slot) {
    if constexpr (!DEQ) {
      const uint32_t fold = (TAIL && s == nfull) ? tail_fold : 0u;
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        const char* base = reinterpret_cast<const char*>(pl ? a.B2 : a.B) + (size_t)s * (KS * 2);
#pragma unroll
        for (int j = 0; j < BN / 8 / NW; ++j) {
          const int r0 = (j * NW + wid) * 8;
          const uint32_t off = (uint32_t)min(n0 + r0 + lrow8, N - 1) * (uint32_t)K * 2u + (uint32_t)gunit * 16u;
          dma16(base, off - fold, lds_addr(&Bs[slot][pl][r0 * KS]));
        }
      }
    }
  };
  // codes (32 bytes per row and stage, two 16-byte halves per lane pair) and the
  // per-row scalars of stage s
  auto issue_codes = [&](int s, int cslot, int xslot) {
    if constexpr (DEQ) {
      const bool tail = TAIL && s == nfull;
#pragma unroll
      for (int i = 0; i < JPW; ++i) {
        const int job = wid * JPW + i;   // wave-uniform
        if (job < 4) {
          const int r = 32 * job + (lane >> 1);
          const uint32_t n = (uint32_t)min(n0 + r, N - 1);
          const uint32_t half = tail ? 0u : (uint32_t)(lane & 1) * 16u;
          const uint8_t* src = (BK == B_INT4) ? a.P : a.codes;
          dma16(src + (size_t)s * (KS / 2), n * (uint32_t)(K >> 1) + half, lds_addr(&Cs[cslot][1024 * job]));
        } else if constexpr (BK == B_INT4) {
          int x = job - 4;
          if (x >= 8) x -= 4;                                  // repeated zero-point loads (g = 32)
          const int is_z = (G == 32) ? (x >= 4) : (x >= 2);
          const int gi = (G == 32) ? ((x >> 1) & 1) : 0;
          const int rh = 64 * (x & 1);
          const uint32_t n = (uint32_t)min(n0 + rh + lane, N - 1);
          const uint32_t g = (uint32_t)min((s * KS + 32 * gi) / G, ngroups - 1);
          const uint32_t idx = n * (uint32_t)ngroups + g;
          if (is_z) dma1(a.Z, idx, lds_addr(&AX[xslot][1][gi][rh]));
          else dma4(a.S, idx * 4u, lds_addr(&AX[xslot][0][gi][rh]));
        } else {
          const int x = job - 4;
          const int h = x >> 1, rh = 64 * (x & 1);
          const uint32_t n = (uint32_t)min(n0 + rh + lane, N - 1);
          const uint32_t byte = (uint32_t)(s * 4 + 2 * (tail ? 0 : h));   // the tail stage has 2 block scales
          dma2(a.bscale, n * (uint32_t)(K >> 4) + byte, lds_addr(&AX[xslot][0][h][rh]));
        }
      }
    }
  };

  // ---- dequantization: codes of one stage -> bf16 weight tile ----------------
  constexpr int TPR = NT / BN;          // threads per weight row
  constexpr int KPT = KS / TPR;         // k per thread (16 or 32)
  constexpr int WPT = KPT / 8;          // 8-code words (= LDS units) per thread
  const int d_row = tid / TPR, d_part = tid % TPR;
  // `tail`: stage s is the 32-wide tail (only its first 32 k are dequantized)
  auto dequant = [&](int cslot, int xslot, int bbuf, bool tail) {
    if constexpr (DEQ) {
      if (tail && d_part * KPT >= 32) return;
      uint32_t w[WPT];
      const uint8_t* cp = &Cs[cslot][d_row * 32 + d_part * (KPT / 2)];
      if constexpr (WPT == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(cp);
        w[0] = v.x; w[1] = v.y;
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(cp);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
      }
      u32x4* dst = reinterpret_cast<u32x4*>(&Bs[bbuf][0][0]);
      if constexpr (BK == B_INT4) {
        const int gi = (G == 32) ? (d_part * KPT) / 32 : 0;
        const float zf = (float)AX[xslot][1][gi][d_row];
#pragma unroll
        for (int u = 0; u < WPT; ++u) {
          uint32_t lo = w[u] & 0x0F0F0F0Fu, hi = (w[u] >> 4) & 0x0F0F0F0Fu;
          // opaque to the optimizer, so each code converts with one v_cvt_f32_ubyteN
          asm("" : "+v"(lo), "+v"(hi));
          uint32_t o[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float ql = (float)((lo >> (8 * b)) & 0xFFu), qh = (float)((hi >> (8 * b)) & 0xFFu);
            o[b] = pack_bf16_exact(ql - zf, qh - zf);
          }
          dst[swz(d_row, d_part * WPT + u)] = u32x4{o[0], o[1], o[2], o[3]};
        }
      } else {
#pragma unroll
        for (int u = 0; u < WPT; ++u) {
          // 16-element block of word u: (d_part KPT + 8 u) / 16 within the stage
          const int blk = (d_part * KPT + 8 * u) >> 4;
          const uint32_t two = AX[xslot][0][blk >> 1][d_row];
          const float sc = (blk & 1) ? __builtin_amdgcn_cvt_f32_fp8((int)two, 1) : __builtin_amdgcn_cvt_f32_fp8((int)two, 0);
          uint32_t o[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            uint32_t e2;
            switch (b) {
              case 0: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 0)); break;
              case 1: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 1)); break;
              case 2: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 2)); break;
              default: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 3)); break;
            }
            o[b] = pack_bf16_exact(bf16_lo(e2) * sc, bf16_hi(e2) * sc);
          }
          dst[swz(d_row, d_part * WPT + u)] = u32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
  };

  // ---- accumulators: 32x32 output blocks (mi, ni) of the 64 x 64 wave tile ----
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int l32 = lane & 31;
  const int lh = lane >> 5;           // k half of a 16-wide MFMA step
  const u32x4* Av = reinterpret_cast<const u32x4*>(&As[0][0]);
  const u32x4* Bv = reinterpret_cast<const u32x4*>(&Bs[0][0][0]);
  constexpr int A_BUF = BM * KS / 8, B_BUF = (DEQ ? 1 : 2) * BN * KS / 8, B_PLANE = BN * KS / 8;  // 16-byte units

  // NKS: 16-wide MFMA steps of stage s (4, or 2 in the tail); NXT: the same for the
  // stage whose weights are dequantized here (0 for the last stage)
  auto run_stage = [&](int s, auto nk_tag, auto nx_tag) {
    constexpr int NKS = decltype(nk_tag)::value;
    constexpr int NXT = decltype(nx_tag)::value;
    const int abuf = s % NA;
    const int bbuf = s & 1;
    const int xs = s & 3;
    // 1. prefetch: codes / scalars of stage s + 3, activations of stage s + 2 (SPLIT:
    //    activations and planes of stage s + 1)
    const bool more_c = DEQ && s + CD < nstage;
    const bool more_a = s + PD < nstage;
    if (more_c) issue_codes(s + CD, (s + CD) % 3, (s + CD) & 3);
    if (more_a) {
      issue_a(s + PD, (s + PD) % NA);
      issue_planes(s + PD, (s + PD) & 1);
    }
    // 2. fragments of this stage
    bf16x8 af[2][NKS], bf[2][NKS], bf2[2][NKS];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        af[mi][ks] = __builtin_bit_cast(bf16x8, Av[abuf * A_BUF + swz(wm * 64 + 32 * mi + l32, 2 * ks + lh)]);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int row = wn * 64 + 32 * ni + l32;
        bf[ni][ks] = __builtin_bit_cast(bf16x8, Bv[bbuf * B_BUF + swz(row, 2 * ks + lh)]);
        if constexpr (!DEQ) bf2[ni][ks] = __builtin_bit_cast(bf16x8, Bv[bbuf * B_BUF + B_PLANE + swz(row, 2 * ks + lh)]);
      }
    // 3. MFMAs
    if constexpr (BK == B_INT4) {
      constexpr int NG = (G == 32) ? NKS / 2 : 1;   // group partials per block in this stage
      constexpr int KPG = NKS / NG;
      float sc[2][NG];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) sc[ni][gi] = __builtin_bit_cast(float, AX[xs][0][gi][wn * 64 + 32 * ni + l32]);
      // (group, block) pairs in order; each block's rescale runs one pair behind its MFMAs
      f32x16 tprev;
#pragma unroll
      for (int it = 0; it < 4 * NG; ++it) {
        const int gi = it >> 2, mi = (it >> 1) & 1, ni = it & 1;
        f32x16 tp;
#pragma unroll
        for (int k = 0; k < KPG; ++k) {
          const int ks = gi * KPG + k;
          const f32x16 zero = {};
          tp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][ks], bf[ni][ks], k == 0 ? zero : tp, 0, 0, 0);
        }
        if (it > 0) {
          const int pg = (it - 1) >> 2, pm = ((it - 1) >> 1) & 1, pn = (it - 1) & 1;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[pm][pn][v] = __builtin_fmaf(sc[pn][pg], tprev[v], acc[pm][pn][v]);
        }
        tprev = tp;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[1][1][v] = __builtin_fmaf(sc[1][NG - 1], tprev[v], acc[1][1][v]);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int mi = b >> 1, ni = b & 1;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][ks], bf[ni][ks], acc[mi][ni], 0, 0, 0);
          if constexpr (!DEQ)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][ks], bf2[ni][ks], acc[mi][ni], 0, 0, 0);
        }
      }
    }
    // 4. weights of the next stage (its codes were published one barrier ago)
    if constexpr (DEQ && NXT > 0) dequant((s + 1) % 3, (s + 1) & 3, bbuf ^ 1, NXT == 2);
    // 5. wait until only this stage's loads are outstanding (loads complete in order),
    //    and for this wave's LDS writes; then publish
    //    (SPLIT prefetches one stage ahead: everything issued so far is needed next)
    if (DEQ && more_c) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(JPW + A_DMA));
    else if (DEQ && more_a) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(A_DMA));
    else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
    stage_barrier();
  };

  // ---- prologue --------------------------------------------------------------
  if constexpr (DEQ) {
    // P0 = stage 0 (codes, activations), P1 = stage 1 (codes, activations), P2 = codes of stage 2
    issue_codes(0, 0, 0);
    issue_a(0, 0);
    if (nstage > 1) {
      issue_codes(1, 1, 1);
      issue_a(1, 1);
    }
    if (nstage > 2) issue_codes(2, 2, 2);
    if (nstage > 2) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(2 * JPW + A_DMA));
    else if (nstage > 1) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(JPW + A_DMA));
    else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
    stage_barrier();
    dequant(0, 0, 0, TAIL && nfull == 0);
    if (nstage > 2) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(JPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
    stage_barrier();
  } else {
    issue_a(0, 0);
    issue_planes(0, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
    stage_barrier();
  }
  using IC4 = std::integral_constant<int, 4>;
  using IC2 = std::integral_constant<int, 2>;
  using IC0 = std::integral_constant<int, 0>;
  for (int s = 0; s + 1 < nfull; ++s) run_stage(s, IC4{}, IC4{});
  if constexpr (TAIL) {
    if (nfull > 0) run_stage(nfull - 1, IC4{}, IC2{});
    run_stage(nfull, IC2{}, IC0{});
  } else {
    run_stage(nfull - 1, IC4{}, IC0{});
  }

  // ---- epilogue --------------------------------------------------------------
  // result i of block (mi, ni): row 8 (i / 4) + 4 lh + (i % 4), column l32
  if constexpr (BK == B_SPLIT) {
    double ss = 0.0;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int n = n0 + wn * 64 + 32 * ni + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * 64 + 32 * mi + 8 * (v >> 2) + 4 * lh + (v & 3);
          const double d = (double)acc[mi][ni][v];
          if (m < M && n < N) ss = __builtin_fma(d, d, ss);
        }
      }
    ss = wave_sum(ss);
    __shared__ double wsum[NW];
    if (lane == 0) wsum[wid] = ss;
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += wsum[w];
      a.partial[t] = tot;
    }
  } else {
    const bool full = (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int n = n0 + wn * 64 + 32 * ni + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * 64 + 32 * mi + 8 * (v >> 2) + 4 * lh + (v & 3);
          const float y = (BK == B_FP4) ? acc[mi][ni][v] * a.ts : acc[mi][ni][v];
          if (full || (m < M && n < N)) __builtin_nontemporal_store(y, &a.Y[(int64_t)m * N + n]);
        }
      }
  }
}

int tiles(int M, int N, int bm) { return ((M + bm - 1) / bm) * ((N + BN - 1) / BN); }

// 256-row tiles (8 waves) once M fills them; 128-row tiles (4 waves) for small M.
constexpr int kWideM = 192;

template <int BK, int G, bool TAIL>
hipError_t launch_tail(const GemmArgs& a, hipStream_t stream) {
  if (a.M > kWideM) {
    hipLaunchKernelGGL((gemm_kernel<BK, G, TAIL, 4>), dim3(tiles(a.M, a.N, 256)), dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL((gemm_kernel<BK, G, TAIL, 2>), dim3(tiles(a.M, a.N, 128)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int BK, int G>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t stream) {
  if (a.K % KS) return launch_tail<BK, G, true>(a, stream);
  return launch_tail<BK, G, false>(a, stream);
}

}  // namespace

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
  return launch_tiles<B_FP4, 64>(a, stream);
}

int sumsq_gemm_blocks(int M, int N) { return M > kWideM ? tiles(M, N, 256) : tiles(M, N, 128); }  // SPLIT tiles

hipError_t launch_sumsq_gemm(const uint16_t* X, int M, int K, const uint16_t* E, int N, double* partial,
                             hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.B = E; a.B2 = E + (size_t)N * K; a.partial = partial;
  return launch_tiles<B_SPLIT, 64>(a, stream);
}

}  // namespace aq

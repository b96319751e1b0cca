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
// Pipeline (per 256-thread block, 4 waves in a 2 x 2 grid, wave tile WM x 64 of
// 16x16 v_mfma_f32_16x16x32_bf16 blocks):
//   * K advances in stages of 64 (one INT4 group at g = 64) through two LDS
//     buffers; one barrier per stage.
//   * Activation rows (and the SPLIT planes) go global -> LDS directly with
//     global_load_lds_dwordx4, issued one stage ahead; no registers, no VALU.
//   * INT4 / FP4 weight codes are loaded one stage ahead into registers and
//     dequantized exactly once per block into LDS, shared by both waves of a
//     column.
//   * LDS rows are 128 bytes (64 bf16, 8 units of 16 bytes) with unit u of row r
//     stored at u ^ (r & 7): the 8 rows read by each 8-lane phase of a
//     ds_read_b128 hit 8 different bank groups.
//   * Block order is XCD-aware: block b runs on XCD b % 8; each XCD gets a
//     contiguous range of a grouped tile order (a few row tiles, all column
//     tiles), so the blocks it runs together share their activation and weight
//     tiles in its L2.
//   * INT4: the MFMAs of one group run block by block into a 4-register
//     temporary that is rescaled by S[n, g] straight into the VGPR-resident
//     output (one v_fmac per output element per group); a group wider than a
//     stage (g = 128) is rescaled once per stage with the same S.
// A lane of a 16x16x32 MFMA holds row (lane % 16) and k = 8 (lane / 16) .. +7 of
// each operand; its 4 results are column (lane % 16), rows 4 (lane / 16) + v,
// so they share one weight row n and need one S per 16x16 block per group.
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

// gfx9 s_waitcnt immediate that waits for vmcnt <= n and lgkmcnt == 0 (expcnt untouched).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// Workgroup barrier for the stage hand-off.  The caller has already waited for
// what the next stage reads (its own LDS writes: lgkmcnt(0); its direct LDS loads
// of the next stage: vmcnt(n)).  A __syncthreads() here would also wait for the
// direct loads of the stage after next (vmcnt(0)) and cost the prefetch depth; the
// asm's memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Tile index of block b under the XCD-aware order (b runs on XCD b % 8).
__device__ __forceinline__ int tile_of_block(int b, int nblk) {
  const int per = nblk >> 3, rem = nblk & 7;
  const int x = b & 7, local = b >> 3;
  const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + local;
}

template <int BK, int MI, int G, bool TAIL>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs a) {
  constexpr int WM = 16 * MI, BM = 2 * WM;
  constexpr int PLANES = (BK == B_SPLIT) ? 2 : 1;
  constexpr int A_INST = BM / 8 / 4;             // direct-load instructions per wave per stage (8 rows each)
  constexpr int B_INST = BN / 8 / 4;
  // activation ring: NA buffers, prefetched NA - 1 stages ahead (3 when LDS allows)
  constexpr int NA = (BK == B_SPLIT) ? 2 : 3;

  __shared__ __attribute__((aligned(16))) uint16_t As[NA][BM * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][PLANES][BN * KS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
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

  // ---- direct global -> LDS loads of the activation tile (and SPLIT planes) ----
  // instruction j of wave w covers tile rows R0 = (j * 4 + w) * 8 .. + 8; lane l
  // lands at LDS unit (R0 + l / 8, l % 8) and fetches global unit (l % 8) ^ (row & 7).
  // Offsets are 32-bit byte offsets of the stage-0 unit (M * K and N * K < 2^30).
  const int lrow8 = lane >> 3, lunit = lane & 7;
  const int gunit = lunit ^ lrow8;   // row & 7 == lane / 8 since R0 is a multiple of 8
  uint32_t aoff[A_INST];
#pragma unroll
  for (int j = 0; j < A_INST; ++j) {
    const int row = (j * 4 + wid) * 8 + lrow8;
    aoff[j] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)K * 2u + (uint32_t)gunit * 16u;
  }
  // byte offset of stage s for this lane's unit; in the 32-wide tail stage the upper
  // four units are folded back onto the lower four (loaded, never multiplied)
  auto stage_off = [&](int s) -> uint32_t {
    const uint32_t base = (uint32_t)s * (KS * 2);
    return (TAIL && s == nfull && gunit >= 4) ? base - 64u : base;
  };
  auto issue_a = [&](int s, int abuf) {
    const char* xb = reinterpret_cast<const char*>(a.X);
    const uint32_t so = stage_off(s);
    uint16_t* dst = &As[abuf][0];
#pragma unroll
    for (int j = 0; j < A_INST; ++j) {
      const int r0 = (j * 4 + wid) * 8;
      __builtin_amdgcn_global_load_lds((const void*)(xb + aoff[j] + so), (lds_void*)&dst[r0 * KS], 16, 0, 0);
    }
  };
  auto issue_b_planes = [&](int s, int buf) {
    if constexpr (BK == B_SPLIT) {
      const uint32_t so = stage_off(s);
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int j = 0; j < B_INST; ++j) {
          const int r0 = (j * 4 + wid) * 8;
          const uint32_t off = (uint32_t)min(n0 + r0 + lrow8, N - 1) * (uint32_t)K * 2u + (uint32_t)gunit * 16u;
          const char* base = reinterpret_cast<const char*>(pl ? a.B2 : a.B);
          __builtin_amdgcn_global_load_lds((const void*)(base + off + so), (lds_void*)&Bs[buf][pl][r0 * KS], 16, 0, 0);
        }
    }
  };

  // ---- weight codes: one 16-byte load per thread per stage, dequantized into LDS ----
  const int b_row = tid >> 1;       // tile row (weight row n0 + b_row)
  const int b_half = tid & 1;       // k half of the stage: 32 values = 4 units
  const int b_n = min(n0 + b_row, N - 1);
  u32x4 braw;
  uint32_t bzb = 0;                 // INT4 zero point of the half's group (raw byte)
  float bsc0 = 0.0f, bsc1 = 0.0f;   // FP4 block scales of the half's two 16-blocks
  auto load_b = [&](int s) {
    if constexpr (BK != B_SPLIT) {
      int k0 = s * KS + b_half * 32;
      if (TAIL && k0 >= K) k0 -= 32;
      if constexpr (BK == B_INT4) {
        braw = *reinterpret_cast<const u32x4*>(a.P + (int64_t)b_n * (K >> 1) + (k0 >> 1));
        bzb = a.Z[(int64_t)b_n * (K / G) + k0 / G];
      } else {
        braw = *reinterpret_cast<const u32x4*>(a.codes + (int64_t)b_n * (K >> 1) + (k0 >> 1));
        const uint32_t two = *reinterpret_cast<const uint16_t*>(a.bscale + (int64_t)b_n * (K >> 4) + (k0 >> 4));
        bsc0 = __builtin_amdgcn_cvt_f32_fp8((int)two, 0);
        bsc1 = __builtin_amdgcn_cvt_f32_fp8((int)two, 1);
      }
    }
  };
  auto store_b = [&](int buf) {
    if constexpr (BK != B_SPLIT) {
      const float bz = (float)bzb;
      uint32_t w[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = braw[d] & 0x0F0F0F0Fu, hi = (braw[d] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          if constexpr (BK == B_INT4) {
            const float ql = (float)((lo >> (8 * bb)) & 0xFFu), qh = (float)((hi >> (8 * bb)) & 0xFFu);
            w[4 * d + bb] = pack_bf16_exact(ql - bz, qh - bz);
          } else {
            uint32_t e2;
            switch (bb) {
              case 0: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(braw[d], 1.0f, 0)); break;
              case 1: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(braw[d], 1.0f, 1)); break;
              case 2: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(braw[d], 1.0f, 2)); break;
              default: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(braw[d], 1.0f, 3)); break;
            }
            const float sc = d < 2 ? bsc0 : bsc1;
            w[4 * d + bb] = pack_bf16_exact(bf16_lo(e2) * sc, bf16_hi(e2) * sc);
          }
        }
      }
      u32x4* dst = reinterpret_cast<u32x4*>(&Bs[buf][0][0]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dst[swz(b_row, b_half * 4 + u)] = u32x4{w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]};
    }
  };

  // ---- accumulators: 16x16 output blocks of v_mfma_f32_16x16x32_bf16 ----------
  // lane l holds column (l % 16) and k = 8 (l / 16) .. +7 of each operand; its 4
  // results are rows 4 (l / 16) + v, column (l % 16).
  constexpr int MB = MI, NB = 4;   // 16x16 blocks per wave tile (wave tile WM x 64)
  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  const int l16 = lane & 15;
  const int lq = lane >> 4;           // k quarter: 8 values of a 32-wide MFMA step
  const int ngroups = K / G;
  const int ncol0 = n0 + wn * 64 + l16;
  const u32x4* Bv = reinterpret_cast<const u32x4*>(&Bs[0][0][0]);
  constexpr int A_BUF = BM * KS / 8, B_BUF = PLANES * BN * KS / 8, B_PLANE = BN * KS / 8;  // in 16-byte units
  // direct loads issued per stage by one wave (activations, plus the SPLIT planes)
  constexpr int DIRECT = A_INST + (BK == B_SPLIT ? 2 * B_INST : 0);

  // group steps S[n, g] of the (one or two) groups a stage touches, per n-block
  auto load_gs = [&](int s, float (&out)[2][NB]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int g = min((s * KS + 32 * ks) / G, ngroups - 1);
#pragma unroll
      for (int j = 0; j < NB; ++j) out[ks][j] = a.S[(int64_t)min(ncol0 + 16 * j, N - 1) * ngroups + g];
    }
  };
  float gs[2][NB];
  if constexpr (BK == B_INT4) load_gs(0, gs);

  auto run_stage = [&](int s, auto nk_tag) {
    constexpr int nk32 = decltype(nk_tag)::value;   // 32-wide MFMA steps in this stage
    const int abuf = s % NA;                          // activation buffer
    const int buf = s & 1;                            // weight buffer
    const u32x4* Av = reinterpret_cast<const u32x4*>(&As[abuf][0]);
    const bool more = s + 1 < nstage;
    // register loads of the next stage first (weight codes, zero points, group
    // steps), pinned ahead of the direct activation loads: loads complete in order,
    // so waiting for them never waits for the activation prefetch behind them
    if (more) load_b(s + 1);
    float gs_next[2][NB];
    if constexpr (BK == B_INT4) {
      if (more) load_gs(s + 1, gs_next);
    }
    asm volatile("" ::: "memory");
    bool issued = false;
    if constexpr (NA == 3) {
      if (s + 2 < nstage) {
        issue_a(s + 2, (s + 2) % NA);
        issued = true;
      }
    } else if (more) {
      issue_a(s + 1, abuf ^ 1);
      issue_b_planes(s + 1, buf ^ 1);
      issued = true;
    }
    asm volatile("" ::: "memory");
    bf16x8 bfr[NB][2], bf2[NB][2];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int ks = 0; ks < nk32; ++ks) {
        const int row = wn * 64 + 16 * j + l16;
        bfr[j][ks] = __builtin_bit_cast(bf16x8, Bv[buf * B_BUF + swz(row, 4 * ks + lq)]);
        if constexpr (BK == B_SPLIT)
          bf2[j][ks] = __builtin_bit_cast(bf16x8, Bv[buf * B_BUF + B_PLANE + swz(row, 4 * ks + lq)]);
      }
    // software pipeline over the m-blocks: the A fragments of block i + 1 are read
    // while block i's MFMAs run, and block i - 1 is rescaled after block i's MFMAs
    // are issued (hides LDS and MFMA latency with one wave per SIMD).
    auto load_af = [&](int i, bf16x8* af) {
      const int arow = wm * WM + 16 * i + l16;
#pragma unroll
      for (int ks = 0; ks < nk32; ++ks) af[ks] = __builtin_bit_cast(bf16x8, Av[swz(arow, 4 * ks + lq)]);
    };
    bf16x8 afc[2], afn[2];
    load_af(0, afc);
    if constexpr (BK == B_INT4) {
      constexpr bool ONE_GROUP = (G >= KS) && (nk32 == 2);   // both 32-steps share one group
      constexpr int NT = ONE_GROUP ? 1 : nk32;                // partial sums per block per stage
      f32x4 tpp[NT][NB];                                      // previous block's partials
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (i + 1 < MB) load_af(i + 1, afn);
        f32x4 tpc[NT][NB];
#pragma unroll
        for (int ks = 0; ks < nk32; ++ks) {
          const int tix = ONE_GROUP ? 0 : ks;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const f32x4 zero = {};
            tpc[tix][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afc[ks], bfr[j][ks],
                                                                 (ONE_GROUP && ks == 1) ? tpc[tix][j] : zero, 0, 0, 0);
          }
        }
        if (i > 0) {
#pragma unroll
          for (int tix = 0; tix < NT; ++tix)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
              for (int v = 0; v < 4; ++v)
                acc[i - 1][j][v] = __builtin_fmaf(gs[tix][j], tpp[tix][j][v], acc[i - 1][j][v]);
        }
#pragma unroll
        for (int tix = 0; tix < NT; ++tix)
#pragma unroll
          for (int j = 0; j < NB; ++j) tpp[tix][j] = tpc[tix][j];
        if (i + 1 < MB) {
          afc[0] = afn[0];
          afc[1] = afn[1];
        }
      }
#pragma unroll
      for (int tix = 0; tix < NT; ++tix)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[MB - 1][j][v] = __builtin_fmaf(gs[tix][j], tpp[tix][j][v], acc[MB - 1][j][v]);
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (i + 1 < MB) load_af(i + 1, afn);
#pragma unroll
        for (int ks = 0; ks < nk32; ++ks)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afc[ks], bfr[j][ks], acc[i][j], 0, 0, 0);
            if constexpr (BK == B_SPLIT)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afc[ks], bf2[j][ks], acc[i][j], 0, 0, 0);
          }
        if (i + 1 < MB) {
          afc[0] = afn[0];
          afc[1] = afn[1];
        }
      }
    }
    if (more) store_b(buf ^ 1);
    if constexpr (BK == B_INT4) {
      if (more) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < NB; ++j) gs[ks][j] = gs_next[ks][j];
      }
    }
    // this wave's direct loads for the next stage have landed (loads return in order;
    // the ones issued during this stage, for the stage after next, may still fly)
    if (NA == 3 && issued) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(DIRECT));
    else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
    stage_barrier();
  };

  // ---- prologue and main loop ------------------------------------------------
  load_b(0);
  issue_a(0, 0);
  issue_b_planes(0, 0);
  if (NA == 3 && nstage > 1) issue_a(1, 1);
  store_b(0);
  if (NA == 3 && nstage > 1) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(DIRECT));
  else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
  stage_barrier();
  for (int s = 0; s < nfull; ++s) run_stage(s, std::integral_constant<int, 2>{});
  if constexpr (TAIL) run_stage(nfull, std::integral_constant<int, 1>{});

  // ---- epilogue --------------------------------------------------------------
  if constexpr (BK == B_SPLIT) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + wn * 64 + 16 * j + l16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = m0 + wm * WM + 16 * i + 4 * lq + v;
          const double d = (double)acc[i][j][v];
          if (m < M && n < N) ss = __builtin_fma(d, d, ss);
        }
      }
    ss = wave_sum(ss);
    __shared__ double wsum[4];
    if (lane == 0) wsum[wid] = ss;
    __syncthreads();
    if (tid == 0) a.partial[t] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  } else {
    const bool full = (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + wn * 64 + 16 * j + l16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = m0 + wm * WM + 16 * i + 4 * lq + v;
          const float y = (BK == B_FP4) ? acc[i][j][v] * a.ts : acc[i][j][v];
          if (full || (m < M && n < N)) a.Y[(int64_t)m * N + n] = y;
        }
      }
  }
}

int tiles(int M, int N, int bm) { return ((M + bm - 1) / bm) * ((N + BN - 1) / BN); }

template <int BK, int G, bool TAIL>
hipError_t launch_tail(const GemmArgs& a, hipStream_t stream) {
  const dim3 block(256);
  // INT4 keeps the running output and the group partials in VGPRs: 128-row tiles at
  // two waves per SIMD.  FP4 / SPLIT accumulate straight into MFMA registers and use
  // 256-row tiles for large M.
  if constexpr (BK != B_INT4) {
    if (a.M >= 2048) {
      hipLaunchKernelGGL((gemm_kernel<BK, 8, G, TAIL>), dim3(tiles(a.M, a.N, 256)), block, 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<BK, 4, G, TAIL>), dim3(tiles(a.M, a.N, 128)), block, 0, stream, a);
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

int sumsq_gemm_blocks(int M, int N) { return M >= 2048 ? tiles(M, N, 256) : tiles(M, N, 128); }  // SPLIT tiles

hipError_t launch_sumsq_gemm(const uint16_t* X, int M, int K, const uint16_t* E, int N, double* partial,
                             hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.B = E; a.B2 = E + (size_t)N * K; a.partial = partial;
  return launch_tiles<B_SPLIT, 64>(a, stream);
}

}  // namespace aq

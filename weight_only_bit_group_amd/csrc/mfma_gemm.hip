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
//   GRAM  the same two-plane pipeline for the search's Gram form: A = E_hi, B = the
//         two bf16 planes of H = X^T X, so the tile holds F = E_hi H; the epilogue
//         returns the fp64 sum of F * (E_hi + 2 E_lo) over the tile, read from the
//         error planes at each output's (row, column).
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
//     stored at u ^ ((r >> 1) & 7): the 16 consecutive rows read by each 16-lane
//     phase of a ds_read_b128 (the same unit of each) hit all 16 groups of four
//     banks once (rows r and r + 8 would collide under u ^ (r & 7)).
//   * Block order is XCD-aware: block b runs on XCD b % 8; each XCD gets a
//     contiguous range of a grouped tile order (a few row tiles, all column
//     tiles), so the blocks it runs together share their activation and weight
//     tiles in its L2.
//   * Persistent grid (K % 64 == 0, at least four stages): one block per compute
//     unit runs tiles b, b + grid, ...; the last three stages of a tile already
//     load the next tile's first stages, so the load pipeline never drains.
//   * INT4: the MFMAs of one group run block by block into a temporary that is
//     rescaled by S[n, g] straight into the VGPR-resident output (one v_fma per
//     output element per group), software-pipelined one block behind the MFMAs
//     and interleaved with them (a slice of the rescale after each MFMA, so the
//     VALU work overlaps the matrix core).  A group wider than a stage (g = 128)
//     is rescaled once per stage with the same S.
//   * Output stores address the tile from a uniform base plus one 32-bit lane
//     offset (N < 2^22), so the epilogue holds no 64-bit address per store.
// A lane of a 32x32x16 MFMA holds row (lane % 32) and k = 8 (lane / 32) .. +7 of
// each operand; its 16 results are column (lane % 32), rows
// 8 (i / 4) + 4 (lane / 32) + (i % 4), so they share one weight row n and need
// one S per block per group.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "aq_device.h"
#include "aq_kernels.h"
#include "gemm_lds.h"

namespace aq {

// Compute units of the current device (queried once per device, 256 if the query fails).
int device_cu_count() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// B operand kinds: INT4 / FP4 codes dequantized in the kernel; INT4S / FP4S the same
// weights dequantized beforehand into a bf16 staging matrix (loaded like the SPLIT
// planes); SPLIT the search's two bf16 planes; GRAM the search's Gram-form product.
enum BKind { B_INT4 = 0, B_SPLIT = 1, B_FP4 = 2, B_INT4S = 3, B_FP4S = 4, B_GRAM = 5 };

struct GemmArgs {
  const uint16_t* X;
  int M, N, K;
  // row stride in k of X, of the weight arrays and of the staged / plane matrices (= K
  // unless the contraction is split); K slice: ks blocks along y each take kslice k
  // (K is the slice length then) and write their fp32 output ystride floats apart
  int ld;
  int kslice;
  int64_t ystride;
  // INT4
  const uint8_t* P;
  const float* S;
  const uint8_t* Z;
  // SPLIT: the two bf16 planes of E; INT4S / FP4S: the staged bf16 weights in B
  const uint16_t* B;
  const uint16_t* B2;
  // GRAM: the E_lo plane (E_hi is X), [M, N] with N contiguous
  const uint16_t* Elo;
  // FP4
  const uint8_t* codes;
  const uint8_t* bscale;
  float ts;
  // outputs
  float* Y;           // [M, N] fp32 (INT4, FP4)
  double* partial;    // [number of blocks] fp64 sums of squares (SPLIT) or weighted sums (GRAM)
};

namespace {

using namespace gemm;

constexpr int KS = 64;            // k per stage
constexpr int BN = 128;           // block tile columns (weight rows)
constexpr int ROW_UNITS = KS / 8;  // 16-byte units per LDS row

__device__ __forceinline__ int swz(int row, int unit) { return row * ROW_UNITS + (unit ^ ((row >> 1) & 7)); }

template <int BK, int G, bool TAIL, int WGM>
__global__ __launch_bounds__(128 * WGM, 1) void gemm_kernel(GemmArgs a) {
  if (gridDim.y > 1) {
    // K slice blockIdx.y: operands from its first k on, its own output buffer
    const int k0 = (int)blockIdx.y * a.kslice;
    a.K = min(a.kslice, a.K - k0);
    a.X += k0;
    if (a.P) a.P += k0 >> 1;
    if (a.B) a.B += k0;
    if (a.B2) a.B2 += k0;
    if (a.codes) a.codes += k0 >> 1;
    if (a.bscale) a.bscale += k0 >> 4;
    if (a.S) a.S += k0 / G;
    if (a.Z) a.Z += k0 / G;
    a.Y += (int64_t)blockIdx.y * a.ystride;
  }
  constexpr int NW = 2 * WGM, NT = 64 * NW;
  constexpr int BM = 64 * WGM;
  constexpr bool DEQ = BK == B_INT4 || BK == B_FP4;        // codes dequantized here
  constexpr bool SPLIT = BK == B_SPLIT || BK == B_GRAM;    // two B planes into one accumulator
  constexpr bool GRAM = BK == B_GRAM;
  constexpr bool STAGED = BK == B_INT4S || BK == B_FP4S;   // bf16 weights from global memory
  constexpr bool RESCALE = BK == B_INT4 || BK == B_INT4S;  // per-group steps applied to partials
  constexpr bool TSCALE = BK == B_FP4 || BK == B_FP4S;     // fp32 tensor scale on the output
  constexpr int PLANES = SPLIT ? 2 : 1;
  constexpr int NA = SPLIT ? 2 : 3;                 // activation ring
  constexpr int NB = STAGED ? 3 : 2;                // weight-tile ring
  constexpr int PD = 2;                             // stage s loads the activations of stage s + 2
  constexpr int CD = 3;                             // code / per-row scalar prefetch distance
  constexpr int A_DMA = BM / 8 / NW;                // activation loads per wave per stage (8 rows each)
  constexpr int B_DMA = PLANES * (BN / 8) / NW * (DEQ ? 0 : 1);  // plane loads per wave per stage
  // code + per-row scalar loads per stage: 4 code loads (1 KB each) and the scalars
  // (INT4: steps and zero points, two 64-row halves per group, one or two groups per
  // stage, the zero-point loads repeated at g = 32 so every wave issues the same
  // number; FP4: two ushorts of block scales per row)
  constexpr int NAUX = (BK == B_INT4 && G == 32) ? 12 : 4;
  constexpr int JOBS = DEQ ? 4 + NAUX : 0;
  constexpr int JPW = JOBS / NW;
  static_assert(!DEQ || JOBS % NW == 0, "scalar loads must split evenly over the waves");

  __shared__ __attribute__((aligned(16))) uint16_t As[NA][BM * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NB][PLANES][BN * KS];
  __shared__ __attribute__((aligned(16))) uint8_t Cs[DEQ ? 3 : 1][DEQ ? BN * KS / 2 : 16];
  // per-row scalars: [slot][INT4: 0 = S bits, 1 = zero point | FP4: 0][group in stage or FP4 half][row]
  __shared__ __attribute__((aligned(16))) uint32_t AX[(DEQ || RESCALE) ? 4 : 1][DEQ ? 2 : 1][2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 1, wn = wid & 1;
  const int M = a.M, N = a.N, K = a.K, LD = a.ld;
  const int GLD = LD / G;   // row stride of the group steps and zero points
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = (M + BM - 1) / BM;
  const int ntiles = tiles_m * tiles_n;
  const int nfull = K / KS;                    // full 64-wide stages; TAIL adds one 32-wide stage
  const int nstage = nfull + (TAIL ? 1 : 0);
  const int ngroups = K / G;
  // The block runs tiles blockIdx.x, blockIdx.x + gridDim.x, ... (a persistent grid of
  // one block per CU, or one tile per block).  Virtual block vb maps to a tile by the
  // XCD-aware order (vb runs on XCD vb % 8 when the grid is a multiple of 8): an
  // XCD-contiguous linear index, then groups of GM row tiles walked column by column,
  // so the tiles an XCD runs at once share their activation and weight tiles in its L2.
  struct TileXY { int m0, n0, t; };
  auto coords = [&](int i) -> TileXY {
    const int t = tile_of_block(blockIdx.x + i * (int)gridDim.x, ntiles);
    const int GM = max(1, (tiles_m + 7) / 8);
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int within = t - group * GM * tiles_n;
    // wave-uniform: keep the coordinates in scalar registers
    return TileXY{__builtin_amdgcn_readfirstlane((first_m + within % gm) * BM),
                  __builtin_amdgcn_readfirstlane((within / gm) * BN), __builtin_amdgcn_readfirstlane(t)};
  };
  const int ntl = (ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;   // tiles of this block

  // ---- LDS-DMA loads --------------------------------------------------------
  // Tile rows: load j of wave w covers the 8 rows from R0 = 8 r8, r8 = j NW + w; lane l
  // lands at LDS unit (R0 + l / 8, l % 8), which holds logical unit
  // (l % 8) ^ (((R0 + l / 8) >> 1) & 7) = (l % 8) ^ ((4 r8 + l / 16) & 7): the global
  // unit it fetches.  Load addresses are a 64-bit base at the block's first row (and
  // the stage's first column) plus a 32-bit lane offset within the block's rows, which
  // stays below 2^32 for K < 2^22.  In the 32-wide tail stage
  // the upper four units are folded back onto the lower four (loaded, never
  // multiplied), so no load runs past a row.
  const int lrow8 = lane >> 3;
  auto gunit_of = [&](int r8) { return (lane & 7) ^ ((4 * r8 + (lane >> 4)) & 7); };
  auto fold_of = [&](int r8) -> uint32_t { return (TAIL && gunit_of(r8) >= 4) ? 64u : 0u; };
  // lane offsets of the activation loads for the tile at row m0 (rows past M clamped)
  uint32_t aoff[A_DMA];
  auto set_aoff = [&](int m0) {
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
      const int r8 = j * NW + wid;
      aoff[j] = (uint32_t)(min(m0 + 8 * r8 + lrow8, M - 1) - m0) * (uint32_t)LD * 2u + (uint32_t)gunit_of(r8) * 16u;
    }
  };
  // activations of stage s of the tile at row m0 (aoff set for that tile)
  auto issue_a = [&](int m0, int s, int slot) {
    const char* base = reinterpret_cast<const char*>(a.X + (size_t)m0 * LD) + (size_t)s * (KS * 2);
    const bool tail = TAIL && s == nfull;
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
      const int r8 = j * NW + wid;
      dma16(base, aoff[j] - (tail ? fold_of(r8) : 0u), lds_addr(&As[slot][8 * r8 * KS]));
    }
  };
  // lane offsets of the SPLIT plane / staged weight loads for the tile at column n0
  // (rows past N clamped); plane loads q and q + PER share one
  constexpr int PER = BN / 8 / NW;   // plane loads per plane and wave
  uint32_t boff[PER];
  auto set_boff = [&](int n0) {
    if constexpr (!DEQ) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int r8 = j * NW + wid;
        boff[j] = (uint32_t)(min(n0 + 8 * r8 + lrow8, N - 1) - n0) * (uint32_t)LD * 2u + (uint32_t)gunit_of(r8) * 16u;
      }
    }
  };
  // codes (32 bytes per row and stage, two 16-byte halves per lane pair) and the
  // per-row scalars of stage s: job i (0 <= i < JPW) of this wave
  auto issue_job = [&](int n0, int s, int cslot, int xslot, int i) {
    if constexpr (DEQ) {
      const bool tail = TAIL && s == nfull;
      const int job = wid * JPW + i;   // wave-uniform
      if (job < 4) {
        const int r = 32 * job + (lane >> 1);
        const uint32_t n = (uint32_t)(min(n0 + r, N - 1) - n0);
        const uint32_t half = tail ? 0u : (uint32_t)(lane & 1) * 16u;
        const uint8_t* src = ((BK == B_INT4) ? a.P : a.codes) + (size_t)n0 * (LD >> 1) + (size_t)s * (KS / 2);
        dma16(src, n * (uint32_t)(LD >> 1) + half, lds_addr(&Cs[cslot][1024 * job]));
      } else if constexpr (BK == B_INT4) {
        int x = job - 4;
        if (x >= 8) x -= 4;                                  // repeated zero-point loads (g = 32)
        const int is_z = (G == 32) ? (x >= 4) : (x >= 2);
        const int gi = (G == 32) ? ((x >> 1) & 1) : 0;
        const int rh = 64 * (x & 1);
        const uint32_t n = (uint32_t)(min(n0 + rh + lane, N - 1) - n0);
        const uint32_t g = (uint32_t)min((s * KS + 32 * gi) / G, ngroups - 1);
        const uint32_t idx = n * (uint32_t)GLD + g;
        if (is_z) dma1(a.Z + (size_t)n0 * GLD, idx, lds_addr(&AX[xslot][1][gi][rh]));
        else dma4(a.S + (size_t)n0 * GLD, idx * 4u, lds_addr(&AX[xslot][0][gi][rh]));
      } else {
        const int x = job - 4;
        const int h = x >> 1, rh = 64 * (x & 1);
        const uint32_t n = (uint32_t)(min(n0 + rh + lane, N - 1) - n0);
        const uint32_t byte = (uint32_t)(s * 4 + 2 * (tail ? 0 : h));   // the tail stage has 2 block scales
        dma2(a.bscale + (size_t)n0 * (LD >> 4), n * (uint32_t)(LD >> 4) + byte, lds_addr(&AX[xslot][0][h][rh]));
      }
    }
  };
  auto issue_codes = [&](int n0, int s, int cslot, int xslot) {
#pragma unroll
    for (int i = 0; i < JPW; ++i) issue_job(n0, s, cslot, xslot, i);
  };
  // one activation load (j < A_DMA) / one SPLIT plane load (q < B_DMA) of stage s
  auto issue_a_one = [&](int m0, int s, int slot, int j) {
    const char* base = reinterpret_cast<const char*>(a.X + (size_t)m0 * LD) + (size_t)s * (KS * 2);
    const int r8 = j * NW + wid;
    dma16(base, aoff[j] - ((TAIL && s == nfull) ? fold_of(r8) : 0u), lds_addr(&As[slot][8 * r8 * KS]));
  };
  auto issue_plane_one = [&](int n0, int s, int slot, int q) {
    if constexpr (!DEQ) {
      const int pl = q / PER, j = q % PER, r8 = j * NW + wid;
      const char* base = reinterpret_cast<const char*>((pl ? a.B2 : a.B) + (size_t)n0 * LD) + (size_t)s * (KS * 2);
      dma16(base, boff[j] - ((TAIL && s == nfull) ? fold_of(r8) : 0u), lds_addr(&Bs[slot][pl][8 * r8 * KS]));
    }
  };
  auto issue_planes = [&](int n0, int s, int slot) {
#pragma unroll
    for (int q = 0; q < B_DMA; ++q) issue_plane_one(n0, s, slot, q);
  };

  // staged INT4: the group steps of stage s (one dword per row, 64 rows per load, one
  // or two groups per stage)
  auto issue_steps = [&](int n0, int s, int slot) {
    if constexpr (BK == B_INT4S) {
      // every wave issues one (no branch in the stage body): wave w loads part w % NL,
      // so each part is loaded by several waves with the same bytes
      constexpr int NL = (G == 32) ? 4 : 2;
      const int part = wid % NL;
      const int gi = part >> 1, rh = 64 * (part & 1);
      const uint32_t n = (uint32_t)(min(n0 + rh + lane, N - 1) - n0);
      const uint32_t g = (uint32_t)min((s * KS + 32 * gi) / G, ngroups - 1);
      dma4(a.S + (size_t)n0 * GLD, (n * (uint32_t)GLD + g) * 4u, lds_addr(&AX[slot][0][gi][rh]));
    }
  };

  // ---- dequantization: codes of one stage -> bf16 weight tile ----------------
  // Thread t converts KPT codes of weight row t / TPR (WPT words of 8 codes, each one
  // 16-byte LDS unit of bf16 values), in four parts so the work can be spread over a
  // stage.  dq_load reads the codes and per-row scalars; dq_part(p) converts pairs
  // [p WPT, (p + 1) WPT) and stores each unit once its four pairs are done.
  constexpr int TPR = NT / BN;          // threads per weight row
  constexpr int KPT = KS / TPR;         // k per thread (16 or 32)
  constexpr int WPT = KPT / 8;          // 8-code words (= LDS units) per thread
  const int d_row = tid / TPR, d_part = tid % TPR;
  uint32_t dq_w[WPT], dq_lo[WPT], dq_hi[WPT], dq_o[WPT][4];
  float dq_z = 0.0f;
  uint32_t dq_sc2[2] = {0u, 0u};
  auto dq_load = [&](int cslot, int xslot) {
    if constexpr (DEQ) {
      const uint8_t* cp = &Cs[cslot][d_row * 32 + d_part * (KPT / 2)];
      if constexpr (WPT == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(cp);
        dq_w[0] = v.x; dq_w[1] = v.y;
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(cp);
        dq_w[0] = v[0]; dq_w[1] = v[1]; dq_w[2] = v[2]; dq_w[3] = v[3];
      }
      if constexpr (BK == B_INT4) {
        const int gi = (G == 32) ? (d_part * KPT) / 32 : 0;
        dq_z = (float)AX[xslot][1][gi][d_row];
      } else {
        // the 16-element blocks of this thread's codes: (d_part KPT + 8 u) / 16
        dq_sc2[0] = AX[xslot][0][0][d_row];
        dq_sc2[1] = AX[xslot][0][1][d_row];
      }
    }
  };
  auto dq_part = [&](int p, int bbuf, bool tail) {
    if constexpr (DEQ) {
      if (tail && d_part * KPT >= 32) return;   // the tail stage has 32 k
      u32x4* dst = reinterpret_cast<u32x4*>(&Bs[bbuf][0][0]);
#pragma unroll
      for (int q = p * WPT; q < (p + 1) * WPT; ++q) {
        const int u = q >> 2, b = q & 3;
        if constexpr (BK == B_INT4) {
          if (b == 0) {
            dq_lo[u] = dq_w[u] & 0x0F0F0F0Fu;
            dq_hi[u] = (dq_w[u] >> 4) & 0x0F0F0F0Fu;
            // opaque to the optimizer, so each code converts with one v_cvt_f32_ubyteN
            asm("" : "+v"(dq_lo[u]), "+v"(dq_hi[u]));
          }
          const float ql = (float)((dq_lo[u] >> (8 * b)) & 0xFFu), qh = (float)((dq_hi[u] >> (8 * b)) & 0xFFu);
          dq_o[u][b] = pack_bf16_exact(ql - dq_z, qh - dq_z);
        } else {
          const int blk = (d_part * KPT + 8 * u) >> 4;   // block of word u within the stage
          const uint32_t two = dq_sc2[blk >> 1];
          const float sc = (blk & 1) ? __builtin_amdgcn_cvt_f32_fp8((int)two, 1) : __builtin_amdgcn_cvt_f32_fp8((int)two, 0);
          uint32_t e2;
          switch (b) {
            case 0: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dq_w[u], 1.0f, 0)); break;
            case 1: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dq_w[u], 1.0f, 1)); break;
            case 2: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dq_w[u], 1.0f, 2)); break;
            default: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dq_w[u], 1.0f, 3)); break;
          }
          dq_o[u][b] = pack_bf16_exact(bf16_lo(e2) * sc, bf16_hi(e2) * sc);
        }
        if (b == 3) dst[swz(d_row, d_part * WPT + u)] = u32x4{dq_o[u][0], dq_o[u][1], dq_o[u][2], dq_o[u][3]};
      }
    }
  };
  auto dequant = [&](int cslot, int xslot, int bbuf, bool tail) {
    dq_load(cslot, xslot);
#pragma unroll
    for (int p = 0; p < 4; ++p) dq_part(p, bbuf, tail);
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
  constexpr int A_BUF = BM * KS / 8, B_BUF = PLANES * BN * KS / 8, B_PLANE = BN * KS / 8;  // 16-byte units
  static_assert(A_DMA == 4 && JPW <= 4 && B_DMA % 2 == 0, "loads are spread over the parts of a stage");

  // INT4: the group partial of block (1, 1) from a stage's last part, with its step,
  // rescaled by the next stage's first part (or the tile epilogue); zero at the start
  f32x16 tcar;
  float scar = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) tcar[v] = 0.0f;

  // ---- one stage ----------------------------------------------------------------
  // The workgroup barrier sits in the middle of a stage: stage s reads all its
  // fragments, runs blocks (0,0) and (0,1), waits for its loads and passes barrier
  // M_s, then runs blocks (1,0) and (1,1) from registers.  M_s publishes stage s + 1
  // (its activations landed, its weights dequantized), so the next stage's reads are
  // issued right behind the MFMAs of blocks (1,*) and there is MFMA work queued on
  // both sides of every barrier.
  //   Buffers: stage s's tiles are read only before M_s, so after M_s they take stage
  //   s + 2's weights (dequantized during parts 2, 3 of stage s and parts 0, 1 of
  //   stage s + 1) and, for SPLIT (two-deep rings), its planes and activations.
  //   INT4 / FP4 activations use a three-deep ring: stage s + 2's are loaded during
  //   all of stage s.  Codes and per-row scalars of stage s + 3 load at its start.
  //   M_s waits for every load except those issued in stage s before it.
  // Tags: NKS = 16-wide MFMA steps of stage s (4, or 2 in the tail); NX1 / NX2 = the
  // same for stages s + 1 / s + 2 (0: none), whose dequantization parts 2, 3 / 0, 1
  // run here; MA: load activations (INT4, FP4: stage s + 2) or activations and planes
  // (SPLIT: stage s + 2, after M_s); MC: load codes and scalars of stage s + 3.
  // q: the block's stage index (ring slots); (m2, n2, s2): tile and tile stage of stage
  // q + 2, (n3, s3): weight rows and tile stage of stage q + 3 (prefetch targets).
  auto run_stage = [&](int q, int m2, int n2, int s2, int n3, int s3, auto nk_tag, auto nx1_tag, auto nx2_tag,
                       auto mc_tag, auto ma_tag) {
    constexpr int NKS = decltype(nk_tag)::value;
    constexpr int NX1 = decltype(nx1_tag)::value;
    constexpr int NX2 = decltype(nx2_tag)::value;
    constexpr bool MC = DEQ && decltype(mc_tag)::value;
    constexpr bool MA = decltype(ma_tag)::value;
    constexpr int NG = (RESCALE && G == 32) ? NKS / 2 : 1;   // group partials per block (INT4)
    constexpr int KPG = NKS / NG;
    const int abuf = q % NA;
    const int bbuf = q % NB;
    const int xs = q & 3;
    if constexpr (MC) issue_codes(n3, s3, (q + CD) % 3, (q + CD) & 3);
    __builtin_amdgcn_sched_barrier(0);
    // LDS reads: this stage's fragments (m-block 1's during part 0) and group steps
    bf16x8 af[2][NKS], bf[2][NKS], bf2[2][NKS];
    auto read_a = [&](int mi) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        af[mi][ks] = __builtin_bit_cast(bf16x8, Av[abuf * A_BUF + swz(wm * 64 + 32 * mi + l32, 2 * ks + lh)]);
    };
    // in the order the first block's MFMAs consume them (the operand pair of each k step,
    // then n-block 1), so the first MFMA waits for two reads, not for all of them
    auto read_b = [&](int ni, int ks) {
      const int row = wn * 64 + 32 * ni + l32;
      bf[ni][ks] = __builtin_bit_cast(bf16x8, Bv[bbuf * B_BUF + swz(row, 2 * ks + lh)]);
      if constexpr (SPLIT) bf2[ni][ks] = __builtin_bit_cast(bf16x8, Bv[bbuf * B_BUF + B_PLANE + swz(row, 2 * ks + lh)]);
    };
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      af[0][ks] = __builtin_bit_cast(bf16x8, Av[abuf * A_BUF + swz(wm * 64 + l32, 2 * ks + lh)]);
      read_b(0, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) read_b(1, ks);
    float sc[2][2];
    if constexpr (RESCALE) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) sc[ni][gi] = __builtin_bit_cast(float, AX[xs][0][gi][wn * 64 + 32 * ni + l32]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Parts: INT4 runs one (group, block) item per part, item it = (group it / 4,
    // block it % 4), so NPART = 4 NG; each part rescales the previous part's item (part
    // 0: the item carried from the previous stage, always block (1, 1)).  The other
    // kinds run one block per part.  Loads and dequantization are spread over the
    // parts in four steps (pp = 0 .. 3, one every NPART / 4 parts).
    constexpr int NPART = RESCALE ? 4 * NG : 4;
    constexpr int PSTEP = NPART / 4;
    f32x16 tprev = tcar;
    float sprev = scar;
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      if constexpr (RESCALE) {
        const int gi = part >> 2, blk = part & 3, mi = blk >> 1, ni = blk & 1;
        const int pblk = part == 0 ? 3 : ((part - 1) & 3), qm = pblk >> 1, qn = pblk & 1;
        // The item's MFMAs interleaved with the previous item's rescale: slice k of the
        // rescale (V of its 16 outputs) runs after MFMA k and before MFMA k + 1, so the
        // VALU work overlaps the matrix core.  Empty asm statements fix the order (the
        // compiler would otherwise group the rescale ahead of the MFMAs, or sink it to
        // the end of the stage): each ties the accumulator elements of slices k - 1 and
        // k and the A operand of MFMA k.
        constexpr int V = 16 / KPG;
        float e[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) e[v] = acc[qm][qn][v];
        f32x16 tp;
#pragma unroll
        for (int k = 0; k < KPG; ++k) {
          const int ks = gi * KPG + k;
#pragma unroll
          for (int v = (k > 0 ? (k - 1) * V : 0); v < (k + 1) * V; ++v) asm volatile("" : "+v"(e[v]));
          asm volatile("" : "+v"(af[mi][ks]));
          const f32x16 zero = {};
          tp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][ks], bf[ni][ks], k == 0 ? zero : tp, 0, 0, 0);
#pragma unroll
          for (int v = k * V; v < (k + 1) * V; ++v) e[v] = __builtin_fmaf(sprev, tprev[v], e[v]);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[qm][qn][v] = e[v];
        asm volatile("" : "+v"(acc[qm][qn]));
        tprev = tp;
        sprev = sc[ni][gi];
      } else {
        const int mi = part >> 1, ni = part & 1;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][ks], bf[ni][ks], acc[mi][ni], 0, 0, 0);
          if constexpr (SPLIT)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][ks], bf2[ni][ks], acc[mi][ni], 0, 0, 0);
        }
      }
      // m-block 1 is first used by block 2 (part 2): read in part 1
      if (part == 1) read_a(1);
      if (part % PSTEP == 0) {
        const int pp = part / PSTEP;
        if constexpr (DEQ) {
          // dequantization: steps 0, 1 finish stage q + 1 (into the other weight buffer);
          // steps 2, 3 start stage q + 2 (into this stage's buffer, free after M_s)
          if (pp < 2) {
            if constexpr (NX1 > 0) dq_part(pp + 2, bbuf ^ 1, NX1 == 2);
          } else {
            if constexpr (NX2 > 0) {
              if (pp == 2) dq_load((q + 2) % 3, (q + 2) & 3);
              dq_part(pp - 2, bbuf, NX2 == 2);
            }
          }
        }
        if constexpr (DEQ && MA) {
          issue_a_one(m2, s2, (q + PD) % NA, pp);
        } else if constexpr (STAGED && MA) {
          // stage q + 2's activations over all four steps, its weights in steps 0, 1,
          // its group steps in step 2 (after M_s, so they are not counted there)
          issue_a_one(m2, s2, (q + 2) % 3, pp);
          if (pp < 2) {
#pragma unroll
            for (int qq = pp * (B_DMA / 2); qq < (pp + 1) * (B_DMA / 2); ++qq)
              issue_plane_one(n2, s2, (q + 2) % 3, qq);
          }
          if (pp == 2) issue_steps(n2, s2, (q + 2) & 3);
        } else if constexpr (MA) {
          // SPLIT: stage q + 2's activations and planes go into this stage's buffers,
          // after M_s
          if (pp >= 2) {
#pragma unroll
            for (int j = (pp - 2) * (A_DMA / 2); j < (pp - 1) * (A_DMA / 2); ++j) issue_a_one(m2, s2, bbuf, j);
#pragma unroll
            for (int qq = (pp - 2) * (B_DMA / 2); qq < (pp - 1) * (B_DMA / 2); ++qq)
              issue_plane_one(n2, s2, bbuf, qq);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (part == NPART / 2 - 1) {
        // M_s: only the loads issued in this stage so far may still be in flight (loads
        // complete in order); this wave's LDS writes are done
        constexpr int KEEP = DEQ ? (MC ? JPW : 0) + (MA ? 2 : 0) : STAGED ? (MA ? 2 + B_DMA : 0) : 0;
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(KEEP));
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (RESCALE) {
      tcar = tprev;   // the last item (block (1, 1)) is rescaled by the next stage or the epilogue
      scar = sprev;
    }
  };

  // ---- tile epilogue ----------------------------------------------------------------
  // Applies the last carried group partials, writes the tile's outputs (SPLIT: its fp64
  // sum of squares; GRAM: its weighted sum) and clears the accumulators for the block's
  // next tile.
  // Result i of block (mi, ni): row 8 (i / 4) + 4 lh + (i % 4), column l32.
  __shared__ double wsum[NW];
  auto finish_tile = [&](const TileXY& tt) {
    if constexpr (RESCALE) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[1][1][v] = __builtin_fmaf(scar, tcar[v], acc[1][1][v]);
      scar = 0.0f;
    }
    const int m0 = tt.m0, n0 = tt.n0;
    // this lane's first output row and column; opaque to the optimizer so no part of the
    // epilogue's addressing is hoisted out of the tile loop into registers held by the
    // whole main loop
    int lrow = wm * 64 + 4 * lh, lcol = wn * 64 + l32;
    asm volatile("" : "+v"(lrow), "+v"(lcol));
    if constexpr (SPLIT) {
      double ss = 0.0;
      if constexpr (GRAM) {
        // weight of output (m, n): E_hi[m, n] + 2 E_lo[m, n], exact in fp32 (E_lo is at
        // most half an ulp of E_hi).  Outputs past the matrix load the tile's first
        // element and weigh 0, so every load is in bounds and unconditional: the loads
        // of an m-block (two output blocks, both planes) are all issued before the
        // first is used.
        const uint16_t* eh = a.X + (int64_t)m0 * N + n0;
        const uint16_t* el = a.Elo + (int64_t)m0 * N + n0;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          uint32_t off[2][16];
          bool in[2][16];
          uint16_t hv[2][16], lv[2][16];
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int cn = lcol + 32 * ni;
              const int rm = lrow + 32 * mi + 8 * (v >> 2) + (v & 3);
              in[ni][v] = m0 + rm < M && n0 + cn < N;
              off[ni][v] = in[ni][v] ? (uint32_t)rm * (uint32_t)N + (uint32_t)cn : 0u;
            }
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              hv[ni][v] = eh[off[ni][v]];
              lv[ni][v] = el[off[ni][v]];
            }
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float w = bf16_to_f32(hv[ni][v]) + 2.0f * bf16_to_f32(lv[ni][v]);
              ss = __builtin_fma((double)acc[mi][ni][v], (double)(in[ni][v] ? w : 0.0f), ss);
            }
        }
      } else {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const int n = n0 + lcol + 32 * ni;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int m = m0 + lrow + 32 * mi + 8 * (v >> 2) + (v & 3);
              const double d = (double)acc[mi][ni][v];
              if (m < M && n < N) ss = __builtin_fma(d, d, ss);
            }
          }
      }
      ss = wave_sum(ss);
      if (lane == 0) wsum[wid] = ss;
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the LDS write is done (loads stay in flight)
      stage_barrier();
      if (tid == 0) {
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += wsum[w];
        a.partial[tt.t] = tot;
      }
    } else {
      // store addresses: the tile's base (uniform) plus a 32-bit byte offset per lane,
      // which stays below 2^32 for N < 2^22
      char* yt = reinterpret_cast<char*>(a.Y + (int64_t)m0 * N + n0);
      const uint32_t lbase = ((uint32_t)lrow * (uint32_t)N + (uint32_t)lcol) * 4u;
      const uint32_t rstride = (uint32_t)N * 4u;
      auto out = [&](int mi, int ni, int v) { return TSCALE ? acc[mi][ni][v] * a.ts : acc[mi][ni][v]; };
      auto addr = [&](int mi, int ni, int v) {
        const int dm = 32 * mi + 8 * (v >> 2) + (v & 3);
        return reinterpret_cast<float*>(yt + (lbase + (uint32_t)dm * rstride + 128u * (uint32_t)ni));
      };
      if ((m0 + BM <= M) && (n0 + BN <= N)) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) __builtin_nontemporal_store(out(mi, ni, v), addr(mi, ni, v));
      } else {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int dm = 32 * mi + 8 * (v >> 2) + (v & 3);
              if (m0 + lrow + dm < M && n0 + lcol + 32 * ni < N) __builtin_nontemporal_store(out(mi, ni, v), addr(mi, ni, v));
            }
      }
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
  };

  // ---- prologue ----------------------------------------------------------------
  // Loads of stages 0 and 1 of the first tile (and the codes of stage 2), stage 0's
  // weights and the first half of stage 1's dequantized; SPLIT: stages 0 and 1.
  TileXY tc = coords(0);                       // tile of stage q
  TileXY tn = ntl > 1 ? coords(1) : tc;        // the block's next tile
  set_aoff(tc.m0);
  set_boff(tc.n0);
  if constexpr (DEQ) {
    issue_codes(tc.n0, 0, 0, 0);
    issue_a(tc.m0, 0, 0);
    if (nstage > 1) {
      issue_codes(tc.n0, 1, 1, 1);
      issue_a(tc.m0, 1, 1);
    }
    if (nstage > 2) issue_codes(tc.n0, 2, 2, 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
    stage_barrier();
    dequant(0, 0, 0, TAIL && nfull == 0);
    if (nstage > 1) {
      dq_load(1, 1);
      dq_part(0, 1, TAIL && nfull == 1);
      dq_part(1, 1, TAIL && nfull == 1);
    }
  } else {
    issue_a(tc.m0, 0, 0);
    issue_planes(tc.n0, 0, 0);
    issue_steps(tc.n0, 0, 0);
    if (nstage > 1) {
      issue_a(tc.m0, 1, 1);
      issue_planes(tc.n0, 1, 1);
      issue_steps(tc.n0, 1, 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
  stage_barrier();

  using IC4 = std::integral_constant<int, 4>;
  using IC2 = std::integral_constant<int, 2>;
  using IC0 = std::integral_constant<int, 0>;
  using YES = std::true_type;
  using NO = std::false_type;
  // The block's tiles run back to back; q, the block's stage count, indexes the LDS
  // rings across tiles.  Within a tile the steady loop runs the full stages whose
  // prefetch targets (stage s + 2's activations and weights, stage s + 3's codes) lie
  // in the same tile; a tile's last three stages are peeled: with a next tile they
  // load its first stages, so the pipeline does not drain between tiles, and on the
  // block's last tile they run it down (loads and dequantization depend on the
  // position).  A block with several tiles has full stages only (K % 64 == 0 and at
  // least four stages per tile).
  auto kind = [&](int t) { return t >= nstage ? 0 : (TAIL && t == nfull) ? 2 : 4; };
  const int steady = max(0, nstage - 3);
  int q = 0;
  for (int i = 0; i + 1 < ntl; ++i) {
    for (int s = 0; s < steady; ++s, ++q)
      run_stage(q, tc.m0, tc.n0, s + 2, tc.n0, s + 3, IC4{}, IC4{}, IC4{}, YES{}, YES{});
    run_stage(q, tc.m0, tc.n0, nstage - 1, tn.n0, 0, IC4{}, IC4{}, IC4{}, YES{}, YES{});
    ++q;
    set_aoff(tn.m0);   // activation and weight loads move to the next tile
    set_boff(tn.n0);
    run_stage(q, tn.m0, tn.n0, 0, tn.n0, 1, IC4{}, IC4{}, IC4{}, YES{}, YES{});
    ++q;
    run_stage(q, tn.m0, tn.n0, 1, tn.n0, 2, IC4{}, IC4{}, IC4{}, YES{}, YES{});
    ++q;
    finish_tile(tc);
    tc = tn;
    if (i + 2 < ntl) tn = coords(i + 2);
  }
  // the block's last tile
  const int m0 = tc.m0, n0 = tc.n0;
  for (int s = 0; s < steady; ++s, ++q)
    run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC4{}, IC4{}, YES{}, YES{});
  for (int s = steady; s < nstage; ++s, ++q) {
    const int k0 = kind(s), k1 = kind(s + 1), k2 = kind(s + 2);
    const bool ma = s + 2 < nstage;   // codes are never loaded here (s + 3 >= nstage)
    if (k0 == 2) {
      run_stage(q, m0, n0, s + 2, n0, s + 3, IC2{}, IC0{}, IC0{}, NO{}, NO{});
    } else if (k1 == 0) {
      run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC0{}, IC0{}, NO{}, NO{});
    } else if (k1 == 2) {
      run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC2{}, IC0{}, NO{}, NO{});
    } else if (k2 == 0) {
      run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC4{}, IC0{}, NO{}, NO{});
    } else if (k2 == 2) {
      if (ma) run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC4{}, IC2{}, NO{}, YES{});
      else run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC4{}, IC2{}, NO{}, NO{});
    } else {
      if (ma) run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC4{}, IC4{}, NO{}, YES{});
      else run_stage(q, m0, n0, s + 2, n0, s + 3, IC4{}, IC4{}, IC4{}, NO{}, NO{});
    }
  }
  finish_tile(tc);
}

// Staged weights: the codes of one weight matrix dequantized once into a bf16 matrix
// W16[N, K] (K contiguous) that the INT4S / FP4S GEMMs load like activations.  INT4:
// the exact integer q - z (group step applied in the GEMM); FP4: the exact product
// e2m1(code) * e4m3(block scale).  One thread converts 16 codes (8 bytes in, 32 out)
// of a range of `rows` rows with rows * K / 16 <= 2^30 (the launcher splits larger
// matrices), so the thread's row and chunk come from 32-bit arithmetic.
template <bool FP4>
__global__ __launch_bounds__(256) void stage_weights_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ aux, int rows, int K,
                                                            int gshift, uint16_t* __restrict__ W16) {
  const uint32_t cpr = (uint32_t)K >> 4;                        // 16-code chunks per row
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= (uint32_t)rows * cpr) return;
  const uint32_t n = idx / cpr, c = idx - n * cpr;
  const uint2 wv = *reinterpret_cast<const uint2*>(codes + (size_t)n * (uint32_t)(K >> 1) + c * 8u);
  const uint32_t w[2] = {wv.x, wv.y};
  uint32_t o[8];
  if constexpr (!FP4) {
    const float z = (float)aux[(size_t)n * (uint32_t)(K >> gshift) + ((c << 4) >> gshift)];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t lo = w[u] & 0x0F0F0F0Fu, hi = (w[u] >> 4) & 0x0F0F0F0Fu;
      asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        o[4 * u + b] = pack_bf16_exact((float)((lo >> (8 * b)) & 0xFFu) - z, (float)((hi >> (8 * b)) & 0xFFu) - z);
    }
  } else {
    const float sc = __builtin_amdgcn_cvt_f32_fp8((int)aux[(size_t)n * (uint32_t)(K >> 4) + c], 0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t e2;
        switch (b) {
          case 0: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 0)); break;
          case 1: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 1)); break;
          case 2: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 2)); break;
          default: e2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], 1.0f, 3)); break;
        }
        o[4 * u + b] = pack_bf16_exact(bf16_lo(e2) * sc, bf16_hi(e2) * sc);
      }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(W16 + (size_t)n * (uint32_t)K + c * 16u);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

// 8-bit codes: the exact integer q - z (|q - z| <= 255 has at most 8 significant
// bits, exact in bf16); one thread converts 16 code bytes (16 in, 32 out), 32-bit
// indexing over a row range as above.
__global__ __launch_bounds__(256) void stage_weights8_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ zeros, int rows, int K,
                                                             int gshift, uint16_t* __restrict__ W16) {
  const uint32_t cpr = (uint32_t)K >> 4;
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= (uint32_t)rows * cpr) return;
  const uint32_t n = idx / cpr, c = idx - n * cpr;
  const u32x4 w = *reinterpret_cast<const u32x4*>(codes + (size_t)n * (uint32_t)K + c * 16u);
  const float z = (float)zeros[(size_t)n * (uint32_t)(K >> gshift) + ((c << 4) >> gshift)];
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = pack_bf16_exact(ubyte_f32<0>(w[i]) - z, ubyte_f32<1>(w[i]) - z);
    o[2 * i + 1] =
        pack_bf16_exact(ubyte_f32<2>(w[i]) - z, ubyte_f32<3>(w[i]) - z);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(W16 + (size_t)n * (uint32_t)K + c * 16u);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

int log2_group(int G) { return G == 16 ? 4 : G == 32 ? 5 : G == 64 ? 6 : 7; }

// The staging kernels over row ranges of at most 2^30 chunks (32-bit indexing).
// FP4 passes G = 16 (one block scale per 16 codes).
template <bool FP4>
hipError_t stage_weights(const uint8_t* codes, const uint8_t* aux, int N, int K, int G, uint16_t* W16,
                         hipStream_t stream) {
  const int gshift = log2_group(G);
  const int64_t cpr = K >> 4;
  const int64_t max_rows = cpr > 0 ? std::max<int64_t>(1, (int64_t(1) << 30) / cpr) : N;
  for (int64_t n0 = 0; n0 < N; n0 += max_rows) {
    const int rows = (int)std::min<int64_t>(max_rows, N - n0);
    const int64_t chunks = rows * cpr;
    hipLaunchKernelGGL((stage_weights_kernel<FP4>), dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                       codes + n0 * (K >> 1), aux + n0 * (K >> gshift), rows, K, gshift, W16 + n0 * K);
  }
  return hipGetLastError();
}

int tiles(int M, int N, int bm) { return ((M + bm - 1) / bm) * ((N + BN - 1) / BN); }

// 256-row tiles (8 waves) once M fills them; 128-row tiles (4 waves) for small M.
constexpr int kWideM = 192;

// K slices for launches with few tiles (the q / k / v / o / down shapes at a few hundred
// rows leave most CUs idle otherwise, and a lone block runs ~1.1 us per 64-k stage on its
// load latency): at most kSplitMax slices, enough to bring the blocks to about
// kSplitTargetBlocks, each at least kSplitMinStages 64-k stages and a whole number of
// groups.  Measured on gfx950 (GEMM + fixed-order sum, us): [512, 2048, 2048] 35.6 unsplit,
// 19.2 / 18.4 / 19.8 with 4 / 6 / 8 slices; [512, 2048, 11008] 166 -> 43.9 / 43.0 with 6 / 8;
// [512, 256, 2048] 34.7 -> 13.6 with 8; splitting the 172 tiles of [512, 11008, 2048] is
// slower (41 -> 60).  Planned against the 256 CUs of an MI355X, so the workspace size is a
// function of the sizes alone.
constexpr int64_t kSplitMaxTiles = 128;
constexpr int64_t kSplitTargetBlocks = 192;
constexpr int64_t kSplitMax = 8;
constexpr int64_t kSplitMinStages = 4;

// Grid: one block per CU looping over the tiles (persistent) when every tile has at
// least four full stages, else one block per tile.
template <int BK, int G, bool TAIL>
hipError_t launch_tail(const GemmArgs& a, hipStream_t stream, int slices) {
  const bool wide = a.M > kWideM;
  const int nt = tiles(a.M, a.N, wide ? 256 : 128);
  const int grid = (!TAIL && a.K / KS >= 4) ? min(nt, device_cu_count()) : nt;
  if (wide) {
    hipLaunchKernelGGL((gemm_kernel<BK, G, TAIL, 4>), dim3(grid, slices), dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL((gemm_kernel<BK, G, TAIL, 2>), dim3(grid, slices), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

// slices > 1: K split into slices of a.kslice k along the grid's y (K % KS == 0)
template <int BK, int G>
hipError_t launch_tiles(GemmArgs a, hipStream_t stream, int slices = 1) {
  if (a.ld == 0) a.ld = a.K;
  if (a.K % KS) return launch_tail<BK, G, true>(a, stream, 1);
  return launch_tail<BK, G, false>(a, stream, slices);
}

// Y[i] = sum over s of P[s][i], s in order (deterministic); four outputs per thread,
// as 16-byte accesses when every slice and Y are 16-byte aligned (vec)
__global__ __launch_bounds__(256) void ksplit_sum_kernel(const float* __restrict__ P, int slices, int64_t count,
                                                          float* __restrict__ Y, bool vec) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= count) return;
  if (vec) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(P + i0);
    for (int sl = 1; sl < slices; ++sl) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(P + (int64_t)sl * count + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(Y + i0));
  } else {
    for (int64_t i = i0; i < min(count, i0 + 4); ++i) {
      float acc = P[i];
      for (int sl = 1; sl < slices; ++sl) acc += P[(int64_t)sl * count + i];
      Y[i] = acc;
    }
  }
}

}  // namespace

int gemm_k_slices(int64_t M, int64_t N, int64_t K, int group, int* kslice) {
  *kslice = (int)K;
  if (K <= 0 || K % KS || K % group || M <= 0 || N <= 0) return 1;
  const int64_t bm = M > kWideM ? 256 : 128;
  const int64_t nt = ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
  if (nt > kSplitMaxTiles) return 1;
  const int64_t stages = K / KS, unit = (group > KS ? group : KS) / KS;   // stages per slice granule
  int64_t sl = std::min<int64_t>({kSplitMax, (kSplitTargetBlocks + nt - 1) / nt, stages / kSplitMinStages});
  if (sl < 2) return 1;
  int64_t per = (stages + sl - 1) / sl;
  per = (per + unit - 1) / unit * unit;
  sl = (stages + per - 1) / per;
  if (sl < 2) return 1;
  *kslice = (int)(per * KS);
  return (int)sl;
}

hipError_t launch_w4a16_gemm(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                             const uint8_t* Z, int N, int group, float* Y, uint16_t* staged, float* partial,
                             hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.ld = K; a.P = P; a.S = S; a.Z = Z; a.Y = Y;
  int kslice = K;
  const int slices = partial ? gemm_k_slices(M, N, K, group, &kslice) : 1;
  if (slices > 1) {
    a.Y = partial;
    a.kslice = kslice;
    a.ystride = (int64_t)M * N;
  }
  hipError_t e = hipSuccess;
  if (staged) {
    e = stage_weights<false>(P, Z, N, K, group, staged, stream);
    if (e != hipSuccess) return e;
    a.B = staged;
    switch (group) {
      case 32: e = launch_tiles<B_INT4S, 32>(a, stream, slices); break;
      case 64: e = launch_tiles<B_INT4S, 64>(a, stream, slices); break;
      case 128: e = launch_tiles<B_INT4S, 128>(a, stream, slices); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (group) {
      case 32: e = launch_tiles<B_INT4, 32>(a, stream, slices); break;
      case 64: e = launch_tiles<B_INT4, 64>(a, stream, slices); break;
      case 128: e = launch_tiles<B_INT4, 128>(a, stream, slices); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess || slices == 1) return e;
  const int64_t count = (int64_t)M * N;
  const bool vec = (count & 3) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(partial) & 15) == 0;
  hipLaunchKernelGGL(ksplit_sum_kernel, dim3((unsigned)((count + 1023) / 1024)), dim3(256), 0, stream, partial,
                     slices, count, Y, vec);
  return hipGetLastError();
}

hipError_t launch_w8a16_gemm(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z,
                             int N, int group, float* Y, uint16_t* staged, hipStream_t stream) {
  // always staged: the 8-bit codes are dequantized once into the bf16 matrix, then
  // the staged INT4 GEMM (same per-group step rescale) runs on it
  const int gshift = log2_group(group);
  const int64_t cpr = K >> 4;
  const int64_t max_rows = cpr > 0 ? std::max<int64_t>(1, (int64_t(1) << 30) / cpr) : N;
  for (int64_t n0 = 0; n0 < N; n0 += max_rows) {   // row ranges of at most 2^30 chunks (32-bit indexing)
    const int rows = (int)std::min<int64_t>(max_rows, N - n0);
    const int64_t chunks = rows * cpr;
    hipLaunchKernelGGL(stage_weights8_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                       C + n0 * K, Z + n0 * (K >> gshift), rows, K, gshift, staged + n0 * K);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.S = S; a.Y = Y; a.B = staged;
  switch (group) {
    case 32: return launch_tiles<B_INT4S, 32>(a, stream);
    case 64: return launch_tiles<B_INT4S, 64>(a, stream);
    case 128: return launch_tiles<B_INT4S, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fp4_gemm(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale,
                           float ts, int N, float* Y, uint16_t* staged, hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.codes = codes; a.bscale = bscale; a.ts = ts; a.Y = Y;
  if (staged) {
    hipError_t e = stage_weights<true>(codes, bscale, N, K, 16, staged, stream);
    if (e != hipSuccess) return e;
    a.B = staged;
    return launch_tiles<B_FP4S, 64>(a, stream);
  }
  return launch_tiles<B_FP4, 64>(a, stream);
}

// SPLIT tiles (64-bit: the caller bounds the count before launching)
int64_t sumsq_gemm_blocks(int64_t M, int64_t N) {
  const int64_t bm = M > kWideM ? 256 : 128;
  return ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
}

hipError_t launch_sumsq_gemm(const uint16_t* X, int M, int K, const uint16_t* E, int N, double* partial,
                             hipStream_t stream) {
  GemmArgs a = {};
  a.X = X; a.M = M; a.N = N; a.K = K; a.B = E; a.B2 = E + (size_t)N * K; a.partial = partial;
  return launch_tiles<B_SPLIT, 64>(a, stream);
}

hipError_t launch_gram_gemm(const uint16_t* E, int M, int K, const uint16_t* H, double* partial,
                            hipStream_t stream) {
  GemmArgs a = {};
  a.X = E; a.Elo = E + (size_t)M * K; a.M = M; a.N = K; a.K = K;
  a.B = H; a.B2 = H + (size_t)K * K; a.partial = partial;
  return launch_tiles<B_GRAM, 64>(a, stream);
}

hipError_t launch_bf16_gemm(const uint16_t* A, int M, int K, const uint16_t* Bm, int N, float* Y,
                            hipStream_t stream) {
  // the staged-weight kind with a unit output scale (multiplying by 1 is exact)
  GemmArgs a = {};
  a.X = A; a.M = M; a.N = N; a.K = K; a.B = Bm; a.ts = 1.0f; a.Y = Y;
  return launch_tiles<B_FP4S, 64>(a, stream);
}

}  // namespace aq

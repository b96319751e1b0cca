// Internal launch functions of libaq (host side).  Each enqueues its kernels on
// `stream` and returns the launch status; arguments are validated by the C ABI
// layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

// sym: the symmetric variant (S = max |v| / 7, codes q + 8, zero point 8)
hipError_t launch_quant_pack(const void* W, bool w_bf16, const float* chan_scale, uint8_t* packed, float* scales,
                             uint8_t* zeros, int64_t N, int64_t K, int group, bool sym, hipStream_t stream);
// E = (q - z) S * chan_rcp - W as two bf16 planes; chan_rcp[k] = fl32(1 / chan_scale[k])
hipError_t launch_quant_error(const void* W, bool w_bf16, const float* chan_scale, const float* chan_rcp, uint16_t* E,
                              int64_t N, int64_t K, int group, hipStream_t stream);
hipError_t launch_w4a16_gemv(const uint16_t* X, int M, int K, const uint8_t* P, const float* S, const uint8_t* Z,
                             int N, int group, float* Y, hipStream_t stream);
// the same products on the matrix cores, M <= 16 (used by the launch_*_gemv dispatchers
// from a few rows up); FP4 needs K % 64 == 0
// true where the LDS-staged matrix-core decode kernel serves a W4A16 product (K = 2048, N >= 8192, M >= 4)
bool w4a16_lds_decode(int M, int N, int K);
hipError_t launch_w4a16_gemv_mfma(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream);
hipError_t launch_w8a16_gemv_mfma(const uint16_t* X, int M, int K, const uint8_t* C, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream);
hipError_t launch_fp4_gemv_mfma(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale,
                                float ts, int N, float* Y, hipStream_t stream);
// the VALU kernels only (any M <= 16)
hipError_t launch_w8a16_gemv_valu(const uint16_t* X, int M, int K, const uint8_t* C, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream);
hipError_t launch_fp4_gemv_valu(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale,
                                float ts, int N, float* Y, hipStream_t stream);
// the VALU kernel only (any M <= 16)
hipError_t launch_w4a16_gemv_valu(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                                  const uint8_t* Z, int N, int group, float* Y, hipStream_t stream);
// `staged`: NULL for the fused kernel, else N * K bf16 of device memory that first
// receives the dequantized weights (the staged GEMM then loads them like activations)
// K slices of a W4A16 GEMM with few output tiles (1: none); *kslice = k per slice.  The
// split GEMM writes slices x M x N fp32 partials to `partial` and adds them in order.
int gemm_k_slices(int64_t M, int64_t N, int64_t K, int group, int* kslice);
hipError_t launch_w4a16_gemm(const uint16_t* X, int M, int K, const uint8_t* P, const float* S,
                             const uint8_t* Z, int N, int group, float* Y, uint16_t* staged, float* partial,
                             hipStream_t stream);
// 8-bit codes [N, K] (one byte per weight), S / z as the INT4 format
hipError_t launch_quant_pack8(const void* W, bool w_bf16, const float* chan_scale, uint8_t* codes, float* scales,
                              uint8_t* zeros, int64_t N, int64_t K, int group, hipStream_t stream);
hipError_t launch_w8a16_gemv(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z,
                             int N, int group, float* Y, hipStream_t stream);
// `staged`: N * K bf16 of device memory (always used)
hipError_t launch_w8a16_gemm(const uint16_t* X, int M, int K, const uint8_t* C, const float* S, const uint8_t* Z,
                             int N, int group, float* Y, uint16_t* staged, hipStream_t stream);
hipError_t launch_fp4_gemv(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale, float ts,
                           int N, float* Y, hipStream_t stream);
hipError_t launch_fp4_gemm(const uint16_t* X, int M, int K, const uint8_t* codes, const uint8_t* bscale, float ts,
                           int N, float* Y, uint16_t* staged, hipStream_t stream);
size_t fp4_quantize_workspace_bytes(int64_t N, int64_t K);
// ts: one fp32 on the device (written); partial: fp4_quantize_workspace_bytes of device memory
hipError_t launch_fp4_quantize(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* codes, uint8_t* bscale,
                               float* ts, float* partial, hipStream_t stream);
// compute units of the current device (cached per device)
int device_cu_count();
int64_t sumsq_gemm_blocks(int64_t M, int64_t N);
hipError_t launch_sumsq_gemm(const uint16_t* X, int M, int K, const uint16_t* E, int N, double* partial,
                             hipStream_t stream);
// Gram form of the search's error GEMM: E = the [2][M, K] error planes, H = the [2][K, K]
// bf16 planes of X^T X; partial[sumsq_gemm_blocks(M, K)] gets each tile's sum of
// (E_hi H)[m, j] (E_hi + 2 E_lo)[m, j]
hipError_t launch_gram_gemm(const uint16_t* E, int M, int K, const uint16_t* H, double* partial, hipStream_t stream);
// Y[M, N] = A[M, K] Bm[N, K]^T, bf16 operands (K contiguous, K % 32 == 0), fp32 output
hipError_t launch_bf16_gemm(const uint16_t* A, int M, int K, const uint16_t* Bm, int N, float* Y, hipStream_t stream);
// Xt[K, Tp] = X[T, K]^T with rows T .. Tp - 1 of X taken as zero (Tp % 64 == 0, K % 8 == 0)
hipError_t launch_transpose_pad(const uint16_t* X, int64_t T, int64_t K, int64_t Tp, uint16_t* Xt, hipStream_t stream);
// H[n] (fp32) -> planes[0][n] = bf16(H), planes[1][n] = bf16(H - planes[0]), n < count (count % 4 == 0)
hipError_t launch_split_planes(const float* H, int64_t count, uint16_t* planes, hipStream_t stream);
int absmean_row_slices(int64_t T, int64_t K);
// the allocation-free entry point's scratch: its size, and its device address on the
// current device (looked up once per device)
size_t absmean_scratch_bytes();
hipError_t absmean_scratch(double** ptr);
hipError_t launch_act_absmean(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, float* mean, int64_t count,
                              double* work, hipStream_t stream);
hipError_t launch_fold_norm(const void* w, bool w_bf16, const float* s, int K, float* out, hipStream_t stream);
hipError_t launch_search_select(const double* partial, int nblocks, int n_grid, double count, const float* sgrid,
                                int K, double* mse, int32_t* best, float* best_scale, hipStream_t stream);

}  // namespace aq

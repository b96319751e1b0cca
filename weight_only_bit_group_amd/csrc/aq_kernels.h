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
hipError_t launch_quant_error(const void* W, bool w_bf16, const float* chan_scale, uint16_t* E, int64_t N, int64_t K,
                              int group, hipStream_t stream);
hipError_t launch_w4a16_gemv(const uint16_t* X, int M, int K, const uint8_t* P, const float* S, const uint8_t* Z,
                             int N, int group, float* Y, hipStream_t stream);
// the same products on the matrix cores, M <= 16 (used by the launch_*_gemv dispatchers
// from a few rows up); FP4 needs K % 64 == 0
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
hipError_t launch_w4a16_gemm(const uint16_t* X, int M, int K, const uint8_t* P, const float* S, const uint8_t* Z,
                             int N, int group, float* Y, uint16_t* staged, hipStream_t stream);
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
int sumsq_gemm_blocks(int M, int N);
hipError_t launch_sumsq_gemm(const uint16_t* X, int M, int K, const uint16_t* E, int N, double* partial,
                             hipStream_t stream);
int absmean_row_slices(int64_t T, int64_t K);
hipError_t launch_act_absmean(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, float* mean, int64_t count,
                              double* work, hipStream_t stream);
hipError_t launch_search_select(const double* partial, int nblocks, int n_grid, double count, const float* sgrid,
                                int K, double* mse, int32_t* best, float* best_scale, hipStream_t stream);

}  // namespace aq

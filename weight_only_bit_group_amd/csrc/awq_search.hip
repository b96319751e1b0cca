// AWQ alpha-grid search: device-side reduction of the per-block sums of squares
// into the MSE of every candidate, the argmin, and the winning scale vector.
//
// The method ("Lance-Quant", zingnex.cn, grid-search / grouped packing section;
// "Quantization：模型量化", xingyuwang.me, section 7 AWQ): for each alpha the
// candidate channel scale s = mean|x|^alpha / sqrt(max * min) is applied to W,
// W * diag(s) is quantize-dequantized group-wise, and the output MSE of
// (X / s) Q(W s)^T against X W^T -- which equals X E^T with E = Q(W s) / s - W --
// scores the candidate.  The smallest MSE wins (ties to the smallest alpha) and
// W * diag(s_best) is packed.
#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

// One block per candidate: the per-tile sums of squares are added by 256 threads
// (each a fixed stride of tiles) and combined by a fixed-order tree, then divided by
// the number of outputs.
__global__ __launch_bounds__(256) void search_mse_kernel(const double* __restrict__ partial, int nblocks,
                                                         double count, double* __restrict__ mse) {
  __shared__ double sm[256];
  const int t = threadIdx.x;
  const double* p = partial + (int64_t)blockIdx.x * nblocks;
  double s = 0.0;
  for (int b = t; b < nblocks; b += 256) s += p[b];
  sm[t] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) sm[t] = sm[t] + sm[t + w];
    __syncthreads();
  }
  if (t == 0) mse[blockIdx.x] = sm[0] / count;
}

// Argmin (first minimum wins) and the winning scale vector.
__global__ __launch_bounds__(256) void search_pick_kernel(const double* __restrict__ mse, int n_grid,
                                                          const float* __restrict__ sgrid, int K,
                                                          int32_t* __restrict__ best, float* __restrict__ best_scale) {
  __shared__ int sbest;
  if (threadIdx.x == 0) {
    int bi = 0;
    for (int i = 1; i < n_grid; ++i)
      if (mse[i] < mse[bi]) bi = i;
    sbest = bi;
    best[0] = bi;
  }
  __syncthreads();
  const float* src = sgrid + (int64_t)sbest * K;
  for (int k = threadIdx.x; k < K; k += 256) best_scale[k] = src[k];
}

// The RMSNorm fold of the chosen channel scale: the norm's consumers hold
// Q(W diag(s)), so the norm's output is divided by s through its weight,
// w'_k = fl32(w_k / s_k), one IEEE fp32 division per channel ("Lance-Quant",
// grid-search / grouping section: the scale is folded into the preceding norm).
template <bool BF16>
__global__ __launch_bounds__(256) void fold_norm_kernel(const void* __restrict__ w, const float* __restrict__ s,
                                                        int K, float* __restrict__ out) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const float wk = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(w)[k]) : static_cast<const float*>(w)[k];
  out[k] = wk / s[k];
}

hipError_t launch_fold_norm(const void* w, bool w_bf16, const float* s, int K, float* out, hipStream_t stream) {
  const dim3 grid((unsigned)((K + 255) / 256));
  if (w_bf16) hipLaunchKernelGGL(fold_norm_kernel<true>, grid, dim3(256), 0, stream, w, s, K, out);
  else hipLaunchKernelGGL(fold_norm_kernel<false>, grid, dim3(256), 0, stream, w, s, K, out);
  return hipGetLastError();
}

// ---- Gram form of the search's MSE --------------------------------------------
// For T > K the numerator sum_{t,n} (X E^T)[t, n]^2 equals sum_n e_n H e_n^T with the
// K x K Gram matrix H = X^T X, formed once per search: K^2 N multiply-adds per
// candidate instead of T K N.  H comes from the bf16 GEMM on X^T (its products are
// exact, its sums fp32), split into two bf16 planes (about 16 significant bits) for
// the per-candidate GEMM.

// Xt[K, Tp] = X[T, K]^T, rows t >= T of X read as zero.  A block moves one 64 x 64
// tile through LDS: 16-byte loads along k, 16-byte stores along t.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t K,
                                                            int64_t Tp, uint16_t* __restrict__ Xt) {
  __shared__ uint16_t tile[64][72];
  const int64_t k0 = (int64_t)blockIdx.x * 64, t0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = threadIdx.x + 256 * h, r = u >> 3, c = u & 7;   // tile row r (t), unit c (8 k)
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t0 + r < T && k0 + 8 * c < K) v = *reinterpret_cast<const u32x4*>(X + (t0 + r) * K + k0 + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[r][8 * c + 2 * i] = (uint16_t)(v[i] & 0xFFFFu);
      tile[r][8 * c + 2 * i + 1] = (uint16_t)(v[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = threadIdx.x + 256 * h, r = u >> 3, c = u & 7;   // output row r (k), unit c (8 t)
    if (k0 + r >= K) continue;
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (uint32_t)tile[8 * c + 2 * i][r] | ((uint32_t)tile[8 * c + 2 * i + 1][r] << 16);
    *reinterpret_cast<u32x4*>(Xt + (k0 + r) * Tp + t0 + 8 * c) = v;
  }
}

hipError_t launch_transpose_pad(const uint16_t* X, int64_t T, int64_t K, int64_t Tp, uint16_t* Xt,
                                hipStream_t stream) {
  if (Tp % 64 || K % 8 || Tp < T) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((K + 63) / 64), (unsigned)(Tp / 64));
  hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, stream, X, T, K, Tp, Xt);
  return hipGetLastError();
}

// planes[0] = bf16(H) and planes[1] = bf16(H - planes[0]), both round to nearest even;
// four values per thread.
__global__ __launch_bounds__(256) void split_planes_kernel(const float* __restrict__ H, int64_t count,
                                                           uint16_t* __restrict__ planes) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  const f32x4 h = *reinterpret_cast<const f32x4*>(H + i);
  uint32_t hi[2], lo[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16x2 a = {(__bf16)h[2 * j], (__bf16)h[2 * j + 1]};
    hi[j] = __builtin_bit_cast(uint32_t, a);
    const bf16x2 b = {(__bf16)(h[2 * j] - bf16_lo(hi[j])), (__bf16)(h[2 * j + 1] - bf16_hi(hi[j]))};
    lo[j] = __builtin_bit_cast(uint32_t, b);
  }
  *reinterpret_cast<uint2*>(planes + i) = uint2{hi[0], hi[1]};
  *reinterpret_cast<uint2*>(planes + count + i) = uint2{lo[0], lo[1]};
}

hipError_t launch_split_planes(const float* H, int64_t count, uint16_t* planes, hipStream_t stream) {
  if (count % 4) return hipErrorInvalidValue;
  const int64_t threads = count / 4;
  hipLaunchKernelGGL(split_planes_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, H, count,
                     planes);
  return hipGetLastError();
}

hipError_t launch_search_select(const double* partial, int nblocks, int n_grid, double count, const float* sgrid,
                                int K, double* mse, int32_t* best, float* best_scale, hipStream_t stream) {
  hipLaunchKernelGGL(search_mse_kernel, dim3(n_grid), dim3(256), 0, stream, partial, nblocks, count, mse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(search_pick_kernel, dim3(1), dim3(256), 0, stream, mse, n_grid, sgrid, K, best, best_scale);
  return hipGetLastError();
}

}  // namespace aq

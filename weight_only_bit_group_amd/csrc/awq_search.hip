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

hipError_t launch_search_select(const double* partial, int nblocks, int n_grid, double count, const float* sgrid,
                                int K, double* mse, int32_t* best, float* best_scale, hipStream_t stream) {
  hipLaunchKernelGGL(search_mse_kernel, dim3(n_grid), dim3(256), 0, stream, partial, nblocks, count, mse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(search_pick_kernel, dim3(1), dim3(256), 0, stream, mse, n_grid, sgrid, K, best, best_scale);
  return hipGetLastError();
}

}  // namespace aq

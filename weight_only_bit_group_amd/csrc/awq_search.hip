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

__global__ __launch_bounds__(64) void search_select_kernel(const double* __restrict__ partial, int nblocks, int n_grid,
                                                           double count, const float* __restrict__ sgrid, int K,
                                                           double* __restrict__ mse, int32_t* __restrict__ best,
                                                           float* __restrict__ best_scale) {
  __shared__ double sm[64];
  __shared__ int sbest;
  const int t = threadIdx.x;
  if (t < n_grid) {
    double s = 0.0;
    const double* p = partial + (int64_t)t * nblocks;
    for (int b = 0; b < nblocks; ++b) s += p[b];
    s = s / count;
    sm[t] = s;
    mse[t] = s;
  }
  __syncthreads();
  if (t == 0) {
    int bi = 0;
    for (int i = 1; i < n_grid; ++i)
      if (sm[i] < sm[bi]) bi = i;  // strict: the first minimum wins
    sbest = bi;
    best[0] = bi;
  }
  __syncthreads();
  const float* src = sgrid + (int64_t)sbest * K;
  for (int k = t; k < K; k += 64) best_scale[k] = src[k];
}

hipError_t launch_search_select(const double* partial, int nblocks, int n_grid, double count, const float* sgrid,
                                int K, double* mse, int32_t* best, float* best_scale, hipStream_t stream) {
  hipLaunchKernelGGL(search_select_kernel, dim3(1), dim3(64), 0, stream, partial, nblocks, n_grid, count, sgrid, K,
                     mse, best, best_scale);
  return hipGetLastError();
}

}  // namespace aq

// Per-input-channel sum and mean of |x| (the AWQ calibration statistic), gfx950.
//
// What it computes ("Lance-Quant", zingnex.cn, calibration section: hooks on the
// target linears keep each input channel's average absolute activation, and
// statistics of several runs are merged): sum_abs[k] += sum_t |X[t, k]| in fp64,
// and optionally mean[k] = fl32(sum_abs[k] / count).
//
// Design (HBM-bound): the grid is (K / 512 column slices) x (T row slices).  A
// lane owns 8 consecutive channels (one 16-byte load per row) and the wave's 64
// lanes cover a contiguous 1 KiB of each row; the 4 waves of a block stride over
// the block's rows.  Every |x| (bf16, 8 significant bits) is added in fp64, so
// the partial sums are exact unless a value is ~2^45 times smaller than its
// channel's total.  Partials go to a workspace [row slices][K] (about 1024 blocks
// in all) and a second kernel adds them in a fixed order, so the result is
// deterministic.
#include <mutex>

#include "aq_device.h"
#include "aq_kernels.h"

namespace aq {

// Scratch of the allocation-free entry point: the fp64 partial sums [row slices][K],
// a file-scope device array (one copy per GPU, held until the process ends).  Host
// code never passes the array's name to a kernel (on the host it is only a stand-in
// symbol): its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and cached.
constexpr size_t kScratchDoubles = size_t(1) << 20;   // 8 MiB
static __device__ __align__(256) double scratch[kScratchDoubles];

size_t absmean_scratch_bytes() { return kScratchDoubles * sizeof(double); }

hipError_t absmean_scratch(double** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static double* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<double*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

constexpr int kColsPerBlock = 512;

int absmean_row_slices(int64_t T, int64_t K) {
  const int64_t kx = (K + kColsPerBlock - 1) / kColsPerBlock;
  int64_t ts = (T + 127) / 128;                 // at least 128 rows (32 per wave) per block
  const int64_t target = (1024 + kx - 1) / kx;  // about 1024 blocks in total
  if (ts > target) ts = target;
  if (ts < 1) ts = 1;
  return (int)ts;
}

__global__ __launch_bounds__(256) void absmean_partial_kernel(const uint16_t* __restrict__ X, int64_t T, int K,
                                                              int64_t rows_per_slice, double* __restrict__ part) {
  __shared__ double sm[4][kColsPerBlock];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int col0 = blockIdx.x * kColsPerBlock + lane * 8;
  const bool live = col0 < K;
  const int64_t t0 = (int64_t)blockIdx.y * rows_per_slice;
  const int64_t t1 = min(T, t0 + rows_per_slice);
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  if (live) {
    const uint16_t* base = X + col0;
    int64_t t = t0 + wid;
    for (; t + 28 < t1; t += 32) {
      u32x4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = *reinterpret_cast<const u32x4*>(base + (t + 4 * u) * (int64_t)K);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += (double)fabsf(bf16_lo(w[u][i]));
          acc[2 * i + 1] += (double)fabsf(bf16_hi(w[u][i]));
        }
    }
    for (; t < t1; t += 4) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + t * (int64_t)K);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += (double)fabsf(bf16_lo(w[i]));
        acc[2 * i + 1] += (double)fabsf(bf16_hi(w[i]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sm[wid][lane * 8 + i] = acc[i];
  __syncthreads();
  for (int c = threadIdx.x; c < kColsPerBlock; c += 256) {
    const int col = blockIdx.x * kColsPerBlock + c;
    if (col < K) part[(int64_t)blockIdx.y * K + col] = ((sm[0][c] + sm[1][c]) + sm[2][c]) + sm[3][c];
  }
}

// Finish: 16 channels per block, 16 threads per channel each adding every 16th row
// slice (eight loads in flight per batch); the 16 partial sums are then combined in
// a fixed order (deterministic).
__global__ __launch_bounds__(256) void absmean_finish_kernel(const double* __restrict__ part, int slices, int K,
                                                             double* __restrict__ sum_abs, float* __restrict__ mean,
                                                             double count) {
  __shared__ double sm[16][17];
  const int c = threadIdx.x & 15, r = threadIdx.x >> 4;
  const int k = blockIdx.x * 16 + c;
  double s = 0.0;
  if (k < K) {
    int i = r;
    for (; i + 16 * 7 < slices; i += 16 * 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(i + 16 * u) * K + k];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; i < slices; i += 16) s += part[(int64_t)i * K + k];
  }
  sm[r][c] = s;
  __syncthreads();
  if (r == 0 && k < K) {
    double tot_chunk = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) tot_chunk += sm[j][c];
    const double tot = sum_abs[k] + tot_chunk;
    sum_abs[k] = tot;
    if (mean) mean[k] = (float)(tot / count);
  }
}

hipError_t launch_act_absmean(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, float* mean,
                              int64_t count, double* work, hipStream_t stream) {
  const int slices = absmean_row_slices(T, K);
  const int64_t rows = (T + slices - 1) / slices;
  const dim3 grid((unsigned)((K + kColsPerBlock - 1) / kColsPerBlock), (unsigned)slices);
  hipLaunchKernelGGL(absmean_partial_kernel, grid, dim3(256), 0, stream, X, T, (int)K, rows, work);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(absmean_finish_kernel, dim3((unsigned)((K + 15) / 16)), dim3(256), 0, stream, work, slices,
                     (int)K, sum_abs, mean, (double)count);
  return hipGetLastError();
}

}  // namespace aq

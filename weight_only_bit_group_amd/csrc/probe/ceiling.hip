// Ceiling microbenchmarks of the MI355X (gfx950) for the roofline fractions the
// benchmark reports next to the nameplate ones.  Not part of the library's C ABI
// (libaq.so); built into libaq_probe.so and loaded by the benchmark only.
//
//   aqp_empty        an empty kernel at a given grid: the launch / dispatch floor that
//                    every kernel duration contains
//   aqp_stream_read  a pure streaming read of `bytes` bytes (16-byte nontemporal loads,
//                    every lane's loads issued before any is used), at a given grid of
//                    256-thread blocks: the fastest a kernel that reads exactly those
//                    bytes once can be, at that launch shape
//   aqp_mfma_loop    back-to-back independent bf16 MFMAs (32x32x16 or 16x16x32) on every
//                    SIMD, no memory traffic: the sustained dense bf16 MFMA rate
//
// Every kernel keeps its results alive with a store that is taken only for a value
// the inputs cannot produce, so the loads and MFMAs are not removed and nothing is
// written in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__global__ void empty_kernel() {}

// Thread t reads units t, t + T, ..., t + (U - 1) T of this pass (T = threads in the
// grid), all requested before any is combined; passes repeat until `units` are read.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t units,
                                                          uint32_t* __restrict__ sink) {
  const int64_t T = (int64_t)gridDim.x * 256;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (int64_t base = t; base < units; base += T * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * T;
      v[u] = i < units ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u && t == 0x7FFFFFFF) sink[0] = acc;   // never taken for t < 2^31 - 1 threads
}

// NACC independent accumulators per wave, `iters` rounds of one MFMA into each.
template <bool BIG, int NACC>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((lane + i) & 7);
    b[i] = (__bf16)(float)((lane * 3 + i) & 7);
  }
  float tot = 0.0f;
  if constexpr (BIG) {
    f32x16 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NACC; ++j) tot += acc[j][0] + acc[j][15];
  } else {
    f32x4 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[j][v] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NACC; ++j) tot += acc[j][0] + acc[j][3];
  }
  if (tot == -1.0f) sink[threadIdx.x] = tot;   // the sums are non-negative
}

}  // namespace

extern "C" {

int aqp_empty(int blocks, int threads, void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

// src: at least `bytes` bytes (a multiple of 16) of device memory; sink: 4 bytes.
int aqp_stream_read(const void* src, int64_t bytes, int blocks, int unroll, uint32_t* sink, void* stream) {
  if (bytes <= 0 || bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
  const int64_t units = bytes / 16;
  const u32x4* p = static_cast<const u32x4*>(src);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, p, units, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, p, units, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, p, units, sink); break;
    case 5: hipLaunchKernelGGL(stream_read_kernel<5>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, p, units, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, p, units, sink); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// big: 32x32x16 (else 16x16x32); blocks of 256 threads (4 waves); sink: 256 floats.
int aqp_mfma_loop(int big, int blocks, int iters, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  if (big) hipLaunchKernelGGL((mfma_loop_kernel<true, 4>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  else hipLaunchKernelGGL((mfma_loop_kernel<false, 8>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}

}  // extern "C"

// C ABI of libaq: argument validation, status codes, workspace sizing, the
// host-side candidate scales of the AWQ search, and dispatch to the gfx950
// kernels.  Every check runs before the first launch, so a call that returns
// AQ_EINVAL has written nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <system_error>
#include <thread>
#include <vector>

#include "../../include/aq.h"
#include "aq_kernels.h"

namespace {

thread_local std::string g_last_error;

aq_status fail(aq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

aq_status ok() {
  g_last_error.clear();
  return AQ_OK;
}

// AQ_FAULT_INJECT=launch makes every entry point report a runtime failure after
// validation, without touching the GPU (exercises the AQ_ERUNTIME path).
bool fault_injected() {
  const char* v = std::getenv("AQ_FAULT_INJECT");
  return v && std::strcmp(v, "launch") == 0;
}

aq_status runtime_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(AQ_ERUNTIME, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define AQ_REQUIRE(cond, ...) \
  do {                        \
    if (!(cond)) return fail(AQ_EINVAL, __VA_ARGS__); \
  } while (0)

#define AQ_PTR(p, a, name)                                                          \
  do {                                                                              \
    if ((p) == nullptr) return fail(AQ_EINVAL, "%s must not be NULL", name);        \
    if (!aligned((p), (a))) return fail(AQ_EINVAL, "%s must be %d-byte aligned", name, (int)(a)); \
  } while (0)

constexpr int64_t kDimLimit = int64_t(1) << 30;
// MFMA GEMMs: 32-bit offsets within a block's rows (loads) and within its output
// tile (stores) need K < 2^22 and N < 2^22.
constexpr int64_t kGemmDimLimit = int64_t(1) << 22;
// Smallest M for which the staged GEMM path (weights dequantized once into a bf16
// staging matrix) is used when the caller provides the workspace.
constexpr int64_t kStagedMinM = 2048;

bool valid_group(int32_t g) { return g == 32 || g == 64 || g == 128; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct SearchLayout {
  size_t sgrid, rgrid, e, partial, xt, h, hp, total;
  int64_t tp;    // Gram form: token count padded to the GEMM's 64-wide stages
  int nblocks;   // error-GEMM tiles (one fp64 partial each, per candidate)
  bool gram;
};

// The MSE numerator sum (X E^T)^2 either directly (T K N multiply-adds per candidate)
// or as sum_n e_n H e_n^T with H = X^T X formed once (K K N per candidate): the Gram
// form when T > K, its padded token count within the GEMM limit.
bool use_gram(int64_t T, int64_t K) { return T > K && (int64_t)round_up((size_t)T, 64) < kGemmDimLimit; }

// The error GEMM takes T (direct) or N (Gram) as its M: T, N and K below 2^22 keep its
// 32-bit load / store offsets and its tile count (below 2^29) in range.
bool search_dims_ok(int64_t T, int64_t N, int64_t K) {
  if (!(T > 0 && N > 0 && K > 0 && T < kGemmDimLimit && N < kGemmDimLimit && K < kGemmDimLimit)) return false;
  return use_gram(T, K) ? aq::sumsq_gemm_blocks(N, K) < (int64_t(1) << 30)
                        : aq::sumsq_gemm_blocks(T, N) < (int64_t(1) << 30);
}

SearchLayout search_layout(int64_t T, int64_t N, int64_t K, int32_t n_grid) {
  SearchLayout L;
  L.gram = use_gram(T, K);
  L.tp = (int64_t)round_up((size_t)T, 64);
  L.nblocks = (int)(L.gram ? aq::sumsq_gemm_blocks(N, K) : aq::sumsq_gemm_blocks(T, N));
  L.sgrid = 0;
  L.rgrid = round_up((size_t)n_grid * (size_t)K * sizeof(float), 256);   // fl32(1 / s), right after s
  L.e = L.rgrid + round_up((size_t)n_grid * (size_t)K * sizeof(float), 256);
  L.partial = L.e + round_up((size_t)N * (size_t)K * 2 * 2, 256);   // E_hi and E_lo planes
  L.xt = round_up(L.partial + (size_t)n_grid * (size_t)L.nblocks * sizeof(double), 256);
  if (L.gram) {
    L.h = L.xt + round_up((size_t)K * (size_t)L.tp * 2, 256);        // X^T, bf16 [K, tp]
    L.hp = L.h + round_up((size_t)K * (size_t)K * sizeof(float), 256);  // H fp32 [K, K]
    L.total = L.hp + (size_t)K * (size_t)K * 2 * 2;                  // H_hi, H_lo planes
  } else {
    L.h = L.hp = L.total = L.xt;
  }
  return L;
}

// Candidate scales of alphas i = 0 .. n_grid - 1 (alpha = i / n_grid), fp64 libm:
// t = max(m, 1e-8)^alpha, s = fl32(t / sqrt(max t * min t)); out[i K + k] = s and
// out[(n_grid + i) K + k] = fl32(1 / s).  The alphas are shared among up to eight
// threads (each value comes from the same libm calls whichever thread computes it).
void candidate_grid(const float* absmean, int64_t K, int32_t n_grid, float* out) {
  std::atomic<int32_t> next{0};
  auto work = [&]() {
    std::vector<double> t((size_t)K);
    for (int32_t i = next.fetch_add(1); i < n_grid; i = next.fetch_add(1)) {
      const double alpha = (double)i / (double)n_grid;
      double tmax = -INFINITY, tmin = INFINITY;
      for (int64_t k = 0; k < K; ++k) {
        double m = (double)absmean[k];
        if (m < 1e-8) m = 1e-8;
        t[k] = std::pow(m, alpha);
        tmax = std::max(tmax, t[k]);
        tmin = std::min(tmin, t[k]);
      }
      const double den = std::sqrt(tmax * tmin);
      for (int64_t k = 0; k < K; ++k) {
        const float sk = (float)(t[k] / den);
        out[(size_t)i * K + k] = sk;
        out[((size_t)n_grid + i) * K + k] = (float)(1.0 / (double)sk);
      }
    }
  };
  const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  const int nth = (int)std::min<unsigned>({8u, hw, (unsigned)n_grid});
  std::vector<std::thread> pool;
  for (int j = 1; j < nth; ++j) {
    try {
      pool.emplace_back(work);
    } catch (const std::system_error&) {
      break;   // fewer helpers: the calling thread takes the remaining alphas
    }
  }
  work();
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

const char* aq_last_error(void) { return g_last_error.c_str(); }

static aq_status quantize_pack_common(const char* fn, int mode, const void* W, int32_t w_dtype, int64_t N,
                                      int64_t K, int32_t group, const float* chan_scale, uint8_t* packed,
                                      float* scales, uint8_t* zeros, void* stream) {
  AQ_REQUIRE(w_dtype == AQ_F32 || w_dtype == AQ_BF16, "%s: w_dtype must be AQ_F32 or AQ_BF16 (got %d)", fn, w_dtype);
  AQ_REQUIRE(valid_group(group), "%s: group must be 32, 64 or 128 (got %d)", fn, group);
  AQ_REQUIRE(N >= 0 && N < kDimLimit, "%s: N out of range (%lld)", fn, (long long)N);
  AQ_REQUIRE(K > 0 && K < kDimLimit, "%s: K out of range (%lld)", fn, (long long)K);
  AQ_REQUIRE(K % group == 0, "%s: K (%lld) must be a multiple of group (%d)", fn, (long long)K, group);
  AQ_PTR(W, 16, "W");
  if (chan_scale) AQ_REQUIRE(aligned(chan_scale, 16), "%s: chan_scale must be 16-byte aligned", fn);
  AQ_PTR(packed, 16, "packed");
  AQ_PTR(scales, 4, "scales");
  AQ_PTR(zeros, 1, "zeros");
  if (fault_injected()) return fail(AQ_ERUNTIME, "%s: injected launch failure", fn);
  if (N == 0) return ok();
  const bool bf16 = w_dtype == AQ_BF16;
  const hipError_t e =
      mode == 2 ? aq::launch_quant_pack8(W, bf16, chan_scale, packed, scales, zeros, N, K, group, (hipStream_t)stream)
                : aq::launch_quant_pack(W, bf16, chan_scale, packed, scales, zeros, N, K, group, mode == 1,
                                        (hipStream_t)stream);
  return runtime_status(e, fn);
}

aq_status aq_quantize_pack(const void* W, int32_t w_dtype, int64_t N, int64_t K, int32_t group,
                           const float* chan_scale, uint8_t* packed, float* scales, uint8_t* zeros,
                           void* stream) {
  return quantize_pack_common("aq_quantize_pack", 0, W, w_dtype, N, K, group, chan_scale, packed, scales, zeros,
                              stream);
}

aq_status aq_quantize_pack_sym(const void* W, int32_t w_dtype, int64_t N, int64_t K, int32_t group,
                               const float* chan_scale, uint8_t* packed, float* scales, uint8_t* zeros,
                               void* stream) {
  return quantize_pack_common("aq_quantize_pack_sym", 1, W, w_dtype, N, K, group, chan_scale, packed, scales,
                              zeros, stream);
}

aq_status aq_quantize_pack8(const void* W, int32_t w_dtype, int64_t N, int64_t K, int32_t group,
                            const float* chan_scale, uint8_t* codes, float* scales, uint8_t* zeros, void* stream) {
  return quantize_pack_common("aq_quantize_pack8", 2, W, w_dtype, N, K, group, chan_scale, codes, scales, zeros,
                              stream);
}

size_t aq_fp4_quantize_workspace(int64_t N, int64_t K) {
  if (N < 0 || K <= 0 || K % 16 || N >= kDimLimit || K >= kDimLimit) return 0;
  return aq::fp4_quantize_workspace_bytes(N, K);
}

aq_status aq_fp4_quantize(const void* W, int32_t w_dtype, int64_t N, int64_t K, uint8_t* codes,
                          uint8_t* block_scales, float* tensor_scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
  AQ_REQUIRE(w_dtype == AQ_F32 || w_dtype == AQ_BF16, "aq_fp4_quantize: w_dtype must be AQ_F32 or AQ_BF16 (got %d)",
             w_dtype);
  AQ_REQUIRE(N >= 0 && N < kDimLimit, "aq_fp4_quantize: N out of range (%lld)", (long long)N);
  AQ_REQUIRE(K > 0 && K < kDimLimit && K % 16 == 0, "aq_fp4_quantize: K must be a positive multiple of 16 (got %lld)",
             (long long)K);
  AQ_PTR(W, 16, "W");
  AQ_PTR(codes, 8, "codes");
  AQ_PTR(block_scales, 1, "block_scales");
  AQ_PTR(tensor_scale, 4, "tensor_scale");
  AQ_PTR(workspace, 4, "workspace");
  AQ_REQUIRE(workspace_bytes >= aq_fp4_quantize_workspace(N, K),
             "aq_fp4_quantize: workspace too small (%zu < %zu bytes)", workspace_bytes,
             aq_fp4_quantize_workspace(N, K));
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_fp4_quantize: injected launch failure");
  return runtime_status(aq::launch_fp4_quantize(W, w_dtype == AQ_BF16, N, K, codes, block_scales, tensor_scale,
                                                static_cast<float*>(workspace), (hipStream_t)stream),
                        "aq_fp4_quantize");
}

static aq_status check_product(const char* fn, const uint16_t* X, int64_t M, int64_t K, const uint8_t* packed,
                               const float* scales, const uint8_t* zeros, int64_t N, int32_t group, float* Y) {
  AQ_REQUIRE(valid_group(group), "%s: group must be 32, 64 or 128 (got %d)", fn, group);
  AQ_REQUIRE(K > 0 && K < kDimLimit, "%s: K out of range (%lld)", fn, (long long)K);
  AQ_REQUIRE(K % group == 0, "%s: K (%lld) must be a multiple of group (%d)", fn, (long long)K, group);
  AQ_REQUIRE(N >= 0 && N < kDimLimit, "%s: N out of range (%lld)", fn, (long long)N);
  AQ_PTR(X, 16, "X");
  AQ_PTR(packed, 16, "packed");
  AQ_PTR(scales, 4, "scales");
  AQ_PTR(zeros, 1, "zeros");
  AQ_PTR(Y, 4, "Y");
  (void)M;
  return AQ_OK;
}

aq_status aq_w4a16_gemv(const uint16_t* X, int64_t M, int64_t K, const uint8_t* packed, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* stream) {
  AQ_REQUIRE(M >= 1 && M <= 16, "aq_w4a16_gemv: M must be in 1..16 (got %lld)", (long long)M);
  aq_status st = check_product("aq_w4a16_gemv", X, M, K, packed, scales, zeros, N, group, Y);
  if (st != AQ_OK) return st;
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_w4a16_gemv: injected launch failure");
  if (N == 0) return ok();
  return runtime_status(aq::launch_w4a16_gemv(X, (int)M, (int)K, packed, scales, zeros, (int)N, group, Y,
                                              (hipStream_t)stream),
                        "aq_w4a16_gemv");
}

// Bytes of the bf16 staging matrix the MFMA GEMMs use at this size (0: fused path).
static size_t staged_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < kStagedMinM || N <= 0 || K <= 0 || N >= kGemmDimLimit || K >= kGemmDimLimit) return 0;
  return (size_t)N * (size_t)K * sizeof(uint16_t);
}

// The staging matrix when the caller's workspace holds it, else NULL (fused path).
static aq_status staging(const char* fn, int64_t M, int64_t N, int64_t K, void* workspace, size_t bytes,
                         uint16_t** out) {
  *out = nullptr;
  const size_t need = staged_bytes(M, N, K);
  if (workspace == nullptr || need == 0 || bytes < need) return AQ_OK;
  AQ_REQUIRE(aligned(workspace, 256), "%s: workspace must be 256-byte aligned", fn);
  *out = static_cast<uint16_t*>(workspace);
  return AQ_OK;
}

aq_status aq_w8a16_gemv(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* stream) {
  AQ_REQUIRE(M >= 1 && M <= 16, "aq_w8a16_gemv: M must be in 1..16 (got %lld)", (long long)M);
  aq_status st = check_product("aq_w8a16_gemv", X, M, K, codes, scales, zeros, N, group, Y);
  if (st != AQ_OK) return st;
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_w8a16_gemv: injected launch failure");
  if (N == 0) return ok();
  return runtime_status(aq::launch_w8a16_gemv(X, (int)M, (int)K, codes, scales, zeros, (int)N, group, Y,
                                              (hipStream_t)stream),
                        "aq_w8a16_gemv");
}

size_t aq_w8a16_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (!valid_group(group) || M < 0 || N <= 0 || K <= 0 || K % group || N >= kGemmDimLimit || K >= kGemmDimLimit)
    return 0;
  return (size_t)N * (size_t)K * sizeof(uint16_t);
}

aq_status aq_w8a16_gemm(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  AQ_REQUIRE(M >= 0 && M < kDimLimit, "aq_w8a16_gemm: M out of range (%lld)", (long long)M);
  aq_status st = check_product("aq_w8a16_gemm", X, M, K, codes, scales, zeros, N, group, Y);
  if (st != AQ_OK) return st;
  AQ_REQUIRE(K < kGemmDimLimit && N < kGemmDimLimit, "aq_w8a16_gemm: K and N must be below 2^22 (got %lld, %lld)",
             (long long)K, (long long)N);
  AQ_PTR(workspace, 256, "workspace");
  AQ_REQUIRE(workspace_bytes >= (size_t)N * (size_t)K * sizeof(uint16_t),
             "aq_w8a16_gemm: workspace too small (%zu < %zu bytes)", workspace_bytes,
             (size_t)N * (size_t)K * sizeof(uint16_t));
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_w8a16_gemm: injected launch failure");
  if (N == 0 || M == 0) return ok();
  return runtime_status(aq::launch_w8a16_gemm(X, (int)M, (int)K, codes, scales, zeros, (int)N, group, Y,
                                              static_cast<uint16_t*>(workspace), (hipStream_t)stream),
                        "aq_w8a16_gemm");
}

// The W4A16 GEMM's workspace: the staging matrix (large M), then the K-slice partials
// (launches with few output tiles), 256-byte aligned.
struct GemmWorkspace {
  size_t staged, partial, total;
};

static GemmWorkspace gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t group) {
  GemmWorkspace w = {0, 0, 0};
  if (!valid_group(group) || K <= 0 || K % group || M <= 0 || N <= 0 || K >= kGemmDimLimit || N >= kGemmDimLimit)
    return w;
  w.staged = staged_bytes(M, N, K);
  int kslice = 0;
  const int slices = aq::gemm_k_slices(M, N, K, group, &kslice);
  if (slices > 1) w.partial = (size_t)slices * (size_t)M * (size_t)N * sizeof(float);
  w.total = (w.partial ? round_up(w.staged, 256) : w.staged) + w.partial;
  return w;
}

size_t aq_w4a16_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t group) {
  return gemm_workspace(M, N, K, group).total;
}

aq_status aq_w4a16_gemm(const uint16_t* X, int64_t M, int64_t K, const uint8_t* packed, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  AQ_REQUIRE(M >= 0 && M < kDimLimit, "aq_w4a16_gemm: M out of range (%lld)", (long long)M);
  aq_status st = check_product("aq_w4a16_gemm", X, M, K, packed, scales, zeros, N, group, Y);
  if (st != AQ_OK) return st;
  AQ_REQUIRE(K < kGemmDimLimit && N < kGemmDimLimit, "aq_w4a16_gemm: K and N must be below 2^22 (got %lld, %lld)",
             (long long)K, (long long)N);
  // the whole plan when the workspace holds it; else the staging matrix alone when it
  // fits; else the fused path without K slices (workspace untouched)
  uint16_t* staged = nullptr;
  float* partial = nullptr;
  const GemmWorkspace w = gemm_workspace(M, N, K, group);
  if (workspace != nullptr && w.total > 0 && workspace_bytes >= w.total) {
    AQ_REQUIRE(aligned(workspace, 256), "aq_w4a16_gemm: workspace must be 256-byte aligned");
    char* base = static_cast<char*>(workspace);
    if (w.staged) staged = reinterpret_cast<uint16_t*>(base);
    if (w.partial) partial = reinterpret_cast<float*>(base + round_up(w.staged, 256));
  } else {
    st = staging("aq_w4a16_gemm", M, N, K, workspace, workspace_bytes, &staged);
    if (st != AQ_OK) return st;
  }
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_w4a16_gemm: injected launch failure");
  if (N == 0 || M == 0) return ok();
  return runtime_status(aq::launch_w4a16_gemm(X, (int)M, (int)K, packed, scales, zeros, (int)N, group, Y, staged,
                                              partial, (hipStream_t)stream),
                        "aq_w4a16_gemm");
}

size_t aq_act_absmean_workspace(int64_t T, int64_t K) {
  if (T <= 0 || K <= 0) return 0;
  return (size_t)aq::absmean_row_slices(T, K) * (size_t)K * sizeof(double);
}

aq_status aq_act_absmean(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, float* mean_out,
                         int64_t total_count, void* workspace, size_t workspace_bytes, void* stream) {
  AQ_REQUIRE(T > 0, "aq_act_absmean: empty calibration data (T = %lld)", (long long)T);
  AQ_REQUIRE(T < (int64_t(1) << 40), "aq_act_absmean: T out of range");
  AQ_REQUIRE(K > 0 && K < kDimLimit && K % 8 == 0, "aq_act_absmean: K must be a positive multiple of 8 (got %lld)",
             (long long)K);
  AQ_REQUIRE(total_count >= T, "aq_act_absmean: total_count (%lld) must include this chunk's T (%lld)",
             (long long)total_count, (long long)T);
  AQ_PTR(X, 16, "X");
  AQ_PTR(sum_abs, 8, "sum_abs");
  if (mean_out) AQ_REQUIRE(aligned(mean_out, 4), "mean_out must be 4-byte aligned");
  AQ_PTR(workspace, 16, "workspace");
  const size_t need = aq_act_absmean_workspace(T, K);
  AQ_REQUIRE(workspace_bytes >= need, "aq_act_absmean: workspace too small (%zu < %zu bytes)", workspace_bytes, need);
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_act_absmean: injected launch failure");
  return runtime_status(aq::launch_act_absmean(X, T, K, sum_abs, mean_out, total_count,
                                               static_cast<double*>(workspace), (hipStream_t)stream),
                        "aq_act_absmean");
}

aq_status aq_act_absmean_noalloc(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, float* mean_out,
                                 int64_t total_count, void* stream) {
  AQ_REQUIRE(T > 0, "aq_act_absmean_noalloc: empty calibration data (T = %lld)", (long long)T);
  AQ_REQUIRE(T < (int64_t(1) << 40), "aq_act_absmean_noalloc: T out of range");
  AQ_REQUIRE(K > 0 && K < kDimLimit && K % 8 == 0,
             "aq_act_absmean_noalloc: K must be a positive multiple of 8 (got %lld)", (long long)K);
  AQ_REQUIRE(total_count >= T, "aq_act_absmean_noalloc: total_count (%lld) must include this chunk's T (%lld)",
             (long long)total_count, (long long)T);
  AQ_PTR(X, 16, "X");
  AQ_PTR(sum_abs, 8, "sum_abs");
  if (mean_out) AQ_REQUIRE(aligned(mean_out, 4), "mean_out must be 4-byte aligned");
  const size_t need = aq_act_absmean_workspace(T, K);
  AQ_REQUIRE(need <= aq::absmean_scratch_bytes(),
             "aq_act_absmean_noalloc: %lld channels need %zu bytes of partial sums, beyond the %zu-byte scratch",
             (long long)K, need, aq::absmean_scratch_bytes());
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_act_absmean_noalloc: injected launch failure");
  double* scratch = nullptr;
  const hipError_t e = aq::absmean_scratch(&scratch);
  if (e != hipSuccess) return runtime_status(e, "aq_act_absmean_noalloc: scratch address");
  return runtime_status(aq::launch_act_absmean(X, T, K, sum_abs, mean_out, total_count, scratch, (hipStream_t)stream),
                        "aq_act_absmean_noalloc");
}

size_t aq_awq_search_workspace(int64_t T, int64_t N, int64_t K, int32_t group, int32_t n_grid) {
  if (n_grid < 1 || n_grid > 64 || !valid_group(group) || !search_dims_ok(T, N, K)) return 0;
  return search_layout(T, N, K, n_grid).total;
}

aq_status aq_awq_search(const uint16_t* X_sub, int64_t T, const float* absmean_host, const void* W,
                        int32_t w_dtype, int64_t N, int64_t K, int32_t group, int32_t n_grid, double* mse,
                        int32_t* best, float* best_scale, uint8_t* packed, float* scales, uint8_t* zeros,
                        void* workspace, size_t workspace_bytes, void* stream) {
  AQ_REQUIRE(T > 0, "aq_awq_search: empty calibration data (T = %lld)", (long long)T);
  AQ_REQUIRE(T < kGemmDimLimit, "aq_awq_search: T must be below 2^22 (got %lld)", (long long)T);
  AQ_REQUIRE(w_dtype == AQ_F32 || w_dtype == AQ_BF16, "aq_awq_search: bad w_dtype %d", w_dtype);
  AQ_REQUIRE(valid_group(group), "aq_awq_search: group must be 32, 64 or 128 (got %d)", group);
  AQ_REQUIRE(n_grid >= 1 && n_grid <= 64, "aq_awq_search: n_grid must be in 1..64 (got %d)", n_grid);
  AQ_REQUIRE(N > 0 && N < kGemmDimLimit, "aq_awq_search: N must be in 1 .. 2^22 - 1 (got %lld)", (long long)N);
  AQ_REQUIRE(K > 0 && K < kGemmDimLimit && K % group == 0,
             "aq_awq_search: K (%lld) must be a multiple of group (%d) below 2^22", (long long)K, group);
  AQ_REQUIRE(search_dims_ok(T, N, K), "aq_awq_search: too many error-GEMM tiles for T = %lld, N = %lld",
             (long long)T, (long long)N);
  AQ_PTR(X_sub, 16, "X_sub");
  AQ_REQUIRE(absmean_host != nullptr, "absmean_host must not be NULL");
  AQ_PTR(W, 16, "W");
  AQ_PTR(mse, 8, "mse");
  AQ_PTR(best, 4, "best");
  AQ_PTR(best_scale, 16, "best_scale");
  AQ_PTR(packed, 16, "packed");
  AQ_PTR(scales, 4, "scales");
  AQ_PTR(zeros, 1, "zeros");
  AQ_PTR(workspace, 256, "workspace");
  const SearchLayout L = search_layout(T, N, K, n_grid);
  AQ_REQUIRE(workspace_bytes >= L.total, "aq_awq_search: workspace too small (%zu < %zu bytes)", workspace_bytes,
             L.total);
  for (int64_t k = 0; k < K; ++k)
    AQ_REQUIRE(std::isfinite(absmean_host[k]) && absmean_host[k] >= 0.0f,
               "aq_awq_search: absmean_host[%lld] must be finite and >= 0", (long long)k);
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_awq_search: injected launch failure");

  char* ws = static_cast<char*>(workspace);
  float* d_sgrid = reinterpret_cast<float*>(ws + L.sgrid);
  float* d_rgrid = reinterpret_cast<float*>(ws + L.rgrid);
  uint16_t* d_e = reinterpret_cast<uint16_t*>(ws + L.e);
  double* d_partial = reinterpret_cast<double*>(ws + L.partial);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  uint16_t* d_hp = reinterpret_cast<uint16_t*>(ws + L.hp);
  if (L.gram) {
    // H = X^T X and its two bf16 planes, queued before the host work below
    uint16_t* d_xt = reinterpret_cast<uint16_t*>(ws + L.xt);
    float* d_h = reinterpret_cast<float*>(ws + L.h);
    e = aq::launch_transpose_pad(X_sub, T, K, L.tp, d_xt, s);
    if (e == hipSuccess) e = aq::launch_bf16_gemm(d_xt, (int)K, (int)L.tp, d_xt, (int)K, d_h, s);
    if (e == hipSuccess) e = aq::launch_split_planes(d_h, K * K, d_hp, s);
    if (e != hipSuccess) return runtime_status(e, "aq_awq_search: Gram matrix");
  }
  // candidate scales s (then fl32(1 / s), which the error matrix multiplies by), one copy
  std::vector<float> sgrid((size_t)2 * n_grid * (size_t)K);
  candidate_grid(absmean_host, K, n_grid, sgrid.data());
  e = hipMemcpyAsync(d_sgrid, sgrid.data(), (size_t)n_grid * K * sizeof(float), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(d_rgrid, sgrid.data() + (size_t)n_grid * K, (size_t)n_grid * K * sizeof(float),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return runtime_status(e, "aq_awq_search: candidate-scale upload");
  const bool bf16 = w_dtype == AQ_BF16;
  for (int32_t i = 0; i < n_grid; ++i) {
    e = aq::launch_quant_error(W, bf16, d_sgrid + (size_t)i * K, d_rgrid + (size_t)i * K, d_e, N, K, group, s);
    if (e != hipSuccess) return runtime_status(e, "aq_awq_search: error-matrix kernel");
    double* part = d_partial + (size_t)i * L.nblocks;
    e = L.gram ? aq::launch_gram_gemm(d_e, (int)N, (int)K, d_hp, part, s)
               : aq::launch_sumsq_gemm(X_sub, (int)T, (int)K, d_e, (int)N, part, s);
    if (e != hipSuccess) return runtime_status(e, "aq_awq_search: error GEMM");
  }
  e = aq::launch_search_select(d_partial, L.nblocks, n_grid, (double)T * (double)N, d_sgrid, (int)K, mse, best,
                               best_scale, s);
  if (e != hipSuccess) return runtime_status(e, "aq_awq_search: select kernel");
  return runtime_status(aq::launch_quant_pack(W, bf16, best_scale, packed, scales, zeros, N, K, group, false, s),
                        "aq_awq_search: final pack");
}

aq_status aq_awq_fold_norm(const void* norm_w, int32_t w_dtype, const float* chan_scale, int64_t K, float* folded,
                           void* stream) {
  AQ_REQUIRE(w_dtype == AQ_F32 || w_dtype == AQ_BF16, "aq_awq_fold_norm: w_dtype must be AQ_F32 or AQ_BF16 (got %d)",
             w_dtype);
  AQ_REQUIRE(K > 0 && K < kDimLimit, "aq_awq_fold_norm: K out of range (%lld)", (long long)K);
  AQ_PTR(norm_w, w_dtype == AQ_BF16 ? 2 : 4, "norm_w");
  AQ_PTR(chan_scale, 4, "chan_scale");
  AQ_PTR(folded, 4, "folded");
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_awq_fold_norm: injected launch failure");
  return runtime_status(aq::launch_fold_norm(norm_w, w_dtype == AQ_BF16, chan_scale, (int)K, folded,
                                             (hipStream_t)stream),
                        "aq_awq_fold_norm");
}

size_t aq_fp4_gemm_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || K % 32) return 0;
  return staged_bytes(M, N, K);
}

aq_status aq_fp4_gemm(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const uint8_t* block_scales,
                      float tensor_scale, int64_t N, float* Y, void* workspace, size_t workspace_bytes,
                      void* stream) {
  AQ_REQUIRE(M >= 0 && M < kDimLimit, "aq_fp4_gemm: M out of range (%lld)", (long long)M);
  AQ_REQUIRE(K > 0 && K < kDimLimit && K % 32 == 0, "aq_fp4_gemm: K must be a positive multiple of 32 (got %lld)",
             (long long)K);
  AQ_REQUIRE(N >= 0 && N < kDimLimit, "aq_fp4_gemm: N out of range (%lld)", (long long)N);
  AQ_REQUIRE(std::isfinite(tensor_scale), "aq_fp4_gemm: tensor_scale must be finite");
  AQ_PTR(X, 16, "X");
  AQ_PTR(codes, 16, "codes");
  AQ_PTR(block_scales, 2, "block_scales");
  AQ_PTR(Y, 4, "Y");
  if (M > 16)
    AQ_REQUIRE(K < kGemmDimLimit && N < kGemmDimLimit,
               "aq_fp4_gemm: K and N must be below 2^22 for M > 16 (got %lld, %lld)", (long long)K, (long long)N);
  uint16_t* staged = nullptr;
  if (M > 16) {
    const aq_status st = staging("aq_fp4_gemm", M, N, K, workspace, workspace_bytes, &staged);
    if (st != AQ_OK) return st;
  }
  if (fault_injected()) return fail(AQ_ERUNTIME, "aq_fp4_gemm: injected launch failure");
  if (N == 0 || M == 0) return ok();
  hipError_t e;
  if (M <= 16)
    e = aq::launch_fp4_gemv(X, (int)M, (int)K, codes, block_scales, tensor_scale, (int)N, Y, (hipStream_t)stream);
  else
    e = aq::launch_fp4_gemm(X, (int)M, (int)K, codes, block_scales, tensor_scale, (int)N, Y, staged,
                            (hipStream_t)stream);
  return runtime_status(e, "aq_fp4_gemm");
}

}  // extern "C"

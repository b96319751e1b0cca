/*
 * libaq -- group-wise INT4 (W4A16) weight quantization, AWQ calibration and an
 * FP4 decode path for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller (the library
 *     never allocates or frees device memory; calls that need scratch space take
 *     a caller-provided workspace sized by the matching *_workspace() query).
 *     The only host pointer is `absmean_host` of aq_awq_search.
 *   - Every tensor is row-major and dense.  bf16 tensors are passed as uint16_t
 *     bit patterns.  Weights follow the linear-layer convention W[N, K]
 *     (N = out features, K = in features, K contiguous).
 *   - Quantized INT4 weights ("packed triple"):
 *       packed [N, K/2] uint8 : two 4-bit codes per byte, k even in the low
 *                               nibble, k odd in the high nibble;
 *       scales [N, K/g] fp32  : the group step S;
 *       zeros  [N, K/g] uint8 : the zero point z, 0..15;
 *     groups are g consecutive k inside one row, g in {32, 64, 128}; the
 *     dequantized weight is (q - z) * S.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream).  Only aq_awq_search synchronises `stream`, once, to
 *     upload its candidate scales.
 *   - Status codes mirror the 0 / 1 / 2 exit-code convention of the llm-quantize
 *     CLI ("模型量化指南", blog.yoooo.fun, section "用 CLI 量化", exit-code convention): AQ_OK; AQ_EINVAL when an
 *     argument fails validation -- validation runs before any launch, so on
 *     AQ_EINVAL no output byte is written; AQ_ERUNTIME when the HIP runtime
 *     reports a launch or copy failure.  aq_last_error() returns a thread-local
 *     description of the last non-OK status.
 *   - Pointers must be non-NULL (unless stated) and aligned: 16 bytes for X, W,
 *     packed, codes, chan_scale and workspaces; 8 for fp64 outputs; 4 for other
 *     fp32 / int32 tensors.
 *   - Inputs must be finite (documented precondition, not checked).
 *   - An empty output dimension (N == 0, or M == 0 for the products) is a valid
 *     no-op.
 */
#ifndef AQ_H_
#define AQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { AQ_OK = 0, AQ_EINVAL = 1, AQ_ERUNTIME = 2 } aq_status;
typedef enum { AQ_F32 = 0, AQ_BF16 = 1 } aq_dtype;

/*
 * Group-wise asymmetric INT4 quantization and packing.
 * Source: "Quantization：模型量化" (xingyuwang.me), section 2 (asymmetric
 * quantization q = round(x/s) + z, dequantization (q - z) s, clipping to the
 * integer range) and section 3 (per-group scales); "Lance-Quant" (zingnex.cn),
 * grid-search / grouping section (INT4 packed by groups; min-max when no
 * activation statistics exist; o_proj / down_proj get plain group quantization).
 *
 * For every row n and group j of g consecutive k:
 *   v_k = fl32(w_nk * chan_scale[k])   (v_k = w_nk when chan_scale == NULL)
 *   S = fl32(fl32(max v - min v) / 15), z = clamp(rne(fl32(-min v / S)), 0, 15),
 *   q_k = clamp(rne(fl32(v_k / S)) + z, 0, 15); a constant group stores
 *   S = 0, z = 0, q = 0.  Divisions are IEEE fp32, rounding is half-to-even.
 *
 * W          [N, K] fp32 or bf16 (w_dtype), device
 * chan_scale [K] fp32 AWQ scale, device, or NULL
 * packed/scales/zeros: the packed triple (outputs), device
 * Errors: EINVAL for bad dtype, group not in {32,64,128}, K <= 0 or K % group,
 *         NULL / misaligned pointers, N < 0.
 */
aq_status aq_quantize_pack(const void* W, int32_t w_dtype, int64_t N, int64_t K, int32_t group,
                           const float* chan_scale, uint8_t* packed, float* scales, uint8_t* zeros,
                           void* stream);

/*
 * Group-wise symmetric INT4 quantization and packing (the same packed format).
 * Source: "Quantization：模型量化" (xingyuwang.me), section 2 (symmetric
 * quantization: a symmetric integer range with zero mapped to integer zero,
 * q = round(x/s), dequantization q s, clipping to the range) and section 3.
 *
 * For every row n and group j of g consecutive k (v as above):
 *   S = fl32(max |v| / 7),  q_k = clamp(rne(fl32(v_k / S)), -7, 7),
 *   stored code q_k + 8 and zero point 8, so (code - z) S = q S and
 *   aq_w4a16_gemv / aq_w4a16_gemm decode it unchanged; an all-zero group stores
 *   S = 0 and codes 8.
 * Arguments, layout and errors as aq_quantize_pack.
 */
aq_status aq_quantize_pack_sym(const void* W, int32_t w_dtype, int64_t N, int64_t K, int32_t group,
                               const float* chan_scale, uint8_t* packed, float* scales, uint8_t* zeros,
                               void* stream);

/*
 * W4A16 decode GEMV, 1 <= M <= 16 activation rows.  For a few rows a VALU kernel
 * (HBM-bound at M = 1); from 5 rows a matrix-core kernel
 * (16x16x32 bf16 MFMA on the exact integers q - z), whose time grows little with M.
 * Source: "模型量化指南" (blog.yoooo.fun), common conventions (the packed linear
 * dequantizes in memory and equals the original layer with W replaced by its
 * dequantized value); "Quantization：模型量化" (xingyuwang.me), sections 4 (W4A16)
 * and 13 (compressed weights are read, dequantized inside the kernel, then
 * contracted; decode is memory-bound).
 *
 *   Y[m, n] = sum_g S[n,g] * sum_{k in g} X[m,k] * (q[n,k] - z[n,g])  (fp32)
 *
 * X [M, K] bf16, device; packed triple for W[N, K]; Y [M, N] fp32 (output).
 * Errors: EINVAL for M outside 1..16, group not in {32,64,128}, K <= 0 or
 *         K % group, N < 0, NULL / misaligned pointers, K or N >= 2^30.
 */
aq_status aq_w4a16_gemv(const uint16_t* X, int64_t M, int64_t K, const uint8_t* packed, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* stream);

/*
 * W4A16 prefill GEMM, any M >= 0 (tuned for M >= 64): bf16 MFMA on the exact
 * integer operand (q - z), fp32 group-step rescale per group, fp32 output.
 * Same sources, arguments and formula as aq_w4a16_gemv.
 *
 * Two paths with identical results (bit-identical outputs): fused (the kernel
 * dequantizes each weight tile in LDS) and staged (a first kernel writes the
 * exact bf16 (q - z) of every weight into `workspace`, the GEMM then streams it;
 * used for M >= 2048).  Launches with few output tiles (small M or N: at most
 * 128 tiles of 256 or 128 rows x 128 columns) also split K into up to 8 slices
 * of whole 64-k stages and groups: each slice writes an fp32 partial
 * [M, N] into `workspace` and a second kernel adds the slices in order
 * (deterministic; the sum order differs from the unsplit GEMM's, so the results
 * differ from it by fp32 rounding).
 * aq_w4a16_gemm_workspace(M, N, K, group) gives the bytes of both (staging
 * matrix, then 256-byte aligned partials); it depends on the sizes only.  With
 * workspace_bytes at least that, both are used; else, with room for the staging
 * matrix, the staged path alone; else the fused path without slices, and
 * workspace is not touched.
 * workspace: caller-owned device memory, 256-byte aligned, used only during the
 * call on `stream` (its contents afterwards are unspecified).
 * Errors: EINVAL for M < 0 or M >= 2^30, K or N >= 2^22, a misaligned workspace, and
 *         as aq_w4a16_gemv otherwise.
 */
size_t aq_w4a16_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t group);
aq_status aq_w4a16_gemm(const uint16_t* X, int64_t M, int64_t K, const uint8_t* packed, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Per-input-channel |x| statistic for AWQ calibration.
 * Source: "Lance-Quant" (zingnex.cn), calibration section (hooks store each
 * input channel's average absolute activation; statistics of several runs are
 * merged); "BNB/GPTQ/AWQ量化全面支持" (maplevalley.com.cn), AWQ paragraph.
 *
 *   sum_abs[k] += sum_{t < T} |X[t, k]|        (fp64, ACCUMULATED: the caller
 *                                               zeroes sum_abs once, then feeds
 *                                               chunks / tasks)
 *   mean_out[k] = fl32(sum_abs[k] / total_count)   (skipped when mean_out == NULL)
 *
 * X [T, K] bf16, device; sum_abs [K] fp64, device; mean_out [K] fp32 or NULL;
 * total_count = tokens accumulated so far including this chunk (>= T);
 * workspace >= aq_act_absmean_workspace(T, K) bytes, device.
 * Partial sums are reduced in a fixed order: results are deterministic.
 * Errors: EINVAL for T <= 0 (empty calibration data), K <= 0 or K % 8,
 *         total_count < T, small workspace, NULL / misaligned pointers.
 */
size_t aq_act_absmean_workspace(int64_t T, int64_t K);
aq_status aq_act_absmean(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, float* mean_out,
                         int64_t total_count, void* workspace, size_t workspace_bytes, void* stream);

/*
 * aq_act_absmean without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid allocation).  Same arguments (less the workspace), results (bit for
 * bit) and errors as aq_act_absmean.  The partial sums live in a file-scope
 * device array of the library (8 MiB per GPU, held until the process ends), so:
 *   - it serves any (T, K) with aq_act_absmean_workspace(T, K) <= 8 MiB (every
 *     K up to 2^20 channels, any T); larger sizes return AQ_EINVAL;
 *   - every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (different streams, or host threads without ordering) race and give
 *     wrong sums; calls ordered on one stream are safe (each call rewrites every
 *     partial it reads, nothing has to start at zero);
 *   - it uses the array of the current device: `stream` must belong to it.
 * No device memory is allocated or freed by the call.
 */
aq_status aq_act_absmean_noalloc(const uint16_t* X, int64_t T, int64_t K, double* sum_abs, float* mean_out,
                                 int64_t total_count, void* stream);

/*
 * AWQ alpha-grid search and final packing.
 * Source: "Lance-Quant" (zingnex.cn), grid-search / grouping section (grid
 * search of the AWQ scale for a norm and its consuming linears, then INT4 group
 * packing); "Quantization：模型量化" (xingyuwang.me), section 7 (AWQ uses activation
 * statistics to protect salient channels by scaling); OmniQuant tutorial
 * (cyqw.cn), section 2.2.2 (the per-channel equivalent transform is exact).
 *
 * For i = 0 .. n_grid-1, alpha = i / n_grid:
 *   t_k = max(absmean_host[k], 1e-8)^alpha      (fp64 libm pow, on the host)
 *   s_k = fl32(t_k / sqrt(max t * min t))
 *   E   = Q(W diag(s)) / s - W                   (Q: aq_quantize_pack + dequant)
 *   mse[i] = mean over (t, n) of (X_sub E^T)[t, n]^2
 *          (= output MSE of (X/s) Q(W s)^T against X W^T)
 * best[0] = first index of the minimum; best_scale = s of that index;
 * packed/scales/zeros = aq_quantize_pack(W, chan_scale = best_scale).
 * E is formed in fp32 and split into two bf16 planes (hi + lo, ~16 significant
 * bits) for the bf16-MFMA product; the MSE is accumulated in fp64 with a fixed
 * reduction order.
 *
 * X_sub [T, K] bf16, device; absmean_host [K] fp32, HOST; W [N, K] fp32/bf16,
 * device; mse [n_grid] fp64, best [1] int32, best_scale [K] fp32 and the packed
 * triple are device outputs; workspace >= aq_awq_search_workspace(...) bytes.
 * Synchronises `stream` once (candidate-scale upload) before the first launch.
 * Errors: EINVAL for T <= 0 (empty calibration data), n_grid outside 1..64,
 *         K % group, group not in {32,64,128}, T, N or K >= 2^22 (the error
 *         GEMM's 32-bit offsets), small workspace, NULL / misaligned pointers,
 *         non-finite or negative absmean values.  The workspace query returns 0
 *         for arguments the search refuses.
 */
size_t aq_awq_search_workspace(int64_t T, int64_t N, int64_t K, int32_t group, int32_t n_grid);
aq_status aq_awq_search(const uint16_t* X_sub, int64_t T, const float* absmean_host, const void* W,
                        int32_t w_dtype, int64_t N, int64_t K, int32_t group, int32_t n_grid, double* mse,
                        int32_t* best, float* best_scale, uint8_t* packed, float* scales, uint8_t* zeros,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The RMSNorm fold of the AWQ channel scale.
 * Source: "Lance-Quant" (zingnex.cn), grid-search / grouping section (the scale
 * chosen for a normalisation and its consuming linears is folded into that
 * RMSNorm: the linears hold Q(W diag(s)), the norm weight becomes w / s, so the
 * layer computes the same function); OmniQuant tutorial (cyqw.cn), section 2.2.2
 * (the per-channel equivalent transform (X / s)(s W) = X W).
 *
 *   folded[k] = fl32(norm_w[k] / chan_scale[k])      (one IEEE fp32 division)
 *
 * norm_w [K] fp32 or bf16 (w_dtype), chan_scale [K] fp32 (aq_awq_search's
 * best_scale), folded [K] fp32 output; all device pointers (4-byte aligned,
 * 2 for a bf16 norm_w).  A zero chan_scale entry gives an infinite result
 * (aq_awq_search's scales are positive).
 * Errors: EINVAL for a bad w_dtype, K <= 0 or K >= 2^30, NULL / misaligned
 *         pointers.
 */
aq_status aq_awq_fold_norm(const void* norm_w, int32_t w_dtype, const float* chan_scale, int64_t K, float* folded,
                           void* stream);

/*
 * Group-wise asymmetric INT8 quantization (one code byte per weight).
 * Source: "Quantization：模型量化" (xingyuwang.me), sections 2 and 3 (the
 * asymmetric formulas with the integer range setting the clip; per-group
 * scales); "模型量化指南" (blog.yoooo.fun), "混合精度（按层 4/8-bit）" (a per-layer
 * policy keeps key layers at 8 bits, the rest at 4).
 *
 *   S = fl32(fl32(max v - min v) / 255), z = clamp(rne(fl32(-min v / S)), 0, 255),
 *   q_k = clamp(rne(fl32(v_k / S)) + z, 0, 255); a constant group stores S = 0,
 *   z = 0, q = 0 (v as in aq_quantize_pack, with the optional chan_scale).
 * codes [N, K] uint8 (one byte per weight), scales [N, K/g] fp32, zeros
 * [N, K/g] uint8.  Arguments and errors as aq_quantize_pack.
 */
aq_status aq_quantize_pack8(const void* W, int32_t w_dtype, int64_t N, int64_t K, int32_t group,
                            const float* chan_scale, uint8_t* codes, float* scales, uint8_t* zeros, void* stream);

/*
 * W8A16 products of the INT8 format: Y[m, n] = sum_g S[n, g] sum_{k in g}
 * X[m, k] (q[n, k] - z[n, g]), fp32 Y [M, N], X [M, K] bf16.
 * aq_w8a16_gemv: 1 <= M <= 16; VALU kernel up to 3 rows (HBM-bound at M = 1),
 * 16x16x32 bf16 MFMA on the exact integers q - z from 4 rows.
 * aq_w8a16_gemm: any M; the codes are first dequantized exactly into the bf16
 * matrix (q - z) in `workspace` (N * K * 2 bytes, aq_w8a16_gemm_workspace,
 * 256-byte aligned, caller-owned, contents unspecified afterwards), then a
 * bf16-MFMA GEMM applies the fp32 group steps to per-group partials.
 * Source: as aq_quantize_pack8; the products as aq_w4a16_gemv / aq_w4a16_gemm.
 * Errors: as aq_w4a16_gemv / aq_w4a16_gemm; aq_w8a16_gemm also for a NULL,
 *         misaligned or small workspace.
 */
aq_status aq_w8a16_gemv(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* stream);
size_t aq_w8a16_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t group);
aq_status aq_w8a16_gemm(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const float* scales,
                        const uint8_t* zeros, int64_t N, int32_t group, float* Y, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * FP4 decode product: E2M1 codes with an FP8-E4M3 scale per 16-element block
 * and an fp32 tensor scale.  M <= 16 runs a decode kernel (VALU up to 2 rows,
 * 16x16x32 bf16 MFMA from 3 rows when K % 64 == 0), larger M a bf16-MFMA GEMM; all
 * use the exact bf16 value e2m1 * e4m3.
 * Source: "Lance-Quant" (zingnex.cn), grid-search / grouping section (NVFP4 =
 * E2M1 codes + FP8 E4M3 scale per 16 elements, block_size 16);
 * "Quantization：模型量化" (xingyuwang.me), section 12 (E4M3 = 1 + 4 + 3 bits).
 *
 *   Y[m, n] = tensor_scale * sum_k X[m, k] * e2m1(c[n, k]) * e4m3(b[n, k / 16])
 *
 * X [M, K] bf16; codes [N, K/2] uint8 (k even in the low nibble; bit 3 of a
 * code is the sign, bits 2..1 the exponent with bias 1, bit 0 the mantissa);
 * block_scales [N, K/16] uint8 E4M3 (OCP "FN": bias 7, no infinities, 0x7F /
 * 0xFF are NaN); Y [M, N] fp32 output.
 * For M > 16 the GEMM has the same fused and staged paths as aq_w4a16_gemm
 * (staged: the exact bf16 weights written to `workspace` first), selected the
 * same way with aq_fp4_gemm_workspace(M, N, K).
 * Errors: EINVAL for M < 0, K <= 0 or K % 32, non-finite tensor_scale, N < 0,
 *         NULL / misaligned pointers, K or N >= 2^30, K or N >= 2^22 when M > 16.
 */
size_t aq_fp4_gemm_workspace(int64_t M, int64_t N, int64_t K);
aq_status aq_fp4_gemm(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const uint8_t* block_scales,
                      float tensor_scale, int64_t N, float* Y, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * FP4 encoder: W [N, K] (fp32 or bf16) -> the codes, block scales and tensor
 * scale that aq_fp4_gemm decodes.
 * Source: "Lance-Quant" (zingnex.cn), grid-search / grouping section (nvfp4_apply
 * packs E2M1 codes with an FP8 E4M3 scale per 16-element block);
 * "Quantization：模型量化" (xingyuwang.me), section 12 (E4M3 = 1 + 4 + 3 bits).
 *
 *   ts   = fl32(max |W| / 2688)              (2688 = 6 * 448); 1 if W is all zero
 *   b    = E4M3(fl32(max_block |w| / fl32(6 ts)))   nearest, ties to the even
 *          code, saturating at 448; one byte per 16 consecutive k of a row
 *   code = nearest E2M1 magnitude of fl32(|w| / fl32(e4m3(b) ts)), ties to the
 *          even code, saturating at 6 (0 when the block scale is 0); bit 3 set
 *          for negative w with a non-zero magnitude
 * Outputs: codes [N, K/2] uint8 (k even in the low nibble), block_scales
 * [N, K/16] uint8, tensor_scale: one fp32 on the device.  Every fp32 operation
 * is an IEEE operation in the order above (deterministic, bit-reproducible).
 * workspace: device memory of at least aq_fp4_quantize_workspace(N, K) bytes
 * (the partial maxima), 4-byte aligned, used only during the call.
 * Errors: EINVAL for w_dtype not AQ_F32 / AQ_BF16, N < 0, K <= 0 or K % 16,
 *         K or N >= 2^30, a small workspace, NULL / misaligned pointers (W 16,
 *         codes 8, tensor_scale and workspace 4 bytes).  Inputs must be finite.
 */
size_t aq_fp4_quantize_workspace(int64_t N, int64_t K);
aq_status aq_fp4_quantize(const void* W, int32_t w_dtype, int64_t N, int64_t K, uint8_t* codes,
                          uint8_t* block_scales, float* tensor_scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Thread-local text for the last non-OK status of this thread ("" if none). */
const char* aq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AQ_H_ */

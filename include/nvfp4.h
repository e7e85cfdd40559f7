/*
 * libnvfp4 — NVFP4 quantisation and block-scale selection on AMD Instinct MI355X (gfx950).
 *
 * NVFP4 stores a tensor as 4-bit E2M1 codes in blocks of 16 consecutive values, one FP8
 * (E4M3) scale per block and one FP32 scale per tensor. Pages this library follows
 * (titles translated):
 *  [QAD] "Why NVFP4 inference loses accuracy, and what QAD actually repairs"
 *        (czchanglian.com/news/46648), sections 1, 2.1, 2.3, 3.2, 4.2;
 *  [BT]  "Baseten on high-quality NVFP4 quantization" (attain.fans translation),
 *        sections "Why do we need a scale", "Block scaling", "Why blocks";
 *  [LH]  "How much dumber does 4-bit make a model? The answer is in the scale shared by
 *        every 16 weights" (2kiu.com/news/4970560), a write-up of NVIDIA Model Optimizer's
 *        "Improving NVFP4 Accuracy with Local-Hessian Weight Scales": sections "NVFP4
 *        structure", the paragraph on max / Four-Over-Six / MSE selection, and "Change the
 *        objective".
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller; nothing is allocated,
 *    retained or freed by the library. Host-side validation happens before any launch.
 *  - Layout is row-major and contiguous. `cols` is the contiguous dimension and must be a
 *    multiple of 16; blocks are 16 consecutive values along it ([BT] "Block scaling").
 *    `batch` stacks independent tensors of identical shape (e.g. MoE experts); each has
 *    its own tensor scale S[batch].
 *  - Element tensors (x, w, y) must be 16-byte aligned; packed codes 8-byte aligned.
 *  - Block scales are E4M3FN bytes [batch][rows][cols/16]: 0x01..0x7E are the 126
 *    positive candidates of [LH]; 0x00 marks an all-zero block.
 *  - Codes are packed two per byte [batch][rows][cols/2]: element 2j in the low nibble of
 *    byte j. A code is sign<<3 | k, with k indexing {0, 0.5, 1, 1.5, 2, 3, 4, 6}
 *    ([BT] "Why do we need a scale"); a zero magnitude never carries the sign bit.
 *  - Rounding: the block byte is the E4M3 value nearest to amax_b/(6 S) ([QAD] 2.3),
 *    saturating at 448 ([QAD] 4.2) and at least 0x01 for a non-zero block; an element's
 *    code is the E2M1 value nearest to |x|/(s S) ([QAD] 2.1), saturating at 6. Both are
 *    decided on the exact real quotient, ties to the even byte / even grid index.
 *  - Dequantised value: +-fp32(G_k * s * S), one rounding of the exact product; bf16
 *    output rounds that to nearest-even.
 *  - Inputs must be finite; the tensor scale S must be a positive normal fp32 number.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call is asynchronous on it.
 *  - Return value: NVFP4_OK or an error code below. Calls with an empty tensor (a zero
 *    dimension) validate their shape and return NVFP4_OK without launching.
 *  - The *_workspace_size queries return 0 for arguments their entry point rejects.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define NVFP4_API __attribute__((visibility("default")))
#else
#define NVFP4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* element dtypes */
#define NVFP4_DTYPE_F32 0
#define NVFP4_DTYPE_BF16 1

/* status codes */
#define NVFP4_OK 0
#define NVFP4_ERR_NULL 1      /* a required pointer is NULL */
#define NVFP4_ERR_SHAPE 2     /* negative dimension, cols % 16 != 0, or size overflow */
#define NVFP4_ERR_DTYPE 3     /* unknown dtype */
#define NVFP4_ERR_ALIGN 4     /* a pointer lacks the alignment stated above */
#define NVFP4_ERR_WORKSPACE 5 /* workspace NULL or smaller than *_workspace_size */
#define NVFP4_ERR_HIP 6       /* a HIP launch failed */
#define NVFP4_ERR_ARG 7       /* another argument is out of range */

/* Human-readable name of a status code (static string). */
NVFP4_API const char *nvfp4_status_string(int status);

/* Library ABI version (major * 100 + minor). */
NVFP4_API int nvfp4_version(void);

/*
 * Per-tensor FP32 scale ([BT] "Why do we need a scale": a second, FP32 scaling level
 * exists; its formula is not given there). For each b < batch:
 *   S[b] = fp32(amax(|x[b]|) / 2688), 2688 = 6 * 448, so the largest block maps onto the
 *   top E4M3 value; S[b] = 1 for an all-zero tensor; raised to FLT_MIN if smaller.
 * x: [batch][n] elements of `dtype`, 16-byte aligned, n % 8 == 0. S: [batch] fp32 (out).
 */
NVFP4_API int nvfp4_global_scale(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                       void *stream);

/*
 * The same S in two launches instead of three, with a caller workspace of at least
 * nvfp4_global_scale_workspace_size(batch, n) bytes, 4-byte aligned, that receives one
 * partial maximum per workgroup (no initialisation needed; its contents after the call are
 * unspecified). Calls that share a workspace must not overlap. Same arguments and errors as
 * nvfp4_global_scale, plus NVFP4_ERR_WORKSPACE.
 */
NVFP4_API size_t nvfp4_global_scale_workspace_size(int64_t batch, int64_t n);
NVFP4_API int nvfp4_global_scale_ws(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Max scaling ([QAD] 2.3, [LH] default selector): block byte = E4M3 nearest to
 * amax_b / (6 S[b]). w: [batch][rows][cols]; S: [batch]; scales: [batch][rows][cols/16].
 */
NVFP4_API int nvfp4_scale_search_max(const void *w, int dtype, int64_t batch, int64_t rows,
                           int64_t cols, const float *S, uint8_t *scales, void *stream);

/*
 * MSE scale search ([LH] paragraph on the MSE selector): every block tries all 126
 * positive E4M3 bytes and keeps the first with the smallest squared weight error,
 *   obj(c) = fp32 sum over i = 0..15 of e_i^2, e_i = fp32(dq_i(c) - w_i),
 *   accumulated as acc = fmaf(e_i, e_i, acc) in ascending i.
 * An all-zero block gets byte 0x00 and objective 0. obj (nullable): [batch][rows][cols/16]
 * fp32, the winning objective.
 */
NVFP4_API int nvfp4_scale_search_mse(const void *w, int dtype, int64_t batch, int64_t rows,
                           int64_t cols, const float *S, uint8_t *scales, float *obj,
                           void *stream);

/*
 * Four Over Six scale selection ([LH] paragraph on max / Four-Over-Six / MSE selection:
 * one of two candidate scales per block). Reading: the candidates are the E4M3 bytes
 * nearest amax_b / (6 S[b]) (max scaling) and amax_b / (4 S[b]) (the block max on the E2M1
 * magnitude 4), each saturating at 448 and at least 0x01; the one with the smaller MSE
 * objective (as for nvfp4_scale_search_mse) wins, ties to the smaller byte. An all-zero
 * block gets 0x00 and objective 0. Shapes, alignment and errors as for
 * nvfp4_scale_search_mse; obj (nullable) receives the winning objective.
 */
/*
 * Static activation calibration ([BT] "Calibration": the activation distribution recorded
 * over sample inputs sets the clipping range -- the min/max, or percentile / histogram
 * methods that clip a few outliers). Reading:
 *  - nvfp4_calib_histogram adds the magnitudes of x [n] (n % 8 == 0, 16-byte aligned) to
 *    hist [NVFP4_CALIB_BINS] (device uint64, 8-byte aligned, caller-zeroed once and then
 *    accumulated over calibration batches): bin = (fp32 bits of |x|) >> 16, i.e. one bin per
 *    bf16 magnitude. Counts are integers, so the result does not depend on launch order.
 *  - nvfp4_calib_scale writes S[0] (device fp32): with N the total count and k =
 *    ceil(fraction * N), the clip value is the lower edge of the first bin whose cumulative
 *    count reaches k (the k-th smallest magnitude, rounded toward zero to bf16; exact for
 *    bf16 data, and fraction = 1 gives the max), and S = fp32(clip / 2688) as for
 *    nvfp4_global_scale (1 for an empty or all-zero histogram). fraction must lie in
 *    (0, 1], else NVFP4_ERR_ARG.
 */
/*
 * Fake-quant training support ([QAD] sec. 3.2: forward through the quantiser, gradient
 * handed straight back -- a straight-through estimator -- and clamped to a reasonable range
 * in practice; sec. 4.1: a moving-average scale, momentum about 0.9).
 *  - nvfp4_ste_backward: grad_out = clamp(grad, -clip, clip) elementwise, computed in fp32
 *    (bf16 results rounded to nearest even); clip = +inf gives the plain straight-through
 *    gradient; clip must be > 0 (else NVFP4_ERR_ARG). n % 8 == 0, 16-byte aligned; grad_out
 *    may equal grad.
 *  - nvfp4_scale_ema: for each of batch entries, S = fmaf(m, S, fp32(fp32(1 - m) *
 *    S_batch)) (reading: the moving average is kept on the per-tensor fp32 scale);
 *    momentum in [0, 1], else NVFP4_ERR_ARG.
 */
NVFP4_API int nvfp4_ste_backward(const void *grad, int dtype, int64_t n, float clip,
                       void *grad_out, void *stream);
NVFP4_API int nvfp4_scale_ema(float *S, const float *S_batch, int64_t batch, float momentum,
                    void *stream);

#define NVFP4_CALIB_BINS 32768
NVFP4_API int nvfp4_calib_histogram(const void *x, int dtype, int64_t n, uint64_t *hist,
                          void *stream);
NVFP4_API int nvfp4_calib_scale(const uint64_t *hist, double fraction, float *S, void *stream);

NVFP4_API int nvfp4_scale_search_four_over_six(const void *w, int dtype, int64_t batch,
                           int64_t rows, int64_t cols, const float *S, uint8_t *scales,
                           float *obj, void *stream);

/*
 * Block-diagonal calibration Gram matrix ([LH] "Change the objective": the output error
 * ||dX||^2 = tr(d XX^T d^T) is weighted by XX^T; only its 16x16 diagonal blocks are kept):
 *   H[g][b][i][j] (+)= sum over the tokens t of group g of x[t][16b+i] * x[t][16b+j].
 * x: [tokens][cols] (one token per row; bf16 products are exact, accumulation is fp32).
 * Dense form: groups == 1, group_offsets == NULL, token_ids == NULL (all tokens).
 * Grouped form (MoE experts): group_offsets [groups+1] (device, non-decreasing, last
 *   equal to n_ids) and token_ids [n_ids] (device, each in [0, tokens)); group g sums
 *   rows token_ids[group_offsets[g] .. group_offsets[g+1]).
 * H: [groups][cols/16][16][16] fp32 (out). accumulate != 0 adds to the existing H.
 * The workspace holds per-chunk partial sums, reduced in a fixed order, so results are
 * bitwise reproducible. workspace_bytes must be >= nvfp4_block_hessian_workspace_size().
 */
NVFP4_API size_t nvfp4_block_hessian_workspace_size(int64_t tokens, int64_t cols, int64_t groups,
                                          int64_t n_ids);
NVFP4_API int nvfp4_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols,
                        int64_t groups, const int32_t *group_offsets,
                        const int32_t *token_ids, int64_t n_ids, float *H, int accumulate,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Allocation-free form of nvfp4_block_hessian, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight calibration or serving loops, harnesses that
 * forbid hipMalloc). Arguments, checks and results are those of nvfp4_block_hessian without
 * the workspace: the scratch comes from a static device array of NVFP4_STATIC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends. A call whose
 * nvfp4_block_hessian_workspace_size() exceeds that returns NVFP4_ERR_WORKSPACE before any
 * launch. All calls on a device share the array (it keeps the last call's contents, which
 * no call reads): calls that overlap on one device, e.g. on two streams, race and must be
 * ordered by the caller. Nothing is allocated or freed; NVFP4_ERR_HIP if the array's device
 * address cannot be obtained.
 */
#define NVFP4_STATIC_SCRATCH_BYTES (64u << 20)
NVFP4_API int nvfp4_block_hessian_noalloc(const void *x, int dtype, int64_t tokens, int64_t cols,
                                          int64_t groups, const int32_t *group_offsets,
                                          const int32_t *token_ids, int64_t n_ids, float *H,
                                          int accumulate, void *stream);

/*
 * Local-Hessian scale search ([LH] "Change the objective"): for every (row, block) of
 * every batch entry, all 126 positive E4M3 bytes are tried and the first with the
 * smallest d H_b d^T wins, with d_i = fp32(dq_i(c) - w_i) and H_b the block's 16x16
 * matrix shared by all rows (the block-diagonal approximation). The objective is
 * evaluated as y_i = sum_j H_ij d_j, obj = sum_i d_i y_i in double precision, ascending
 * indices, one fused multiply-add per term. A block with an all-zero H_b takes the MSE choice
 * (objective reported as 0); an all-zero block gets 0x00.
 * w: [batch][rows][cols]; S: [batch]; H: [batch][cols/16][16][16] fp32;
 * scales: [batch][rows][cols/16]; obj (nullable): same shape, double.
 */
NVFP4_API int nvfp4_scale_search_local_hessian(const void *w, int dtype, int64_t batch, int64_t rows,
                                     int64_t cols, const float *S, const float *H,
                                     uint8_t *scales, double *obj, void *stream);

/*
 * Quantise to NVFP4 ([QAD] 1, 2.1; [BT] "Block scaling"): codes from the given block bytes
 * (scales_in != NULL, e.g. chosen by a search) or from max scaling (scales_in == NULL, in
 * which case the chosen bytes are written to scales_out when it is non-NULL).
 * codes: [batch][rows][cols/2] packed.
 */
NVFP4_API int nvfp4_quantize(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                   const float *S, const uint8_t *scales_in, uint8_t *codes,
                   uint8_t *scales_out, void *stream);

/*
 * Dequantise packed codes ([QAD] 3.2: value times scale) into y of out_dtype.
 */
NVFP4_API int nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *S,
                     int64_t batch, int64_t rows, int64_t cols, void *y, int out_dtype,
                     void *stream);

/*
 * Fake quantisation, the quantise -> dequantise round trip of [QAD] 3.2 in one pass:
 * y has the dtype and shape of x. Block bytes as in nvfp4_quantize. codes_out and
 * scales_out are optional (nullable) side outputs.
 */
NVFP4_API int nvfp4_fakequant(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                    const float *S, const uint8_t *scales_in, void *y, uint8_t *codes_out,
                    uint8_t *scales_out, void *stream);

/*
 * Routing groups for per-expert Hessians: from a top-k routing table expert_ids
 * [tokens][topk] (device int32), write offsets [experts+1] (prefix sums of per-expert
 * counts) and token_ids [tokens*topk] with every expert's tokens in ascending token order
 * (a stable counting sort). Ids outside [0, experts) are skipped (not routed); the tail
 * of token_ids beyond offsets[experts] is then left unwritten.
 * workspace_bytes must be >= nvfp4_route_groups_workspace_size().
 */
NVFP4_API size_t nvfp4_route_groups_workspace_size(int64_t tokens, int64_t topk, int64_t experts);
NVFP4_API int nvfp4_route_groups(const int32_t *expert_ids, int64_t tokens, int64_t topk,
                       int64_t experts, int32_t *offsets, int32_t *token_ids,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Full Gram matrix H = X^T X of a layer input ([LH] "Change the objective": the output
 * error is tr(dW X X^T dW^T); Local-Hessian needs only its 16x16 diagonal blocks, GPTQ
 * rounding -- which the same page says combines with Local-Hessian -- needs all of it).
 * x: [tokens][cols] bf16 or fp32 (bf16 products are exact, accumulation is fp32);
 * cols % 16 == 0. H: [cols][cols] fp32 (out), exactly symmetric; accumulate != 0 adds to
 * the existing H (streaming over calibration batches). Partial sums per token chunk are
 * added in a fixed order, so results are bitwise reproducible on a given device model (the
 * chunking follows its compute-unit count).
 * workspace_bytes must be >= nvfp4_full_hessian_workspace_size(), queried with the device
 * that runs the call current (the size depends on its compute-unit count).
 */
NVFP4_API size_t nvfp4_full_hessian_workspace_size(int64_t tokens, int64_t cols);
NVFP4_API int nvfp4_full_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, float *H,
                                 int accumulate, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * GPTQ's factor (GPTQ, Frantar et al. 2022, as combined with Local-Hessian in [LH]'s closing
 * paragraphs): U upper triangular, positive diagonal, with U^T U = (H + lambda I)^-1, where
 * lambda = damp * (sum of diag H, in index order) / cols. A zero diagonal sum (all-zero
 * inputs) gives H + lambda I := I. Computed in double precision. Only the lower triangle of
 * H [cols][cols] (fp32) is read; U: [cols][cols] double (out, zeros below the diagonal).
 * status (nullable, device int32): 0, or non-zero if H + lambda I is not positive definite
 * (U is then not usable). damp >= 0 and finite, else NVFP4_ERR_ARG.
 * workspace_bytes must be >= nvfp4_gptq_factor_workspace_size().
 */
NVFP4_API size_t nvfp4_gptq_factor_workspace_size(int64_t cols);
NVFP4_API int nvfp4_gptq_factor(const float *H, int64_t cols, double damp, double *U,
                                int32_t *status, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * GPTQ rounding at fixed block scales: columns of w [rows][cols] in order; column j of each
 * row is rounded (the element rule of nvfp4_quantize, on the double-precision updated
 * value, exact comparisons) at its block byte scales[row][j/16] and S[0], then
 * e = (v_j - q_j) / U_jj and v_k -= e U_jk for k > j. The block bytes are an input (for
 * example from nvfp4_scale_search_local_hessian): GPTQ changes rounding, not scale.
 * codes: [rows][cols/2] packed (out, 8-byte aligned). U from nvfp4_gptq_factor.
 * workspace_bytes must be >= nvfp4_gptq_workspace_size().
 */
NVFP4_API size_t nvfp4_gptq_workspace_size(int64_t rows, int64_t cols);
NVFP4_API int nvfp4_gptq(const void *w, int dtype, int64_t rows, int64_t cols, const float *S,
                         const uint8_t *scales, const double *U, uint8_t *codes,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Input checks for debugging. Inputs must be finite and tensor scales S positive and
 * finite; other inputs give unspecified (but memory-safe) results. S lives in device memory,
 * so host-side validation cannot see it. With the environment variable NVFP4_DEBUG_CHECKS=1,
 * every entry point that reads floating-point tensors (x, w, grad, H) or S first scans them
 * on its stream and raises a device-side flag if any value is NaN or infinite, or any S is
 * not a positive finite number.
 * nvfp4_debug_nonfinite synchronises `stream`, writes the flag (0 or 1) to *flag_out (host
 * memory) and clears it; it returns NVFP4_ERR_ARG when NVFP4_DEBUG_CHECKS is not 1. The
 * flag is shared by all callers in the process.
 */
NVFP4_API int nvfp4_debug_nonfinite(int32_t *flag_out, void *stream);

/*
 * Search statistics (diagnostics; not part of the method). While switched on with
 * nvfp4_search_stats_enable(1), the MSE and Local-Hessian searches (and the MSE fallback of
 * Local-Hessian blocks whose H_b is zero) add to process-wide device counters the work they
 * do and the path each (row, block) takes; nvfp4_search_stats_enable(0) switches counting
 * off (the default: counting adds atomics to the searches). nvfp4_search_stats_read
 * synchronises `stream`, copies the NVFP4_STATS_N counters to out[] (host memory) and
 * clears them. Counters are shared by every caller in the process; concurrent searches add
 * to the same totals. Indices:
 *  NVFP4_STAT_MSE_BLOCKS     non-zero blocks searched by the MSE search
 *  NVFP4_STAT_MSE_EVALS      MSE candidate objectives evaluated (of 126 per block)
 *  NVFP4_STAT_LH_PAIRS       (row, block) pairs with a non-zero block and H_b searched
 *  NVFP4_STAT_LH_ZERO_H      non-zero blocks whose H_b is zero (the MSE choice)
 *  NVFP4_STAT_LH_REL         pairs screened with the error bound relative to the objective
 *  NVFP4_STAT_LH_ABS         pairs screened with the absolute error bound
 *  NVFP4_STAT_LH_NOPRUNE     pairs whose H_b rules out the pruning below the max byte
 *  NVFP4_STAT_LH_RESCAN      pairs rescanned exactly (three or more screen survivors, or
 *                            values outside the screen's range)
 *  NVFP4_STAT_LH_TWO         pairs with two screen survivors (two exact evaluations)
 *  NVFP4_STAT_LH_SCREENED    (pair, candidate) objectives evaluated on the fp32 screen
 *  NVFP4_STAT_LH_EXACT       (pair, candidate) objectives evaluated exactly in fp64
 */
#define NVFP4_STATS_N 16
#define NVFP4_STAT_MSE_BLOCKS 0
#define NVFP4_STAT_MSE_EVALS 1
#define NVFP4_STAT_LH_PAIRS 2
#define NVFP4_STAT_LH_ZERO_H 3
#define NVFP4_STAT_LH_REL 4
#define NVFP4_STAT_LH_ABS 5
#define NVFP4_STAT_LH_NOPRUNE 6
#define NVFP4_STAT_LH_RESCAN 7
#define NVFP4_STAT_LH_TWO 8
#define NVFP4_STAT_LH_SCREENED 9
#define NVFP4_STAT_LH_EXACT 10
NVFP4_API int nvfp4_search_stats_enable(int on);
NVFP4_API int nvfp4_search_stats_read(int64_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */

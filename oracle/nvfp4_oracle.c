/*
 * NVFP4 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. The product path (the HIP library and its Python binding)
 * never links, imports or calls it, and shares no code, tables or helpers with it.
 *
 * It is a plain, slow, obviously correct restatement of what the engine computes. Every
 * rounding decision (block-scale byte, element code) is taken on exact real numbers:
 * all products compared below have at most 31 significant bits, so double arithmetic
 * holds them exactly. Where floating point decides an index (the MSE and Local-Hessian
 * argmins), the precision and order are stated with the function.
 *
 * Pages followed (titles translated; sections as they appear on each page):
 *  [QAD]  "Why NVFP4 inference loses accuracy, and what QAD actually repairs"
 *         (czchanglian.com/news/46648): sec. 1 (E2M1 is 1 sign, 2 exponent and 1 mantissa
 *         bit; one FP8 scale shared by 16 elements), sec. 2.1 (values go to the nearest
 *         representable level), sec. 2.3 (block scale = block max / 6), sec. 3.2 (the
 *         fake-quant sketch: blocks of 16, amax, divide by 6, clamp, quantise, multiply
 *         back; straight-through gradient, clamped in practice), sec. 4.1 (moving-average
 *         scale), sec. 4.2 (clamp the scale at the FP8 maximum).
 *  [BT]   "Baseten on high-quality NVFP4 quantization" (attain.fans translation):
 *         "Why do we need a scale" (the 16 FP4 values; an FP32 per-tensor scale also
 *         exists), "Block scaling" (16 consecutive values per block), "Why blocks"
 *         (worked example: max 84 gives scale 14 and magnitudes 0..84), "Calibration"
 *         (activation ranges from sample inputs; min/max or outlier-clipping ranges).
 *  [LH]   "How much dumber does 4-bit make a model? The answer is in the scale shared by
 *         every 16 weights" (2kiu.com/news/4970560), a write-up of NVIDIA Model
 *         Optimizer's "Improving NVFP4 Accuracy with Local-Hessian Weight Scales":
 *         "NVFP4 structure", the max / Four-Over-Six / MSE paragraph (two candidate
 *         scales; all 126 positive non-zero FP8 scales), "Change the objective" (E(s) = ||dX||^2 = tr(d XX^T d^T); block-
 *         diagonal 16x16 H_b, 126 candidates per block).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - tensor scale S = fp32(amax_tensor / (6 * 448)); S = 1 for an all-zero tensor;
 *    S is raised to FLT_MIN if the quotient is smaller;
 *  - block byte = E4M3 round-half-even of amax_b / (6 S), saturating at 448 (byte 0x7E);
 *    a non-zero block never gets byte 0 (raised to 0x01); an all-zero block gets 0x00;
 *  - element code: round-half-even to the E2M1 grid of |x| / (s S), saturating at 6;
 *    the sign bit is set only for negative x with a non-zero magnitude;
 *  - dequantised value = +-fp32(G_k * s * S) (one rounding of the exact product);
 *  - nibble order: element 2j in the low nibble of byte j;
 *  - MSE objective: fp32, e_i = fp32(dq_i - x_i), acc = fmaf(e_i, e_i, acc) for i = 0..15;
 *  - Local-Hessian objective: d_i = fp32(dq_i - w_i); y_i = sum_j H_ij d_j and
 *    obj = sum_i d_i y_i, both in double, ascending index, each term added with a fused
 *    multiply-add (one rounding per term);
 *  - argmins take the first (smallest byte) minimum; a block whose H_b is all zero
 *    takes the MSE choice;
 *  - Four Over Six's two candidates are the bytes nearest amax_b / (6 S) and amax_b / (4 S);
 *  - calibration clip value: the k-th smallest |x| (k = ceil(p N)) rounded toward zero to
 *    bf16, from an exact histogram with one bin per bf16 magnitude;
 *  - straight-through backward: clamp to [-c, c] in fp32; scale moving average
 *    S = fmaf(m, S, fp32(fp32(1 - m) * S_batch));
 *  - GPTQ rounding at fixed block scales (the page names GPTQ; its steps follow the
 *    published algorithm, Frantar et al. 2022): damping lambda = damp * mean(diag H),
 *    columns in natural order, every decision on the double-precision updated weight.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* E2M1 magnitudes by 3-bit index: [BT] "Why do we need a scale", [LH] "NVFP4 structure". */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by the parallel loops from now on (timing runs on one thread). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Value of an OCP E4M3FN byte (bias 7, 3 mantissa bits, no infinities): bytes 0x00..0x7E
 * are 0 and the 126 positive values [LH] counts; 0x7F is NaN. Sign bit ignored. */
double oracle_e4m3_value(int byte)
{
    int e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp((double)(8 + m), e - 10);
}

/* Signed E2M1 value of a 4-bit code: sign bit 3, magnitude index bits 0..2 ([QAD] sec. 1). */
double oracle_e2m1_value(int code)
{
    double v = E2M1_MAG[code & 7];
    return (code & 8) ? -v : v;
}

/* Round-half-to-even of an fp32 value to bf16 (returns the 16-bit pattern). */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf / nan */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void oracle_bf16_rne_array(const float *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(y[i]);
}

/* Per-tensor FP32 scale ([BT] "Why do we need a scale": a second, FP32 level exists;
 * the formula is a reading: the largest block of the tensor maps to E4M3's top). */
float oracle_tensor_scale(const float *x, int64_t n)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) return 1.0f;
    float S = amax / 2688.0f; /* IEEE fp32 division, 2688 = 6 * 448 */
    if (S < FLT_MIN) S = FLT_MIN;
    return S;
}

/* Max-scaling block byte: E4M3 round-half-even of amax / (6 S) ([QAD] sec. 2.3 and 4.2,
 * [BT] "Why blocks", [LH] max scaling). Exact: v_b * 6S and midpoints * 6S have at most
 * 31 significant bits. */
/* E4M3 byte nearest to amax / (k S), ties to the even byte, saturating at 0x7E, at least
 * 0x01 (k = 6 for max scaling, 4 for the second Four Over Six candidate; value * k * S has
 * at most 31 significant bits, so the comparisons are exact in double). */
int oracle_byte_for_divisor(float amax, float S, double k)
{
    if (amax == 0.0f) return 0;
    double a = amax, kS = k * (double)S;
    int b = 0; /* largest byte whose value * kS <= amax */
    while (b < 126 && oracle_e4m3_value(b + 1) * kS <= a) ++b;
    if (b < 126) {
        double mid = 0.5 * (oracle_e4m3_value(b) + oracle_e4m3_value(b + 1)) * kS;
        if (a > mid || (a == mid && (b & 1))) ++b; /* ties to the even byte */
    }
    return b == 0 ? 1 : b;
}

/* Straight-through estimator for fake-quant training ([QAD] sec. 3.2: the forward pass goes
 * through the quantiser, the backward pass hands the gradient straight back; in practice
 * the gradient is clamped to a reasonable range; sec. 4.1: the scale is smoothed with a
 * moving average, momentum about 0.9). Readings: the backward clamps each gradient value to
 * [-c, c] (c = +inf: identity), in fp32 after widening, with bf16 output rounded to nearest
 * even; the moving average is kept on the per-tensor fp32 scale S as
 * S = fmaf(m, S, fp32(fp32(1 - m) * S_batch)). */
float oracle_ste_clamp(float g, float c)
{
    if (g > c) return c;
    if (g < -c) return -c;
    return g;
}

float oracle_scale_ema(float S_prev, float S_batch, float m)
{
    float a = 1.0f - m;
    float b = a * S_batch;
    return fmaf(m, S_prev, b);
}

/* Static activation calibration ([BT] "Calibration": feed representative inputs, record the
 * activation distribution, pick a clipping range -- min/max, or percentile / histogram
 * methods that clip a few outliers -- then scale each block). Reading: an exact histogram
 * of |x| with one bin per bf16 magnitude, bin = (fp32 bits of |x|) >> 16 (32768 bins),
 * accumulated over calibration batches; the clip value for a fraction p in (0, 1] is the
 * lower edge of the first bin whose cumulative count reaches ceil(p N), i.e. the k-th
 * smallest magnitude rounded toward zero to bf16 (exact for bf16 data; p = 1 gives amax);
 * the tensor scale is the tensor-scale formula applied to the clip value. */
void oracle_calib_histogram(const float *x, int64_t n, uint64_t *hist)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        hist[(u & 0x7FFFFFFFu) >> 16] += 1;
    }
}

float oracle_calib_scale(const uint64_t *hist, double fraction)
{
    uint64_t total = 0;
    for (int b = 0; b < 32768; ++b) total += hist[b];
    if (total == 0) return 1.0f;
    uint64_t k = (uint64_t)ceil(fraction * (double)total);
    if (k < 1) k = 1;
    if (k > total) k = total;
    uint64_t cum = 0;
    int b = 0;
    for (; b < 32768; ++b) {
        cum += hist[b];
        if (cum >= k) break;
    }
    uint32_t u = (uint32_t)b << 16;
    float clip;
    memcpy(&clip, &u, 4);
    if (clip == 0.0f) return 1.0f;
    float S = clip / 2688.0f;
    if (S < FLT_MIN) S = FLT_MIN;
    return S;
}

int oracle_max_byte(float amax, float S)
{
    return oracle_byte_for_divisor(amax, S, 6.0);
}

/* A block byte as an E4M3FN magnitude: the sign bit plays no part in a scale, and 0x7F is
 * NaN, not one of the 126 candidates; such a block (like an all-zero one, byte 0) is coded
 * as zeros. Bytes 0x00..0x7E are returned unchanged. */
static int given_byte(int byte)
{
    int m = byte & 0x7F;
    return m == 0x7F ? 0 : m;
}

/* E2M1 code of x under block byte `byte` and tensor scale S: round half to even on the
 * exact ratio |x| / (s S), saturating at 6 ([QAD] sec. 2.1). */
int oracle_e2m1_code(float x, int byte, float S)
{
    byte = given_byte(byte);
    if (byte == 0) return 0;
    double ax = fabs((double)x);
    double sS = oracle_e4m3_value(byte) * (double)S; /* exact, <= 28 bits */
    int k = 0; /* largest index whose grid value * sS <= |x| */
    while (k < 7 && E2M1_MAG[k + 1] * sS <= ax) ++k;
    if (k < 7) {
        double mid = 0.5 * (E2M1_MAG[k] + E2M1_MAG[k + 1]) * sS;
        if (ax > mid || (ax == mid && (k & 1))) ++k; /* ties to the even index */
    }
    return (x < 0.0f && k > 0) ? (8 | k) : k;
}

/* Dequantised value: +-fp32(G_k * s * S), a single rounding of the exact product
 * ([QAD] sec. 3.2: the quantised value times its scale). */
float oracle_dequant_value(int code, int byte, float S)
{
    int k = code & 7;
    byte = given_byte(byte);
    if (byte == 0 || k == 0) return 0.0f;
    double mag = E2M1_MAG[k] * oracle_e4m3_value(byte) * (double)S; /* exact */
    float d = (float)mag;
    return (code & 8) ? -d : d;
}

static float block_amax(const float *x)
{
    float m = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float a = fabsf(x[i]);
        if (a > m) m = a;
    }
    return m;
}

/* Max-scaling bytes for a row-major [rows, cols] tensor, blocks of 16 along cols
 * ([BT] "Block scaling"). scales is [rows, cols/16]. */
void oracle_scales_max(const float *x, int64_t rows, int64_t cols, float S, uint8_t *scales)
{
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            scales[r * nb + b] = (uint8_t)oracle_max_byte(block_amax(x + r * cols + b * 16), S);
}

/* Packed codes [rows, cols/2]: element 2j in the low nibble of byte j. */
void oracle_quantize(const float *x, int64_t rows, int64_t cols, float S,
                     const uint8_t *scales, uint8_t *codes)
{
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; c += 2) {
            int byte = scales[r * nb + c / 16];
            int lo = oracle_e2m1_code(x[r * cols + c], byte, S);
            int hi = oracle_e2m1_code(x[r * cols + c + 1], byte, S);
            codes[(r * cols + c) / 2] = (uint8_t)(lo | (hi << 4));
        }
}

void oracle_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                       int64_t cols, float S, float *y)
{
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int byte = scales[r * nb + c / 16];
            uint8_t pair = codes[(r * cols + c) / 2];
            int code = (c & 1) ? (pair >> 4) : (pair & 15);
            y[r * cols + c] = oracle_dequant_value(code, byte, S);
        }
}

/* Squared weight error of one block under byte `byte` (the MSE objective; [LH] the MSE
 * selector keeps the scale with the smallest weight error). fp32, fixed order. */
float oracle_block_sq_error(const float *x, int byte, float S)
{
    float acc = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float dq = oracle_dequant_value(oracle_e2m1_code(x[i], byte, S), byte, S);
        float e = dq - x[i];
        acc = fmaf(e, e, acc);
    }
    return acc;
}

/* MSE scale search: every positive E4M3 byte 0x01..0x7E is tried on every block; the
 * first byte with the smallest objective wins ([LH] the MSE selector). obj may be NULL. */
void oracle_scales_mse(const float *w, int64_t rows, int64_t cols, float S,
                       uint8_t *scales, float *obj)
{
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *x = w + r * cols + b * 16;
            int best_b = 0;
            float best = 0.0f;
            if (block_amax(x) != 0.0f) {
                best = INFINITY;
                for (int c = 1; c <= 126; ++c) {
                    float e = oracle_block_sq_error(x, c, S);
                    if (e < best) {
                        best = e;
                        best_b = c;
                    }
                }
            }
            scales[r * nb + b] = (uint8_t)best_b;
            if (obj) obj[r * nb + b] = best;
        }
}

/* Block-diagonal Gram matrix H_b = sum_t x_t,b x_t,b^T for every 16-channel block b
 * ([LH] "Change the objective": XX^T weighs the output error; only its 16x16 diagonal
 * blocks are kept). X is row-major [tokens, cols] (one token per row). If token_ids is
 * non-NULL only those rows are summed, in the order given. Accumulates in double over
 * ascending position into H [cols/16][16][16] (which is overwritten). */
/* Four Over Six ([LH], the paragraph on max / Four-Over-Six / MSE selection: one of two
 * candidate scales per block). Reading (the page names only "two candidates"): the bytes
 * nearest amax_b / (6 S) and amax_b / (4 S), i.e. the block max on the E2M1 magnitudes 6
 * and 4; the one with the smaller MSE objective (as in oracle_scales_mse) wins, ties to
 * the smaller byte. An all-zero block gets 0x00 and objective 0. */
void oracle_scales_four_over_six(const float *w, int64_t rows, int64_t cols, float S,
                                 uint8_t *scales, float *obj)
{
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *x = w + r * cols + b * 16;
            float amax = block_amax(x);
            int best_b = 0;
            float best = 0.0f;
            if (amax != 0.0f) {
                int c6 = oracle_byte_for_divisor(amax, S, 6.0);
                int c4 = oracle_byte_for_divisor(amax, S, 4.0);
                float e6 = oracle_block_sq_error(x, c6, S);
                float e4 = oracle_block_sq_error(x, c4, S);
                /* c4 >= c6; on equal objectives the smaller byte wins */
                if (e4 < e6) {
                    best_b = c4;
                    best = e4;
                } else {
                    best_b = c6;
                    best = e6;
                }
            }
            scales[r * nb + b] = (uint8_t)best_b;
            if (obj) obj[r * nb + b] = best;
        }
}

void oracle_block_hessian(const float *X, int64_t tokens, int64_t cols,
                          const int32_t *token_ids, int64_t n_ids, double *H)
{
    int64_t nb = cols / 16;
    int64_t n = token_ids ? n_ids : tokens;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        double *h = H + b * 256;
        for (int i = 0; i < 256; ++i) h[i] = 0.0;
        for (int64_t p = 0; p < n; ++p) {
            int64_t t = token_ids ? token_ids[p] : p;
            const float *x = X + t * cols + b * 16;
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; ++j) h[i * 16 + j] += (double)x[i] * (double)x[j];
        }
    }
}

/* Local-Hessian objective of one block under byte `byte`: d H d^T with d the fp32 weight
 * error and H the block's 16x16 matrix (fp32 input, evaluated in double). */
double oracle_block_lh_objective(const float *w, int byte, float S, const float *Hb)
{
    double d[16];
    for (int i = 0; i < 16; ++i) {
        float dq = oracle_dequant_value(oracle_e2m1_code(w[i], byte, S), byte, S);
        d[i] = (double)(dq - w[i]); /* fp32 subtraction, widened exactly */
    }
    double obj = 0.0;
    for (int i = 0; i < 16; ++i) {
        double y = 0.0;
        for (int j = 0; j < 16; ++j) y = fma((double)Hb[i * 16 + j], d[j], y);
        obj = fma(d[i], y, obj);
    }
    return obj;
}

/* Local-Hessian scale search ([LH] "Change the objective"): for every (row, block), all
 * 126 positive E4M3 bytes are tried and the first byte with the smallest d H_b d^T wins.
 * H is [cols/16][16][16] fp32, shared by every row. An all-zero H_b falls back to the MSE
 * choice. obj (NULL allowed) receives the winning objective. */
void oracle_scales_local_hessian(const float *w, int64_t rows, int64_t cols, float S,
                                 const float *H, uint8_t *scales, double *obj)
{
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *x = w + r * cols + b * 16;
            const float *Hb = H + b * 256;
            int zero_h = 1;
            for (int i = 0; i < 256; ++i)
                if (Hb[i] != 0.0f) zero_h = 0;
            int best_b = 0;
            double best = 0.0;
            if (block_amax(x) != 0.0f) {
                if (zero_h) {
                    float bm = INFINITY;
                    for (int c = 1; c <= 126; ++c) {
                        float e = oracle_block_sq_error(x, c, S);
                        if (e < bm) {
                            bm = e;
                            best_b = c;
                        }
                    }
                } else {
                    best = INFINITY;
                    for (int c = 1; c <= 126; ++c) {
                        double o = oracle_block_lh_objective(x, c, S, Hb);
                        if (o < best) {
                            best = o;
                            best_b = c;
                        }
                    }
                }
            }
            scales[r * nb + b] = (uint8_t)best_b;
            if (obj) obj[r * nb + b] = zero_h ? 0.0 : best;
        }
}

/* Token lists per expert from a top-k routing table expert_ids [tokens, topk]:
 * offsets [experts + 1] (prefix sums of the counts) and token_ids [tokens * topk], each
 * expert's tokens in ascending token order. Returns 0, or -1 on an id out of range. */
int oracle_route_groups(const int32_t *expert_ids, int64_t tokens, int64_t topk,
                        int64_t experts, int32_t *offsets, int32_t *token_ids)
{
    for (int64_t e = 0; e <= experts; ++e) offsets[e] = 0;
    for (int64_t i = 0; i < tokens * topk; ++i) {
        int32_t e = expert_ids[i];
        if (e < 0 || e >= experts) return -1;
        offsets[e + 1] += 1;
    }
    for (int64_t e = 0; e < experts; ++e) offsets[e + 1] += offsets[e];
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(experts > 0 ? experts : 1));
    if (!fill) return -1;
    for (int64_t e = 0; e < experts; ++e) fill[e] = offsets[e];
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t k = 0; k < topk; ++k) {
            int32_t e = expert_ids[t * topk + k];
            token_ids[fill[e]++] = (int32_t)t;
        }
    free(fill);
    return 0;
}

/* ------------------------------------------------------------------ GPTQ ([LH] "Change the
 * objective" gives the layer-output error tr(dW X X^T dW^T); the closing paragraphs of the
 * same page say GPTQ changes the rounding where Local-Hessian changes the scale, and that
 * the two can be combined. GPTQ itself is Frantar et al., 2022.) */

/* Full Gram matrix H[i][j] = sum_t x[t][i] x[t][j], double, ascending t (all of X X^T; the
 * Local-Hessian search uses only its 16x16 diagonal blocks). */
void oracle_full_hessian(const float *X, int64_t tokens, int64_t cols, double *H)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < cols; ++i)
        for (int64_t j = i; j < cols; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < tokens; ++t)
                acc += (double)X[t * cols + i] * (double)X[t * cols + j];
            H[i * cols + j] = acc;
            H[j * cols + i] = acc;
        }
}

/* E2M1 code of a double value: the element rule above (round half to even on the exact
 * ratio |v| / (s S), saturating at 6), applied to GPTQ's updated weights, which are not fp32.
 * The products mid * s * S are exact in double, so the comparisons are exact. */
int oracle_e2m1_code_d(double v, int byte, float S)
{
    byte = given_byte(byte);
    if (byte == 0) return 0;
    double av = fabs(v);
    double sS = oracle_e4m3_value(byte) * (double)S;
    int k = 0;
    while (k < 7 && E2M1_MAG[k + 1] * sS <= av) ++k;
    if (k < 7) {
        double mid = 0.5 * (E2M1_MAG[k] + E2M1_MAG[k + 1]) * sS;
        if (av > mid || (av == mid && (k & 1))) ++k;
    }
    return (v < 0.0 && k > 0) ? (8 | k) : k;
}

/* Lower Cholesky factor in place (A = L L^T, lower triangle read); returns 0, or 1 + the
 * first column whose pivot is not positive. */
static int64_t chol_lower(double *A, int64_t n)
{
    for (int64_t j = 0; j < n; ++j) {
        double d = A[j * n + j];
        for (int64_t k = 0; k < j; ++k) d -= A[j * n + k] * A[j * n + k];
        if (!(d > 0.0)) return 1 + j;
        double ljj = sqrt(d);
        A[j * n + j] = ljj;
#pragma omp parallel for schedule(static)
        for (int64_t i = j + 1; i < n; ++i) {
            double s = A[i * n + j];
            for (int64_t k = 0; k < j; ++k) s -= A[i * n + k] * A[j * n + k];
            A[i * n + j] = s / ljj;
        }
    }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = i + 1; j < n; ++j) A[i * n + j] = 0.0;
    return 0;
}

/* GPTQ's factor: U upper triangular with U^T U = (H + lambda I)^{-1}, computed the way the
 * algorithm states it: Cholesky of the damped H, its inverse, then the upper Cholesky
 * factor of that inverse. lambda = damp * (sum_j H_jj, index order) / n; an all-zero
 * diagonal (all-zero inputs) gives H + lambda I := I, so GPTQ reduces to plain rounding.
 * H is read from its lower triangle. Returns 0, or 1 + a failing pivot's column. */
int64_t oracle_gptq_factor(const double *H, int64_t n, double damp, double *U)
{
    double *L = (double *)malloc(sizeof(double) * n * n);
    double *Li = (double *)malloc(sizeof(double) * n * n); /* row c = column c of L^{-1} */
    if (!L || !Li) { free(L); free(Li); return -1; }
    double tr = 0.0;
    for (int64_t j = 0; j < n; ++j) tr += H[j * n + j];
    double lambda = damp * (tr / (double)n);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            double h = tr == 0.0 ? (i == j ? 1.0 : 0.0) : H[i * n + j];
            L[i * n + j] = (i == j && tr != 0.0) ? h + lambda : h;
        }
    int64_t rc = chol_lower(L, n);
    if (rc) { free(L); free(Li); return rc; }
    /* columns of L^{-1} by forward substitution: y_c = 1 / L_cc, y_i = -(sum_k L_ik y_k) / L_ii */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t c = 0; c < n; ++c) {
        double *y = Li + c * n;
        for (int64_t i = 0; i < c; ++i) y[i] = 0.0;
        y[c] = 1.0 / L[c * n + c];
        for (int64_t i = c + 1; i < n; ++i) {
            double s = 0.0;
            for (int64_t k = c; k < i; ++k) s += L[i * n + k] * y[k];
            y[i] = -s / L[i * n + i];
        }
    }
    /* Hinv = L^{-T} L^{-1}: Hinv_ij = sum_{k >= max(i,j)} (L^{-1})_ki (L^{-1})_kj, lower part */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            double s = 0.0;
            for (int64_t k = i; k < n; ++k) s += Li[i * n + k] * Li[j * n + k];
            L[i * n + j] = s;
        }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = i + 1; j < n; ++j) L[i * n + j] = 0.0;
    rc = chol_lower(L, n); /* Hinv = L2 L2^T, so U = L2^T */
    if (!rc)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t j = 0; j < n; ++j) U[i * n + j] = L[j * n + i];
    free(L);
    free(Li);
    return rc;
}

/* The other rounding of v at a near-tie: the grid neighbour of `code` on the side of |v|
 * (a value within a hair of a midpoint may round either way once the sums that made it are
 * reordered). Same sign as v; a zero magnitude carries none (R6); saturated codes and an
 * all-zero block keep their code. */
static int oracle_other_rounding(double v, int code, int byte, float S)
{
    if (byte == 0) return code;
    double sS = oracle_e4m3_value(byte) * (double)S;
    double ax = fabs(v), g = E2M1_MAG[code & 7] * sS;
    int k = code & 7, alt = k;
    if (ax > g && k < 7) alt = k + 1;
    else if (ax < g && k > 0) alt = k - 1;
    return alt == 0 ? 0 : (alt | (v < 0 ? 8 : 0));
}

/* GPTQ's column loop for each row (rows are independent): v = w; for j = 0..n-1 the code
 * of v_j is taken at the block's byte and S, e = (v_j - q_j) / U_jj with q_j the exact
 * dequantised value, and v_k -= e U_jk for every k > j. codes use the packed layout;
 * vout (optional) receives each v_j as it was rounded. flips (optional, [rows][nflip],
 * -1 = unused) names columns where the row takes the other rounding instead (test use:
 * following a row past a near-tie that was resolved the other way). */
void oracle_gptq_rows_flip(const float *w, int64_t rows, int64_t n, float S,
                           const uint8_t *scales, const double *U, uint8_t *codes, double *vout,
                           const int64_t *flips, int64_t nflip)
{
    int64_t nb = n / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        double *v = (double *)malloc(sizeof(double) * n);
        for (int64_t k = 0; k < n; ++k) v[k] = (double)w[r * n + k];
        for (int64_t j = 0; j < n; ++j) {
            int byte = given_byte(scales[r * nb + j / 16]);
            int code = oracle_e2m1_code_d(v[j], byte, S);
            if (flips)
                for (int64_t f = 0; f < nflip; ++f)
                    if (flips[r * nflip + f] == j) code = oracle_other_rounding(v[j], code, byte, S);
            if (vout) vout[r * n + j] = v[j];
            double q = E2M1_MAG[code & 7] * oracle_e4m3_value(byte) * (double)S; /* exact */
            if (code & 8) q = -q;
            double e = (v[j] - q) / U[j * n + j];
            for (int64_t k = j + 1; k < n; ++k) v[k] -= e * U[j * n + k];
            uint8_t *cb = codes + r * (n / 2) + j / 2;
            if (j & 1) *cb = (uint8_t)((*cb & 0x0F) | (code << 4));
            else *cb = (uint8_t)code;
        }
        free(v);
    }
}

void oracle_gptq_rows(const float *w, int64_t rows, int64_t n, float S, const uint8_t *scales,
                      const double *U, uint8_t *codes, double *vout)
{
    oracle_gptq_rows_flip(w, rows, n, S, scales, U, codes, vout, NULL, 0);
}

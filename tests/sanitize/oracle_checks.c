/* The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every function on
 * small seeded inputs that include zeros, signed zeros, subnormals, large values, every
 * block byte 0x00..0xFF and routing ids out of range. Exit status 0 unless a result breaks
 * a basic range property; the sanitizers abort on any memory error or undefined behaviour. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_value(int byte);
double oracle_e2m1_value(int code);
uint16_t oracle_bf16_rne(float f);
void oracle_bf16_rne_array(const float *y, int64_t n, uint16_t *out);
float oracle_tensor_scale(const float *x, int64_t n);
int oracle_byte_for_divisor(float amax, float S, double k);
float oracle_ste_clamp(float g, float c);
float oracle_scale_ema(float S_prev, float S_batch, float m);
void oracle_calib_histogram(const float *x, int64_t n, uint64_t *hist);
float oracle_calib_scale(const uint64_t *hist, double fraction);
int oracle_max_byte(float amax, float S);
int oracle_e2m1_code(float x, int byte, float S);
float oracle_dequant_value(int code, int byte, float S);
void oracle_scales_max(const float *x, int64_t rows, int64_t cols, float S, uint8_t *scales);
void oracle_quantize(const float *x, int64_t rows, int64_t cols, float S, const uint8_t *scales,
                     uint8_t *codes);
void oracle_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       float S, float *out);
float oracle_block_sq_error(const float *x, int byte, float S);
void oracle_scales_mse(const float *w, int64_t rows, int64_t cols, float S, uint8_t *scales, float *obj);
void oracle_scales_four_over_six(const float *w, int64_t rows, int64_t cols, float S, uint8_t *scales,
                                 float *obj);
void oracle_block_hessian(const float *X, int64_t tokens, int64_t cols, const int32_t *token_ids,
                          int64_t n_ids, double *H);
double oracle_block_lh_objective(const float *w, int byte, float S, const float *Hb);
void oracle_scales_local_hessian(const float *w, int64_t rows, int64_t cols, float S, const float *H,
                                 uint8_t *scales, double *obj);
int oracle_route_groups(const int32_t *expert_ids, int64_t tokens, int64_t topk, int64_t experts,
                        int32_t *offsets, int32_t *token_ids);
void oracle_full_hessian(const float *X, int64_t tokens, int64_t cols, double *H);
int oracle_e2m1_code_d(double v, int byte, float S);
int64_t oracle_gptq_factor(const double *H, int64_t n, double damp, double *U);
void oracle_gptq_rows(const float *w, int64_t rows, int64_t n, float S, const uint8_t *scales,
                      const double *U, uint8_t *codes, double *vout);

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double uni(void) { /* xorshift64*, in [0, 1) */
    st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
    return (double)((st * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}

static void fill(float *x, int64_t n, double scale) {
    for (int64_t i = 0; i < n; ++i) {
        double u = uni();
        float v = (float)((2.0 * uni() - 1.0) * scale);
        if (u < 0.02) v = 0.0f;
        else if (u < 0.04) v = -0.0f;
        else if (u < 0.06) v = 1e-40f * (float)(1 + i % 7);   /* subnormal */
        else if (u < 0.07) v = (float)(scale * 1e3);
        x[i] = v;
    }
}

static int bad = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "line %d: %s\n", __LINE__, #c); ++bad; } } while (0)

int main(void) {
    enum { R = 24, C = 96, T = 200, NB = C / 16 };
    float *w = malloc(sizeof(float) * R * C), *x = malloc(sizeof(float) * T * C);
    fill(w, R * C, 0.05);
    fill(x, T * C, 1.0);
    float S = oracle_tensor_scale(w, R * C);
    CHECK(S > 0.0f);
    CHECK(oracle_tensor_scale(w, 0) == 1.0f);

    for (int b = 0; b < 256; ++b) {
        (void)oracle_e4m3_value(b);
        for (int k = 0; k < 16; ++k) {
            int c = oracle_e2m1_code(w[k], b, S);
            CHECK(c >= 0 && c < 16);
            (void)oracle_dequant_value(c, b, S);
            CHECK(oracle_e2m1_code_d((double)w[k] * 1.5, b, S) < 16);
        }
    }
    for (int c = 0; c < 16; ++c) (void)oracle_e2m1_value(c);
    uint16_t h[64];
    oracle_bf16_rne_array(w, 64, h);
    (void)oracle_bf16_rne(INFINITY);
    CHECK(oracle_byte_for_divisor(1.0f, 1e-30f, 6.0) == 126);
    CHECK(oracle_byte_for_divisor(1e-30f, 1.0f, 4.0) == 1);
    CHECK(oracle_max_byte(0.0f, S) == 0);
    (void)oracle_ste_clamp(NAN, 1.0f);
    (void)oracle_ste_clamp(-INFINITY, 1.0f);
    (void)oracle_scale_ema(1.0f, 2.0f, 0.9f);

    uint64_t *hist = calloc(32768, sizeof(uint64_t));
    oracle_calib_histogram(x, T * C, hist);
    CHECK(oracle_calib_scale(hist, 1.0) > 0.0f);
    (void)oracle_calib_scale(hist, 1e-9);
    memset(hist, 0, 32768 * sizeof(uint64_t));
    CHECK(oracle_calib_scale(hist, 0.5) == 1.0f);

    uint8_t *sc = malloc(R * NB), *codes = malloc(R * C / 2);
    float *dq = malloc(sizeof(float) * R * C), *obj = malloc(sizeof(float) * R * NB);
    double *objd = malloc(sizeof(double) * R * NB);
    oracle_scales_max(w, R, C, S, sc);
    oracle_quantize(w, R, C, S, sc, codes);
    oracle_dequantize(codes, sc, R, C, S, dq);
    for (int i = 0; i < R * NB; ++i) sc[i] = (uint8_t)(i * 37);   /* every byte value */
    oracle_quantize(w, R, C, S, sc, codes);
    oracle_dequantize(codes, sc, R, C, S, dq);
    oracle_scales_mse(w, R, C, S, sc, obj);
    for (int i = 0; i < R * NB; ++i) CHECK(sc[i] <= 126);
    (void)oracle_block_sq_error(w, 0x38, S);
    oracle_scales_four_over_six(w, R, C, S, sc, obj);

    double *H = malloc(sizeof(double) * NB * 256);
    float *Hf = malloc(sizeof(float) * NB * 256);
    oracle_block_hessian(x, T, C, NULL, 0, H);
    int32_t ids[50];
    for (int i = 0; i < 50; ++i) ids[i] = (i * 7) % T;
    oracle_block_hessian(x, T, C, ids, 50, H);
    for (int i = 0; i < NB * 256; ++i) Hf[i] = (float)H[i];
    for (int i = 0; i < 256; ++i) Hf[256 + i] = 0.0f;   /* a zero block: the MSE choice */
    oracle_scales_local_hessian(w, R, C, S, Hf, sc, objd);
    (void)oracle_block_lh_objective(w, 0x40, S, Hf);

    int32_t eids[T * 2], off[9], tok[T * 2];
    for (int i = 0; i < T * 2; ++i) eids[i] = (int32_t)(uni() * 8);
    CHECK(oracle_route_groups(eids, T, 2, 8, off, tok) == 0);
    eids[5] = 9;
    CHECK(oracle_route_groups(eids, T, 2, 8, off, tok) != 0);

    enum { N = 48 };
    double *G = malloc(sizeof(double) * N * N), *U = malloc(sizeof(double) * N * N);
    oracle_full_hessian(x, T, N, G);
    CHECK(oracle_gptq_factor(G, N, 0.01, U) == 0);
    memset(G, 0, sizeof(double) * N * N);
    CHECK(oracle_gptq_factor(G, N, 0.01, U) == 0);
    for (int i = 0; i < N * N; ++i) G[i] = (i % (N + 1) == 0) ? -1.0 : 0.0;
    CHECK(oracle_gptq_factor(G, N, 0.0, U) != 0);
    oracle_full_hessian(x, T, N, G);
    CHECK(oracle_gptq_factor(G, N, 0.01, U) == 0);
    float *wg = malloc(sizeof(float) * 5 * N);
    uint8_t *scg = malloc(5 * N / 16), *cg = malloc(5 * N / 2);
    double *vout = malloc(sizeof(double) * 5 * N);
    fill(wg, 5 * N, 0.05);
    for (int i = 0; i < 5 * N / 16; ++i) scg[i] = (uint8_t)(0x30 + 41 * i);
    oracle_gptq_rows(wg, 5, N, S, scg, U, cg, vout);
    oracle_gptq_rows(wg, 5, N, S, scg, U, cg, NULL);

    free(w); free(x); free(hist); free(sc); free(codes); free(dq); free(obj); free(objd);
    free(H); free(Hf); free(G); free(U); free(wg); free(scg); free(cg); free(vout);
    if (bad) { fprintf(stderr, "%d check(s) failed\n", bad); return 1; }
    printf("oracle checks passed\n");
    return 0;
}

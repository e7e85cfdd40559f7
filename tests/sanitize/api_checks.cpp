// Host-side checks of libnvfp4's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer:
// every entry point's argument validation and every workspace-size query, with bad, extreme
// and empty arguments. No call here reaches a kernel launch (validation fails first, or the
// tensor is empty), so the program needs no GPU. Exit status 0 when every return code is
// the documented one; the sanitizers abort on any memory error or undefined behaviour.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nvfp4.h"

static int failures = 0;

#define EXPECT(call, want)                                                                   \
  do {                                                                                       \
    const int got_ = (call);                                                                 \
    if (got_ != (want)) {                                                                    \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, want); \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

int main() {
  // never dereferenced: validation rejects the call or returns before any use
  void *F = reinterpret_cast<void *>(uintptr_t(0x7F0000000000ull));
  char *Fc = static_cast<char *>(F);
  const float *S = static_cast<const float *>(F);
  uint8_t *B = static_cast<uint8_t *>(F);
  const int64_t big = INT64_MAX, neg = -1;

  for (int s = -3; s < 12; ++s)
    if (!nvfp4_status_string(s) || !strlen(nvfp4_status_string(s))) ++failures;
  EXPECT(nvfp4_version(), 100);

  // tensor scale
  EXPECT(nvfp4_global_scale(F, 1, 1, 12, (float *)F, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_global_scale(F, 5, 1, 16, (float *)F, nullptr), NVFP4_ERR_DTYPE);
  EXPECT(nvfp4_global_scale(F, 1, big, big, (float *)F, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_global_scale(F, 1, neg, 16, (float *)F, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_global_scale(Fc + 2, 1, 1, 16, (float *)F, nullptr), NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_global_scale(F, 1, 1, 16, nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_global_scale(nullptr, 1, 0, 16, nullptr, nullptr), NVFP4_OK);
  {
    const size_t need = nvfp4_global_scale_workspace_size(1, 1 << 20);
    EXPECT(nvfp4_global_scale_ws(F, 1, 1, 12, (float *)F, F, need, nullptr), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_global_scale_ws(F, 1, big, big, (float *)F, F, need, nullptr), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_global_scale_ws(F, 1, 1, 1 << 20, (float *)F, nullptr, need, nullptr), NVFP4_ERR_WORKSPACE);
    EXPECT(nvfp4_global_scale_ws(F, 1, 1, 1 << 20, (float *)F, F, need - 1, nullptr), NVFP4_ERR_WORKSPACE);
    EXPECT(nvfp4_global_scale_ws(F, 1, 1, 1 << 20, (float *)F, Fc + 2, need, nullptr), NVFP4_ERR_ALIGN);
    EXPECT(nvfp4_global_scale_ws(nullptr, 1, 0, 16, nullptr, nullptr, 0, nullptr), NVFP4_OK);
  }

  // searches and quantisation: shapes, dtypes, nulls, alignment, overflow, empty tensors
  const int64_t shapes[][3] = {{1, 4, 17}, {neg, 4, 16}, {1, neg, 16}, {1, 4, neg},
                               {big, big, 16}, {1, big, big}, {1 << 20, 1 << 20, 1 << 20},
                               {70000, 1, 16}};
  for (auto &sh : shapes) {
    EXPECT(nvfp4_scale_search_max(F, 1, sh[0], sh[1], sh[2], S, B, nullptr), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_scale_search_mse(F, 1, sh[0], sh[1], sh[2], S, B, nullptr, nullptr), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_scale_search_four_over_six(F, 1, sh[0], sh[1], sh[2], S, B, nullptr, nullptr),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_scale_search_local_hessian(F, 1, sh[0], sh[1], sh[2], S, S, B, nullptr, nullptr),
           NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_quantize(F, 1, sh[0], sh[1], sh[2], S, nullptr, B, nullptr, nullptr), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_dequantize(B, B, S, sh[0], sh[1], sh[2], F, 1, nullptr), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_fakequant(F, 1, sh[0], sh[1], sh[2], S, nullptr, F, nullptr, nullptr, nullptr),
           NVFP4_ERR_SHAPE);
  }
  EXPECT(nvfp4_fakequant(F, 9, 1, 4, 16, S, nullptr, F, nullptr, nullptr, nullptr), NVFP4_ERR_DTYPE);
  EXPECT(nvfp4_fakequant(nullptr, 1, 1, 4, 16, S, nullptr, F, nullptr, nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_fakequant(F, 1, 1, 4, 16, nullptr, nullptr, F, nullptr, nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_fakequant(F, 1, 1, 4, 16, S, nullptr, nullptr, nullptr, nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_fakequant(Fc + 8, 1, 1, 4, 16, S, nullptr, F, nullptr, nullptr, nullptr), NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_fakequant(F, 1, 1, 4, 16, S, nullptr, F, B + 4, nullptr, nullptr), NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_quantize(F, 1, 1, 4, 16, S, nullptr, B + 2, nullptr, nullptr), NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_scale_search_mse(F, 1, 1, 4, 16, S, B, (float *)(Fc + 2), nullptr), NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_scale_search_local_hessian(F, 1, 1, 4, 16, S, nullptr, B, nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_scale_search_local_hessian(F, 1, 1, 4, 16, S, S, B, (double *)(Fc + 4), nullptr),
         NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_fakequant(nullptr, 1, 1, 0, 16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), NVFP4_OK);
  EXPECT(nvfp4_scale_search_mse(nullptr, 0, 0, 4, 16, nullptr, nullptr, nullptr, nullptr), NVFP4_OK);
  EXPECT(nvfp4_dequantize(nullptr, nullptr, nullptr, 1, 4, 0, nullptr, 0, nullptr), NVFP4_OK);

  // training support and calibration
  EXPECT(nvfp4_ste_backward(F, 1, 12, 1.0f, F, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_ste_backward(F, 1, 16, 0.0f, F, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_ste_backward(F, 1, 16, __builtin_nanf(""), F, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_ste_backward(F, 1, 16, 1.0f, nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_ste_backward(nullptr, 1, 0, 1.0f, nullptr, nullptr), NVFP4_OK);
  EXPECT(nvfp4_scale_ema((float *)F, S, neg, 0.9f, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_scale_ema((float *)F, S, 4, 1.5f, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_scale_ema((float *)F, S, 0, 0.5f, nullptr), NVFP4_OK);
  EXPECT(nvfp4_calib_histogram(F, 1, 12, (uint64_t *)F, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_calib_histogram(F, 1, 16, nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_calib_histogram(F, 1, 16, (uint64_t *)(Fc + 4), nullptr), NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_calib_histogram(nullptr, 1, 0, (uint64_t *)F, nullptr), NVFP4_OK);
  EXPECT(nvfp4_calib_scale((const uint64_t *)F, 0.0, (float *)F, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_calib_scale((const uint64_t *)F, 2.0, (float *)F, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_calib_scale((const uint64_t *)F, __builtin_nan(""), (float *)F, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_calib_scale(nullptr, 0.5, (float *)F, nullptr), NVFP4_ERR_NULL);

  // workspace sizes: extreme and negative arguments must not overflow
  const int64_t dims[] = {neg, 0, 1, 15, 16, 4096, 131072, 1ll << 31, 1ll << 40, big};
  for (int64_t a : dims)
    for (int64_t b : dims) {
      (void)nvfp4_block_hessian_workspace_size(a, b, 1, 0);
      (void)nvfp4_block_hessian_workspace_size(a, 2048, b, a);
      (void)nvfp4_route_groups_workspace_size(a, 8, b);
      (void)nvfp4_gptq_workspace_size(a, b);
      (void)nvfp4_gptq_factor_workspace_size(b);
      (void)nvfp4_global_scale_workspace_size(a, b);
    }

  // block Hessian (workspace and allocation-free forms)
  const size_t need = nvfp4_block_hessian_workspace_size(4096, 512, 1, 0);
  if (need == 0) ++failures;
  float *H = static_cast<float *>(F);
  EXPECT(nvfp4_block_hessian(F, 1, 4096, 512, 1, nullptr, nullptr, 0, H, 0, F, need - 1, nullptr),
         NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_block_hessian(F, 1, 4096, 512, 1, nullptr, nullptr, 0, H, 0, nullptr, need, nullptr),
         NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_block_hessian(F, 1, 4096, 512, 2, nullptr, nullptr, 0, H, 0, F, need, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_block_hessian(F, 1, 4096, 500, 1, nullptr, nullptr, 0, H, 0, F, need, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_block_hessian(F, 1, big, big, 1, nullptr, nullptr, 0, H, 0, F, need, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_block_hessian(F, 1, 4096, 512, 2, (const int32_t *)F, nullptr, 10, H, 0, F, need, nullptr),
         NVFP4_ERR_NULL);
  EXPECT(nvfp4_block_hessian(F, 1, 4096, 512, 1, nullptr, nullptr, 0, H, 0, Fc + 16, need, nullptr),
         NVFP4_ERR_ALIGN);
  EXPECT(nvfp4_block_hessian(F, 1, 4096, 0, 1, nullptr, nullptr, 0, nullptr, 0, nullptr, 0, nullptr), NVFP4_OK);
  EXPECT(nvfp4_block_hessian_noalloc(F, 1, 1ll << 20, 16384, 1, nullptr, nullptr, 0, H, 0, nullptr),
         NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_block_hessian_noalloc(F, 7, 4096, 512, 1, nullptr, nullptr, 0, H, 0, nullptr), NVFP4_ERR_DTYPE);
  EXPECT(nvfp4_block_hessian_noalloc(F, 1, 4096, 512, 1, nullptr, nullptr, 0, nullptr, 0, nullptr), NVFP4_ERR_NULL);

  // routing
  const size_t rneed = nvfp4_route_groups_workspace_size(1000, 8, 128);
  int32_t *I = static_cast<int32_t *>(F);
  EXPECT(nvfp4_route_groups(I, 1000, 8, 0, I, I, F, rneed, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_route_groups(I, 1000, 8, 20000, I, I, F, rneed, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_route_groups(I, 1000, 8, 128, I, I, F, rneed - 1, nullptr), NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_route_groups(I, big, big, 128, I, I, F, rneed, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_route_groups(I, 1000, 8, 128, nullptr, I, F, rneed, nullptr), NVFP4_ERR_NULL);

  // GPTQ: full Gram matrix, factor, rounding
  EXPECT(nvfp4_full_hessian(F, 1, 100, 48, H, 0, nullptr, 0, nullptr), NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_full_hessian(F, 1, 100, 50, H, 0, F, 1 << 30, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_full_hessian(F, 1, 100, 1 << 20, H, 0, F, 1 << 30, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_full_hessian(F, 1, big, 16, H, 0, F, 1 << 30, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gptq_factor(S, 50, 0.01, (double *)F, nullptr, F, 1 << 30, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gptq_factor(S, 64, -1.0, (double *)F, nullptr, F, 1 << 30, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_gptq_factor(S, 64, __builtin_inf(), (double *)F, nullptr, F, 1 << 30, nullptr), NVFP4_ERR_ARG);
  EXPECT(nvfp4_gptq_factor(S, 64, 0.01, (double *)F, nullptr, nullptr, 0, nullptr), NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_gptq_factor(S, 0, 0.01, nullptr, nullptr, nullptr, 0, nullptr), NVFP4_OK);
  EXPECT(nvfp4_gptq(F, 1, 64, 50, S, B, (const double *)F, B, F, 1 << 30, nullptr), NVFP4_ERR_SHAPE);
  EXPECT(nvfp4_gptq(F, 1, 64, 64, S, B, (const double *)F, B, nullptr, 0, nullptr), NVFP4_ERR_WORKSPACE);
  EXPECT(nvfp4_gptq(F, 1, 64, 64, S, nullptr, (const double *)F, B, F, 1 << 30, nullptr), NVFP4_ERR_NULL);

  // statistics switches (host state only) and the debug flag without the environment switch
  EXPECT(nvfp4_search_stats_enable(1), NVFP4_OK);
  EXPECT(nvfp4_search_stats_enable(0), NVFP4_OK);
  EXPECT(nvfp4_search_stats_read(nullptr, nullptr), NVFP4_ERR_NULL);
  EXPECT(nvfp4_debug_nonfinite(nullptr, nullptr), NVFP4_ERR_NULL);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("api checks passed\n");
  return 0;
}

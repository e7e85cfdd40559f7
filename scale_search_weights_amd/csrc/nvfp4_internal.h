// Internal launchers behind the C ABI (not exported). Arguments are validated by the
// entry points in nvfp4_api.hip before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

int launch_global_scale(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                        hipStream_t st);
size_t scale_workspace_size(int64_t batch, int64_t n);
int launch_global_scale_ws(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                             void *workspace, hipStream_t st);
int launch_quant(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                 const float *S, const uint8_t *scales_in, uint8_t *codes, uint8_t *scales_out,
                 void *y, hipStream_t st);
int launch_dequant(const uint8_t *codes, const uint8_t *scales, const float *S, int64_t batch,
                   int64_t rows, int64_t cols, void *y, int out_dtype, hipStream_t st);
int launch_ste_backward(const void *g, int dtype, int64_t n, float clip, void *out,
                        hipStream_t st);
int launch_scale_ema(float *S, const float *S_batch, int64_t batch, float m, hipStream_t st);
int launch_calib_histogram(const void *x, int dtype, int64_t n, unsigned long long *hist,
                           hipStream_t st);
int launch_calib_scale(const unsigned long long *hist, double fraction, float *S, hipStream_t st);
int launch_four_over_six(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         const float *S, uint8_t *scales, float *obj, hipStream_t st);
int launch_mse(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
               const float *S, uint8_t *scales, float *obj, hipStream_t st);
int launch_local_hessian(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         const float *S, const float *H, uint8_t *scales, double *obj,
                         hipStream_t st);

size_t hessian_workspace_size(int64_t tokens, int64_t cols, int64_t groups, int64_t n_ids);
int launch_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t groups,
                         const int32_t *group_offsets, const int32_t *token_ids, int64_t n_ids,
                         float *H, int accumulate, void *workspace, hipStream_t st);

int check_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t groups,
                        const int32_t *group_offsets, const int32_t *token_ids, int64_t n_ids,
                        const float *H, bool *empty);
int run_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t groups,
                      const int32_t *group_offsets, const int32_t *token_ids, int64_t n_ids,
                      float *H, int accumulate, void *workspace, void *stream);

void search_stats_enable(bool on);
int search_stats_read(int64_t *out, hipStream_t st);

bool debug_checks_enabled();
void debug_check_finite(const void *x, int dtype, int64_t n, hipStream_t st);
void debug_check_scale(const float *S, int64_t n, hipStream_t st);
int debug_read_flag(int32_t *out, hipStream_t st);

size_t gram_workspace_size(int64_t tokens, int64_t cols);
int launch_full_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, float *H,
                        int accumulate, void *workspace, hipStream_t st);
size_t gptq_factor_workspace_size(int64_t n);
int launch_gptq_factor(const float *H, int64_t n, double damp, double *U, int32_t *status,
                       void *workspace, hipStream_t st);
size_t gptq_rows_workspace_size(int64_t rows, int64_t n);
int launch_gptq_rows(const void *w, int dtype, int64_t rows, int64_t n, const float *S,
                     const uint8_t *scales, const double *U, uint8_t *codes, void *workspace,
                     hipStream_t st);

size_t route_workspace_size(int64_t tokens, int64_t topk, int64_t experts);
int launch_route_groups(const int32_t *expert_ids, int64_t tokens, int64_t topk, int64_t experts,
                        int32_t *offsets, int32_t *token_ids, void *workspace, hipStream_t st);

}  // namespace nvfp4

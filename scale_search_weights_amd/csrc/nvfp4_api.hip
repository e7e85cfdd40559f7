// C-ABI entry points of libnvfp4 (declared in include/nvfp4.h). Each validates its
// arguments on the host — dtype, shape, pointer presence and alignment, workspace size —
// before anything is launched, then forwards to the kernel launchers.
#include <limits.h>

#include "nvfp4_internal.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxGridY = 65535;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// shape checks shared by the tensor entry points; *empty is set if there is nothing to do
int check_tensor(int dtype, int64_t batch, int64_t rows, int64_t cols, bool *empty) {
  if (dtype != NVFP4_DTYPE_F32 && dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_DTYPE;
  if (batch < 0 || rows < 0 || cols < 0 || (cols % 16) != 0) return NVFP4_ERR_SHAPE;
  int64_t n1, n2, bytes;
  if (!mul_ok(batch, rows, &n1) || !mul_ok(n1, cols, &n2) || !mul_ok(n2, 4, &bytes))
    return NVFP4_ERR_SHAPE;
  if (batch > kMaxGridY) return NVFP4_ERR_SHAPE;
  *empty = (n2 == 0);
  return NVFP4_OK;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

namespace nvfp4 {

// Host checks shared by the block-Hessian entry points (all but the workspace): *empty is
// set when there is nothing to launch.
int check_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t groups,
                        const int32_t *group_offsets, const int32_t *token_ids, int64_t n_ids,
                        const float *H, bool *empty) {
  *empty = false;
  if (dtype != NVFP4_DTYPE_F32 && dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_DTYPE;
  if (tokens < 0 || cols < 0 || (cols % 16) != 0 || groups < 0 || n_ids < 0)
    return NVFP4_ERR_SHAPE;
  int64_t t1, t2;
  if (!mul_ok(tokens, cols, &t1) || !mul_ok(t1, 4, &t2)) return NVFP4_ERR_SHAPE;
  if (groups > kMaxGridY || n_ids > INT32_MAX || tokens > INT32_MAX) return NVFP4_ERR_SHAPE;
  const bool grouped = group_offsets != nullptr || token_ids != nullptr;
  if (grouped && (!group_offsets || !token_ids)) return NVFP4_ERR_NULL;
  if (!grouped && groups != 1) return NVFP4_ERR_ARG;
  if (cols == 0 || groups == 0) {
    *empty = true;
    return NVFP4_OK;
  }
  if (!H || (tokens > 0 && !x)) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(H, 4) || !aligned(group_offsets, 4) || !aligned(token_ids, 4))
    return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int run_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t groups,
                      const int32_t *group_offsets, const int32_t *token_ids, int64_t n_ids,
                      float *H, int accumulate, void *workspace, void *stream) {
  const bool grouped = group_offsets != nullptr;
  debug_check_finite(x, dtype, tokens * cols, as_stream(stream));
  return launch_block_hessian(x, dtype, tokens, cols, groups, grouped ? group_offsets : nullptr,
                              grouped ? token_ids : nullptr, n_ids, H, accumulate, workspace,
                              as_stream(stream));
}

}  // namespace nvfp4

extern "C" {

const char *nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: bad dimension (negative, cols % 16 != 0, or too large)";
    case NVFP4_ERR_DTYPE: return "NVFP4_ERR_DTYPE: unknown dtype";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: pointer not aligned (16 B elements, 8 B codes)";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE: workspace missing or too small";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: a HIP launch failed";
    case NVFP4_ERR_ARG: return "NVFP4_ERR_ARG: argument out of range";
    default: return "unknown nvfp4 status";
  }
}

int nvfp4_version(void) { return 100; }

static int check_global_scale(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                              bool *empty) {
  *empty = false;
  if (dtype != NVFP4_DTYPE_F32 && dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_DTYPE;
  if (batch < 0 || n < 0 || (n % 8) != 0 || batch > kMaxGridY) return NVFP4_ERR_SHAPE;
  int64_t tot, bytes;
  if (!mul_ok(batch, n, &tot) || !mul_ok(tot, 4, &bytes)) return NVFP4_ERR_SHAPE;
  if (batch == 0) {
    *empty = true;
    return NVFP4_OK;
  }
  if (!S || (n > 0 && !x)) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(S, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int nvfp4_global_scale(const void *x, int dtype, int64_t batch, int64_t n, float *S, void *stream) {
  bool empty;
  const int rc = check_global_scale(x, dtype, batch, n, S, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  debug_check_finite(x, dtype, batch * n, as_stream(stream));
  return launch_global_scale(x, dtype, batch, n, S, as_stream(stream));
}

size_t nvfp4_global_scale_workspace_size(int64_t batch, int64_t n) {
  int64_t tot, bytes;
  if (batch <= 0 || n < 0 || (n % 8) != 0 || batch > kMaxGridY) return 0;
  if (!mul_ok(batch, n, &tot) || !mul_ok(tot, 4, &bytes)) return 0;
  return scale_workspace_size(batch, n);
}

int nvfp4_global_scale_ws(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                          void *workspace, size_t workspace_bytes, void *stream) {
  bool empty;
  const int rc = check_global_scale(x, dtype, batch, n, S, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!workspace || workspace_bytes < nvfp4_global_scale_workspace_size(batch, n))
    return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return NVFP4_ERR_ALIGN;
  debug_check_finite(x, dtype, batch * n, as_stream(stream));
  return launch_global_scale_ws(x, dtype, batch, n, S, workspace, as_stream(stream));
}

int nvfp4_scale_search_max(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                           const float *S, uint8_t *scales, void *stream) {
  bool empty = false;
  int rc = check_tensor(dtype, batch, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!w || !S || !scales) return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(S, 4)) return NVFP4_ERR_ALIGN;
  debug_check_finite(w, dtype, batch * rows * cols, as_stream(stream));
  debug_check_scale(S, batch, as_stream(stream));
  return launch_quant(w, dtype, batch, rows, cols, S, nullptr, nullptr, scales, nullptr,
                      as_stream(stream));
}

int nvfp4_scale_search_mse(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                           const float *S, uint8_t *scales, float *obj, void *stream) {
  bool empty = false;
  int rc = check_tensor(dtype, batch, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!w || !S || !scales) return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(S, 4) || !aligned(obj, 4)) return NVFP4_ERR_ALIGN;
  if (rows * (cols / 16) / 256 + 1 > (int64_t)UINT_MAX) return NVFP4_ERR_SHAPE;
  debug_check_finite(w, dtype, batch * rows * cols, as_stream(stream));
  debug_check_scale(S, batch, as_stream(stream));
  return launch_mse(w, dtype, batch, rows, cols, S, scales, obj, as_stream(stream));
}

int nvfp4_scale_search_four_over_six(const void *w, int dtype, int64_t batch, int64_t rows,
                                     int64_t cols, const float *S, uint8_t *scales, float *obj,
                                     void *stream) {
  bool empty = false;
  int rc = check_tensor(dtype, batch, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!w || !S || !scales) return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(S, 4) || !aligned(obj, 4)) return NVFP4_ERR_ALIGN;
  if (rows * (cols / 16) / 256 + 1 > (int64_t)UINT_MAX) return NVFP4_ERR_SHAPE;
  debug_check_finite(w, dtype, batch * rows * cols, as_stream(stream));
  debug_check_scale(S, batch, as_stream(stream));
  return launch_four_over_six(w, dtype, batch, rows, cols, S, scales, obj, as_stream(stream));
}

int nvfp4_ste_backward(const void *grad, int dtype, int64_t n, float clip, void *grad_out,
                       void *stream) {
  if (dtype != NVFP4_DTYPE_F32 && dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_DTYPE;
  if (n < 0 || (n % 8) != 0) return NVFP4_ERR_SHAPE;
  if (!(clip > 0.0f)) return NVFP4_ERR_ARG;  // also rejects NaN
  if (n == 0) return NVFP4_OK;
  if (!grad || !grad_out) return NVFP4_ERR_NULL;
  if (!aligned(grad, 16) || !aligned(grad_out, 16)) return NVFP4_ERR_ALIGN;
  debug_check_finite(grad, dtype, n, as_stream(stream));
  return launch_ste_backward(grad, dtype, n, clip, grad_out, as_stream(stream));
}

int nvfp4_scale_ema(float *S, const float *S_batch, int64_t batch, float momentum,
                    void *stream) {
  if (batch < 0) return NVFP4_ERR_SHAPE;
  if (!(momentum >= 0.0f && momentum <= 1.0f)) return NVFP4_ERR_ARG;
  if (batch == 0) return NVFP4_OK;
  if (!S || !S_batch) return NVFP4_ERR_NULL;
  if (!aligned(S, 4) || !aligned(S_batch, 4)) return NVFP4_ERR_ALIGN;
  return launch_scale_ema(S, S_batch, batch, momentum, as_stream(stream));
}

int nvfp4_calib_histogram(const void *x, int dtype, int64_t n, uint64_t *hist, void *stream) {
  if (dtype != NVFP4_DTYPE_F32 && dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_DTYPE;
  if (n < 0 || (n % 8) != 0) return NVFP4_ERR_SHAPE;
  if (!hist || (n > 0 && !x)) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(hist, 8)) return NVFP4_ERR_ALIGN;
  if (n == 0) return NVFP4_OK;
  debug_check_finite(x, dtype, n, as_stream(stream));
  return launch_calib_histogram(x, dtype, n, reinterpret_cast<unsigned long long *>(hist),
                                as_stream(stream));
}

int nvfp4_calib_scale(const uint64_t *hist, double fraction, float *S, void *stream) {
  if (!hist || !S) return NVFP4_ERR_NULL;
  if (!(fraction > 0.0 && fraction <= 1.0)) return NVFP4_ERR_ARG;
  if (!aligned(hist, 8) || !aligned(S, 4)) return NVFP4_ERR_ALIGN;
  return launch_calib_scale(reinterpret_cast<const unsigned long long *>(hist), fraction, S,
                            as_stream(stream));
}

size_t nvfp4_block_hessian_workspace_size(int64_t tokens, int64_t cols, int64_t groups,
                                          int64_t n_ids) {
  // 0 for arguments nvfp4_block_hessian rejects (every size below then fits in 64 bits)
  int64_t t1, t2;
  if (tokens < 0 || cols < 0 || groups < 0 || n_ids < 0) return 0;
  if (!mul_ok(tokens, cols, &t1) || !mul_ok(t1, 4, &t2)) return 0;
  if (groups > kMaxGridY || n_ids > INT32_MAX || tokens > INT32_MAX) return 0;
  const size_t dense = hessian_workspace_size(tokens, cols, groups, -1);
  const size_t grouped = hessian_workspace_size(tokens, cols, groups, n_ids);
  return dense > grouped ? dense : grouped;
}

int nvfp4_block_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t groups,
                        const int32_t *group_offsets, const int32_t *token_ids, int64_t n_ids,
                        float *H, int accumulate, void *workspace, size_t workspace_bytes,
                        void *stream) {
  bool empty = false;
  const int rc = check_block_hessian(x, dtype, tokens, cols, groups, group_offsets, token_ids,
                                     n_ids, H, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  const size_t need = nvfp4_block_hessian_workspace_size(tokens, cols, groups, n_ids);
  if (!workspace || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  return run_block_hessian(x, dtype, tokens, cols, groups, group_offsets, token_ids, n_ids, H,
                           accumulate, workspace, stream);
}

int nvfp4_scale_search_local_hessian(const void *w, int dtype, int64_t batch, int64_t rows,
                                     int64_t cols, const float *S, const float *H, uint8_t *scales,
                                     double *obj, void *stream) {
  bool empty = false;
  int rc = check_tensor(dtype, batch, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!w || !S || !H || !scales) return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(S, 4) || !aligned(H, 4) || !aligned(obj, 8))
    return NVFP4_ERR_ALIGN;
  if (cols / 16 > kMaxGridY || rows / 256 + 1 > (int64_t)UINT_MAX) return NVFP4_ERR_SHAPE;
  debug_check_finite(w, dtype, batch * rows * cols, as_stream(stream));
  debug_check_finite(H, NVFP4_DTYPE_F32, batch * (cols / 16) * 256, as_stream(stream));
  debug_check_scale(S, batch, as_stream(stream));
  return launch_local_hessian(w, dtype, batch, rows, cols, S, H, scales, obj, as_stream(stream));
}

int nvfp4_quantize(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                   const float *S, const uint8_t *scales_in, uint8_t *codes, uint8_t *scales_out,
                   void *stream) {
  bool empty = false;
  int rc = check_tensor(dtype, batch, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!x || !S || !codes) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(S, 4) || !aligned(codes, 8)) return NVFP4_ERR_ALIGN;
  debug_check_finite(x, dtype, batch * rows * cols, as_stream(stream));
  debug_check_scale(S, batch, as_stream(stream));
  return launch_quant(x, dtype, batch, rows, cols, S, scales_in, codes,
                      scales_in ? nullptr : scales_out, nullptr, as_stream(stream));
}

int nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *S, int64_t batch,
                     int64_t rows, int64_t cols, void *y, int out_dtype, void *stream) {
  bool empty = false;
  int rc = check_tensor(out_dtype, batch, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!codes || !scales || !S || !y) return NVFP4_ERR_NULL;
  if (!aligned(codes, 8) || !aligned(S, 4) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
  debug_check_scale(S, batch, as_stream(stream));
  return launch_dequant(codes, scales, S, batch, rows, cols, y, out_dtype, as_stream(stream));
}

int nvfp4_fakequant(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                    const float *S, const uint8_t *scales_in, void *y, uint8_t *codes_out,
                    uint8_t *scales_out, void *stream) {
  bool empty = false;
  int rc = check_tensor(dtype, batch, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (!x || !S || !y) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(S, 4) || !aligned(y, 16) || !aligned(codes_out, 8))
    return NVFP4_ERR_ALIGN;
  debug_check_finite(x, dtype, batch * rows * cols, as_stream(stream));
  debug_check_scale(S, batch, as_stream(stream));
  return launch_quant(x, dtype, batch, rows, cols, S, scales_in, codes_out,
                      scales_in ? nullptr : scales_out, y, as_stream(stream));
}

size_t nvfp4_route_groups_workspace_size(int64_t tokens, int64_t topk, int64_t experts) {
  // 0 for arguments nvfp4_route_groups rejects
  int64_t pairs;
  if (tokens < 0 || topk < 0 || experts <= 0 || experts > 16384) return 0;
  if (!mul_ok(tokens, topk, &pairs) || pairs > INT32_MAX) return 0;
  return route_workspace_size(tokens, topk, experts);
}

int nvfp4_route_groups(const int32_t *expert_ids, int64_t tokens, int64_t topk, int64_t experts,
                       int32_t *offsets, int32_t *token_ids, void *workspace,
                       size_t workspace_bytes, void *stream) {
  if (tokens < 0 || topk < 0 || experts <= 0) return NVFP4_ERR_SHAPE;
  if (experts > 16384) return NVFP4_ERR_ARG;
  int64_t pairs;
  if (!mul_ok(tokens, topk, &pairs) || pairs > INT32_MAX) return NVFP4_ERR_SHAPE;
  if (!offsets) return NVFP4_ERR_NULL;
  if (pairs > 0 && (!expert_ids || !token_ids)) return NVFP4_ERR_NULL;
  if (!aligned(expert_ids, 4) || !aligned(offsets, 4) || !aligned(token_ids, 4))
    return NVFP4_ERR_ALIGN;
  const size_t need = route_workspace_size(tokens, topk, experts);
  if (!workspace || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return NVFP4_ERR_ALIGN;
  return launch_route_groups(expert_ids, tokens, topk, experts, offsets, token_ids, workspace,
                             as_stream(stream));
}

int nvfp4_search_stats_enable(int on) {
  search_stats_enable(on != 0);
  return NVFP4_OK;
}

int nvfp4_search_stats_read(int64_t *out, void *stream) {
  if (!out) return NVFP4_ERR_NULL;
  return search_stats_read(out, as_stream(stream));
}

int nvfp4_debug_nonfinite(int32_t *flag_out, void *stream) {
  if (!flag_out) return NVFP4_ERR_NULL;
  if (!debug_checks_enabled()) return NVFP4_ERR_ARG;
  return debug_read_flag(flag_out, as_stream(stream));
}

size_t nvfp4_full_hessian_workspace_size(int64_t tokens, int64_t cols) {
  if (tokens < 0 || cols <= 0) return 0;
  return gram_workspace_size(tokens, cols);
}

int nvfp4_full_hessian(const void *x, int dtype, int64_t tokens, int64_t cols, float *H,
                       int accumulate, void *workspace, size_t workspace_bytes, void *stream) {
  if (dtype != NVFP4_DTYPE_F32 && dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_DTYPE;
  if (tokens < 0 || cols < 0 || (cols % 16) != 0) return NVFP4_ERR_SHAPE;
  int64_t t1, t2, h1;
  if (!mul_ok(tokens, cols, &t1) || !mul_ok(t1, 4, &t2) || !mul_ok(cols, cols, &h1))
    return NVFP4_ERR_SHAPE;
  if (cols > 65536 || tokens > INT32_MAX) return NVFP4_ERR_SHAPE;
  if (cols == 0) return NVFP4_OK;
  if (!H || (tokens > 0 && !x)) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(H, 4)) return NVFP4_ERR_ALIGN;
  if (!workspace || workspace_bytes < gram_workspace_size(tokens, cols)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  debug_check_finite(x, dtype, tokens * cols, as_stream(stream));
  return launch_full_hessian(x, dtype, tokens, cols, H, accumulate, workspace, as_stream(stream));
}

size_t nvfp4_gptq_factor_workspace_size(int64_t cols) {
  if (cols <= 0 || cols > 65536) return 0;
  return gptq_factor_workspace_size(cols);
}

int nvfp4_gptq_factor(const float *H, int64_t cols, double damp, double *U, int32_t *status,
                      void *workspace, size_t workspace_bytes, void *stream) {
  if (cols < 0 || (cols % 16) != 0 || cols > 65536) return NVFP4_ERR_SHAPE;
  if (!(damp >= 0.0) || damp > 1e300) return NVFP4_ERR_ARG;  // also rejects NaN and inf
  if (cols == 0) return NVFP4_OK;
  if (!H || !U) return NVFP4_ERR_NULL;
  if (!aligned(H, 4) || !aligned(U, 16) || !aligned(status, 4)) return NVFP4_ERR_ALIGN;
  if (!workspace || workspace_bytes < gptq_factor_workspace_size(cols)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  debug_check_finite(H, NVFP4_DTYPE_F32, cols * cols, as_stream(stream));
  return launch_gptq_factor(H, cols, damp, U, status, workspace, as_stream(stream));
}

size_t nvfp4_gptq_workspace_size(int64_t rows, int64_t cols) {
  // 0 for arguments nvfp4_gptq rejects
  int64_t r1, r2;
  if (rows < 0 || cols <= 0 || cols > 65536) return 0;
  if (!mul_ok(rows, cols, &r1) || !mul_ok(r1, 4, &r2) || (rows + 63) / 64 > INT32_MAX) return 0;
  return gptq_rows_workspace_size(rows, cols);
}

int nvfp4_gptq(const void *w, int dtype, int64_t rows, int64_t cols, const float *S,
               const uint8_t *scales, const double *U, uint8_t *codes, void *workspace,
               size_t workspace_bytes, void *stream) {
  bool empty = false;
  int rc = check_tensor(dtype, 1, rows, cols, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (cols > 65536 || (rows + 63) / 64 > INT32_MAX) return NVFP4_ERR_SHAPE;
  if (!w || !S || !scales || !U || !codes) return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(S, 4) || !aligned(U, 16) || !aligned(codes, 8))
    return NVFP4_ERR_ALIGN;
  if (!workspace || workspace_bytes < gptq_rows_workspace_size(rows, cols)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  debug_check_finite(w, dtype, rows * cols, as_stream(stream));
  debug_check_scale(S, 1, as_stream(stream));
  return launch_gptq_rows(w, dtype, rows, cols, S, scales, U, codes, workspace, as_stream(stream));
}

}  // extern "C"

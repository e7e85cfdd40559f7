// Optional input checks. Inputs must be finite and tensor scales positive; with
// NVFP4_DEBUG_CHECKS=1 in the environment, every entry point first scans its floating-point
// inputs (and its S) and raises a device flag if any value is NaN or infinite (or any S is
// not a positive finite number). nvfp4_debug_nonfinite() reads and clears the flag.
#include <stdlib.h>

#include "nvfp4_internal.h"

namespace nvfp4 {

__device__ int g_nonfinite_flag;

template <int DT>
__global__ void __launch_bounds__(256) k_check_finite(const void *__restrict__ x, int64_t n) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    unsigned bits;
    if (DT == NVFP4_DTYPE_BF16)
      bits = (unsigned)static_cast<const uint16_t *>(x)[i] << 16;
    else
      bits = __float_as_uint(static_cast<const float *>(x)[i]);
    bad |= (bits & 0x7F800000u) == 0x7F800000u;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(&g_nonfinite_flag, 1);
}

// tensor scales must be finite and positive
__global__ void __launch_bounds__(256) k_check_scale(const float *__restrict__ S, int64_t n) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float v = S[i];
    bad |= !(v > 0.0f && v <= 3.4028235e38f);
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(&g_nonfinite_flag, 1);
}

bool debug_checks_enabled() {
  const char *e = getenv("NVFP4_DEBUG_CHECKS");
  return e != nullptr && e[0] == '1';
}

void debug_check_finite(const void *x, int dtype, int64_t n, hipStream_t st) {
  if (!x || n <= 0 || !debug_checks_enabled()) return;
  int64_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_check_finite<NVFP4_DTYPE_BF16>, dim3((unsigned)g), dim3(256), 0, st, x, n);
  else
    hipLaunchKernelGGL(k_check_finite<NVFP4_DTYPE_F32>, dim3((unsigned)g), dim3(256), 0, st, x, n);
}

void debug_check_scale(const float *S, int64_t n, hipStream_t st) {
  if (!S || n <= 0 || !debug_checks_enabled()) return;
  const int64_t g = n < 256 * 64 ? (n + 255) / 256 : 64;
  hipLaunchKernelGGL(k_check_scale, dim3((unsigned)g), dim3(256), 0, st, S, n);
}

int debug_read_flag(int32_t *out, hipStream_t st) {
  if (hipStreamSynchronize(st) != hipSuccess) return NVFP4_ERR_HIP;
  int v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_nonfinite_flag), sizeof(int), 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return NVFP4_ERR_HIP;
  const int zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_nonfinite_flag), &zero, sizeof(int), 0,
                        hipMemcpyHostToDevice) != hipSuccess)
    return NVFP4_ERR_HIP;
  *out = v;
  return NVFP4_OK;
}

}  // namespace nvfp4

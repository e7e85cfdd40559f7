// Peak-rate probes for the benchmark (not part of the NVFP4 library): loops of independent
// matrix-core or vector instructions, so the benchmark can report each kernel against the
// rate this device actually sustains as well as against the datasheet figure.
//   kind 0: v_mfma_f64_16x16x4_f64      (2048 flops per wave instruction)
//   kind 1: v_mfma_f32_32x32x16_bf16    (32768 flops)
//   kind 2: v_mfma_f32_16x16x4_f32      (2048 flops)
//   kind 3: v_fma_f32, non-packed       (64 lane-ops per wave instruction)
// Every wave issues 8 independent chains per loop iteration; `out` (blocks * 256 doubles)
// receives a value derived from every chain so nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef double pr_v4d __attribute__((ext_vector_type(4)));
typedef float pr_v4f __attribute__((ext_vector_type(4)));
typedef float pr_v16f __attribute__((ext_vector_type(16)));
typedef __bf16 pr_v8bf __attribute__((ext_vector_type(8)));

constexpr int NCH = 8;

__global__ void __launch_bounds__(256) k_probe_f64(double *out, int iters) {
  pr_v4d acc[NCH];
  for (int i = 0; i < NCH; ++i) acc[i] = (pr_v4d){0.0, 0.0, 0.0, 0.0};
  const double a = 1e-3 * (threadIdx.x + 1), b = 1e-3 * (blockIdx.x + 1);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < NCH; ++i) acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[i], 0, 0, 0);
  double s = 0.0;
  for (int i = 0; i < NCH; ++i) s += acc[i][0] + acc[i][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) k_probe_bf16(double *out, int iters) {
  pr_v16f acc[NCH];
  for (int i = 0; i < NCH; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  pr_v8bf a, b;
  for (int r = 0; r < 8; ++r) {
    a[r] = (__bf16)(1e-3f * (float)(threadIdx.x + r));
    b[r] = (__bf16)(1e-3f * (float)(blockIdx.x + r));
  }
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < NCH; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  float s = 0.0f;
  for (int i = 0; i < NCH; ++i) s += acc[i][0] + acc[i][15];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) k_probe_f32(double *out, int iters) {
  pr_v4f acc[NCH];
  for (int i = 0; i < NCH; ++i) acc[i] = (pr_v4f){0.0f, 0.0f, 0.0f, 0.0f};
  const float a = 1e-3f * (threadIdx.x + 1), b = 1e-3f * (blockIdx.x + 1);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < NCH; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
  float s = 0.0f;
  for (int i = 0; i < NCH; ++i) s += acc[i][0] + acc[i][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) k_probe_valu(double *out, int iters) {
  float x[NCH];
  for (int i = 0; i < NCH; ++i) x[i] = 1e-3f * (float)(threadIdx.x + i);
  const float m = 0.999f, c = 1e-4f * (float)(blockIdx.x + 1);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < NCH; ++i) x[i] = __builtin_fmaf(x[i], m, c);
  float s = 0.0f;
  for (int i = 0; i < NCH; ++i) s += x[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

extern "C" __attribute__((visibility("default"))) int nvfp4_probe_run(int kind, int blocks, int iters,
                                                                      double *out, void *stream) {
  if (blocks <= 0 || iters <= 0 || !out) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_probe_f64, dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 1: hipLaunchKernelGGL(k_probe_bf16, dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 2: hipLaunchKernelGGL(k_probe_f32, dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 3: hipLaunchKernelGGL(k_probe_valu, dim3(blocks), dim3(256), 0, st, out, iters); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Training support for fake-quant (QAD page, sec. 3.2: the forward pass runs through the
// quantiser, the backward pass hands the gradient straight back, clamped to a reasonable
// range in practice; sec. 4.1: the scale is smoothed with a moving average).
//  * k_ste_clamp: grad_out = clamp(grad, -c, c) in fp32 (bf16 rounded back to nearest even),
//    16 bytes per lane, may run in place. c = +inf is the plain straight-through gradient.
//  * k_scale_ema: S = fmaf(m, S, fp32(fp32(1 - m) * S_batch)) per batch entry.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

// Comparisons rather than fmin/fmax so that a NaN gradient passes through unchanged.
__device__ __forceinline__ float clampg(float g, float c) {
  return g > c ? c : (g < -c ? -c : g);
}

template <int DT>
__global__ void __launch_bounds__(256)
    k_ste_clamp(const void *__restrict__ g, int64_t nvec, float c, void *__restrict__ out) {
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    if (DT == NVFP4_DTYPE_BF16) {  // 8 values per 16 bytes
      const uint4 q = reinterpret_cast<const uint4 *>(g)[v];
      const unsigned w[4] = {q.x, q.y, q.z, q.w};
      unsigned r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = clampg(bf16_lo(w[k]), c);
        const float b = clampg(bf16_hi(w[k]), c);
        r[k] = bf16x2_bits(a, b);
      }
      reinterpret_cast<uint4 *>(out)[v] = make_uint4(r[0], r[1], r[2], r[3]);
    } else {  // 4 values per 16 bytes
      float4 q = reinterpret_cast<const float4 *>(g)[v];
      q.x = clampg(q.x, c);
      q.y = clampg(q.y, c);
      q.z = clampg(q.z, c);
      q.w = clampg(q.w, c);
      reinterpret_cast<float4 *>(out)[v] = q;
    }
  }
}

__global__ void k_scale_ema(float *__restrict__ S, const float *__restrict__ S_batch,
                            int64_t batch, float m) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch) return;
  const float a = 1.0f - m;
  const float b = a * S_batch[i];
  S[i] = __builtin_fmaf(m, S[i], b);
}

int launch_ste_backward(const void *g, int dtype, int64_t n, float clip, void *out,
                        hipStream_t st) {
  const int64_t per_vec = dtype == NVFP4_DTYPE_BF16 ? 8 : 4;
  const int64_t nvec = n / per_vec;
  int64_t wgs = (nvec + 255) / 256;
  if (wgs > (1 << 20)) wgs = 1 << 20;
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_ste_clamp<NVFP4_DTYPE_BF16>, dim3((unsigned)wgs), dim3(256), 0, st, g,
                       nvec, clip, out);
  else
    hipLaunchKernelGGL(k_ste_clamp<NVFP4_DTYPE_F32>, dim3((unsigned)wgs), dim3(256), 0, st, g, nvec,
                       clip, out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int launch_scale_ema(float *S, const float *S_batch, int64_t batch, float m, hipStream_t st) {
  hipLaunchKernelGGL(k_scale_ema, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, st, S,
                     S_batch, batch, m);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

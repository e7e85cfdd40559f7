// Static activation calibration (Baseten page, "Calibration": record the activation
// distribution over sample inputs, choose a clipping range -- min/max, or percentile /
// histogram methods that clip a few outliers -- then scale blocks from it).
//
// Reading: an exact histogram of |x| with one bin per bf16 magnitude, bin = (fp32 bits of
// |x|) >> 16 (32768 bins), accumulated over calibration batches. For a fraction p in (0, 1]
// the clip value is the lower edge of the first bin whose cumulative count reaches
// ceil(p N): the k-th smallest magnitude rounded toward zero to bf16 (exact for bf16 data;
// p = 1 gives the max). The tensor scale is the tensor-scale formula applied to it.
//
//  * k_calib_hist: one workgroup of 1024 threads per CU counts its share of the values in a
//    32-bit LDS histogram (128 KiB), then adds its non-zero bins to the global 64-bit
//    histogram with atomics. Integer counts: the result does not depend on order. (Smaller
//    workgroups with 16-bit counters and 4x more flushes took 2.5x longer.)
//  * k_calib_scale: one workgroup; each wave sums 2048 consecutive bins (coalesced loads), a
//    scan over the 16 wave totals finds the wave holding the crossing bin, and that wave
//    regroups its bins through LDS (32 consecutive bins per lane), scans its lanes and lets
//    the one lane whose bins reach ceil(p N) find the crossing bin.
#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int CAL_BINS = 32768;

constexpr int CAL_THREADS = 1024;

template <int DT>
__global__ void __launch_bounds__(CAL_THREADS)
    k_calib_hist(const void *__restrict__ x, int64_t n, unsigned long long *__restrict__ hist) {
  __shared__ unsigned cnt[CAL_BINS];  // 128 KiB: one workgroup per CU
  for (int i = threadIdx.x; i < CAL_BINS; i += blockDim.x) cnt[i] = 0u;
  __syncthreads();
  const int64_t nv = n / 8;  // vectors of 8 values
  const int64_t per = (nv + gridDim.x - 1) / gridDim.x;
  const int64_t v1 = min(nv, (int64_t)blockIdx.x * per + per);
  const int64_t step = blockDim.x;
  int64_t v = (int64_t)blockIdx.x * per + threadIdx.x;
  auto add8 = [&](const unsigned w[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) atomicAdd(&cnt[w[j]], 1u);
  };
  if (DT == NVFP4_DTYPE_BF16) {
    // bf16 magnitude bits are the bin; four 16-byte loads in flight per lane
    auto bins = [](const uint4 &q, unsigned w[8]) {
      const unsigned u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[2 * j] = u[j] & 0x7FFFu;
        w[2 * j + 1] = (u[j] >> 16) & 0x7FFFu;
      }
    };
    for (; v + 3 * step < v1; v += 4 * step) {
      uint4 q[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) q[k] = reinterpret_cast<const uint4 *>(x)[v + k * step];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        unsigned w[8];
        bins(q[k], w);
        add8(w);
      }
    }
    for (; v < v1; v += step) {
      unsigned w[8];
      bins(reinterpret_cast<const uint4 *>(x)[v], w);
      add8(w);
    }
  } else {
    for (; v < v1; v += step) {
      const uint4 *p = reinterpret_cast<const uint4 *>(x) + 2 * v;
      const uint4 a = p[0], b = p[1];
      unsigned w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = (w[j] & 0x7FFFFFFFu) >> 16;
      add8(w);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < CAL_BINS; i += blockDim.x) {
    const unsigned c = cnt[i];
    if (c) atomicAdd(&hist[i], (unsigned long long)c);
  }
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ void __launch_bounds__(1024)
    k_calib_scale(const unsigned long long *__restrict__ hist, double fraction, float *__restrict__ S) {
  constexpr int WB = CAL_BINS / 16;  // consecutive bins per wave
  constexpr int PER = WB / 64;       // 32
  __shared__ unsigned long long pre[17];
  __shared__ unsigned long long stage[WB + WB / PER];  // one wave's bins, padded
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  // coalesced: the wave's bins as 32 rows of 64, lane l holding column l
  unsigned long long v[PER];
  unsigned long long mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    v[j] = hist[w * WB + j * 64 + l];
    mine += v[j];
  }
  const unsigned long long wtot = wave_sum_u64(mine);
  if (l == 0) pre[w + 1] = wtot;
  __syncthreads();
  if (t == 0) {
    pre[0] = 0;
    for (int i = 1; i <= 16; ++i) pre[i] += pre[i - 1];
  }
  __syncthreads();
  const unsigned long long total = pre[16];
  if (total == 0) {
    if (t == 0) *S = 1.0f;
    return;
  }
  unsigned long long k = (unsigned long long)ceil(fraction * (double)total);
  k = k < 1 ? 1 : (k > total ? total : k);
  if (!(pre[w] < k && k <= pre[w + 1])) return;  // exactly one wave holds the crossing bin
  // that wave regroups its bins through LDS so that lane l holds bins 32 l .. 32 l + 31
  // (one pad slot per 32 bins spreads the reads over the banks)
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int b = j * 64 + l;
    stage[b + b / PER] = v[j];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  unsigned long long u[PER];
  unsigned long long run = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    u[i] = stage[l * (PER + 1) + i];
    run += u[i];
  }
  unsigned long long inc = run;  // inclusive scan over the lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_up(inc, off);
    if (l >= off) inc += o;
  }
  unsigned long long c = pre[w] + inc - run;  // count in all bins before this lane's
  if (!(c < k && k <= c + run)) return;       // exactly one lane holds the crossing bin
  int found = 0;  // the first of its bins whose cumulative count reaches k
  bool done = false;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c += u[i];
    if (!done && c >= k) {
      found = i;
      done = true;
    }
  }
  const int b = w * WB + l * PER + found;
  const float clip = __uint_as_float((unsigned)b << 16);
  float s = 1.0f;
  if (clip != 0.0f) {
    s = __fdiv_rn(clip, 2688.0f);
    if (s < 1.17549435e-38f) s = 1.17549435e-38f;
  }
  *S = s;
}

int launch_calib_histogram(const void *x, int dtype, int64_t n, unsigned long long *hist,
                           hipStream_t st) {
  // one workgroup per CU (the LDS histogram fills most of a CU's LDS); each flushes its
  // non-zero bins once, so fewer workgroups mean fewer global atomics
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return NVFP4_ERR_HIP;
  int64_t wgs = (n / 8 + CAL_THREADS - 1) / CAL_THREADS;
  if (wgs > cus) wgs = cus;
  if (wgs > 0) {
    if (dtype == NVFP4_DTYPE_BF16)
      hipLaunchKernelGGL(k_calib_hist<NVFP4_DTYPE_BF16>, dim3((unsigned)wgs), dim3(CAL_THREADS), 0, st, x,
                         n, hist);
    else
      hipLaunchKernelGGL(k_calib_hist<NVFP4_DTYPE_F32>, dim3((unsigned)wgs), dim3(CAL_THREADS), 0, st, x, n,
                         hist);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int launch_calib_scale(const unsigned long long *hist, double fraction, float *S, hipStream_t st) {
  hipLaunchKernelGGL(k_calib_scale, dim3(1), dim3(1024), 0, st, hist, fraction, S);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

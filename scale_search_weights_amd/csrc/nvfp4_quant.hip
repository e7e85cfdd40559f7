// NVFP4 tensor scale, quantise / fake-quantise / dequantise kernels for gfx950.
//
// Fake quantisation is the quantise -> dequantise round trip of the QAD article's sec. 3.2
// sketch (blocks of 16, block max / 6, clamp, round to E2M1, multiply back), here with the
// block scale rounded to E4M3 and a per-tensor FP32 scale, as NVFP4 stores it (Baseten
// on NVFP4 quality, "Why do we need a scale" and "Block scaling").
//
// Work mapping: one lane owns one 16-value block (32 B of bf16 or 64 B of fp32, loaded as
// 16-byte vectors), so the block max needs no cross-lane traffic and a wave streams 2 KiB
// (bf16) of contiguous input. The kernel is HBM-bound; the per-element work is seven fp32
// compares against exact-equivalent thresholds plus selects.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

// ------------------------------------------------------------------ tensor scale

__global__ void k_scale_init(unsigned *amax_bits, int64_t batch) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < batch) amax_bits[i] = 0u;
}

// amax over each batch entry; |x| as uint bits orders like |x| for finite values.
template <int DT>
__global__ void __launch_bounds__(256) k_scale_amax(const void *__restrict__ x, int64_t n,
                                                    unsigned *__restrict__ amax_bits,
                                                    int64_t chunks_per_batch) {
  const int64_t batch = blockIdx.y;
  const int64_t vec_elems = 8;  // 16 B per load for bf16; two loads for fp32
  const int64_t nvec = n / vec_elems;
  unsigned m = 0u;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)chunks_per_batch * blockDim.x) {
    const int64_t e0 = batch * n + v * vec_elems;
    if (DT == NVFP4_DTYPE_BF16) {
      const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + e0);
      const unsigned w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m = max(m, (w[k] & 0x7FFFu) << 16);
        m = max(m, w[k] & 0x7FFF0000u);
      }
    } else {
      const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + e0);
      const float4 a = p[0], b = p[1];
      const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) m = max(m, __float_as_uint(f[k]) & 0x7FFFFFFFu);
    }
  }
  // wave reduce then one atomic per wave
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0 && m) atomicMax(&amax_bits[batch], m);
}

__global__ void k_scale_finalize(unsigned *amax_bits_then_S, int64_t batch) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch) return;
  const float amax = __uint_as_float(amax_bits_then_S[i]);
  float S = 1.0f;
  if (amax != 0.0f) {
    S = __fdiv_rn(amax, 2688.0f);
    if (S < 1.17549435e-38f) S = 1.17549435e-38f;
  }
  reinterpret_cast<float *>(amax_bits_then_S)[i] = S;
}

int launch_global_scale(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                        hipStream_t st) {
  unsigned *bits = reinterpret_cast<unsigned *>(S);
  const int tb = 256;
  hipLaunchKernelGGL(k_scale_init, dim3((unsigned)((batch + tb - 1) / tb)), dim3(tb), 0, st,
                     bits, batch);
  const int64_t nvec = n / 8;
  int64_t chunks = (nvec + tb - 1) / tb;
  const int64_t cap = 2048;
  if (chunks > cap) chunks = cap;
  if (chunks < 1) chunks = 1;
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_scale_amax<NVFP4_DTYPE_BF16>, dim3((unsigned)chunks, (unsigned)batch),
                       dim3(tb), 0, st, x, n, bits, chunks);
  else
    hipLaunchKernelGGL(k_scale_amax<NVFP4_DTYPE_F32>, dim3((unsigned)chunks, (unsigned)batch),
                       dim3(tb), 0, st, x, n, bits, chunks);
  hipLaunchKernelGGL(k_scale_finalize, dim3((unsigned)((batch + tb - 1) / tb)), dim3(tb), 0, st,
                     bits, batch);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ block load / store

template <int DT>
__device__ __forceinline__ void load_block(const void *__restrict__ x, int64_t blk, float v[16]) {
  if (DT == NVFP4_DTYPE_BF16) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + blk * 16);
    const uint4 a = p[0], b = p[1];
    const unsigned w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = bf16_lo(w[k]);
      v[2 * k + 1] = bf16_hi(w[k]);
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + blk * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a = p[k];
      v[4 * k] = a.x;
      v[4 * k + 1] = a.y;
      v[4 * k + 2] = a.z;
      v[4 * k + 3] = a.w;
    }
  }
}

template <int DT>
__device__ __forceinline__ void store_block(void *__restrict__ y, int64_t blk, const float v[16]) {
  if (DT == NVFP4_DTYPE_BF16) {
    unsigned w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = bf16_bits(v[2 * k]) | (bf16_bits(v[2 * k + 1]) << 16);
    uint4 *p = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(y) + blk * 16);
    p[0] = make_uint4(w[0], w[1], w[2], w[3]);
    p[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(y) + blk * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// ------------------------------------------------------------------ quantise / fake-quant

// flags: which outputs exist and whether block bytes are given
enum : int { F_SCALES_IN = 1, F_CODES = 2, F_SCALES_OUT = 4, F_Y = 8 };

template <int DT, int OUT_DT, int FLAGS>
__global__ void __launch_bounds__(256)
    k_quant(const void *__restrict__ x, const float *__restrict__ S_arr,
            const uint8_t *__restrict__ scales_in, uint8_t *__restrict__ codes,
            uint8_t *__restrict__ scales_out, void *__restrict__ y, int64_t blocks_per_batch,
            int64_t total_blocks) {
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < total_blocks;
       blk += (int64_t)gridDim.x * blockDim.x) {
    const float S = S_arr[blk / blocks_per_batch];
    float v[16];
    load_block<DT>(x, blk, v);
    int byte;
    if (FLAGS & F_SCALES_IN) {
      byte = scales_in[blk];
    } else {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
      byte = max_scale_byte(amax, S);
    }
    ScaleTable tb;
    if (byte) make_table(byte, S, tb);
    unsigned lo = 0u, hi = 0u;
    float dq[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float X = fabsf(v[i]);
      float d = 0.0f;
      unsigned k = 0u;
      if (byte) {
#pragma unroll
        for (int j = 0; j < 7; ++j) {
          const bool p = X > tb.t[j];
          d = p ? tb.d[j + 1] : d;
          k += p ? 1u : 0u;
        }
      }
      const unsigned neg = (__float_as_uint(v[i]) >> 31) & (k ? 1u : 0u);
      const unsigned code = k | (neg << 3);
      dq[i] = __uint_as_float(__float_as_uint(d) | (neg << 31));
      if (i < 8) lo |= code << (4 * i);
      else hi |= code << (4 * (i - 8));
    }
    if (FLAGS & F_CODES) reinterpret_cast<uint2 *>(codes)[blk] = make_uint2(lo, hi);
    if (FLAGS & F_SCALES_OUT) scales_out[blk] = (uint8_t)byte;
    if (FLAGS & F_Y) store_block<OUT_DT>(y, blk, dq);
  }
}

static unsigned grid_for(int64_t total_blocks) {
  int64_t g = (total_blocks + 255) / 256;
  const int64_t cap = 1 << 20;
  return (unsigned)(g > cap ? cap : (g < 1 ? 1 : g));
}

template <int DT, int OUT_DT>
static void dispatch_quant(int flags, const void *x, const float *S, const uint8_t *si,
                           uint8_t *codes, uint8_t *so, void *y, int64_t bpb, int64_t total,
                           hipStream_t st) {
  const dim3 g(grid_for(total)), b(256);
#define NVFP4_Q(F)                                                                              \
  case F:                                                                                       \
    hipLaunchKernelGGL((k_quant<DT, OUT_DT, F>), g, b, 0, st, x, S, si, codes, so, y, bpb,     \
                       total);                                                                  \
    break;
  switch (flags) {
    NVFP4_Q(F_CODES)
    NVFP4_Q(F_CODES | F_SCALES_OUT)
    NVFP4_Q(F_SCALES_IN | F_CODES)
    NVFP4_Q(F_SCALES_OUT)
    NVFP4_Q(F_Y)
    NVFP4_Q(F_Y | F_CODES)
    NVFP4_Q(F_Y | F_SCALES_OUT)
    NVFP4_Q(F_Y | F_CODES | F_SCALES_OUT)
    NVFP4_Q(F_SCALES_IN | F_Y)
    NVFP4_Q(F_SCALES_IN | F_Y | F_CODES)
    default:
      break;
  }
#undef NVFP4_Q
}

int launch_quant(const void *x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                 const float *S, const uint8_t *scales_in, uint8_t *codes, uint8_t *scales_out,
                 void *y, hipStream_t st) {
  const int64_t bpb = rows * (cols / 16), total = batch * bpb;
  int flags = 0;
  if (scales_in) flags |= F_SCALES_IN;
  if (codes) flags |= F_CODES;
  if (scales_out && !scales_in) flags |= F_SCALES_OUT;
  if (y) flags |= F_Y;
  if (dtype == NVFP4_DTYPE_BF16)
    dispatch_quant<NVFP4_DTYPE_BF16, NVFP4_DTYPE_BF16>(flags, x, S, scales_in, codes, scales_out,
                                                       y, bpb, total, st);
  else
    dispatch_quant<NVFP4_DTYPE_F32, NVFP4_DTYPE_F32>(flags, x, S, scales_in, codes, scales_out,
                                                     y, bpb, total, st);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ dequantise

template <int OUT_DT>
__global__ void __launch_bounds__(256)
    k_dequant(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
              const float *__restrict__ S_arr, void *__restrict__ y, int64_t blocks_per_batch,
              int64_t total_blocks) {
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < total_blocks;
       blk += (int64_t)gridDim.x * blockDim.x) {
    const float S = S_arr[blk / blocks_per_batch];
    const int byte = scales[blk];
    const uint2 c = reinterpret_cast<const uint2 *>(codes)[blk];
    ScaleTable tb;
    if (byte) make_table(byte, S, tb);
    float dq[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const unsigned code = ((i < 8 ? c.x : c.y) >> (4 * (i & 7))) & 15u;
      const unsigned k = code & 7u;
      float d = 0.0f;
      if (byte) {
#pragma unroll
        for (int j = 1; j < 8; ++j) d = (k == (unsigned)j) ? tb.d[j] : d;
      }
      const unsigned neg = (code >> 3) & (k ? 1u : 0u);
      dq[i] = __uint_as_float(__float_as_uint(d) | (neg << 31));
    }
    store_block<OUT_DT>(y, blk, dq);
  }
}

int launch_dequant(const uint8_t *codes, const uint8_t *scales, const float *S, int64_t batch,
                   int64_t rows, int64_t cols, void *y, int out_dtype, hipStream_t st) {
  const int64_t bpb = rows * (cols / 16), total = batch * bpb;
  const dim3 g(grid_for(total)), b(256);
  if (out_dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_dequant<NVFP4_DTYPE_BF16>, g, b, 0, st, codes, scales, S, y, bpb, total);
  else
    hipLaunchKernelGGL(k_dequant<NVFP4_DTYPE_F32>, g, b, 0, st, codes, scales, S, y, bpb, total);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

// NVFP4 tensor scale, quantise / fake-quantise / dequantise kernels for gfx950.
//
// Fake quantisation is the quantise -> dequantise round trip of the QAD article's sec. 3.2
// sketch (blocks of 16, block max / 6, clamp, round to E2M1, multiply back), here with the
// block scale rounded to E4M3 and a per-tensor FP32 scale, as NVFP4 stores it (Baseten
// on NVFP4 quality, "Why do we need a scale" and "Block scaling").
//
// Work mapping: two lanes own one 16-value block (16 B of bf16 each), so a wave streams
// 1 KiB of contiguous input per load and the block max needs one lane-pair exchange. The
// kernel is HBM-bound. Rounding decisions use the hardware FP8/FP4 converts on two
// bracketing products (nvfp4_device.h); a value whose bracket straddles a midpoint takes
// the exact threshold path. Outputs use non-temporal stores: with ordinary stores the
// kernel itself finishes sooner, but the dirty lines it leaves in the caches are written
// back during the kernels that follow, which then take longer than the time saved.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

// ------------------------------------------------------------------ tensor scale

__global__ void k_scale_init(unsigned *amax_bits, int64_t batch) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < batch) amax_bits[i] = 0u;
}

// amax over each batch entry; |x| as uint bits orders like |x| for finite values.
// Each workgroup strides over its batch entry with four 16-byte loads in flight per lane,
// reduces in registers, across the wave and across the workgroup, then issues a single
// atomicMax, so contention stays at a few hundred atomics per call.
template <int DT>
__device__ __forceinline__ unsigned vec_amax_bits(const void *__restrict__ x, int64_t e0) {
  unsigned m = 0u;
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
  return m;
}

template <int DT>
__global__ void __launch_bounds__(256) k_scale_amax(const void *__restrict__ x, int64_t n,
                                                    unsigned *__restrict__ amax_bits,
                                                    int64_t chunks_per_batch) {
  __shared__ unsigned red[4];
  const int64_t batch = blockIdx.y;
  const int64_t nvec = n / 8;  // 8 elements per vector
  const int64_t stride = chunks_per_batch * blockDim.x;
  const int64_t base = batch * n;
  unsigned m = 0u;
  int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; v + 3 * stride < nvec; v += 4 * stride) {
    const unsigned a = vec_amax_bits<DT>(x, base + v * 8);
    const unsigned b = vec_amax_bits<DT>(x, base + (v + stride) * 8);
    const unsigned c = vec_amax_bits<DT>(x, base + (v + 2 * stride) * 8);
    const unsigned d = vec_amax_bits<DT>(x, base + (v + 3 * stride) * 8);
    m = max(m, max(max(a, b), max(c, d)));
  }
  for (; v < nvec; v += stride) m = max(m, vec_amax_bits<DT>(x, base + v * 8));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (m) atomicMax(&amax_bits[batch], m);
  }
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
  // about 256 workgroups in total: every workgroup ends with one atomicMax on its entry's
  // word, and same-address atomics serialise (2048 of them cost ~15 us)
  int64_t cap = 256 / batch;
  if (cap < 4) cap = 4;
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

// Workspace form: the amax pass writes each workgroup's maximum to its own slot (plain
// stores, no atomics, no initialisation), and one workgroup per batch entry reduces the
// slots and writes S (the launch boundary makes the slots visible). Two launches instead of
// three, and about 512 workgroups with sixteen 16-byte loads in flight per lane instead of
// 256 with four (the single-word atomicMax form must keep its same-address atomics few;
// 512 x 16 was the fastest of 512..4096 workgroups x 4..16 loads on the 4096x4096 and
// 12288x4096 weights, within 8% of the best on the 128-expert stack).
static inline int64_t scale_ws_wgs(int64_t batch, int64_t n) {
  const int64_t nvec = n / 8, per = 256 * 16;  // vectors a workgroup takes per round
  int64_t g = (nvec + per - 1) / per;
  int64_t cap = 512 / (batch > 0 ? batch : 1);  // about 512 workgroups in all
  if (cap < 2) cap = 2;
  if (g > cap) g = cap;
  return g < 1 ? 1 : g;
}

// workspace: one uint32 slot per workgroup, [batch][G]
size_t scale_workspace_size(int64_t batch, int64_t n) {
  return (size_t)4 * (size_t)batch * (size_t)scale_ws_wgs(batch, n);
}

__device__ __forceinline__ unsigned wg_max256(unsigned m, unsigned *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

template <int DT>
__global__ void __launch_bounds__(256)
    k_scale_slots(const void *__restrict__ x, int64_t n, int64_t G, unsigned *__restrict__ slot) {
  __shared__ unsigned red[4];
  const int64_t batch = blockIdx.y, wg = blockIdx.x;
  const int64_t nvec = n / 8, stride = G * 256, base = batch * n;
  unsigned m = 0u;
  int64_t v = wg * 256 + threadIdx.x;
  for (; v + 15 * stride < nvec; v += 16 * stride) {
    unsigned a[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) a[k] = vec_amax_bits<DT>(x, base + (v + k * stride) * 8);
#pragma unroll
    for (int k = 0; k < 16; ++k) m = max(m, a[k]);
  }
  for (; v < nvec; v += stride) m = max(m, vec_amax_bits<DT>(x, base + v * 8));
  m = wg_max256(m, red);
  if (threadIdx.x == 0) slot[batch * G + wg] = m;
}

// one workgroup per batch entry: the maximum of its slots, then S as in k_scale_finalize
__global__ void __launch_bounds__(256)
    k_scale_slots_finalize(const unsigned *__restrict__ slot, int64_t G, float *__restrict__ S) {
  __shared__ unsigned red[4];
  const int64_t batch = blockIdx.x;
  unsigned m = 0u;
  for (int64_t i = threadIdx.x; i < G; i += 256) m = max(m, slot[batch * G + i]);
  m = wg_max256(m, red);
  if (threadIdx.x == 0) {
    const float amax = __uint_as_float(m);
    float s = 1.0f;
    if (amax != 0.0f) {
      s = __fdiv_rn(amax, 2688.0f);
      if (s < 1.17549435e-38f) s = 1.17549435e-38f;
    }
    S[batch] = s;
  }
}

int launch_global_scale_ws(const void *x, int dtype, int64_t batch, int64_t n, float *S,
                           void *workspace, hipStream_t st) {
  const int64_t G = scale_ws_wgs(batch, n);
  unsigned *slot = static_cast<unsigned *>(workspace);
  const dim3 g((unsigned)G, (unsigned)batch), b(256);
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_scale_slots<NVFP4_DTYPE_BF16>, g, b, 0, st, x, n, G, slot);
  else
    hipLaunchKernelGGL(k_scale_slots<NVFP4_DTYPE_F32>, g, b, 0, st, x, n, G, slot);
  hipLaunchKernelGGL(k_scale_slots_finalize, dim3((unsigned)batch), b, 0, st, slot, G, S);
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
    for (int k = 0; k < 8; ++k) w[k] = bf16x2_bits(v[2 * k], v[2 * k + 1]);
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


typedef unsigned nv_u2 __attribute__((ext_vector_type(2)));
typedef unsigned nv_u4 __attribute__((ext_vector_type(4)));
typedef float nv_f4 __attribute__((ext_vector_type(4)));

// outputs are written once and not re-read by this kernel: non-temporal stores
#define NVFP4_ST(ptr, val) __builtin_nontemporal_store((val), (ptr))
__device__ __forceinline__ void st_out(uint2 *p, uint2 v) {
  const nv_u2 t = {v.x, v.y};
  NVFP4_ST(reinterpret_cast<nv_u2 *>(p), t);
}
__device__ __forceinline__ void st_out(uint4 *p, uint4 v) {
  const nv_u4 t = {v.x, v.y, v.z, v.w};
  NVFP4_ST(reinterpret_cast<nv_u4 *>(p), t);
}
__device__ __forceinline__ void st_out(float4 *p, float4 v) {
  const nv_f4 t = {v.x, v.y, v.z, v.w};
  NVFP4_ST(reinterpret_cast<nv_f4 *>(p), t);
}
__device__ __forceinline__ void st_out(uint8_t *p, uint8_t v) { NVFP4_ST(p, v); }

// Two lanes per block: lane 2b+h owns values 8h..8h+7 of block b (16 contiguous bytes of
// bf16), the block max is exchanged between the lane pair, and each lane writes its own
// 4 code bytes and 16 output bytes, so every wave load and store is contiguous and twice
// as many waves are in flight as with one lane per block (measured faster on MI355X).
// Eight consecutive elements as loaded: bf16 uses a (16 bytes), fp32 uses a and b.
struct Raw8 {
  uint4 a, b;
};

template <int DT>
__device__ __forceinline__ Raw8 load_raw8(const void *__restrict__ x, int64_t hb) {
  Raw8 r;
  if (DT == NVFP4_DTYPE_BF16) {
    r.a = reinterpret_cast<const uint4 *>(x)[hb];
    r.b = make_uint4(0u, 0u, 0u, 0u);
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(x) + 2 * hb;
    r.a = p[0];
    r.b = p[1];
  }
  return r;
}

template <int DT>
__device__ __forceinline__ void unpack_raw8(const Raw8 &r, float v[8]) {
  if (DT == NVFP4_DTYPE_BF16) {
    const unsigned w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_lo(w[k]);
      v[2 * k + 1] = bf16_hi(w[k]);
    }
  } else {
    const unsigned w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(w[k]);
  }
}

// Grid: x = chunks of U x 256 half blocks within one tensor, y = batch entry. Every
// workgroup belongs to one tensor, so it builds that tensor's 127-entry byte table (E4M3
// value, the bracket of 1/(sS), and the bracket of 1/(6S)) once in LDS and no lane runs fp64
// work. A lane takes U half blocks a round, U x 256 apart within the round's span of the
// grid, with all U loads issued before the first is used; the first round's loads are in
// flight while the table is built.
template <int DT, int OUT_DT, int FLAGS, int U>
__global__ void __launch_bounds__(256)
    k_quant(const void *__restrict__ x, const float *__restrict__ S_arr,
             const uint8_t *__restrict__ scales_in, uint8_t *__restrict__ codes,
             uint8_t *__restrict__ scales_out, void *__restrict__ y, int64_t blocks_per_batch) {
  const float S = S_arr[blockIdx.y];  // uniform: a scalar load
  const int64_t n_half = 2 * blocks_per_batch;
  const int64_t off = (int64_t)blockIdx.y * n_half;  // the entry's first half block
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t l0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  Raw8 raw[U];
  int given[U];
  // one round's loads, at half blocks base + k stride (clamped to a valid index)
  auto load_round = [&](int64_t base) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t l = base + k * stride;
      const int64_t hb = off + (l < n_half ? l : n_half - 1);
      raw[k] = load_raw8<DT>(x, hb);
      given[k] = (FLAGS & F_SCALES_IN) ? (int)scales_in[hb >> 1] : 0;
    }
  };
  load_round(l0);
  __shared__ Cand tab[127];
  build_cands(tab, S);
  lds_barrier();
  auto block = [&](int64_t hb, const Raw8 &raw, int given) {
    const int64_t blk = hb >> 1;
    float v[8];
    unpack_raw8<DT>(raw, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // the two lanes of a block are lanes 2k and 2k+1 (both active): DPP quad_perm [1,0,3,2]
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1,
                                                                   0xF, 0xF, false)));
    const int byte = (FLAGS & F_SCALES_IN) ? given_byte(given)
                                           : max_scale_byte_fast(amax, tab[0].rlo, tab[0].rhi, S);
    unsigned c = 0u;
    float s = 0.0f;
    if (byte) {
      const Cand e = tab[byte];
      s = e.s;
      const double sS = (double)s * (double)S;
      if (e.rlo >= 0x1p-126f && amax * e.rhi < 0x1p126f) {
        c = fp4_exact_codes8(v, e.rlo, e.rhi, sS);
      } else {
        ScaleTable tb;
        make_table(byte, S, tb);
        c = exact_codes8(v, tb);
      }
      c = fp4_clear_neg_zero(c);
    }
    if (FLAGS & F_CODES) NVFP4_ST(reinterpret_cast<unsigned *>(codes) + hb, c);
    if ((FLAGS & F_SCALES_OUT) && (hb & 1) == 0) st_out(scales_out + blk, (uint8_t)byte);
    if (FLAGS & F_Y) {
      float dq[8];
      fp4_decode8(c, dq);
#pragma unroll
      for (int i = 0; i < 8; ++i) dq[i] = (dq[i] * s) * S;
      if (OUT_DT == NVFP4_DTYPE_BF16) {
        unsigned w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = bf16x2_bits(dq[2 * k], dq[2 * k + 1]);
        st_out(reinterpret_cast<uint4 *>(y) + hb, make_uint4(w[0], w[1], w[2], w[3]));
      } else {
        float4 *p = reinterpret_cast<float4 *>(y) + 2 * hb;
        st_out(p, make_float4(dq[0], dq[1], dq[2], dq[3]));
        st_out(p + 1, make_float4(dq[4], dq[5], dq[6], dq[7]));
      }
    }
  };
  // the two lanes of a block are both in range or both out (stride and n_half are even)
  for (int64_t base = l0;;) {
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (base + k * stride < n_half) block(off + base + k * stride, raw[k], given[k]);
    base += U * stride;
    if (base >= n_half) break;
    load_round(base);
  }
}

static unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  const int64_t cap = 1 << 20;
  return (unsigned)(g > cap ? cap : (g < 1 ? 1 : g));
}

// half blocks a lane of k_quant takes per round: four for the quantise-only forms (about 10%
// faster than one on the 4096x4096 and 12288x4096 weights, 20% on the 128-expert stack);
// one when the fake-quantised tensor is written (four was 8% slower at 8192x4096)
constexpr int quant_u(int flags) { return (flags & F_Y) ? 1 : 4; }

template <int DT, int OUT_DT>
static void dispatch_quant(int flags, const void *x, const float *S, const uint8_t *si,
                           uint8_t *codes, uint8_t *so, void *y, int64_t batch, int64_t bpb,
                           hipStream_t st) {
  const dim3 b(256);
#define NVFP4_Q(F)                                                                              \
  case F:                                                                                       \
    hipLaunchKernelGGL((k_quant<DT, OUT_DT, F, quant_u(F)>),                                    \
                       dim3(grid_for((2 * bpb + quant_u(F) - 1) / quant_u(F)), (unsigned)batch), \
                       b, 0, st, x, S, si, codes, so, y, bpb);                                  \
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
  const int64_t bpb = rows * (cols / 16);
  int flags = 0;
  if (scales_in) flags |= F_SCALES_IN;
  if (codes) flags |= F_CODES;
  if (scales_out && !scales_in) flags |= F_SCALES_OUT;
  if (y) flags |= F_Y;
  if (dtype == NVFP4_DTYPE_BF16)
    dispatch_quant<NVFP4_DTYPE_BF16, NVFP4_DTYPE_BF16>(flags, x, S, scales_in, codes, scales_out,
                                                       y, batch, bpb, st);
  else
    dispatch_quant<NVFP4_DTYPE_F32, NVFP4_DTYPE_F32>(flags, x, S, scales_in, codes, scales_out,
                                                     y, batch, bpb, st);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ dequantise

// Grid: x = chunks of blocks within one tensor, y = batch entry (one S per workgroup).
template <int OUT_DT>
__global__ void __launch_bounds__(256)
    k_dequant(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
              const float *__restrict__ S_arr, void *__restrict__ y, int64_t blocks_per_batch) {
  const float S = S_arr[blockIdx.y];
  const int64_t off = (int64_t)blockIdx.y * blocks_per_batch;
  for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l < blocks_per_batch;
       l += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = off + l;
    const int byte = given_byte(scales[blk]);
    const uint2 c = reinterpret_cast<const uint2 *>(codes)[blk];
    const float s = byte ? e4m3_value(byte) : 0.0f;
    float dq[16];
    fp4_decode8(fp4_clear_neg_zero(c.x), dq);
    fp4_decode8(fp4_clear_neg_zero(c.y), dq + 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[i] = (dq[i] * s) * S;
    store_block<OUT_DT>(y, blk, dq);
  }
}

int launch_dequant(const uint8_t *codes, const uint8_t *scales, const float *S, int64_t batch,
                   int64_t rows, int64_t cols, void *y, int out_dtype, hipStream_t st) {
  const int64_t bpb = rows * (cols / 16);
  const dim3 g(grid_for(bpb), (unsigned)batch), b(256);
  if (out_dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_dequant<NVFP4_DTYPE_BF16>, g, b, 0, st, codes, scales, S, y, bpb);
  else
    hipLaunchKernelGGL(k_dequant<NVFP4_DTYPE_F32>, g, b, 0, st, codes, scales, S, y, bpb);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

// Block-scale searches for gfx950: MSE over the 126 positive E4M3 scales, and
// Local-Hessian selection (Local-Hessian write-up, the paragraph on the MSE selector and
// "Change the objective").
//
// Both searches loop over candidates in a wave-uniform order, so each candidate's rounding
// table (seven exact-equivalent thresholds and eight dequantised magnitudes, which depend
// only on the candidate and the tensor scale) is read from LDS by every lane at the same
// address. One lane owns one (row, block): it keeps its 16 values in registers and runs
// the objective in the same fixed order as the oracle, so chosen bytes and objectives are
// bitwise reproducible.
#include <float.h>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int kTab = 16;  // floats per candidate entry: t[0..6], d[1..7], 2 pad

__device__ __forceinline__ void build_tables(float (*tab)[kTab], float S) {
  for (int c = threadIdx.x; c < 126; c += blockDim.x) {
    ScaleTable tb;
    make_table(c + 1, S, tb);
#pragma unroll
    for (int j = 0; j < 7; ++j) tab[c][j] = tb.t[j];
#pragma unroll
    for (int j = 1; j < 8; ++j) tab[c][6 + j] = tb.d[j];
    tab[c][14] = 0.0f;
    tab[c][15] = 0.0f;
  }
}

// magnitude of the dequantised value of |x| under a candidate's table
__device__ __forceinline__ float rtn_mag(float X, const float *e) {
  float d = 0.0f;
#pragma unroll
  for (int j = 0; j < 7; ++j) d = (X > e[j]) ? e[7 + j] : d;
  return d;
}

template <int DT>
__device__ __forceinline__ void load16(const void *__restrict__ x, int64_t blk, float v[16]) {
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

// MSE objective of one candidate: fp32, e_i = fp32(dq_i - x_i), acc = fma(e_i, e_i, acc).
// With |x| and the magnitude: dq - x = sign(x) (d - |x|) rounds symmetrically, and for a
// zero code (d = 0) it is -x; the square is the same either way.
__device__ __forceinline__ float mse_obj(const float X[16], const float *e) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float err = rtn_mag(X[i], e) - X[i];
    acc = __builtin_fmaf(err, err, acc);
  }
  return acc;
}

__device__ __forceinline__ void mse_search(const float X[16], const float (*tab)[kTab],
                                           int &best_c, float &best) {
  best = INFINITY;
  best_c = 0;
  for (int c = 0; c < 126; ++c) {
    float e[kTab];
#pragma unroll
    for (int j = 0; j < 14; ++j) e[j] = tab[c][j];
    const float acc = mse_obj(X, e);
    if (acc < best) {
      best = acc;
      best_c = c + 1;
    }
  }
}

// ------------------------------------------------------------------ MSE
//
// Exact candidate pruning (the result is the exhaustive search's, bit for bit):
//  * c_z = the smallest byte at which every value of the block rounds to 0 (amax <= s S/4).
//    All bytes >= c_z produce the same codes (0), the same errors (-x) and the same fp32
//    objective, so with first-index ties only c_z itself can win among them.
//  * c_b = the largest byte whose top grid value D7 = fp32(6 s S) is <= amax. For every
//    byte c <= c_b the block max is coded 7 and its error e = fp32(D7(c) - amax) grows as c
//    falls, and the fp32 fma chain never decreases, so obj(c) >= fp32(e*e) =: LB(c), a
//    lower bound that is non-increasing in c. Bytes below c_b are visited downwards until
//    LB exceeds the best objective; then no smaller byte can win.
// Each lane owns one block and walks its own window [max(c_b,1), c_hi], then downwards;
// per-candidate constants (s, the two bracketing reciprocals of s S) come from an LDS table.

struct Cand {
  float s, rlo, rhi, pad;
};

__device__ __forceinline__ void build_cands(Cand *cand, float S) {
  for (int c = threadIdx.x; c < 127; c += blockDim.x) {
    Cand e;
    e.s = c ? e4m3_value(c) : 0.0f;
    e.rlo = e.rhi = 0.0f;
    if (c) recip_bracket((double)e.s * (double)S, e.rlo, e.rhi);
    e.pad = 0.0f;
    cand[c] = e;
  }
}

// fp32 objective of candidate byte c for |x| (codes unsigned): sum of fma(e, e, acc) in order.
// fast_ok: all products x * r stay in the normal fp32 range, so the bracketed hardware
// conversions apply; otherwise the exact threshold table decides every code.
__device__ __forceinline__ float mse_candidate(const float X[16], int c, const Cand &e, float S,
                                               bool fast_ok) {
  unsigned c0, c1;
  if (fast_ok) {
    const double sS = (double)e.s * (double)S;
    c0 = fp4_exact_codes8(X, e.rlo, e.rhi, sS);
    c1 = fp4_exact_codes8(X + 8, e.rlo, e.rhi, sS);
  } else {
    ScaleTable tb;
    make_table(c, S, tb);
    c0 = exact_codes8(X, tb);
    c1 = exact_codes8(X + 8, tb);
  }
  float g[16];
  fp4_decode8(c0, g);
  fp4_decode8(c1, g + 8);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float d = (g[i] * e.s) * S;  // fp32(G s S): G s is exact
    const float err = d - X[i];
    acc = __builtin_fmaf(err, err, acc);
  }
  return acc;
}

template <int DT>
__global__ void __launch_bounds__(256)
    k_mse(const void *__restrict__ w, const float *__restrict__ S_arr, uint8_t *__restrict__ scales,
          float *__restrict__ obj, int64_t blocks_per_batch) {
  __shared__ Cand cand[127];
  const int64_t batch = blockIdx.y;
  const float S = S_arr[batch];
  build_cands(cand, S);
  __syncthreads();
  const int64_t local = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (local >= blocks_per_batch) return;
  const int64_t blk = batch * blocks_per_batch + local;
  float v[16], X[16];
  load16<DT>(w, blk, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    X[i] = fabsf(v[i]);
    amax = fmaxf(amax, X[i]);
  }
  int best_c = 0;
  float best = 0.0f;
  if (amax != 0.0f) {
    const double a = amax, Sd = S;
    // c_z: smallest byte with amax <= s S / 4 (exact); 127 if none
    int cz;
    {
      const float q = fminf(amax * cand[1].rhi * 0x1p-7f, 448.0f);  // ~ 4 amax / S (guess)
      cz = __builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xFF;
      cz = cz < 1 ? 1 : (cz > 126 ? 126 : cz);
      while (cz > 1 && 0.25 * e4m3_value_d(cz - 1) * Sd >= a) --cz;
      while (cz <= 126 && 0.25 * e4m3_value_d(cz) * Sd < a) ++cz;
    }
    // c_b: largest byte with fp32(6 s S) <= amax; 0 if none
    int cb;
    {
      const float q = fminf(amax * cand[1].rlo * 0x1p-9f * (1.0f / 6.0f), 448.0f);
      cb = __builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xFF;
      cb = cb > 126 ? 126 : cb;
      while (cb < 126 && (6.0f * cand[cb + 1].s) * S <= amax) ++cb;
      while (cb >= 1 && (6.0f * cand[cb].s) * S > amax) --cb;
    }
    const int c_hi = cz <= 126 ? cz : 126;
    const int c_lo = cb >= 1 ? cb : 1;
    // the largest products (byte 1) stay finite and the smallest reciprocal (byte 126) normal
    const bool fast_ok = amax * cand[1].rhi < 0x1p126f && cand[126].rlo >= 0x1p-126f;
    best = INFINITY;
    for (int c = c_lo; c <= c_hi; ++c) {
      const float o = mse_candidate(X, c, cand[c], S, fast_ok);
      if (o < best) {
        best = o;
        best_c = c;
      }
    }
    for (int c = c_lo - 1; c >= 1; --c) {
      const float e7 = (6.0f * cand[c].s) * S - amax;
      if (e7 * e7 > best) break;  // LB(c) > best, and LB only grows below
      const float o = mse_candidate(X, c, cand[c], S, fast_ok);
      if (o <= best) {  // ties: the smaller byte wins
        best = o;
        best_c = c;
      }
    }
  }
  scales[blk] = (uint8_t)best_c;
  if (obj) obj[blk] = best;
}

int launch_mse(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
               const float *S, uint8_t *scales, float *obj, hipStream_t st) {
  const int64_t bpb = rows * (cols / 16);
  const dim3 g((unsigned)((bpb + 255) / 256), (unsigned)batch), b(256);
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_mse<NVFP4_DTYPE_BF16>, g, b, 0, st, w, S, scales, obj, bpb);
  else
    hipLaunchKernelGGL(k_mse<NVFP4_DTYPE_F32>, g, b, 0, st, w, S, scales, obj, bpb);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ Local-Hessian

// Grid: x = chunks of 256 rows, y = block column b, z = batch entry. All rows of block
// column b share H_b (the block-diagonal approximation), held in LDS as doubles.
template <int DT>
__global__ void __launch_bounds__(256)
    k_lh_exact(const void *__restrict__ w, const float *__restrict__ S_arr,
               const float *__restrict__ H, uint8_t *__restrict__ scales, double *__restrict__ obj,
               int64_t rows, int64_t nb) {
  __shared__ float tab[126][kTab];
  __shared__ double hb[256];
  const int64_t batch = blockIdx.z, b = blockIdx.y;
  build_tables(tab, S_arr[batch]);
  const float hv = H[(batch * nb + b) * 256 + threadIdx.x];
  hb[threadIdx.x] = (double)hv;
  const int h_nonzero = __syncthreads_or(hv != 0.0f);
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  const int64_t blk = (batch * rows + row) * nb + b;
  float v[16], X[16];
  load16<DT>(w, blk, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    X[i] = fabsf(v[i]);
    amax = fmaxf(amax, X[i]);
  }
  int best_c = 0;
  double best_o = 0.0;
  if (amax != 0.0f) {
    if (!h_nonzero) {
      float bm;
      mse_search(X, tab, best_c, bm);
    } else {
      best_o = INFINITY;
      for (int c = 0; c < 126; ++c) {
        float e[kTab];
#pragma unroll
        for (int j = 0; j < 14; ++j) e[j] = tab[c][j];
        double dl[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float d = rtn_mag(X[i], e);
          const float dq = (v[i] < 0.0f && d > 0.0f) ? -d : d;
          dl[i] = (double)(dq - v[i]);
        }
        // i stays a rolled (wave-uniform) loop so H_b rows stream from LDS instead of
        // being hoisted into registers; dl[i] is a uniform register index
        double o = 0.0;
#pragma unroll 1
        for (int i = 0; i < 16; ++i) {
          double y = 0.0;
#pragma unroll
          for (int j = 0; j < 16; ++j) y = __dadd_rn(y, __dmul_rn(hb[i * 16 + j], dl[j]));
          o = __dadd_rn(o, __dmul_rn(dl[i], y));
        }
        if (o < best_o) {
          best_o = o;
          best_c = c + 1;
        }
      }
    }
  }
  scales[blk] = (uint8_t)best_c;
  if (obj) obj[blk] = best_o;
}

int launch_local_hessian(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         const float *S, const float *H, uint8_t *scales, double *obj,
                         hipStream_t st) {
  const int64_t nb = cols / 16;
  const dim3 g((unsigned)((rows + 255) / 256), (unsigned)nb, (unsigned)batch), b(256);
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_lh_exact<NVFP4_DTYPE_BF16>, g, b, 0, st, w, S, H, scales, obj, rows, nb);
  else
    hipLaunchKernelGGL(k_lh_exact<NVFP4_DTYPE_F32>, g, b, 0, st, w, S, H, scales, obj, rows, nb);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

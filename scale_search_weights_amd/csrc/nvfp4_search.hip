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

// c_z: the smallest byte with amax <= s S / 4 (every value rounds to 0), 127 if none;
// c_b: the largest byte with fp32(6 s S) <= amax (the block max saturates), 0 if none.
// Both start from an FP8-convert guess and are settled by exact comparisons.
__device__ __forceinline__ void window_bounds(float amax, const Cand *cand, float S, int &cz,
                                              int &cb) {
  const double a = amax, Sd = S;
  const float qz = fminf(amax * cand[1].rhi * 0x1p-7f, 448.0f);  // ~ 4 amax / S
  cz = __builtin_amdgcn_cvt_pk_fp8_f32(qz, qz, 0, false) & 0xFF;
  cz = cz < 1 ? 1 : (cz > 126 ? 126 : cz);
  while (cz > 1 && 0.25 * e4m3_value_d(cz - 1) * Sd >= a) --cz;
  while (cz <= 126 && 0.25 * e4m3_value_d(cz) * Sd < a) ++cz;
  const float qb = fminf(amax * cand[1].rlo * 0x1p-9f * (1.0f / 6.0f), 448.0f);  // ~ amax/(6S)
  cb = __builtin_amdgcn_cvt_pk_fp8_f32(qb, qb, 0, false) & 0xFF;
  cb = cb > 126 ? 126 : cb;
  while (cb < 126 && (6.0f * cand[cb + 1].s) * S <= amax) ++cb;
  while (cb >= 1 && (6.0f * cand[cb].s) * S > amax) --cb;
}

// products x * r stay in the normal fp32 range for every candidate
__device__ __forceinline__ bool fast_path_ok(float amax, const Cand *cand) {
  return amax * cand[1].rhi < 0x1p126f && cand[126].rlo >= 0x1p-126f;
}

// Pruned MSE search over |x| (see above); amax > 0.
__device__ __forceinline__ void mse_pruned(const float X[16], float amax, const Cand *cand,
                                           float S, int &best_c, float &best) {
  int cz, cb;
  window_bounds(amax, cand, S, cz, cb);
  const int c_hi = cz <= 126 ? cz : 126;
  const int c_lo = cb >= 1 ? cb : 1;
  const bool fast_ok = fast_path_ok(amax, cand);
  best = INFINITY;
  best_c = 0;
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
  if (amax != 0.0f) mse_pruned(X, amax, cand, S, best_c, best);
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
//
// Grid: x = chunks of 256 rows, y = block column b, z = batch entry. All rows of block
// column b share H_b (the block-diagonal approximation), held in LDS as doubles.
//
// The objective of a candidate is evaluated exactly as the definition fixes it (fp64,
// ascending indices, one fma per term), so bytes and objectives match bit for bit. Only
// candidates that can win are evaluated:
//  * bytes >= c_z (every value rounds to 0) share one objective: only c_z is evaluated;
//  * below c_b the block max saturates; with g_i = H_ii - sum_{j!=i} (|H_ij| + |H_ji|)/2,
//    d H d^T >= sum_i g_i d_i^2 for any d, so when every g_i > 0 the block max's own error
//    e7 gives obj(c) >= g_m e7(c)^2, non-increasing in c. Bytes below c_b are visited
//    downwards until that bound, with a margin covering the fp64 rounding of the objective
//    (gamma_33 times kappa = max_i (H_ii + r_i) / g_i), exceeds the best objective.

__device__ __forceinline__ double lh_candidate(const float v[16], int c, const Cand &e, float S,
                                               bool fast_ok, const double *hb) {
  unsigned c0, c1;
  if (fast_ok) {
    const double sS = (double)e.s * (double)S;
    c0 = fp4_exact_codes8(v, e.rlo, e.rhi, sS);
    c1 = fp4_exact_codes8(v + 8, e.rlo, e.rhi, sS);
  } else {
    ScaleTable tb;
    make_table(c, S, tb);
    c0 = exact_codes8(v, tb);
    c1 = exact_codes8(v + 8, tb);
  }
  float g[16];
  fp4_decode8(fp4_clear_neg_zero(c0), g);
  fp4_decode8(fp4_clear_neg_zero(c1), g + 8);
  double dl[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) dl[i] = (double)((g[i] * e.s) * S - v[i]);  // fp32(dq - w)
  // i stays a rolled, wave-uniform loop so H rows stream from LDS rather than occupying
  // 512 VGPRs; dl[i] becomes a uniform register index
  double o = 0.0;
#pragma unroll 1
  for (int i = 0; i < 16; ++i) {
    double y = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) y = __builtin_fma(hb[i * 16 + j], dl[j], y);
    o = __builtin_fma(dl[i], y, o);
  }
  return o;
}

template <int DT>
__global__ void __launch_bounds__(256)
    k_lh(const void *__restrict__ w, const float *__restrict__ S_arr, const float *__restrict__ H,
         uint8_t *__restrict__ scales, double *__restrict__ obj, int64_t rows, int64_t nb) {
  __shared__ Cand cand[127];
  __shared__ double hb[256];
  __shared__ double gw[16];
  __shared__ double kap[16];
  const int64_t batch = blockIdx.z, b = blockIdx.y;
  const float S = S_arr[batch];
  build_cands(cand, S);
  const float hv = H[(batch * nb + b) * 256 + threadIdx.x];
  hb[threadIdx.x] = (double)hv;
  const int h_nonzero = __syncthreads_or(hv != 0.0f);
  if (threadIdx.x < 16) {
    const int i = threadIdx.x;
    double off = 0.0;
    for (int j = 0; j < 16; ++j)
      if (j != i) off += 0.5 * (fabs(hb[i * 16 + j]) + fabs(hb[j * 16 + i]));
    const double d = hb[i * 17];
    const double g = d - off - 1e-12 * (fabs(d) + off);  // margin for the rounding of these sums
    gw[i] = g;
    kap[i] = g > 0.0 ? (fabs(d) + off) / g : INFINITY;
  }
  __syncthreads();
  double kappa = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) kappa = fmax(kappa, kap[i]);
  // prune only with a well-defined bound; margin on the comparison with fp64 objectives
  const bool prune = kappa < 1e9;
  const double margin = 1.0 + 8e-15 * kappa + 1e-13;

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
  int m = 0;  // first index of the block max
#pragma unroll
  for (int i = 15; i >= 0; --i) m = (X[i] == amax) ? i : m;
  int best_c = 0;
  double best_o = 0.0;
  if (amax != 0.0f) {
    if (!h_nonzero) {
      float bm;
      mse_pruned(X, amax, cand, S, best_c, bm);
    } else {
      int cz, cb;
      window_bounds(amax, cand, S, cz, cb);
      const int c_hi = cz <= 126 ? cz : 126;
      const int c_lo = cb >= 1 ? cb : 1;
      const bool fast_ok = fast_path_ok(amax, cand);
      double gm = gw[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) gm = (m == i) ? gw[i] : gm;
      best_o = INFINITY;
      for (int c = c_lo; c <= c_hi; ++c) {
        const double o = lh_candidate(v, c, cand[c], S, fast_ok, hb);
        if (o < best_o) {
          best_o = o;
          best_c = c;
        }
      }
      for (int c = c_lo - 1; c >= 1; --c) {
        if (prune) {
          const double e7 = (double)((6.0f * cand[c].s) * S - amax);
          if (gm * e7 * e7 > best_o * margin) break;
        }
        const double o = lh_candidate(v, c, cand[c], S, fast_ok, hb);
        if (o <= best_o) {  // ties: the smaller byte wins
          best_o = o;
          best_c = c;
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
    hipLaunchKernelGGL(k_lh<NVFP4_DTYPE_BF16>, g, b, 0, st, w, S, H, scales, obj, rows, nb);
  else
    hipLaunchKernelGGL(k_lh<NVFP4_DTYPE_F32>, g, b, 0, st, w, S, H, scales, obj, rows, nb);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

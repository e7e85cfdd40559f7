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

// ------------------------------------------------------------------ search statistics
//
// Process-wide device counters of the work the searches do (NVFP4_STAT_* indices), filled
// only by the STATS instantiations, which the launchers pick while counting is switched on.
__device__ unsigned long long g_search_stats[NVFP4_STATS_N];
static bool g_stats_on = false;

// sum of v over the wave, added to counter i by lane 0
__device__ __forceinline__ void stat_add(int i, unsigned v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += (unsigned)__shfl_xor((int)v, off, 64);
  if ((threadIdx.x & 63) == 0 && v) atomicAdd(&g_search_stats[i], (unsigned long long)v);
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
//  * Upwards from c_b, the values that round to 0 at byte c (x <= s S / 4) contribute x^2
//    each; the fp32 chain over just those terms is a lower bound that never decreases in c,
//    so the upward walk stops once it exceeds the best objective.
// Each lane owns one block and walks its own window [max(c_b,1), c_hi], then downwards;
// per-candidate constants (s, the two bracketing reciprocals of s S) come from an LDS table.

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
                                           float S, int &best_c, float &best, unsigned &n_eval) {
  int cz, cb;
  window_bounds(amax, cand, S, cz, cb);
  const int c_hi = cz <= 126 ? cz : 126;
  const int c_lo = cb >= 1 ? cb : 1;
  const bool fast_ok = fast_path_ok(amax, cand);
  best = INFINITY;
  best_c = 0;
  for (int c = c_lo; c <= c_hi; ++c) {
    // upward bound: the values that round to 0 at byte c have error -x exactly, so the fp32
    // chain over only those terms (same order, the others zero) is at most obj(c); the set
    // only grows with c, so once this exceeds the best objective no larger byte can win.
    // Checked at every second byte (measured fastest: one more candidate at most)
    if (c > c_lo && ((c - c_lo) & 1) == 0) {
      const float z = cand[c].z;
      float lb = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t = X[i] <= z ? X[i] : 0.0f;
        lb = __builtin_fmaf(t, t, lb);
      }
      if (lb > best) break;
    }
    const float o = mse_candidate(X, c, cand[c], S, fast_ok);
    ++n_eval;
    if (o < best) {
      best = o;
      best_c = c;
    }
  }
  for (int c = c_lo - 1; c >= 1; --c) {
    const float e7 = (6.0f * cand[c].s) * S - amax;
    if (e7 * e7 > best) break;  // LB(c) > best, and LB only grows below
    const float o = mse_candidate(X, c, cand[c], S, fast_ok);
    ++n_eval;
    if (o <= best) {  // ties: the smaller byte wins
      best = o;
      best_c = c;
    }
  }
}

template <int DT, bool STATS>
__global__ void __launch_bounds__(256)
    k_mse(const void *__restrict__ w, const float *__restrict__ S_arr, uint8_t *__restrict__ scales,
          float *__restrict__ obj, int64_t blocks_per_batch) {
  __shared__ Cand cand[127];
  const int64_t batch = blockIdx.y;
  const float S = S_arr[batch];
  const int64_t local = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = local < blocks_per_batch;
  const int64_t blk = batch * blocks_per_batch + (active ? local : 0);
  float v[16], X[16];
  load16<DT>(w, blk, v);  // in flight while the table is built
  build_cands(cand, S);
  lds_barrier();
  if (!STATS && !active) return;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    X[i] = fabsf(v[i]);
    amax = fmaxf(amax, X[i]);
  }
  if (!active) amax = 0.0f;  // (STATS: every lane reaches the wave sums below)
  int best_c = 0;
  float best = 0.0f;
  unsigned n_eval = 0;
  if (amax != 0.0f) mse_pruned(X, amax, cand, S, best_c, best, n_eval);
  if (active) {
    scales[blk] = (uint8_t)best_c;
    if (obj) obj[blk] = best;
  }
  if (STATS) {
    stat_add(NVFP4_STAT_MSE_BLOCKS, amax != 0.0f ? 1u : 0u);
    stat_add(NVFP4_STAT_MSE_EVALS, n_eval);
  }
}

int launch_mse(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
               const float *S, uint8_t *scales, float *obj, hipStream_t st) {
  const int64_t bpb = rows * (cols / 16);
  const dim3 g((unsigned)((bpb + 255) / 256), (unsigned)batch), b(256);
  if (dtype == NVFP4_DTYPE_BF16) {
    if (g_stats_on) hipLaunchKernelGGL((k_mse<NVFP4_DTYPE_BF16, true>), g, b, 0, st, w, S, scales, obj, bpb);
    else hipLaunchKernelGGL((k_mse<NVFP4_DTYPE_BF16, false>), g, b, 0, st, w, S, scales, obj, bpb);
  } else {
    if (g_stats_on) hipLaunchKernelGGL((k_mse<NVFP4_DTYPE_F32, true>), g, b, 0, st, w, S, scales, obj, bpb);
    else hipLaunchKernelGGL((k_mse<NVFP4_DTYPE_F32, false>), g, b, 0, st, w, S, scales, obj, bpb);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ Four Over Six
//
// Local-Hessian write-up, paragraph on max / Four-Over-Six / MSE selection: one of two
// candidate scales per block. Reading: the bytes nearest amax/(6S) and amax/(4S) (block max
// on the E2M1 magnitudes 6 and 4); the smaller MSE objective (the same fp32 chain as the MSE
// search) wins, ties to the smaller byte. One lane per block, as for MSE.

template <int DT>
__global__ void __launch_bounds__(256)
    k_four_over_six(const void *__restrict__ w, const float *__restrict__ S_arr,
                    uint8_t *__restrict__ scales, float *__restrict__ obj,
                    int64_t blocks_per_batch) {
  __shared__ Cand cand[127];
  const int64_t batch = blockIdx.y;
  const float S = S_arr[batch];
  const int64_t local = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = local < blocks_per_batch;
  const int64_t blk = batch * blocks_per_batch + (active ? local : 0);
  float v[16], X[16];
  load16<DT>(w, blk, v);  // in flight while the table is built
  build_cands(cand, S);
  lds_barrier();
  if (!active) return;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    X[i] = fabsf(v[i]);
    amax = fmaxf(amax, X[i]);
  }
  int best_c = 0;
  float best = 0.0f;
  if (amax != 0.0f) {
    // cand[0] brackets 1/(6S); 1/(4S) = 1.5/(6S) keeps the bracket (one rounding < 2^-24)
    const int c6 = max_scale_byte_fast(amax, cand[0].rlo, cand[0].rhi, S, 6.0f);
    const int c4 = max_scale_byte_fast(amax, 1.5f * cand[0].rlo, 1.5f * cand[0].rhi, S, 4.0f);
    const bool fast_ok = fast_path_ok(amax, cand);
    const float o6 = mse_candidate(X, c6, cand[c6], S, fast_ok);
    const float o4 = mse_candidate(X, c4, cand[c4], S, fast_ok);
    const bool take4 = o4 < o6;  // c4 >= c6: on equal objectives the smaller byte wins
    best_c = take4 ? c4 : c6;
    best = take4 ? o4 : o6;
  }
  scales[blk] = (uint8_t)best_c;
  if (obj) obj[blk] = best;
}

int launch_four_over_six(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         const float *S, uint8_t *scales, float *obj, hipStream_t st) {
  const int64_t bpb = rows * (cols / 16);
  const dim3 g((unsigned)((bpb + 255) / 256), (unsigned)batch), b(256);
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_four_over_six<NVFP4_DTYPE_BF16>, g, b, 0, st, w, S, scales, obj, bpb);
  else
    hipLaunchKernelGGL(k_four_over_six<NVFP4_DTYPE_F32>, g, b, 0, st, w, S, scales, obj, bpb);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ Local-Hessian
//
// Grid: x = groups of up to 8 tiles of 64 rows, y = block column b, z = batch entry. All
// rows of block column b share H_b (the block-diagonal approximation), held in LDS as
// doubles. A workgroup first stages its rows' blocks in LDS (one thread per row, with the
// block max, the first index of the max and the candidate window) and sorts the rows by
// window length, so that the 16 pairs of a wave step through windows of about the same
// length; it then takes its rows 64 at a time in that order.
//
// The chosen byte and its objective equal those of the definition evaluated exactly as it
// is written (fp64, ascending indices, one fma per term), bit for bit. Only candidates that
// can win are visited:
//  * bytes >= c_z (every value rounds to 0) share one objective: only c_z is visited;
//  * below c_b the block max saturates; with g_i = H_ii - sum_{j!=i} (|H_ij| + |H_ji|)/2,
//    d H d^T >= sum_i g_i d_i^2 for any d, so when every g_i > 0 the block max's own error
//    e7 gives obj(c) >= g_m e7(c)^2, non-increasing in c. Bytes below c_b are visited
//    downwards until that bound, with a margin covering the fp64 rounding of the objective
//    (gamma_33 times kappa = max_i (H_ii + r_i) / g_i), exceeds the best objective.
//
// A wave handles 16 (row, block) pairs of one block column: lane l owns pair p = l & 15 and the
// four elements 4q..4q+3, q = l >> 4. For a candidate each lane forms its four fp32 weight
// errors d and four v_mfma_f32_16x16x4_f32 compute Y = H_b d for all 16 pairs: in step t the
// K slot of lane group q is element 4q + t, so A = H[p][4q+t] and B = d_p[4q+t] are the
// lane's own values, and the 16x16 result leaves Y_p[4q..4q+3] in the lane that holds
// d_p[4q..4q+3]. A four-term dot and two cross-lane adds give the fp32 objective.
// Screening: |fp32 obj - exact obj| <= 1e-5 A + t, A = sum_ij |d_i||H_ij||d_j|. The constant
// is ~8x the worst-case fp32 rounding of the 16-term products, the four-term dot and the two
// adds; t = 2^-138 (1 + amax) covers roundings in the denormal range (the fp32 MFMA keeps
// denormals). A <= (sum |d_i| a_i)^2 with a_i^2 >= max_j max(|H_ij|, |H_ji|); when every
// g_i > 0 (below), also A <= kappa d H d^T, so for kappa <= 1e4 the bound is relative to the
// objective. Each lane keeps theta = min(obj + err) and the three smallest (obj - err) of
// the candidates it scored (a candidate is scored by one lane of its pair); every
// candidate that can still be the exact argmin has obj - err <= theta (the pair's theta).
// If at most two do, they are re-evaluated in the exact fp64 order (split over the pair's
// four lanes) and the smaller wins; if three or more do, or values are too small or large
// for the fast path or for fp32, the pair is rescanned exactly. The downward pruning
// compares with theta.

// the four fp32 weight errors of this lane's elements under candidate c
__device__ __forceinline__ void lh_delta4(const float v[4], int c, const Cand &e, float S,
                                          bool fast_ok, float d[4], bool act = true) {
  unsigned code;
  if (fast_ok) {
    unsigned a = 0u, b = 0u;
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[0] * e.rlo, v[1] * e.rlo, 1.0f, 0);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[2] * e.rlo, v[3] * e.rlo, 1.0f, 1);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, v[0] * e.rhi, v[1] * e.rhi, 1.0f, 0);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, v[2] * e.rhi, v[3] * e.rhi, 1.0f, 1);
    a &= 0xFFFFu;
    b &= 0xFFFFu;
    if (a != b && act) {
      float v8[8] = {v[0], v[1], v[2], v[3], 0.0f, 0.0f, 0.0f, 0.0f};
      a = fp4_resolve8(v8, a, b, (double)e.s * (double)S);
    }
    code = a;
  } else {
    ScaleTable tb;
    make_table(c, S, tb);
    float v8[8] = {v[0], v[1], v[2], v[3], 0.0f, 0.0f, 0.0f, 0.0f};
    code = exact_codes8(v8, tb) & 0xFFFFu;
  }
  // (a -0 code needs no clearing here: -0 - v and +0 - v are the same error)
  nv_v2f g01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
  nv_v2f g23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 1);
  d[0] = (g01.x * e.s) * S - v[0];
  d[1] = (g01.y * e.s) * S - v[1];
  d[2] = (g23.x * e.s) * S - v[2];
  d[3] = (g23.y * e.s) * S - v[3];
}

// x of rows 0, 1, 2, 3 (same lane within the row), in every lane
__device__ __forceinline__ void rows4(float x, float out[4]) {
  const LanePair a = swap16(x, x);       // rows (0 | 2, 1 | 3)
  const LanePair e = swap32(a.r0, a.r0);  // rows (0, 2)
  const LanePair o = swap32(a.r1, a.r1);  // rows (1, 3)
  out[0] = e.r0;
  out[1] = o.r0;
  out[2] = e.r1;
  out[3] = o.r1;
}

// exact fp64 objective (the definition's order) of the pair, from the four lanes' errors;
// every lane of the pair returns the same value. Row q holds errors 4q..4q+3 in d[0..3].
__device__ __forceinline__ double lh_exact_split(const float d[4], int q, const double *hb) {
  float D[16];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float t[4];
    rows4(d[r], t);
#pragma unroll
    for (int g = 0; g < 4; ++g) D[4 * g + r] = t[g];
  }
  // y_i for this row's four indices i = 4q + r; the source row g stays a rolled, wave-uniform
  // loop so H streams from LDS instead of being hoisted into registers
  double y[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const double dj = (double)D[4 * g + jj];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = __builtin_fma(hb[(4 * q + r) * 16 + 4 * g + jj], dj, y[r]);
    }
  }
  double Y[16];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float lo[4], hi[4];
    rows4(__int_as_float(__double2loint(y[r])), lo);
    rows4(__int_as_float(__double2hiint(y[r])), hi);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      Y[4 * g + r] = __hiloint2double(__float_as_int(hi[g]), __float_as_int(lo[g]));
  }
  double o = 0.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) o = __builtin_fma((double)D[k], Y[k], o);
  return o;
}

// Screening state of one lane: the smallest upper bound and the three smallest lower bounds
// (with the bytes of the first two) over the candidates this lane has scored.
struct Screen {
  float theta, L1, L2, L3;
  int c1, c2;
};

// (selects, no branches: L1 <= L2 <= L3, so L < L1 implies L < L2 < ... ; L = +inf changes
// nothing)
__device__ __forceinline__ void screen_add(Screen &z, float L, float U, int c) {
  z.theta = fminf(z.theta, U);
  const bool b1 = L < z.L1, b2 = L < z.L2, b3 = L < z.L3;
  z.L3 = b2 ? z.L2 : (b3 ? L : z.L3);
  z.L2 = b1 ? z.L1 : (b2 ? L : z.L2);
  z.c2 = b1 ? z.c1 : (b2 ? c : z.c2);
  z.L1 = b1 ? L : z.L1;
  z.c1 = b1 ? c : z.c1;
}

constexpr int LH_TILES = 8;                // tiles of 64 rows per workgroup, at most
constexpr int LH_ROWS_MAX = 64 * LH_TILES;

template <int DT, bool STATS>
__global__ void __launch_bounds__(256)
    k_lh_mfma(const void *__restrict__ w, const float *__restrict__ S_arr,
              const float *__restrict__ H, uint8_t *__restrict__ scales, double *__restrict__ obj,
              int64_t rows, int64_t nb, int64_t tiles_per_wg) {
  __shared__ Cand cand[127];
  __shared__ double hb[256];
  __shared__ double gw[16];
  __shared__ double kap[16];
  __shared__ float aw[16];
  __shared__ int32_t ord[LH_ROWS_MAX];  // this workgroup's rows (offsets), in key order
  __shared__ uint32_t bins[128];
  // per row of the workgroup: its block as stored, the block max, and c_lo | c_hi << 8 |
  // (first index of the max) << 16
  constexpr int VB = DT == NVFP4_DTYPE_BF16 ? 32 : 64;
  __shared__ __attribute__((aligned(16))) unsigned char wv[LH_ROWS_MAX * VB];
  __shared__ float amx[LH_ROWS_MAX];
  __shared__ int32_t meta[LH_ROWS_MAX];
  // Workgroups go to the eight XCDs round-robin by linear id; renumber them so that each XCD
  // takes one contiguous range (neighbouring block columns share 128-byte lines of W and of
  // the scale bytes, and each XCD has its own L2).
  const int64_t gx = gridDim.x, gy = gridDim.y, n_wg = gx * gy * gridDim.z;
  int64_t wid = blockIdx.x + gx * (blockIdx.y + gy * (int64_t)blockIdx.z);
  if ((n_wg & 7) == 0) wid = (wid & 7) * (n_wg >> 3) + (wid >> 3);
  const int64_t wx = wid % gx, batch = wid / (gx * gy), b = (wid / gx) % gy;
  const float S = S_arr[batch];
  build_cands(cand, S);
  const float hv = H[(batch * nb + b) * 256 + threadIdx.x];
  hb[threadIdx.x] = (double)hv;
  const int h_nonzero = __syncthreads_or(hv != 0.0f);
  if (threadIdx.x < 16) {
    const int i = threadIdx.x;
    double off = 0.0, mx = 0.0;
    for (int j = 0; j < 16; ++j) {
      mx = fmax(mx, fmax(fabs(hb[i * 16 + j]), fabs(hb[j * 16 + i])));
      if (j != i) off += 0.5 * (fabs(hb[i * 16 + j]) + fabs(hb[j * 16 + i]));
    }
    const double dg = hb[i * 17];
    const double g = dg - off - 1e-12 * (fabs(dg) + off);
    gw[i] = g;
    kap[i] = g > 0.0 ? (fabs(dg) + off) / g : INFINITY;
    aw[i] = (float)(sqrt(mx) * (1.0 + 0x1p-20));  // a_i^2 >= max |H| along row and column i
  }
  __syncthreads();
  double kappa = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) kappa = fmax(kappa, kap[i]);
  const bool prune = kappa < 1e9;
  const double margin = 1.0 + 8e-15 * kappa + 1e-13;
  // screening error relative to the objective itself when H_b is well conditioned:
  // sum_ij |d_i||H_ij||d_j| <= kappa sum_i g_i d_i^2 <= kappa d H d^T
  const bool rel = prune && kappa <= 1e4;
  float hmax = 0.0f;  // max |H_ij| (up to the 2^-20 margin of a_i)
#pragma unroll
  for (int i = 0; i < 16; ++i) hmax = fmaxf(hmax, aw[i] * aw[i]);
  const float rho = (float)(1.2e-5 * kappa);
  // this workgroup's tiles of 64 rows
  const int64_t n_tiles = (rows + 63) / 64;
  const int64_t tile0 = wx * tiles_per_wg;
  const int64_t tile1 = min(tile0 + tiles_per_wg, n_tiles);

  if (!h_nonzero) {  // every candidate has objective 0: the MSE choice, one lane per row
    const int64_t row_end = min(tile1 * 64, rows);
    unsigned n_zero = 0, n_eval = 0;
    for (int64_t row = tile0 * 64 + threadIdx.x; row < row_end; row += blockDim.x) {
      {
        const int64_t blk = (batch * rows + row) * nb + b;
        float v[16], X[16];
        load16<DT>(w, blk, v);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          X[i] = fabsf(v[i]);
          amax = fmaxf(amax, X[i]);
        }
        int bc = 0;
        float bm = 0.0f;
        if (amax != 0.0f) mse_pruned(X, amax, cand, S, bc, bm, n_eval);
        n_zero += amax != 0.0f ? 1u : 0u;
        scales[blk] = (uint8_t)bc;
        if (obj) obj[blk] = 0.0;
      }
    }
    if (STATS) {
      stat_add(NVFP4_STAT_LH_ZERO_H, n_zero);
      stat_add(NVFP4_STAT_MSE_EVALS, n_eval);
    }
    return;
  }

  // Per row of this workgroup (one thread per row): the block, kept in LDS, its max, the first
  // index of the max and the candidate window [c_lo, c_hi]. The rows are then sorted by the
  // window's length (a counting sort in LDS), so that the 16 pairs of a wave, which step
  // through their windows together, have windows of about the same length. The order does
  // not change any pair's result.
  const int64_t r0 = tile0 * 64;
  const int nr = (int)(min(tile1 * 64, rows) - r0);  // <= LH_ROWS_MAX
  if (threadIdx.x < 128) bins[threadIdx.x] = 0u;
  __syncthreads();
  int key[LH_ROWS_MAX / 256], pos[LH_ROWS_MAX / 256];
#pragma unroll
  for (int k = 0; k < LH_ROWS_MAX / 256; ++k) {
    const int i = (int)threadIdx.x + 256 * k;
    key[k] = -1;
    if (i < nr) {
      const int64_t blk = (batch * rows + r0 + i) * nb + b;
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(w) + blk * VB);
      uint4 *dst = reinterpret_cast<uint4 *>(wv + i * VB);
      float vv[16];
#pragma unroll
      for (int j = 0; j < VB / 16; ++j) {
        const uint4 r = src[j];
        dst[j] = r;
        if (DT == NVFP4_DTYPE_BF16) {
          vv[8 * j + 0] = bf16_lo(r.x); vv[8 * j + 1] = bf16_hi(r.x);
          vv[8 * j + 2] = bf16_lo(r.y); vv[8 * j + 3] = bf16_hi(r.y);
          vv[8 * j + 4] = bf16_lo(r.z); vv[8 * j + 5] = bf16_hi(r.z);
          vv[8 * j + 6] = bf16_lo(r.w); vv[8 * j + 7] = bf16_hi(r.w);
        } else {
          vv[4 * j + 0] = __uint_as_float(r.x); vv[4 * j + 1] = __uint_as_float(r.y);
          vv[4 * j + 2] = __uint_as_float(r.z); vv[4 * j + 3] = __uint_as_float(r.w);
        }
      }
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) am = fmaxf(am, fabsf(vv[j]));
      int li = 16;
#pragma unroll
      for (int j = 15; j >= 0; --j) li = fabsf(vv[j]) == am ? j : li;
      int cz = 127, cb = 0;
      if (am != 0.0f) window_bounds(am, cand, S, cz, cb);
      const int c_hi = cz <= 126 ? cz : 126, c_lo = cb >= 1 ? cb : 1;
      const int n_up = am != 0.0f ? c_hi - c_lo + 1 : 0;
      amx[i] = am;
      meta[i] = c_lo | (c_hi << 8) | (li << 16);
      key[k] = n_up < 0 ? 0 : (n_up > 127 ? 127 : n_up);
      pos[k] = (int)atomicAdd(&bins[key[k]], 1u);
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // exclusive scan of the 128 bin counts, two per lane
    const int l = threadIdx.x;
    const uint32_t b0 = bins[2 * l], b1 = bins[2 * l + 1];
    uint32_t inc = b0 + b1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(inc, d, 64);
      inc += l >= d ? o : 0u;
    }
    bins[2 * l] = inc - b0 - b1;
    bins[2 * l + 1] = inc - b1;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < LH_ROWS_MAX / 256; ++k)
    if (key[k] >= 0) ord[bins[key[k]] + pos[k]] = (int)threadIdx.x + 256 * k;
  __syncthreads();

  const int lane = threadIdx.x & 63, p = lane & 15, q = lane >> 4;
  float ha[4], ab[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    ha[t] = (float)hb[p * 16 + 4 * q + t];
    ab[t] = aw[4 * q + t];
  }
  // statistics (STATS only): pair-path counts kept by lane group 0 of each pair, screened
  // candidates by the lane group that scores them
  unsigned st_pairs = 0, st_rel = 0, st_abs = 0, st_noprune = 0, st_rescan = 0, st_two = 0;
  unsigned st_screened = 0, st_exact = 0;
  for (int64_t tile = tile0; tile < tile1; ++tile) {
  const int idx = (int)(tile - tile0) * 64 + (int)(threadIdx.x >> 6) * 16 + p;
  const bool valid = idx < nr;
  const int64_t row = r0 + (valid ? ord[idx] : 0);
  const int64_t blk = (batch * rows + (valid ? row : 0)) * nb + b;
  const int ri = valid ? ord[idx] : 0;  // the row's slot in LDS
  float v[4];
  if (DT == NVFP4_DTYPE_BF16) {
    uint2 u = make_uint2(0u, 0u);
    if (valid) u = reinterpret_cast<const uint2 *>(wv + ri * VB)[q];
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
  } else {
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) u = reinterpret_cast<const float4 *>(wv + ri * VB)[q];
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  const float amax = valid ? amx[ri] : 0.0f;
  const int mt = meta[ri];
  const int m = mt >> 16;  // first index of the block max
  const bool live = valid && amax != 0.0f;
  const int c_lo = live ? (mt & 0xFF) : 1, c_hi = live ? ((mt >> 8) & 0xFF) : 126;
  const bool fast_ok = fast_path_ok(amax, cand) && amax >= 0x1p-60f;
  const double gm = gw[m < 16 ? m : 0];

  // ---- screen on MFMA, four candidates per step (independent MFMA chains); after the
  // transposing reduction lane group q holds the objective of the step's candidate q
  // Absolute part of the screening error: the fp32 MFMA keeps denormals (gradual underflow),
  // so each rounding below 2^-126 errs by at most 2^-150, scaled by |d_i| <= 4.5 amax.
  const float tiny = 0x1p-138f * (1.0f + amax);
  // fp32 stays finite: sum_ij |d_i||H_ij||d_j| <= hmax (sum_i |d_i|)^2 <= hmax (72 amax)^2
  const float da = 72.0f * amax;
  const bool screen_ok = fast_ok && hmax * da * da < 0x1p100f;
  bool screen = live && screen_ok;
  Screen z = {INFINITY, INFINITY, INFINITY, INFINITY, 0, 0};
  // a step: slot k scores byte base + dir k for the pairs whose bit k of `am` is set
  auto step4 = [&](int base, int dir, unsigned am) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    float P[4], B[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      P[k] = 0.0f;
      B[k] = 0.0f;
      const bool act = (am >> k) & 1u;
      if (!__any(act)) continue;  // a slot no pair of the wave uses
      const int ck = act ? base + dir * k : 1;
      // every lane forms d (an inactive lane with byte 1: finite, since fast_ok holds for
      // every byte); column p of the product depends only on pair p's d, and an inactive
      // pair's objective is not used
      float d[4];
      lh_delta4(v, ck, cand[ck], S, true, d, act);
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ha[t], d[t], acc, 0, 0, 0);
      float op = d[0] * acc[0];
#pragma unroll
      for (int r = 1; r < 4; ++r) op = __builtin_fmaf(d[r], acc[r], op);
      P[k] = op;
      if (!rel) {
        float bp = fabsf(d[0]) * ab[0];
#pragma unroll
        for (int r = 1; r < 4; ++r) bp = __builtin_fmaf(fabsf(d[r]), ab[r], bp);
        B[k] = bp;
      }
    }
    // halves: the lower half sums candidates 0 and 1 over both halves, the upper 2 and 3;
    // then rows: even rows keep the even candidate of their half, odd rows the odd one
    LanePair t = swap32(P[0], P[2]);
    const float A0 = t.r0 + t.r1;
    t = swap32(P[1], P[3]);
    const float A1 = t.r0 + t.r1;
    t = swap16(A0, A1);
    const float o = t.r0 + t.r1;
    float er;
    if (rel) {
      er = rho * fabsf(o) + 2.0f * tiny;
    } else {
      t = swap32(B[0], B[2]);
      const float C0 = t.r0 + t.r1;
      t = swap32(B[1], B[3]);
      const float C1 = t.r0 + t.r1;
      t = swap16(C0, C1);
      const float bb = t.r0 + t.r1;
      er = 1e-5f * bb * bb + tiny;
    }
    const int cq = base + dir * q;  // (arithmetic, not an indexed array: no private memory)
    const bool aq = (am >> q) & 1u;
    screen_add(z, aq ? o - er : INFINITY, aq ? o + er : INFINITY, cq);
    if (STATS) st_screened += aq ? 1u : 0u;
  };
  for (int j = 0;; j += 4) {
    unsigned am = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) am |= (screen && c_lo + j + k <= c_hi) ? 1u << k : 0u;
    if (!__any(am != 0u)) break;
    step4(c_lo + j, 1, am);
  }
  // downward: the bound uses the pair's theta so far (merged over its four lanes)
  bool down = screen;
  for (int c0 = c_lo - 1;; c0 -= 4) {
    LanePair t = swap16(z.theta, z.theta);
    float th = fminf(t.r0, t.r1);
    t = swap32(th, th);
    th = fminf(t.r0, t.r1);
    unsigned am = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 - k;
      bool a = down && c >= 1;
      if (a && prune) {
        const double e7 = (double)((6.0f * cand[c].s) * S - amax);
        if (gm * e7 * e7 > (double)th * margin) a = false;
      }
      down = a;  // the bound is monotone: once pruned, every smaller byte is too
      am |= a ? 1u << k : 0u;
    }
    if (!__any(am != 0u)) break;
    step4(c0, -1, am);
  }
  // ---- the pair's screening result. Each candidate was scored by exactly one of the pair's
  // four lanes, so their lists are disjoint: theta is the smallest upper bound, c1 the byte
  // of the smallest lower bound (ties to the smaller byte), and n the number of listed lower
  // bounds <= theta (a lane lists its three smallest, so n >= 3 means three or more
  // candidates can still be the exact argmin).
  float theta = z.theta, n_le;
  {
    LanePair t = swap16(theta, theta);
    theta = fminf(t.r0, t.r1);
    t = swap32(theta, theta);
    theta = fminf(t.r0, t.r1);
    n_le = (float)((z.L1 <= theta ? 1 : 0) + (z.L2 <= theta ? 1 : 0) + (z.L3 <= theta ? 1 : 0));
    t = swap16(n_le, n_le);
    n_le = t.r0 + t.r1;
    t = swap32(n_le, n_le);
    n_le = t.r0 + t.r1;
  }
  // (L, c) := the smaller of the pair's four (L, c) entries, ties to the smaller byte; the
  // two halves of a swap come in the same order in both lanes, so every lane agrees
  auto pair_min = [](float &L, int &c) {
    LanePair tl = swap16(L, L), tc = swap16(__int_as_float(c), __int_as_float(c));
    bool o = tl.r1 < tl.r0 || (tl.r1 == tl.r0 && __float_as_int(tc.r1) < __float_as_int(tc.r0));
    L = o ? tl.r1 : tl.r0;
    c = __float_as_int(o ? tc.r1 : tc.r0);
    tl = swap32(L, L);
    tc = swap32(__int_as_float(c), __int_as_float(c));
    o = tl.r1 < tl.r0 || (tl.r1 == tl.r0 && __float_as_int(tc.r1) < __float_as_int(tc.r0));
    L = o ? tl.r1 : tl.r0;
    c = __float_as_int(o ? tc.r1 : tc.r0);
  };
  float L1m = z.L1;
  int c1 = z.c1;
  pair_min(L1m, c1);

  // ---- exact decision
  const bool overflow = screen && n_le >= 3.0f;
  const bool slow = live && (!screen_ok || overflow);
  int best_c = 0;
  double best_o = 0.0;
  // (all cross-lane steps below run with the whole wave active; the four lanes of a pair
  // always agree on every per-pair flag)
  const bool sel = screen && !overflow;
  const bool two = sel && n_le >= 2.0f;
  int c2 = 0;
  if (__any(two)) {  // the second smallest: c1's lane offers its next entry, the others their first
    const bool own = z.c1 == c1;
    float L2m = own ? z.L2 : z.L1;
    c2 = own ? z.c2 : z.c1;
    pair_min(L2m, c2);
  }
  const bool need = sel && (two || obj != nullptr);
  if (sel) best_c = c1;
  if (__any(need)) {
    float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (need) lh_delta4(v, c1, cand[c1], S, true, d);
    const double oa = lh_exact_split(d, q, hb);
    if (need) best_o = oa;
    if (__any(two)) {
      float d2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (two) lh_delta4(v, c2, cand[c2], S, true, d2);
      const double ob = lh_exact_split(d2, q, hb);
      if (two && (ob < best_o || (ob == best_o && c2 < c1))) {
        best_o = ob;
        best_c = c2;
      }
    }
  }
  if (__any(slow)) {  // exact scan of every candidate that can win
    double bo = INFINITY;
    int bcx = 0;
    for (int j = 0;; ++j) {
      const int c = c_lo + j;
      const bool act = slow && c <= c_hi;
      if (!__any(act)) break;
      float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (act) lh_delta4(v, c, cand[c], S, fast_ok, d);
      const double o = lh_exact_split(d, q, hb);
      if (STATS && q == 0) st_exact += act ? 1u : 0u;
      if (act && o < bo) {
        bo = o;
        bcx = c;
      }
    }
    bool dn = slow;
    for (int c = c_lo - 1;; --c) {
      bool act = dn && c >= 1;
      if (act && prune) {
        const double e7 = (double)((6.0f * cand[c].s) * S - amax);
        if (gm * e7 * e7 > bo * margin) act = false;
      }
      dn = act;
      if (!__any(act)) break;
      float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (act) lh_delta4(v, c, cand[c], S, fast_ok, d);
      const double o = lh_exact_split(d, q, hb);
      if (STATS && q == 0) st_exact += act ? 1u : 0u;
      if (act && o <= bo) {
        bo = o;
        bcx = c;
      }
    }
    if (slow) {
      best_c = bcx;
      best_o = bo;
    }
  }
  if (valid && q == 0) {
    scales[blk] = (uint8_t)best_c;
    if (obj) obj[blk] = best_c ? best_o : 0.0;
  }
  if (STATS && q == 0 && live) {
    st_pairs += 1;
    st_rel += (screen && rel) ? 1u : 0u;
    st_abs += (screen && !rel) ? 1u : 0u;
    st_noprune += prune ? 0u : 1u;
    st_rescan += slow ? 1u : 0u;
    st_two += two ? 1u : 0u;
    st_exact += (need ? 1u : 0u) + (two ? 1u : 0u);
  }
  }  // tiles
  if (STATS) {
    stat_add(NVFP4_STAT_LH_PAIRS, st_pairs);
    stat_add(NVFP4_STAT_LH_REL, st_rel);
    stat_add(NVFP4_STAT_LH_ABS, st_abs);
    stat_add(NVFP4_STAT_LH_NOPRUNE, st_noprune);
    stat_add(NVFP4_STAT_LH_RESCAN, st_rescan);
    stat_add(NVFP4_STAT_LH_TWO, st_two);
    stat_add(NVFP4_STAT_LH_SCREENED, st_screened);
    stat_add(NVFP4_STAT_LH_EXACT, st_exact);
  }
}

int launch_local_hessian(const void *w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         const float *S, const float *H, uint8_t *scales, double *obj,
                         hipStream_t st) {
  const int64_t nb = cols / 16;
  // up to LH_TILES tiles of 64 rows per workgroup (the H_b analysis and candidate table are
  // shared by them), fewer when that would leave the grid under ~8192 workgroups
  const int64_t n_tiles = (rows + 63) / 64;
  const int64_t cols_batch = nb * batch;
  int64_t tpw = LH_TILES;
  while (tpw > 1 && cols_batch * ((n_tiles + tpw - 1) / tpw) < 8192) tpw >>= 1;
  const dim3 g((unsigned)((n_tiles + tpw - 1) / tpw), (unsigned)nb, (unsigned)batch), b(256);
#define NVFP4_LH(D, ST) \
  hipLaunchKernelGGL((k_lh_mfma<D, ST>), g, b, 0, st, w, S, H, scales, obj, rows, nb, tpw)
  if (dtype == NVFP4_DTYPE_BF16) {
    if (g_stats_on) NVFP4_LH(NVFP4_DTYPE_BF16, true);
    else NVFP4_LH(NVFP4_DTYPE_BF16, false);
  } else {
    if (g_stats_on) NVFP4_LH(NVFP4_DTYPE_F32, true);
    else NVFP4_LH(NVFP4_DTYPE_F32, false);
  }
#undef NVFP4_LH
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

void search_stats_enable(bool on) { g_stats_on = on; }

int search_stats_read(int64_t *out, hipStream_t st) {
  if (hipStreamSynchronize(st) != hipSuccess) return NVFP4_ERR_HIP;
  unsigned long long v[NVFP4_STATS_N];
  if (hipMemcpyFromSymbol(v, HIP_SYMBOL(g_search_stats), sizeof(v), 0, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return NVFP4_ERR_HIP;
  const unsigned long long zero[NVFP4_STATS_N] = {};
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_search_stats), zero, sizeof(zero), 0,
                        hipMemcpyHostToDevice) != hipSuccess)
    return NVFP4_ERR_HIP;
  for (int i = 0; i < NVFP4_STATS_N; ++i) out[i] = (int64_t)v[i];
  return NVFP4_OK;
}

}  // namespace nvfp4

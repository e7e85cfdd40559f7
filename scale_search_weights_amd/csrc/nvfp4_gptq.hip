// GPTQ rounding at fixed NVFP4 block scales, in double precision.
//
// [LH] (closing paragraphs): Local-Hessian picks the block scale, GPTQ picks the rounding,
// and the two combine. GPTQ (Frantar et al., 2022) quantises the columns of W in order and,
// after each column, moves the columns not yet quantised so as to cancel its rounding error
// under the layer's Gram matrix H = X^T X: with U upper triangular and U^T U = (H + lambda I)^-1,
// e_j = (v_j - q_j) / U_jj and v_k -= e_j U_jk for k > j.
//
// MI355X runs fp64 FMA and fp64 MFMA at 78.6 TFLOP/s, so the whole method stays in double:
// the codes then depend on summation order only for values within ~1e-12 (relative) of a
// rounding midpoint. Two entry points:
//  * factor: lambda = damp * mean(diag H) (index-order sum); U from one Cholesky
//    factorisation and one triangular inverse, using the reversal J (J_ij = [i + j = n-1]):
//    if J (H + lambda I) J = L L^T then H + lambda I = R R^T with R = J L J upper, and
//    U = R^-1 = J L^-1 J. Blocked right-looking Cholesky (64 x 64 blocks: per step, each
//    workgroup factors the diagonal block in one wave's registers and solves one panel
//    block; steps go in pairs, and after each pair one fp64 MFMA product with K = 128
//    updates the trailing matrix), then a bottom-up recursive inverse
//    [[A, 0], [B, C]]^-1 = [[A^-1, 0], [-C^-1 B A^-1, C^-1]] (two fp64 MFMA products per level,
//    in 64 x 64 tiles whose K differs by up to a factor nbs: launched longest first, so the
//    device balances them, where one 128 x 128 tile per compute unit waited on the longest).
//  * rows: the column loop in blocks of 64 columns. In a block, sixteen lanes share a row,
//    each holding 4 of its values in registers; for every column the owning lane rounds,
//    forms e and broadcasts it to its row of 16 lanes (DPP row_newbcast), and all of them
//    update their values with the block's row of U from LDS (e uses 1 / U_jj). Errors reach
//    later columns by GPTQ's lazy batch updates on two levels: the same kernel then applies
//    the block's errors to the rest of its 256-column outer block, and after each outer block
//    an fp64 MFMA product V[:, later] -= E U[done, later] updates all later columns at once,
//    so the working copy of W is read and written once per 256 columns.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef double gq_v4d __attribute__((ext_vector_type(4)));

constexpr int DB = 64;       // block edge
constexpr int DP = DB + 1;   // LDS pitch of a K-major tile (doubles)

static inline int64_t pad64(int64_t n) { return (n + DB - 1) / DB * DB; }
static inline int64_t pad128(int64_t n) { return (n + 127) / 128 * 128; }

size_t gptq_factor_workspace_size(int64_t n) {
  const int64_t np = pad64(n);
  return 256 + 2 * sizeof(double) * (size_t)np * (size_t)np;
}

constexpr int OB = 4 * DB;    // outer column block of the two-level lazy update

size_t gptq_rows_workspace_size(int64_t rows, int64_t n) {
  const int64_t rp = pad128(rows), np = pad128(n);  // the working copy, in 128 x 128 tiles
  return sizeof(double) * ((size_t)rp * (size_t)np + (size_t)rp * OB);
}

// ------------------------------------------------------------------ fp64 64x64 tiles
// LDS tiles are K-major: T[k * DP + m]. A workgroup of 256 threads (4 waves) owns one
// 64 x 64 output tile; wave w computes the 32 x 32 quarter (w >> 1, w & 1) as 2 x 2
// v_mfma_f64_16x16x4_f64 tiles (A: lane l holds row l & 15 at k = l >> 4; B likewise for
// columns; D: lane l, register r holds row (l >> 4) + 4 r of column l & 15, unlike the
// fp32 16x16x4 form, whose rows are 4 (l >> 4) + r).

// Tile loads in two halves: into registers (issued before the current chunk's products) and
// from there into LDS (after them), so a chunk's global reads overlap the previous chunk's
// products with one LDS buffer. mk: element (m, k) at src[m * ld + k] (k contiguous); kn:
// element (k, n) at src[k * ld + n] (n contiguous); zero outside the limits
struct DPre {
  double2 v[8];
};

__device__ __forceinline__ void dpre_mk(DPre &r, const double *src, int64_t ld, int mlim, int klim) {
  const int t = threadIdx.x;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int idx = s * 256 + t;
    const int m = idx >> 5, k = (idx & 31) * 2;
    r.v[s] = m < mlim && k < klim ? *reinterpret_cast<const double2 *>(src + (int64_t)m * ld + k)
                                  : make_double2(0.0, 0.0);
  }
}

__device__ __forceinline__ void dput_mk(double *T, const DPre &r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int idx = s * 256 + t;
    const int m = idx >> 5, k = (idx & 31) * 2;
    T[k * DP + m] = r.v[s].x;
    T[(k + 1) * DP + m] = r.v[s].y;
  }
}

__device__ __forceinline__ void dpre_kn(DPre &r, const double *src, int64_t ld, int klim, int nlim) {
  const int t = threadIdx.x;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int idx = s * 256 + t;
    const int k = idx >> 5, n = (idx & 31) * 2;
    r.v[s] = k < klim && n < nlim ? *reinterpret_cast<const double2 *>(src + (int64_t)k * ld + n)
                                  : make_double2(0.0, 0.0);
  }
}

__device__ __forceinline__ void dput_kn(double *T, const DPre &r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int idx = s * 256 + t;
    const int k = idx >> 5, n = (idx & 31) * 2;
    T[k * DP + n] = r.v[s].x;
    T[k * DP + n + 1] = r.v[s].y;
  }
}

struct DAcc {
  gq_v4d c[2][2];
};

__device__ __forceinline__ void dacc_zero(DAcc &a) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) a.c[i][j] = (gq_v4d){0.0, 0.0, 0.0, 0.0};
}

__device__ __forceinline__ void dmma(DAcc &acc, const double *LA, const double *LB) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
#pragma unroll 4
  for (int kk = 0; kk < DB / 4; ++kk) {
    const int kr = kk * 4 + (lane >> 4);
    double a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = LA[kr * DP + wr * 32 + i * 16 + (lane & 15)];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = LB[kr * DP + wc * 32 + j * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc.c[i][j], 0, 0, 0);
  }
}

// visit the tile elements a thread owns: f(row, col, value)
template <class F>
__device__ __forceinline__ void dacc_each(const DAcc &acc, F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        f(wr * 32 + i * 16 + (lane >> 4) + 4 * r, wc * 32 + j * 16 + (lane & 15), acc.c[i][j][r]);
}

// C[0:64, 0:nlim] -= A B over K = 64 * NCH (k < klim): A (m, k) at A[m * lda + k]; B (k, n)
// at B[k * ldb + n] when KN, else at B[n * ldb + k]; zero outside the limits. The 64 x 64
// form of the trailing updates, for launches with fewer 128 x 128 tiles than compute units:
// four times the workgroups, each a quarter as long, two per compute unit. The products run
// over k in the same order as in the wide form, so both give the same bits. C's old values
// are read before the products and used after them.
template <bool KN, int NCH>
__device__ __forceinline__ void d64_sub(double *C, int64_t ldc, int nlim, const double *A,
                                        int64_t lda, const double *B, int64_t ldb, int64_t klim,
                                        double *LA, double *LB) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  double cv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 3, j = (q >> 2) & 1, r = q & 3;
    const int row = wr * 32 + i * 16 + (lane >> 4) + 4 * r, col = wc * 32 + j * 16 + (lane & 15);
    cv[q] = col < nlim ? C[(int64_t)row * ldc + col] : 0.0;
  }
  DAcc acc;
  dacc_zero(acc);
  auto kl = [&](int c) {
    const int64_t kb = (int64_t)c * DB;
    return (int)(klim - kb < DB ? (klim - kb > 0 ? klim - kb : 0) : DB);
  };
  DPre ra, rb;
  dpre_mk(ra, A, lda, DB, kl(0));
  if (KN) dpre_kn(rb, B, ldb, kl(0), nlim);
  else dpre_mk(rb, B, ldb, nlim, kl(0));
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c) __syncthreads();
    dput_mk(LA, ra);
    if (KN) dput_kn(LB, rb);
    else dput_mk(LB, rb);
    __syncthreads();
    if (c + 1 < NCH) {
      const int64_t kb = (int64_t)(c + 1) * DB;
      dpre_mk(ra, A + kb, lda, DB, kl(c + 1));
      if (KN) dpre_kn(rb, B + kb * ldb, ldb, kl(c + 1), nlim);
      else dpre_mk(rb, B + kb, ldb, nlim, kl(c + 1));
    }
    dmma(acc, LA, LB);
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 3, j = (q >> 2) & 1, r = q & 3;
    const int row = wr * 32 + i * 16 + (lane >> 4) + 4 * r, col = wc * 32 + j * 16 + (lane & 15);
    if (col < nlim) C[(int64_t)row * ldc + col] = cv[q] - acc.c[i][j][r];
  }
}

static int gptq_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// Wide tiles: a workgroup of 16 waves owns a 128 x 128 output tile (each wave 32 x 32, as
// 2 x 2 MFMA tiles), K in chunks of 32 staged through two 66 KiB LDS buffers (the next
// chunk's global loads are in flight while the current one is multiplied, one barrier per
// chunk). Four times the work of a 64 x 64 tile per byte loaded; four waves per SIMD hide the
// loads and barriers (eight waves of 32 x 64 were 5% slower, four of 64 x 64 another 15%).
constexpr int T2 = 128;     // wide tile edge
constexpr int KC = 32;      // K chunk
constexpr int P2 = T2 + 1;  // LDS pitch (doubles)
constexpr int W2T = 1024;  // threads of a wide-tile workgroup

struct DAcc2 {
  gq_v4d c[2][2];
};

struct DStage {
  double2 a[2], b[2];
};

__device__ __forceinline__ void d2_zero(DAcc2 &a) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) a.c[i][j] = (gq_v4d){0.0, 0.0, 0.0, 0.0};
}

// A chunk: element (m, k) at A[m * lda + k], m < 128, k < 32; zero outside m < mlim, k < klim
__device__ __forceinline__ void d2_load_a(DStage &st, const double *A, int64_t lda, int mlim, int klim) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int idx = s * W2T + threadIdx.x, m = idx >> 4, k = (idx & 15) * 2;
    st.a[s] = (m < mlim && k < klim) ? *reinterpret_cast<const double2 *>(A + (int64_t)m * lda + k)
                                     : make_double2(0.0, 0.0);
  }
}

__device__ __forceinline__ void d2_store_a(const DStage &st, double *LA) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int idx = s * W2T + threadIdx.x, m = idx >> 4, k = (idx & 15) * 2;
    LA[k * P2 + m] = st.a[s].x;
    LA[(k + 1) * P2 + m] = st.a[s].y;
  }
}

// B chunk, element (k, n): at B[k * ldb + n] when KN, else at B[n * ldb + k]
template <bool KN>
__device__ __forceinline__ void d2_load_b(DStage &st, const double *B, int64_t ldb, int klim, int nlim) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int idx = s * W2T + threadIdx.x;
    if (KN) {
      const int k = idx >> 6, n = (idx & 63) * 2;
      st.b[s] = (k < klim && n < nlim) ? *reinterpret_cast<const double2 *>(B + (int64_t)k * ldb + n)
                                       : make_double2(0.0, 0.0);
    } else {
      const int n = idx >> 4, k = (idx & 15) * 2;
      st.b[s] = (n < nlim && k < klim) ? *reinterpret_cast<const double2 *>(B + (int64_t)n * ldb + k)
                                       : make_double2(0.0, 0.0);
    }
  }
}

template <bool KN>
__device__ __forceinline__ void d2_store_b(const DStage &st, double *LB) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int idx = s * W2T + threadIdx.x;
    if (KN) {
      const int k = idx >> 6, n = (idx & 63) * 2;
      LB[k * P2 + n] = st.b[s].x;
      LB[k * P2 + n + 1] = st.b[s].y;
    } else {
      const int n = idx >> 4, k = (idx & 15) * 2;
      LB[k * P2 + n] = st.b[s].x;
      LB[(k + 1) * P2 + n] = st.b[s].y;
    }
  }
}

__device__ __forceinline__ void d2_mma(DAcc2 &acc, const double *LA, const double *LB) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 2, wc = wave & 3;  // 32 x 32 per wave
  const double *pa = LA + (lane >> 4) * P2 + wr * 32 + (lane & 15);
  const double *pb = LB + (lane >> 4) * P2 + wc * 32 + (lane & 15);
  // the operands of step kk + 1 are read while step kk's four products run
  double a[2][2], b[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[0][i] = pa[i * 16];
    b[0][i] = pb[i * 16];
  }
#pragma unroll
  for (int kk = 0; kk < KC / 4; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < KC / 4) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[cur ^ 1][i] = pa[(kk + 1) * 4 * P2 + i * 16];
        b[cur ^ 1][i] = pb[(kk + 1) * 4 * P2 + i * 16];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[cur][i], b[cur][j], acc.c[i][j], 0, 0, 0);
  }
}

// C[0:mlim, 0:nlim] -= A[:, 0:K] B[0:K, :] with K = NCH * KC (k < klim; A as in d2_load_a,
// B as in d2_load_b), the tile of C in global memory. The tile's old values are read into registers
// a share per chunk, beside that chunk's products, rather than after the last of them: with
// one workgroup per compute unit, reading and writing the 128 KiB tile at the end left the
// matrix cores idle for a third of a short-K update.
template <bool KN, int NCH>
__device__ __forceinline__ void d2_gemm_sub(double *C, int64_t ldc, int mlim, int nlim,
                                            const double *A, int64_t lda, const double *B,
                                            int64_t ldb, int64_t klim, double *L) {
  static_assert(16 % NCH == 0, "the tile's 16 values per thread split evenly over the chunks");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 2, wc = wave & 3;
  auto kl = [&](int64_t kb) { return (int)(klim - kb < KC ? (klim - kb > 0 ? klim - kb : 0) : KC); };
  DAcc2 acc;
  d2_zero(acc);
  DStage st;
  d2_load_a(st, A, lda, mlim, kl(0));
  d2_load_b<KN>(st, B, ldb, kl(0), nlim);
  d2_store_a(st, L);
  d2_store_b<KN>(st, L + KC * P2);
  __syncthreads();
  double cv[16];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    double *cur = L + (c & 1) * 2 * KC * P2, *nxt = L + ((c + 1) & 1) * 2 * KC * P2;
    if (c + 1 < NCH) {
      const int64_t kb = (int64_t)(c + 1) * KC;
      d2_load_a(st, A + kb, lda, mlim, kl(kb));
      d2_load_b<KN>(st, B + (KN ? kb * ldb : kb), ldb, kl(kb), nlim);
    }
#pragma unroll
    for (int q = c * (16 / NCH); q < (c + 1) * (16 / NCH); ++q) {
      const int i = q >> 3, j = (q >> 2) & 1, r = q & 3;
      const int row = wr * 32 + i * 16 + (lane >> 4) + 4 * r, col = wc * 32 + j * 16 + (lane & 15);
      cv[q] = row < mlim && col < nlim ? C[(int64_t)row * ldc + col] : 0.0;
    }
    d2_mma(acc, cur, cur + KC * P2);
    if (c + 1 < NCH) {
      d2_store_a(st, nxt);
      d2_store_b<KN>(st, nxt + KC * P2);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 3, j = (q >> 2) & 1, r = q & 3;
    const int row = wr * 32 + i * 16 + (lane >> 4) + 4 * r, col = wc * 32 + j * 16 + (lane & 15);
    if (row < mlim && col < nlim) C[(int64_t)row * ldc + col] = cv[q] - acc.c[i][j][r];
  }
}

// ------------------------------------------------------------------ factor
// hdr[0] = lambda, hdr[1] = 1 if diag(H) sums to zero (then H + lambda I := I).
// lambda takes the diagonal's sum in index order. When every partial sum of it, in any
// order, is exact in double, a tree sum has the same bits and replaces the 4096-step chain
// of dependent adds: each diagonal entry is an integer multiple of 2^qlo (its lowest set
// bit) with magnitude below 2^(qhi + 1), so every partial sum is a multiple of 2^qlo
// (the smallest qlo) below n 2^(qhi + 1) (the largest qhi); if that is at most 2^53 units
// of 2^qlo, all of them are exact. Otherwise, or with a non-finite entry, the sum runs in
// index order.
__device__ __forceinline__ double block_sum256(double v, double *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ void __launch_bounds__(256)
    k_gptq_lambda(const float *__restrict__ H, int64_t n, double damp, double *__restrict__ hdr,
                  int32_t *__restrict__ status) {
  __shared__ double dg[4096];
  __shared__ int qred[3][4];
  __shared__ double red[4];
  const int t = threadIdx.x;
  int qlo = 1 << 20, qhi = -(1 << 20), bad = 0;
  double part = 0.0;  // this thread's entries, summed in any order (used only when exact)
  for (int64_t i = t; i < n; i += 256) {
    const float h = H[i * n + i];
    const unsigned u = __float_as_uint(h) & 0x7FFFFFFFu;
    if (u >= 0x7F800000u) {
      bad = 1;
    } else if (u != 0u) {
      const int E = (int)(u >> 23);
      const unsigned m = E ? ((u & 0x7FFFFFu) | 0x800000u) : u;  // |h| = m 2^(max(E,1) - 150)
      const int e0 = (E ? E : 1) - 150;
      qlo = min(qlo, e0 + __builtin_ctz(m));
      qhi = max(qhi, e0 + 31 - __builtin_clz(m));
    }
    part += (double)h;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    qlo = min(qlo, __shfl_xor(qlo, off, 64));
    qhi = max(qhi, __shfl_xor(qhi, off, 64));
    bad |= __shfl_xor(bad, off, 64);
  }
  if ((t & 63) == 0) {
    qred[0][t >> 6] = qlo;
    qred[1][t >> 6] = qhi;
    qred[2][t >> 6] = bad;
  }
  __syncthreads();
  qlo = min(min(qred[0][0], qred[0][1]), min(qred[0][2], qred[0][3]));
  qhi = max(max(qred[1][0], qred[1][1]), max(qred[1][2], qred[1][3]));
  bad = qred[2][0] | qred[2][1] | qred[2][2] | qred[2][3];
  const int lg = n > 1 ? 64 - __builtin_clzll((unsigned long long)(n - 1)) : 0;  // ceil(log2 n)
  const bool any_order = !bad && (qhi < qlo || lg + qhi + 1 - qlo <= 53);
  double tr = 0.0;
  if (any_order) {
    tr = block_sum256(part, red);
  } else {
    for (int64_t base = 0; base < n; base += 4096) {
      const int64_t m = n - base < 4096 ? n - base : 4096;
      float h[16];  // this thread's diagonal entries of the chunk, all reads in flight at once
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int64_t i = s * 256 + t;
        h[s] = i < m ? H[(base + i) * n + base + i] : 0.0f;
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) dg[s * 256 + t] = (double)h[s];
      __syncthreads();
      if (t == 0) {
#pragma unroll 16
        for (int64_t i = 0; i < m; ++i) tr += dg[i];  // index order
      }
      __syncthreads();
    }
  }
  if (t == 0) {
    hdr[0] = damp * (tr / (double)n);
    hdr[1] = tr == 0.0 ? 1.0 : 0.0;
    *status = 0;
  }
}

// A (np x np) = J (H + lambda I) J, lower triangle from H's lower triangle, identity padding,
// zero above the diagonal; X zero in its blocks above the diagonal (the inverse reads them as
// zero; the factorisation and the inverse write every other block of X before reading it).
// One 64 x 64 tile per workgroup: A[i][j] = H[n-1-j][n-1-i] reverses and transposes, so the
// tile of H is read along its rows into LDS and written along A's rows from there.
__global__ void __launch_bounds__(256)
    k_gptq_load_h(const float *__restrict__ H, int64_t n, int64_t np,
                  const double *__restrict__ hdr, double *__restrict__ A, double *__restrict__ X) {
  __shared__ float T[DB][DB + 1];  // T[k][m] = H[n-1-(j0+k)][n-1-(i0+m)]
  const int64_t nbt = np / DB;
  const int64_t ti = blockIdx.x / nbt, tj = blockIdx.x % nbt;
  const int64_t i0 = ti * DB, j0 = tj * DB;
  const int t = threadIdx.x;
  if (tj > ti) {  // above the diagonal: zero in A and in X
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int e = s * 256 + t, r = e >> 5, c = (e & 31) * 2;
      *reinterpret_cast<double2 *>(A + (i0 + r) * np + j0 + c) = make_double2(0.0, 0.0);
      *reinterpret_cast<double2 *>(X + (i0 + r) * np + j0 + c) = make_double2(0.0, 0.0);
    }
    return;
  }
  const double lam = hdr[0];
  const bool ident = hdr[1] != 0.0;
  {
    // thread t reads H row n-1-(j0+k) at columns n-1-(i0+63) + (t & 63) upward (m = 63 - (t & 63))
    float h[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int k = s * 4 + (t >> 6), m = DB - 1 - (t & 63);
      const int64_t b = n - 1 - (j0 + k), a = n - 1 - (i0 + m);
      h[s] = (j0 + k < n && i0 + m < n) ? H[b * n + a] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) T[s * 4 + (t >> 6)][DB - 1 - (t & 63)] = h[s];
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int m = s * 4 + (t >> 6), k = t & 63;  // A row i0 + m, column j0 + k
    const int64_t i = i0 + m, j = j0 + k;
    double v = 0.0;
    if (j <= i) {
      if (i >= n) v = i == j ? 1.0 : 0.0;
      else v = ident ? (i == j ? 1.0 : 0.0) : (double)T[k][m] + (i == j ? lam : 0.0);
    }
    A[i * np + j] = v;
  }
}

// value of lane `src` of this lane's quad; src is a compile-time constant at every call
__device__ __forceinline__ double quad_bcast(double x, int src) {
  int lo = __double2loint(x), hi = __double2hiint(x);
  switch (src) {
    case 0:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x00, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x00, 0xF, 0xF, false);
      break;
    case 1:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x55, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x55, 0xF, 0xF, false);
      break;
    case 2:
      lo = __builtin_amdgcn_mov_dpp(lo, 0xAA, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0xAA, 0xF, 0xF, false);
      break;
    default:
      lo = __builtin_amdgcn_mov_dpp(lo, 0xFF, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0xFF, 0xF, 0xF, false);
      break;
  }
  return __hiloint2double(hi, lo);
}

// Waits (s_sleep between reads) until the LDS word at f is above j. The read and its wait
// are in one asm block, and the loop stays out of the compiler's view, so the unrolled column
// loop around it remains one straight-line block (a loop inside it spilled to scratch).
__device__ __forceinline__ void lds_wait_above(int *f, int j) {
  int seen, tmp;
  const unsigned addr = (unsigned)(uintptr_t)f;
  asm volatile(
      "1:\n\t"
      "ds_read_b32 %1, %2\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_readfirstlane_b32 %0, %1\n\t"
      "s_cmp_gt_i32 %0, %3\n\t"
      "s_cbranch_scc1 2f\n\t"
      "s_sleep 1\n\t"
      "s_branch 1b\n\t"
      "2:"
      : "=&s"(seen), "=&v"(tmp)
      : "v"(addr), "s"(j)
      : "scc", "memory");
}

// Step k of the blocked Cholesky factorisation. Workgroups of five waves. Wave 1 of every
// workgroup factors diagonal block k (lane i holds row i in registers) in four panels of 16
// columns: inside a panel column by column (pivot by readlane, its 1 / sqrt one column ahead,
// each scaled column to LDS, updates only within the panel), then the panel's update of the
// columns right of it, L_p L_p^T, on the fp64 matrix cores (16 x 16 tiles, K = 16, the same
// fragments serving as A and B), back into the rows through LDS. It publishes column j by
// setting an LDS counter to j + 1 once the column and 1 / L_jj are written. Workgroup 0
// stores L_kk; in workgroup b >= 1 the other four waves meanwhile solve the 64 rows of panel
// block k + b, x L_kk^T = a, by forward substitution a column pair behind the factorisation:
// four lanes per row, 16 columns each, x_j shared in the quad by DPP. The waits end: the
// factorising wave runs all 64 columns unconditionally (a bad pivot only sets the status)
// and waits only on itself. LDS operations of one wave are performed in order, so a panel
// wave that reads the counter above j then reads column j and 1 / L_jj as written. The
// factorisation is on wave 1 because a fifth wave shares a SIMD with wave 0 (here a panel
// wave); on wave 0 the step took 20.4 instead of 18.9 us.
// L_kk goes to the same place in X, not back into A: with more workgroups than fit on the
// device at once, a late workgroup still reads A_kk itself (the triangular inverse reads
// the diagonal blocks from X).
constexpr int CHOL_THREADS = 320;
constexpr int CHOL_DIAG_WAVE = 1;
__global__ void __launch_bounds__(CHOL_THREADS)
    k_chol_step(double *__restrict__ A, double *__restrict__ X, int64_t np, int64_t k,
                int32_t *__restrict__ status) {
  __shared__ __attribute__((aligned(16))) double Lt[DB * DB];  // Lt[j * 64 + m] = L_kk[m][j]
  __shared__ __attribute__((aligned(16))) double Ub[DB * DB];  // a panel's update, [row][col]
  __shared__ double rinv[DB];
  __shared__ int ready;  // columns published
  const int t = threadIdx.x;
  if (t == 0) ready = 0;
  __syncthreads();
  if ((t >> 6) == CHOL_DIAG_WAVE) {
    const int i = t & 63;
    const double *blk = A + k * DB * np + k * DB;
    double d[DB];
#pragma unroll
    for (int j = 0; j < DB; j += 2) {
      const double2 v = *reinterpret_cast<const double2 *>(blk + (int64_t)i * np + j);
      d[j] = j <= i ? v.x : 0.0;
      d[j + 1] = j + 1 <= i ? v.y : 0.0;
    }
    // 1 / sqrt(piv): the hardware estimate and two Newton steps (about 1 ulp), off the
    // longer sqrt and divide sequences on this step's critical path
    auto rsqrt_nr = [](double piv) {
      double rl = __builtin_amdgcn_rsq(piv);
      rl = rl * __builtin_fma(-0.5 * piv * rl, rl, 1.5);
      rl = rl * __builtin_fma(-0.5 * piv * rl, rl, 1.5);
      return rl;
    };
    bool bad = false;
    double piv = 0.0, rl = 0.0;
    auto pivot_of = [&](int j) {  // column j's pivot (final in lane j's d[j]) and its 1 / sqrt
      const int plo = __builtin_amdgcn_readlane(__double2loint(d[j]), j);
      const int phi = __builtin_amdgcn_readlane(__double2hiint(d[j]), j);
      piv = __hiloint2double(phi, plo);
      bad |= !(piv > 0.0);
      rl = rsqrt_nr(piv);
    };
#pragma unroll
    for (int P = 0; P < 4; ++P) {
      const int c0 = 16 * P;
      pivot_of(c0);
#pragma unroll
      for (int j = c0; j < c0 + 16; ++j) {
        const double ljj = piv * rl;
        d[j] = i == j ? ljj : d[j] * rl;      // right of the diagonal, d holds unused values
        Lt[j * DB + i] = i >= j ? d[j] : 0.0;  // column j of L_kk (zero above the diagonal)
        if (i == j) {  // the pivot's lane: 1 / L_jj, then column j is published
          rinv[j] = rl;
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __hip_atomic_store(&ready, j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (j + 1 < c0 + 16) {
          // the next pivot first: L[j+1][j] read from lane j + 1 is column j + 1's only
          // missing term, so its pivot and 1 / sqrt overlap the LDS round trip and the rest
          // of the panel's update
          const int slo = __builtin_amdgcn_readlane(__double2loint(d[j]), j + 1);
          const int shi = __builtin_amdgcn_readlane(__double2hiint(d[j]), j + 1);
          d[j + 1] = fma(-d[j], __hiloint2double(shi, slo), d[j + 1]);
          const double dj = d[j];
          pivot_of(j + 1);
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          const double *col = Lt + j * DB;
#pragma unroll
          for (int l = j + 2; l < c0 + 16; ++l) d[l] = fma(-dj, col[l], d[l]);
        }
      }
      if (P < 3) {
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // fragment (tile t, step s): lane l holds L_kk[16 t + (l & 15)][c0 + 4 s + (l >> 4)]
        auto frag = [&](int tt, int s) { return Lt[(c0 + 4 * s + (i >> 4)) * DB + 16 * tt + (i & 15)]; };
#pragma unroll
        for (int tm = P + 1; tm < 4; ++tm)
#pragma unroll
          for (int tn = P + 1; tn <= tm; ++tn) {
            double fm[4], fn[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              fm[s] = frag(tm, s);
              fn[s] = tn == tm ? fm[s] : frag(tn, s);
            }
            gq_v4d acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(fm[s], fn[s], acc, 0, 0, 0);
            // D: lane l, register r holds row (l >> 4) + 4 r, column l & 15 of the tile
#pragma unroll
            for (int r = 0; r < 4; ++r) Ub[(16 * tm + (i >> 4) + 4 * r) * DB + 16 * tn + (i & 15)] = acc[r];
          }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // only l <= i matters; the rest of the row holds unused values
#pragma unroll
        for (int l = c0 + 16; l < DB; ++l) d[l] -= Ub[i * DB + l];
      }
    }
    if (blockIdx.x == 0) {
      if (bad && i == 0) atomicCAS(status, 0, (int32_t)(1 + k));
      double *lk = X + k * DB * np + k * DB;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int j = 0; j < DB; j += 2)  // from LDS (zero above the diagonal), so d dies early
        *reinterpret_cast<double2 *>(lk + (int64_t)i * np + j) =
            make_double2(Lt[j * DB + i], Lt[(j + 1) * DB + i]);
    }
    return;
  }
  if (blockIdx.x == 0) return;
  // panel: lane p of row r owns columns 16 p .. 16 p + 15 (read now, so that the read
  // overlaps the first columns of the factorisation)
  const int tp = t >= 64 * (CHOL_DIAG_WAVE + 1) ? t - 64 : t;
  const int p = tp & 3, r = tp >> 2;
  double *ar = A + ((k + blockIdx.x) * DB + r) * np + k * DB + 16 * p;
  double a[16];
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const double2 v = *reinterpret_cast<const double2 *>(ar + j);
    a[j] = v.x;
    a[j + 1] = v.y;
  }
  // columns in pairs: one counter read for both, and the second column's reads can be
  // issued during the first one's update
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    if ((j & 1) == 0) lds_wait_above(&ready, j + 1);
    const int pj = j >> 4, jj = j & 15;
    const double x = quad_bcast(a[jj] * rinv[j], pj);
    const double *lc = Lt + j * DB + 16 * p;  // L_kk[16 p + i][j], zero for 16 p + i < j
    // from column 48 on, only the last lane of a quad has columns right of j
#pragma unroll
    for (int i = (j < 48 ? 0 : jj + 1); i < 16; ++i) a[i] = fma(-x, lc[i], a[i]);
    if (p == pj) a[jj] = x;
  }
#pragma unroll
  for (int j = 0; j < 16; j += 2) *reinterpret_cast<double2 *>(ar + j) = make_double2(a[j], a[j + 1]);
}

// column block k + 1 only: A[bi][k+1] -= L[bi][k] L[k+1][k]^T for bi >= k + 1 (what step
// k + 1 needs before the paired trailing update)
__global__ void __launch_bounds__(256)
    k_chol_colupd(double *__restrict__ A, int64_t np, int64_t k) {
  __shared__ double LA[DB * DP], LB[DB * DP];
  const int64_t bi = k + 1 + blockIdx.x, bj = k + 1;
  d64_sub<false, 1>(A + bi * DB * np + bj * DB, np, DB, A + bi * DB * np + k * DB, np,
                    A + bj * DB * np + k * DB, np, DB, LA, LB);
}

// inverses of the diagonal blocks, in place in X (where the steps left L_bb): column c of
// L_bb^-1 by forward substitution, after the whole block is in LDS
__global__ void __launch_bounds__(64)
    k_trtri_diag(double *__restrict__ X, int64_t np) {
  __shared__ double Lb[DB * DP];
  const int64_t b = blockIdx.x;
  const int c = threadIdx.x;
  const double *src = X + b * DB * np + b * DB;
  {
    double l[DB];  // column c of the block: all 64 reads in flight before the first wait
#pragma unroll
    for (int i = 0; i < DB; ++i) l[i] = src[i * np + c];
#pragma unroll
    for (int i = 0; i < DB; ++i) Lb[i * DP + c] = l[i];
  }
  __syncthreads();
  double y[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    double s = 0.0;
#pragma unroll
    for (int m = 0; m < i; ++m) s = fma(Lb[i * DP + m], y[m], s);  // y[m] = 0 for m < c
    y[i] = i < c ? 0.0 : (i == c ? 1.0 / Lb[i * DP + i] : -s / Lb[i * DP + i]);
  }
  double *dst = X + b * DB * np + b * DB;
#pragma unroll
  for (int i = 0; i < DB; ++i) dst[i * np + c] = y[i];
}

// One level of the recursive inverse. Groups of 2s rows: A-range [a0, a0 + s), C-range
// [c0, c0 + sc). phase 0: T = L[C][A] X[A][A], stored transposed in the Cholesky factor's
// upper triangle (A[A rows][C cols], which nothing reads as L); phase 1: X[C][A] =
// -X[C][C] T. X's own upper triangle stays zero.
__global__ void __launch_bounds__(256)
    k_trtri_level(double *__restrict__ A, double *__restrict__ X, int64_t np, int64_t s,
                  int64_t g, int phase) {
  __shared__ double LA[DB * DP], LB[DB * DP];
  // workgroups in order of decreasing work across all groups (phase 0's tiles take s - 64 jb
  // of K, phase 1's 64 (ib + 1)), so the longest start first and the short ones fill in
  const int64_t nbs = s / DB, per = nbs * g;
  const int64_t q = blockIdx.x / per, rem = blockIdx.x % per, rr = rem % nbs;
  const int64_t a0 = (rem / nbs) * 2 * s, c0 = a0 + s;
  const int64_t sc = np - c0 < s ? np - c0 : s;
  const int64_t jb = phase == 0 ? q : rr, ib = phase == 0 ? rr : nbs - 1 - q;  // C row, A col
  if (ib * DB >= sc) return;
  const int64_t r0 = c0 + ib * DB, q0 = a0 + jb * DB;  // global row / column of the block
  DAcc acc;
  dacc_zero(acc);
  if (phase == 0) {
    // sum over A-range blocks kb >= jb: L[r0][kb] X[kb][q0]
    DPre ra, rb;
    dpre_mk(ra, A + r0 * np + a0 + jb * DB, np, DB, DB);
    dpre_kn(rb, X + (a0 + jb * DB) * np + q0, np, DB, DB);
    for (int64_t kb = jb; kb < nbs; ++kb) {
      __syncthreads();
      dput_mk(LA, ra);
      dput_kn(LB, rb);
      __syncthreads();
      if (kb + 1 < nbs) {
        const int64_t k1 = a0 + (kb + 1) * DB;
        dpre_mk(ra, A + r0 * np + k1, np, DB, DB);
        dpre_kn(rb, X + k1 * np + q0, np, DB, DB);
      }
      dmma(acc, LA, LB);
    }
    dacc_each(acc, [&](int r, int c, double v) { A[(q0 + c) * np + r0 + r] = v; });
  } else {
    // sum over C-range blocks kb <= ib: X[r0][kb] T[kb][q0], T[kb][q0] stored at A[q0][kb]
    DPre ra, rb;
    dpre_mk(ra, X + r0 * np + c0, np, DB, DB);
    dpre_mk(rb, A + q0 * np + c0, np, DB, DB);
    for (int64_t kb = 0; kb <= ib; ++kb) {
      __syncthreads();
      dput_mk(LA, ra);
      dput_mk(LB, rb);
      __syncthreads();
      if (kb + 1 <= ib) {
        const int64_t k1 = c0 + (kb + 1) * DB;
        dpre_mk(ra, X + r0 * np + k1, np, DB, DB);
        dpre_mk(rb, A + q0 * np + k1, np, DB, DB);
      }
      dmma(acc, LA, LB);
    }
    dacc_each(acc, [&](int r, int c, double v) { X[(r0 + r) * np + q0 + c] = -v; });
  }
}

// U[i][j] = X[n-1-i][n-1-j] for i <= j, zero below the diagonal. Thread x of a row writes
// columns 4x .. 4x + 3 (n is a multiple of 16); rows by grid-stride over y, no index division.
__global__ void __launch_bounds__(256)
    k_gptq_store_u(const double *__restrict__ X, int64_t n, int64_t np, double *__restrict__ U) {
  const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (j >= n) return;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const double *src = X + (n - 1 - i) * np + (n - 1 - j);  // column n-1-j, then leftwards
    double u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = i <= j + q ? src[-q] : 0.0;
    *reinterpret_cast<double2 *>(U + i * n + j) = make_double2(u[0], u[1]);
    *reinterpret_cast<double2 *>(U + i * n + j + 2) = make_double2(u[2], u[3]);
  }
}

// trailing update after a pair of steps: for the lower-triangular 128 x 128 tiles of the
// matrix from row / column c on, A[I][J] -= L[I][k0 .. k0 + 128) L[J][k0 .. k0 + 128)^T
__global__ void __launch_bounds__(W2T)
    k_chol_update2(double *__restrict__ A, int64_t np, int64_t c, int64_t k0) {
  __shared__ __attribute__((aligned(16))) double L2[4 * KC * P2];  // two (A, B) chunk buffers
  int64_t e = blockIdx.x, ti = 0;
  while (e > ti) {  // lower-triangular enumeration: tile row ti holds ti + 1 tiles
    e -= ti + 1;
    ++ti;
  }
  const int64_t I = c + ti * T2, J = c + e * T2;
  const int mlim = (int)(np - I < T2 ? np - I : T2), nlim = (int)(np - J < T2 ? np - J : T2);
  d2_gemm_sub<false, 2 * DB / KC>(A + I * np + J, np, mlim, nlim, A + I * np + k0, np,
                                  A + J * np + k0, np, 2 * DB, L2);
}

// the same update with 64 x 64 tiles (the lower-triangular ones from c on)
__global__ void __launch_bounds__(256)
    k_chol_update64(double *__restrict__ A, int64_t np, int64_t c, int64_t k0) {
  __shared__ double LA[DB * DP], LB[DB * DP];
  int64_t e = blockIdx.x, ti = 0;
  while (e > ti) {
    e -= ti + 1;
    ++ti;
  }
  const int64_t I = c + ti * DB, J = c + e * DB;
  d64_sub<false, 2>(A + I * np + J, np, DB, A + I * np + k0, np, A + J * np + k0, np, 2 * DB,
                    LA, LB);
}

int launch_gptq_factor(const float *H, int64_t n, double damp, double *U, int32_t *status,
                       void *workspace, hipStream_t st) {
  const int64_t np = pad64(n), nb = np / DB;
  double *hdr = static_cast<double *>(workspace);
  int32_t *stat = status ? status : reinterpret_cast<int32_t *>(hdr + 2);
  double *A = reinterpret_cast<double *>(static_cast<char *>(workspace) + 256);
  double *X = A + np * np;
  const int64_t cus = gptq_cus();
  hipLaunchKernelGGL(k_gptq_lambda, dim3(1), dim3(256), 0, st, H, n, damp, hdr, stat);
  hipLaunchKernelGGL(k_gptq_load_h, dim3((unsigned)(nb * nb)), dim3(256), 0, st, H, n, np, hdr, A, X);
  // steps in pairs: step k, column block k + 1, step k + 1, then one trailing update with
  // K = 128 over the 128-aligned rest (128 x 128 tiles); an odd last step stands alone
  for (int64_t k = 0; k < nb; k += 2) {
    const int64_t T = nb - k - 1;
    hipLaunchKernelGGL(k_chol_step, dim3((unsigned)(T + 1)), dim3(CHOL_THREADS), 0, st, A, X, np, k,
                       stat);
    if (T == 0) break;
    hipLaunchKernelGGL(k_chol_colupd, dim3((unsigned)T), dim3(256), 0, st, A, np, k);
    hipLaunchKernelGGL(k_chol_step, dim3((unsigned)T), dim3(CHOL_THREADS), 0, st, A, X, np, k + 1,
                       stat);
    const int64_t c = (k + 2) * DB;
    if (c >= np) break;
    const int64_t t2 = (np - c + T2 - 1) / T2;
    if (t2 * (t2 + 1) / 2 >= cus) {
      hipLaunchKernelGGL(k_chol_update2, dim3((unsigned)(t2 * (t2 + 1) / 2)), dim3(W2T), 0, st, A,
                         np, c, k * DB);
    } else {  // too few wide tiles to fill the device
      const int64_t t1 = (np - c) / DB;
      hipLaunchKernelGGL(k_chol_update64, dim3((unsigned)(t1 * (t1 + 1) / 2)), dim3(256), 0, st, A,
                         np, c, k * DB);
    }
  }
  hipLaunchKernelGGL(k_trtri_diag, dim3((unsigned)nb), dim3(64), 0, st, X, np);
  for (int64_t s = DB; s < np; s *= 2) {
    const int64_t groups = (np + 2 * s - 1) / (2 * s);
    int64_t g = groups;
    if (groups * 2 * s - s >= np) --g;  // the last group has no C range
    if (g <= 0) continue;
    const int64_t nbs = s / DB;
    const dim3 grid((unsigned)(nbs * nbs * g));  // (np / 64)^2 / 2 at most
    hipLaunchKernelGGL(k_trtri_level, grid, dim3(256), 0, st, A, X, np, s, g, 0);
    hipLaunchKernelGGL(k_trtri_level, grid, dim3(256), 0, st, A, X, np, s, g, 1);
  }
  hipLaunchKernelGGL(k_gptq_store_u, dim3((unsigned)((n / 4 + 255) / 256), (unsigned)(n < 65535 ? n : 65535)),
                     dim3(256), 0, st, X, n, np, U);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ------------------------------------------------------------------ rows
// the working copy V [rp][np] (fp64) of W [rows][n], zero in the padding. Thread x of a row
// fills columns 4x .. 4x + 3 (n and np are multiples of 16); rows by grid-stride over y.
template <int DT>
__global__ void __launch_bounds__(256)
    k_gptq_init(const void *__restrict__ w, int64_t rows, int64_t n, int64_t rp, int64_t np,
                double *__restrict__ V) {
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= np) return;
  for (int64_t r = blockIdx.y; r < rp; r += gridDim.y) {
    double v[4] = {0.0, 0.0, 0.0, 0.0};
    if (r < rows && c < n) {
      if (DT == NVFP4_DTYPE_BF16) {
        const uint2 h = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(w) + r * n + c);
        v[0] = (double)__uint_as_float(h.x << 16);
        v[1] = (double)__uint_as_float(h.x & 0xFFFF0000u);
        v[2] = (double)__uint_as_float(h.y << 16);
        v[3] = (double)__uint_as_float(h.y & 0xFFFF0000u);
      } else {
        const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(w) + r * n + c);
        v[0] = (double)f.x;
        v[1] = (double)f.y;
        v[2] = (double)f.z;
        v[3] = (double)f.w;
      }
    }
    *reinterpret_cast<double2 *>(V + r * np + c) = make_double2(v[0], v[1]);
    *reinterpret_cast<double2 *>(V + r * np + c + 2) = make_double2(v[2], v[3]);
  }
}

// value of lane `src` of this lane's row of 16 (DPP row_newbcast); src is a compile-time
// constant at every call site (the column loop is unrolled), so the switch folds away
__device__ __forceinline__ double row_bcast16(double x, int src) {
  int lo = __double2loint(x), hi = __double2hiint(x);
#define GQ_BCAST(S)                                              \
  case S:                                                        \
    lo = __builtin_amdgcn_mov_dpp(lo, 0x150 + S, 0xF, 0xF, false); \
    hi = __builtin_amdgcn_mov_dpp(hi, 0x150 + S, 0xF, 0xF, false); \
    break;
  switch (src) {
    GQ_BCAST(0) GQ_BCAST(1) GQ_BCAST(2) GQ_BCAST(3) GQ_BCAST(4) GQ_BCAST(5) GQ_BCAST(6)
    GQ_BCAST(7) GQ_BCAST(8) GQ_BCAST(9) GQ_BCAST(10) GQ_BCAST(11) GQ_BCAST(12) GQ_BCAST(13)
    GQ_BCAST(14) default: GQ_BCAST(15)
  }
#undef GQ_BCAST
  return __hiloint2double(hi, lo);
}

// Column block b (columns 64 b .. 64 b + 63). Sixteen lanes share a row (four rows per
// wave): lane p holds columns 4 p .. 4 p + 3 of the block. Codes go to `codes`, errors e to
// E[r][64 (b % 4) + 4 p + i] (E: [rows][OB]).
__global__ void __launch_bounds__(256)
    k_gptq_block(double *__restrict__ V, int64_t np, int64_t rows, int64_t n,
                 const float *__restrict__ Sp, const uint8_t *__restrict__ scales,
                 const double *__restrict__ U, int64_t b, double *__restrict__ E,
                 uint8_t *__restrict__ codes) {
  __shared__ __attribute__((aligned(16))) double LU[DB * DB];  // U's block, zero below diagonal
  __shared__ double RU[DB];                                    // 1 / U_jj
  const int t = threadIdx.x;
  const int64_t c0 = b * DB;
  // every global read is issued before the first wait: one workgroup per compute unit has
  // no other work to hide their latency behind
  const int p = t & 15;
  const int64_t r = (int64_t)blockIdx.x * 16 + (t >> 4);
  const int64_t cb = c0 + 4 * p;  // first of this lane's 4 columns
  const bool live = r < rows && cb < n;
  const double2 v01 = *reinterpret_cast<const double2 *>(V + r * np + cb);
  const double2 v23 = *reinterpret_cast<const double2 *>(V + r * np + cb + 2);
  const int byte = live ? given_byte(scales[r * (n / 16) + cb / 16]) : 0;
  // the rest of this 256-column outer block (at most 192 columns, 12 tiles of 16), updated
  // after the column loop: wave w takes tiles w, w + 4, w + 8, whose rows of U and values of
  // V are read here (n is a multiple of 16; when any tile follows, all 64 rows of U's block
  // are below n)
  int64_t c_end = (b / 4 + 1) * OB;
  if (c_end > n) c_end = n;
  const int ntiles = c_end > c0 + DB ? (int)((c_end - c0 - DB) / 16) : 0;
  const int lane = t & 63, w = t >> 6, lr = lane >> 4, lc = lane & 15;
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  double ub[3][16], vv[3][4];
#pragma unroll
  for (int qi = 0; qi < 3; ++qi) {
    const int q = w + 4 * qi;
    const int64_t cq = c0 + DB + 16 * q + lc;
#pragma unroll
    for (int s = 0; s < 16; ++s) ub[qi][s] = q < ntiles ? U[(c0 + 4 * s + lr) * n + cq] : 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[qi][i] = q < ntiles ? V[(r0 + lr + 4 * i) * np + cq] : 0.0;
  }
  // U's block: thread t stages rows t / 16 + 16 s, columns 4 (t % 16) .. + 3 (past n: the
  // identity, for the padding columns)
  {
    const int k4 = 4 * (t & 15);
    double2 u[4][2];
    if (c0 + DB <= n) {  // the whole block lies inside U
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const double *src = U + (c0 + (t >> 4) + 16 * s) * n + c0 + k4;
        u[s][0] = *reinterpret_cast<const double2 *>(src);
        u[s][1] = *reinterpret_cast<const double2 *>(src + 2);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = (t >> 4) + 16 * s;
        double e4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t gj = c0 + j, gk = c0 + k4 + i;
          e4[i] = gj < n && gk < n ? U[gj * n + gk] : (gj == gk ? 1.0 : 0.0);
        }
        u[s][0] = make_double2(e4[0], e4[1]);
        u[s][1] = make_double2(e4[2], e4[3]);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      double *dst = LU + ((t >> 4) + 16 * s) * DB + k4;
      *reinterpret_cast<double2 *>(dst) = u[s][0];
      *reinterpret_cast<double2 *>(dst + 2) = u[s][1];
    }
  }
  __syncthreads();
  if (t < DB) RU[t] = 1.0 / LU[t * DB + t];
  __syncthreads();
  double v[4] = {v01.x, v01.y, v23.x, v23.y};
  // s * S (exact in double) and the midpoints between grid values at that scale; a zero
  // byte gives infinite midpoints, so every value rounds to code 0
  double sS = 0.0;
  if (byte != 0) {
    const int ex = (byte >> 3) & 15, mant = byte & 7;
    const double s = ex == 0 ? ldexp((double)mant, -9) : ldexp((double)(8 + mant), ex - 10);
    sS = s * (double)Sp[0];
  }
  const double big = __builtin_inf();
  const double T0 = byte ? 0.25 * sS : big, T1 = byte ? 0.75 * sS : big,
               T2 = byte ? 1.25 * sS : big, T3 = byte ? 1.75 * sS : big,
               T4 = byte ? 2.5 * sS : big, T5 = byte ? 3.5 * sS : big, T6 = byte ? 5.0 * sS : big;
  const double half = 0.5 * sS;
  unsigned cw = 0u;
  double ev[4] = {0.0, 0.0, 0.0, 0.0};
  // kept in registers off the column chain: 1 / U_jj for this lane's own four columns (only
  // the owning lane's e is used), and U's next row, read one column ahead
  double ru[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ru[i] = RU[4 * p + i];
  double2 un01 = *reinterpret_cast<const double2 *>(LU + 4 * p);
  double2 un23 = *reinterpret_cast<const double2 *>(LU + 4 * p + 2);
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    const int pj = j >> 2, jj = j & 3;
    const double2 u01 = un01, u23 = un23;
    if (j + 1 < DB) {
      un01 = *reinterpret_cast<const double2 *>(LU + (j + 1) * DB + 4 * p);
      un23 = *reinterpret_cast<const double2 *>(LU + (j + 1) * DB + 4 * p + 2);
    }
    const double x = v[jj];
    const double a = fabs(x);
    // round half to even onto {0, .5, 1, 1.5, 2, 3, 4, 6} sS: crossing midpoint i moves up
    // one grid step; on a tie, odd i (whose upper neighbour has an even index) moves up
    const int b0 = a > T0, b1 = a >= T1, b2 = a > T2, b3 = a >= T3, b4 = a > T4, b5 = a >= T5,
              b6 = a > T6;
    const int k = b0 + b1 + b2 + b3 + b4 + b5 + b6;
    // grid value in halves of sS: steps of 1/2 up to 2, then 3, 4, 6 (exact: at most 12 sS / 2)
    const double qm = (double)(b0 + b1 + b2 + b3 + 2 * (b4 + b5) + 4 * b6) * half;
    const double q = x < 0.0 ? -qm : qm;
    const unsigned code = (unsigned)k | ((x < 0.0 && k > 0) ? 8u : 0u);
    const double e_own = (x - q) * ru[jj];
    const bool mine = p == pj;
    cw |= mine ? code << (4 * jj) : 0u;
    ev[jj] = mine ? e_own : ev[jj];
    const double e = row_bcast16(e_own, pj);
    v[0] = fma(-e, u01.x, v[0]);
    v[1] = fma(-e, u01.y, v[1]);
    v[2] = fma(-e, u23.x, v[2]);
    v[3] = fma(-e, u23.y, v[3]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (live) *reinterpret_cast<uint16_t *>(codes + r * (n / 2) + cb / 2) = (uint16_t)cw;
  double *er = E + r * OB + (b % 4) * DB + 4 * p;
  *reinterpret_cast<double2 *>(er) = make_double2(ev[0], ev[1]);
  *reinterpret_cast<double2 *>(er + 2) = make_double2(ev[2], ev[3]);

  // the rest of the outer block: V[:, tile] -= E[:, block] U[block, tile] for this
  // workgroup's 16 rows, as 16 fp64 MFMA steps per tile (K = 4 each); A fragments (lane l:
  // row l & 15 at k = l >> 4) come from LDS ([k][row])
  __shared__ double LE[DB * 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) LE[(4 * p + i) * 16 + (t >> 4)] = ev[i];
  __syncthreads();
#pragma unroll
  for (int qi = 0; qi < 3; ++qi) {
    const int q = w + 4 * qi;
    if (q >= ntiles) break;
    gq_v4d acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 16; ++s)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(LE[(4 * s + lr) * 16 + lc], ub[qi][s], acc, 0, 0, 0);
    const int64_t cq = c0 + DB + 16 * q + lc;
#pragma unroll
    for (int i = 0; i < 4; ++i) V[(r0 + lr + 4 * i) * np + cq] = vv[qi][i] - acc[i];
  }
}

// the outer update: V[:, 128-column tiles from c_start] -= E[:, 0 .. 256) U[k0 .. k0 + 256,
// those columns], with rows of U at or beyond n counting as zero
__global__ void __launch_bounds__(W2T)
    k_gptq_update2(double *__restrict__ V, int64_t np, int64_t n, const double *__restrict__ U,
                   const double *__restrict__ E, int64_t k0, int64_t c_start) {
  __shared__ __attribute__((aligned(16))) double L2[4 * KC * P2];  // two (A, B) chunk buffers
  const int64_t r0 = (int64_t)blockIdx.x * T2, c0 = c_start + (int64_t)blockIdx.y * T2;
  const int nlim = (int)(n - c0 < T2 ? n - c0 : T2);
  const int64_t klim = n - k0 < OB ? n - k0 : OB;
  // padding columns of V (n and beyond) are left alone: only their own errors reach them
  d2_gemm_sub<true, OB / KC>(V + r0 * np + c0, np, T2, nlim, E + r0 * OB, OB, U + k0 * n + c0, n,
                             klim, L2);
}

// the same update with 64 x 64 tiles of V (columns at or beyond n are skipped)
__global__ void __launch_bounds__(256)
    k_gptq_update64(double *__restrict__ V, int64_t np, int64_t n, const double *__restrict__ U,
                    const double *__restrict__ E, int64_t k0, int64_t c_start) {
  __shared__ double LA[DB * DP], LB[DB * DP];
  const int64_t r0 = (int64_t)blockIdx.x * DB, c0 = c_start + (int64_t)blockIdx.y * DB;
  if (c0 >= n) return;
  const int nlim = (int)(n - c0 < DB ? n - c0 : DB);
  const int64_t klim = n - k0 < OB ? n - k0 : OB;
  d64_sub<true, OB / DB>(V + r0 * np + c0, np, nlim, E + r0 * OB, OB, U + k0 * n + c0, n, klim,
                         LA, LB);
}

int launch_gptq_rows(const void *w, int dtype, int64_t rows, int64_t n, const float *S,
                     const uint8_t *scales, const double *U, uint8_t *codes, void *workspace,
                     hipStream_t st) {
  const int64_t rp = pad128(rows), np = pad128(n), nbc = pad64(n) / DB;
  double *V = static_cast<double *>(workspace);
  double *E = V + rp * np;
  const int64_t cus = gptq_cus();
  if (dtype == NVFP4_DTYPE_BF16)
    hipLaunchKernelGGL(k_gptq_init<NVFP4_DTYPE_BF16>, dim3((unsigned)((np / 4 + 255) / 256), (unsigned)(rp < 65535 ? rp : 65535)), dim3(256), 0, st, w,
                       rows, n, rp, np, V);
  else
    hipLaunchKernelGGL(k_gptq_init<NVFP4_DTYPE_F32>, dim3((unsigned)((np / 4 + 255) / 256), (unsigned)(rp < 65535 ? rp : 65535)), dim3(256), 0, st, w,
                       rows, n, rp, np, V);
  // blocks of 64 columns; inside an outer block of 256 a block's errors update only the
  // rest of that outer block (within k_gptq_block), and each outer block then updates
  // every later column at once
  for (int64_t b = 0; b < nbc; ++b) {
    hipLaunchKernelGGL(k_gptq_block, dim3((unsigned)(rp / 16)), dim3(256), 0, st, V, np, rows, n, S,
                       scales, U, b, E, codes);
    const int64_t ob_end = (b / 4 + 1) * 4 < nbc ? (b / 4 + 1) * 4 : nbc;  // in blocks
    if (b + 1 == ob_end && ob_end < nbc) {
      const int64_t c_start = ob_end * DB;
      if ((rp / T2) * ((np - c_start) / T2) >= cus)
        hipLaunchKernelGGL(k_gptq_update2, dim3((unsigned)(rp / T2), (unsigned)((np - c_start) / T2)),
                           dim3(W2T), 0, st, V, np, n, U, E, (b / 4) * OB, c_start);
      else  // too few wide tiles to fill the device
        hipLaunchKernelGGL(k_gptq_update64, dim3((unsigned)(rp / DB), (unsigned)((np - c_start) / DB)),
                           dim3(256), 0, st, V, np, n, U, E, (b / 4) * OB, c_start);
    }
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

// Device-side NVFP4 format arithmetic for gfx950.
//
// Every rounding decision is taken on exact reals. The decisive products (grid value or
// midpoint times block scale s times tensor scale S) have at most 31 significant bits, so
// they are exact in double; each is then turned into an fp32 threshold T' with the
// property  (X > T)  <=>  (X > T')  (or (X >= T) <=> (X > T')) for every fp32 X >= 0,
// which lets the per-element work be plain fp32 compares.
//
// E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} and its midpoints {0.25, 0.75, 1.25, 1.75, 2.5,
// 3.5, 5}: Baseten on NVFP4 quality, "Why do we need a scale". E4M3FN bytes 0x01..0x7E
// are the 126 positive candidates of the Local-Hessian write-up.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// A block byte given by the caller, read as an E4M3FN magnitude: the sign bit is ignored,
// and 0x7F (NaN, not one of the 126 candidates) codes its block as zeros, like 0x00.
__device__ __forceinline__ int given_byte(int b) {
  const int m = b & 0x7F;
  return m == 0x7F ? 0 : m;
}

// Value of E4M3FN byte b in 0..126 (exponent bias 7, subnormals m * 2^-9); the sign bit
// of a larger byte is ignored.
__device__ __forceinline__ float e4m3_value(int b) {
  int e = (b >> 3) & 15, m = b & 7;
  return e ? ldexpf(float(8 + m), e - 10) : ldexpf(float(m), -9);
}

__device__ __forceinline__ double e4m3_value_d(int b) { return (double)e4m3_value(b); }

// Largest fp32 f with  X > T  <=>  X > f  for all fp32 X >= 0  (T > 0).
__device__ __forceinline__ float thr_strict(double T) {
  float f = (float)T;
  if ((double)f > T) f = __uint_as_float(__float_as_uint(f) - 1u);
  return f;
}

// Largest fp32 f with  X >= T  <=>  X > f  for all fp32 X >= 0  (T > 0).
__device__ __forceinline__ float thr_nonstrict(double T) {
  float f = (float)T;
  if ((double)f >= T) f = __uint_as_float(__float_as_uint(f) - 1u);
  return f;
}

// Per-scale rounding table: code k = #{j : |x| > t[j]}, magnitude d[k] = fp32(G_k s S).
// Midpoint j lies between grid indices j and j+1; a tie goes to the even index, so even
// midpoints use a strict threshold and odd ones a non-strict one.
struct ScaleTable {
  float t[7];
  float d[8];
};

__device__ __forceinline__ void make_table(int byte, float S, ScaleTable &tb) {
  const double sS = e4m3_value_d(byte) * (double)S;  // exact (<= 28 bits)
  tb.t[0] = thr_strict(0.25 * sS);
  tb.t[1] = thr_nonstrict(0.75 * sS);
  tb.t[2] = thr_strict(1.25 * sS);
  tb.t[3] = thr_nonstrict(1.75 * sS);
  tb.t[4] = thr_strict(2.5 * sS);
  tb.t[5] = thr_nonstrict(3.5 * sS);
  tb.t[6] = thr_strict(5.0 * sS);
  tb.d[0] = 0.0f;
  tb.d[1] = (float)(0.5 * sS);
  tb.d[2] = (float)(1.0 * sS);
  tb.d[3] = (float)(1.5 * sS);
  tb.d[4] = (float)(2.0 * sS);
  tb.d[5] = (float)(3.0 * sS);
  tb.d[6] = (float)(4.0 * sS);
  tb.d[7] = (float)(6.0 * sS);
}

// Max-scaling byte: E4M3 value nearest to amax / (k S), ties to the even byte, saturating
// at 448 (0x7E), at least 0x01 for amax > 0; 0x00 for amax == 0. k = 6 maps the block max
// onto the largest E2M1 magnitude; Four Over Six also tries k = 4. Products value * k * S
// have at most 31 significant bits, so every comparison below is exact in double.
__device__ __forceinline__ int max_scale_byte(float amax, float S, float k = 6.0f) {
  if (amax == 0.0f) return 0;
  const double a = amax, sixS = (double)k * (double)S;  // exact
  // first guess from an fp32 quotient, then exact correction
  const float q = amax / (k * S);
  int b;
  if (!(q < 448.0f)) {
    b = 126;
  } else if (q < 0.015625f) {
    b = (int)(q * 512.0f);
  } else {
    const unsigned u = __float_as_uint(q);
    b = ((int)(u >> 23) - 120) * 8 + (int)((u >> 20) & 7u);
  }
  b = b < 0 ? 0 : (b > 126 ? 126 : b);
  while (b < 126 && e4m3_value_d(b + 1) * sixS <= a) ++b;
  while (b > 0 && e4m3_value_d(b) * sixS > a) --b;
  if (b < 126) {
    const double mid = 0.5 * (e4m3_value_d(b) + e4m3_value_d(b + 1)) * sixS;
    if (a > mid || (a == mid && (b & 1))) ++b;
  }
  return b == 0 ? 1 : b;
}

// ---------------------------------------------------------------- hardware-convert fast path
//
// gfx950's FP4 convert rounds an fp32 value half-to-even onto the E2M1 grid and saturates at
// +-6; its FP8 convert rounds half-to-even onto E4M3FN (inputs clamped to 448 first). They
// decide on the fp32 *input*, whereas the decision must be taken on the exact quotient
// x / (s S). So each value is converted twice, after multiplying by two reciprocals that
// bracket 1/(s S) (relative gap 2^-22 each side of it, above every rounding in the
// products): if both conversions agree, the exact quotient rounds the same way (rounding is
// monotone and a quotient on a midpoint would split the pair). If they differ (a value
// within ~2^-22 of a midpoint) the caller falls back to the exact threshold path.

typedef float nv_v2f __attribute__((ext_vector_type(2)));

// lo < 1/d < hi for an exact double d > 0 (both as fp32). Two Newton steps on v_rcp_f64.
__device__ __forceinline__ void recip_bracket(double d, float &lo, float &hi) {
  double r = __builtin_amdgcn_rcp(d);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  lo = (float)(r * (1.0 - 0x1p-22));
  hi = (float)(r * (1.0 + 0x1p-22));
}

// Max-scaling byte from bracketing multipliers lo < 1/(kS) < hi. The two FP8 conversions
// give the same byte, or two adjacent bytes when amax / (kS) lies within the bracket of the
// midpoint between them; then one exact comparison (products <= 31 bits, exact in double)
// decides, ties to the even byte.
__device__ __forceinline__ int max_scale_byte_fast(float amax, float qlo_mul, float qhi_mul,
                                                   float S, float k = 6.0f) {
  if (amax == 0.0f) return 0;
  const float qlo = fminf(amax * qlo_mul, 448.0f), qhi = fminf(amax * qhi_mul, 448.0f);
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(qlo, qhi, 0, false);
  int b = pk & 0xFF;
  const int b1 = (pk >> 8) & 0xFF;
  if (b != b1) {
    if (b1 == b + 1) {
      const double mid = 0.5 * (e4m3_value_d(b) + e4m3_value_d(b1)) * ((double)k * (double)S);
      const double a = amax;
      b = (a > mid || (a == mid && (b & 1))) ? b1 : b;
    } else {
      b = max_scale_byte(amax, S, k);
    }
  }
  return b == 0 ? 1 : b;
}

// Workgroup barrier that orders LDS only (address-space-qualified fences): global loads
// issued before it stay in flight across it, so a table can be built while they land.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-tensor table of the 127 scale bytes: entry c >= 1 holds s = E4M3(c), the bracket
// lo < 1/(s S) < hi, and z = the largest fp32 <= s S / 4 (for fp32 X >= 0, X <= z exactly
// when X rounds to code 0 at this scale: at s S / 4 itself the tie goes to the even code 0);
// entry 0 holds s = 0 and the bracket of 1/(6 S) used by the max byte.
struct Cand {
  float s, rlo, rhi, z;
};

__device__ __forceinline__ void build_cands(Cand *cand, float S) {
  for (int c = threadIdx.x; c < 127; c += blockDim.x) {
    Cand e;
    e.s = c ? e4m3_value(c) : 0.0f;
    recip_bracket(c ? (double)e.s * (double)S : 6.0 * (double)S, e.rlo, e.rhi);
    const double t = 0.25 * (double)e.s * (double)S;  // exact: at most 28 significant bits
    float z = (float)t;
    if ((double)z > t) z = __uint_as_float(__float_as_uint(z) - 1u);
    e.z = c ? z : 0.0f;
    cand[c] = e;
  }
}

// Midpoint between E2M1 grid indices j and j+1.
__device__ __forceinline__ double e2m1_mid(int j) {
  double m = 0.25;
  m = j == 1 ? 0.75 : m;
  m = j == 2 ? 1.25 : m;
  m = j == 3 ? 1.75 : m;
  m = j == 4 ? 2.5 : m;
  m = j == 5 ? 3.5 : m;
  m = j == 6 ? 5.0 : m;
  return m;
}

// Resolve the nibbles where the codes from the low and high brackets differ: the exact
// code is one of the two adjacent magnitudes, decided by one exact comparison with the
// midpoint between them (ties to the even index). a: codes from lo, b: codes from hi.
__device__ __forceinline__ unsigned fp4_resolve8(const float *v, unsigned a, unsigned b,
                                                 double sS) {
  unsigned d = a ^ b;
  while (d) {
    const int i = __builtin_ctz(d) >> 2;
    const unsigned sh = 4u * (unsigned)i;
    const int j = (int)((a >> sh) & 7u);
    float vi = v[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) vi = (i == k) ? v[k] : vi;
    const double X = fabs((double)vi), T = e2m1_mid(j) * sS;  // T exact (<= 31 bits)
    const bool up = (X > T) || (X == T && (j & 1));
    const unsigned mag = (unsigned)(up ? j + 1 : j);
    const unsigned neg = (__float_as_uint(vi) >> 31) & (mag ? 1u : 0u);
    a = (a & ~(0xFu << sh)) | ((mag | (neg << 3)) << sh);
    d &= ~(0xFu << sh);
  }
  return a;
}

// Signed E2M1 codes of 8 values (element i in nibble i) after scaling by lo (into a) and
// by hi (into b); equal nibbles are the exact codes.
__device__ __forceinline__ void fp4_codes8(const float *v, float lo, float hi, unsigned &a,
                                           unsigned &b) {
  a = 0u;
  b = 0u;
  a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[0] * lo, v[1] * lo, 1.0f, 0);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[2] * lo, v[3] * lo, 1.0f, 1);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[4] * lo, v[5] * lo, 1.0f, 2);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, v[6] * lo, v[7] * lo, 1.0f, 3);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, v[0] * hi, v[1] * hi, 1.0f, 0);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, v[2] * hi, v[3] * hi, 1.0f, 1);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, v[4] * hi, v[5] * hi, 1.0f, 2);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, v[6] * hi, v[7] * hi, 1.0f, 3);
}

// Exact signed codes of 8 values for block scale s (sS = s * S exact in double).
__device__ __forceinline__ unsigned fp4_exact_codes8(const float *v, float lo, float hi,
                                                     double sS) {
  unsigned a, b;
  fp4_codes8(v, lo, hi, a, b);
  if (a != b) a = fp4_resolve8(v, a, b, sS);
  return a;
}

// ---- cross-lane exchange through the VALU (v_permlane16_swap / v_permlane32_swap)
// A "row" is 16 consecutive lanes; rows pair up as {0,1} and {2,3}, halves as {0-31, 32-63}.
// swap16(a, b) returns (r0, r1): in an even row r0 = its own a, r1 = a of the odd row; in an
// odd row r0 = b of the even row, r1 = its own b (swap32 likewise with the two halves).
struct LanePair {
  float r0, r1;
};
__device__ __forceinline__ LanePair swap16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair swap32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// x of the lane 16 (resp. 32) positions away: odd rows take r0, even rows r1
__device__ __forceinline__ float xor16(float x) {
  const LanePair r = swap16(x, x);
  return (threadIdx.x & 16) ? r.r0 : r.r1;
}
__device__ __forceinline__ float xor32(float x) {
  const LanePair r = swap32(x, x);
  return (threadIdx.x & 32) ? r.r0 : r.r1;
}
__device__ __forceinline__ int xor16(int x) { return __float_as_int(xor16(__int_as_float(x))); }
__device__ __forceinline__ int xor32(int x) { return __float_as_int(xor32(__int_as_float(x))); }

// Clear the sign bit of every zero-magnitude nibble (the convert keeps the sign of -0).
__device__ __forceinline__ unsigned fp4_clear_neg_zero(unsigned c) {
  const unsigned m = c & 0x77777777u;
  const unsigned nz = (m + 0x77777777u) & 0x88888888u;  // bit 3 set iff magnitude != 0
  return m | (c & nz);
}

// Signed grid values G of 8 packed codes.
__device__ __forceinline__ void fp4_decode8(unsigned c, float g[8]) {
  nv_v2f t;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  g[0] = t.x; g[1] = t.y;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
  g[2] = t.x; g[3] = t.y;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
  g[4] = t.x; g[5] = t.y;
  t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
  g[6] = t.x; g[7] = t.y;
}

// Exact codes of 8 values from a threshold table (the fallback path).
__device__ __forceinline__ unsigned exact_codes8(const float *v, const ScaleTable &tb) {
  unsigned out = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float X = fabsf(v[i]);
    unsigned k = 0u;
#pragma unroll
    for (int j = 0; j < 7; ++j) k += (X > tb.t[j]) ? 1u : 0u;
    const unsigned neg = (__float_as_uint(v[i]) >> 31) & (k ? 1u : 0u);
    out |= (k | (neg << 3)) << (4 * i);
  }
  return out;
}

// RNE of fp32 to bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 nv_v2bf __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16 (round half to even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  const nv_v2f f = {a, b};
  const nv_v2bf h = __builtin_convertvector(f, nv_v2bf);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace nvfp4

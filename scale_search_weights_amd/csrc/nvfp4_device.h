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

// Value of E4M3FN byte b in 0..126 (exponent bias 7, subnormals m * 2^-9).
__device__ __forceinline__ float e4m3_value(int b) {
  int e = b >> 3, m = b & 7;
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

// Max-scaling byte: E4M3 value nearest to amax / (6 S), ties to the even byte, saturating
// at 448 (0x7E), at least 0x01 for amax > 0; 0x00 for amax == 0.
__device__ __forceinline__ int max_scale_byte(float amax, float S) {
  if (amax == 0.0f) return 0;
  const double a = amax, sixS = 6.0 * (double)S;  // exact
  // first guess from an fp32 quotient, then exact correction
  const float q = amax / (6.0f * S);
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

// RNE of fp32 to bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace nvfp4

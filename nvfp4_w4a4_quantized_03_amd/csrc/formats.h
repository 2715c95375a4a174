// Device helpers for the OCP E4M3 format, shared by every kernel that
// reads or writes E4M3 block scales or FP8 KV codes.
//
// E4M3 is the block-scale format of NVFP4 (explainer page
// "論文解説: Gated DeltaNet はなぜ4bit量子化に耐えるのか", section 前提1); read as
// OCP E4M3FN: exponent bias 7, subnormals m/8 * 2^-6, no infinity, largest
// finite 448 (code 0x7E).  Rounding is to nearest, ties to the even code,
// saturating at 448.
#pragma once

#include <hip/hip_runtime.h>

namespace nvfp4 {

// Value of a non-negative OCP E4M3FN code 0x00..0x7E (bias 7, subnormals
// m/8 * 2^-6, largest finite 448), exactly, in float64.
static __device__ __forceinline__ double e4m3_value(unsigned c) {
  const unsigned e = c >> 3, m = c & 7u;
  return e ? __builtin_ldexp(static_cast<double>(8u + m), static_cast<int>(e) - 10)
           : __builtin_ldexp(static_cast<double>(m), -9);
}

// binary32 value of a non-negative E4M3 code 0x00..0x7E (exact).
static __device__ __forceinline__ float e4m3_f32(unsigned c) {
  return c >= 8u ? __uint_as_float((c << 20) + 0x3C000000u)
                 : static_cast<float>(c) * 0x1p-9f;
}

// A code within one step of RNE_SAT_E4M3(q) for q >= 0: q is rounded to
// binary32 (clamped) and then rounded to 3 mantissa bits in integer form.
static __device__ __forceinline__ unsigned e4m3_candidate(double q) {
  const float f = static_cast<float>(q < 1024.0 ? q : 1024.0);
  const unsigned sub = static_cast<unsigned>(__builtin_rintf(f * 512.0f));
  unsigned b = __float_as_uint(f);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  unsigned norm = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  norm = norm < 0x7Eu ? norm : 0x7Eu;
  return f < 0.015625f ? sub : norm;
}

// Exact RNE_SAT_E4M3(num / den) given a candidate within one code of it.
// Midpoints of adjacent codes have <= 5 significant bits and den (6 g or a
// global) <= 26, so mid * den is exact in float64 and the compares decide
// the rounding without error; ties go to the even code.
static __device__ __forceinline__ unsigned e4m3_settle(unsigned c, double num,
                                                double den) {
  if (c < 0x7Eu) {
    const double t = 0.5 * (e4m3_value(c) + e4m3_value(c + 1)) * den;
    if (num > t || (num == t && ((c + 1) & 1u) == 0)) return c + 1;
  }
  if (c > 0) {
    const double t = 0.5 * (e4m3_value(c - 1) + e4m3_value(c)) * den;
    if (num < t || (num == t && (c & 1u))) return c - 1;
  }
  return c;
}

}  // namespace nvfp4

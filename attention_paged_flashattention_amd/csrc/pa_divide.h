// Correctly rounded float32 division x / s by a divisor shared by many x (the
// per-head scale of the FP8 KV cache: "1Cat-vLLM 1.0.0" README, "Optional
// experimental feature: FP8 KV cache"). Host and device code, so the
// arithmetic can be checked on the CPU against IEEE division.
#pragma once

#include <hip/hip_runtime.h>

namespace pa {

// A divisor s with r = 1/s correctly rounded, and the range [lo, hi] of |x|
// over which x / s can be formed from r (below). The range is empty unless s
// and r are both normal floats (otherwise -- zero, subnormal, infinite or NaN
// s, or a reciprocal that is subnormal or overflows -- every quotient is a
// plain division).
struct Divisor {
  float s, r, lo, hi;
};

__host__ __device__ inline bool is_normal_finite(float v) {
  const float a = __builtin_fabsf(v);
  return a >= 0x1p-126f && a <= 3.40282347e38f;
}

// The shortcut below is exact when |x| >= 2^-100 and 2^-100 <= |x r| <= 2^100
// (Markstein's conditions, see div_fast). lo and hi bound |x| so that both
// hold with a factor of two to spare, whatever the rounding of lo, hi and x r:
// |x| >= lo gives |x r| >= 2^-99 (1 - 2^-24)^2 > 2^-100, and |x| <= hi gives
// |x r| <= 2^99 (1 + 2^-24)^2 < 2^100. hi is finite, so x = inf falls outside.
__host__ __device__ inline Divisor make_divisor(float s) {
  Divisor d;
  d.s = s;
  d.r = 1.0f / s;
  if (is_normal_finite(s) && is_normal_finite(d.r)) {
    const float ar = __builtin_fabsf(d.r);
    d.lo = __builtin_fmaxf(0x1p-100f, 0x1p-99f / ar);
    d.hi = __builtin_fminf(0x1p99f / ar, 3.40282347e38f);
  } else {
    d.lo = __builtin_inff();
    d.hi = 0.0f;
  }
  return d;
}

// Whether div_fast(x, d) is the correctly rounded x / s (false for zeros,
// NaN, infinities, and |x| outside [lo, hi]).
__host__ __device__ inline bool div_fast_ok(float x, const Divisor& d) {
  const float ax = __builtin_fabsf(x);
  return ax >= d.lo && ax <= d.hi;
}

// x / s from r: q = x * r is within an ulp of x / s, the remainder x - s * q
// is exact under fma, and one correction q + r * (x - s q), rounded once, is
// the correctly rounded quotient (Markstein's theorem for round-to-nearest;
// an exact q has a zero remainder and comes back unchanged). Three operations;
// valid where div_fast_ok holds.
__host__ __device__ inline float div_fast(float x, const Divisor& d) {
  const float q = x * d.r;
  const float e = __builtin_fmaf(-q, d.s, x);
  return __builtin_fmaf(e, d.r, q);
}

// x / s, correctly rounded (round to nearest even), equal bit for bit to IEEE
// float32 division: the shortcut where it is exact, the division itself (the
// build makes it correctly rounded) everywhere else.
__host__ __device__ inline float div_rn(float x, const Divisor& d) {
  return div_fast_ok(x, d) ? div_fast(x, d) : x / d.s;
}

}  // namespace pa

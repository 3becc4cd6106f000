// Correctly rounded float32 division x / s by a divisor shared by many x (the
// per-head scale of the FP8 KV cache: "1Cat-vLLM 1.0.0" README, "Optional
// experimental feature: FP8 KV cache"). Host and device code, so the
// arithmetic can be checked on the CPU against IEEE division.
#pragma once

#include <hip/hip_runtime.h>

namespace pa {

// A divisor s with r = 1/s correctly rounded. `fast` holds when s and r are
// both normal floats: then x / s can be formed from r (below); otherwise
// (zero, subnormal, infinite or NaN s, or a reciprocal that is subnormal or
// overflows) every quotient is a plain division.
struct Divisor {
  float s, r;
  bool fast;
};

__host__ __device__ inline bool is_normal_finite(float v) {
  const float a = __builtin_fabsf(v);
  return a >= 0x1p-126f && a <= 3.40282347e38f;
}

__host__ __device__ inline Divisor make_divisor(float s) {
  Divisor d;
  d.s = s;
  d.r = 1.0f / s;
  d.fast = is_normal_finite(s) && is_normal_finite(d.r);
  return d;
}

// x / s, correctly rounded (round to nearest even), equal bit for bit to IEEE
// float32 division. From r: q = x * r is within an ulp of x / s, the
// remainder x - s * q is exact under fma, and one correction q + r * (x - s q)
// rounded once is the correctly rounded quotient (Markstein's theorem for
// round-to-nearest). The theorem needs every step clear of underflow and
// overflow, which holds when s and r are normal, |x| >= 2^-100 and
// 2^-100 <= |q| <= 2^100 (the remainder is then a multiple of at least
// 2^-150 of 24 significant bits, and nothing overflows). An exact q (zero
// remainder) is returned as it is. Everything else -- zeros, tiny or huge
// quotients, infinities, NaN, a divisor outside the fast range -- takes the
// division itself (the build makes it correctly rounded). Three operations
// per element on the fast path.
__host__ __device__ inline float div_rn(float x, const Divisor& d) {
  if (d.fast) {
    const float q = x * d.r;
    const float aq = __builtin_fabsf(q);
    if (aq >= 0x1p-100f && aq <= 0x1p100f && __builtin_fabsf(x) >= 0x1p-100f) {
      const float e = __builtin_fmaf(-q, d.s, x);
      return e == 0.0f ? q : __builtin_fmaf(e, d.r, q);
    }
  }
  return x / d.s;
}

}  // namespace pa

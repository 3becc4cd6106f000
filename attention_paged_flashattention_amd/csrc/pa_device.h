// Device-side helpers shared by the paged-attention kernels (gfx950 only).
//
// FP8 formats are OCP E4M3FN (bias 7, max 448, S.1111.111 = NaN) and E5M2
// (bias 15, max 57344), the two KV-cache formats of "1Cat-vLLM 1.0.0" README,
// "Optional experimental feature: FP8 KV cache".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_divide.h"

namespace pa {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache element formats (compile-time tags).
enum KvFmt : int { KV_F16 = 0, KV_E4M3 = 1, KV_E5M2 = 2 };
// Query element types.
enum QType : int { Q_F16 = 0, Q_BF16 = 1 };
// Output element types.
enum OType : int { O_F32 = 0, O_F16 = 1, O_BF16 = 2 };

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// FP8 -> 16-bit, exact.
//
// E4M3: gfx950's v_cvt_scalef32_pk_f16_fp8 / _bf16_fp8 with scale 1.0 convert
// two OCP E4M3 codes to two fp16 / bf16 values per instruction. Both targets
// hold every E4M3 value exactly (subnormals m * 2^-9 are fp16 normals), and an
// exhaustive check of all 256 codes on the GPU found no difference from the
// format definition (NaN stays NaN).
//
// E5M2 is the upper byte of an fp16 with the same exponent bias, so
// half_bits = code << 8 is the value itself: one byte permute per pair.
// ---------------------------------------------------------------------------

// Two bytes (b0, b1) of w selected by `sel` (a v_perm_b32 selector that places
// them in the high byte of each 16-bit half) -> two fp16 bit patterns (E5M2).
__device__ __forceinline__ uint32_t e5m2x2_to_h2(uint32_t w, uint32_t sel) {
  return __builtin_amdgcn_perm(0u, w, sel);  // (b1 << 24) | (b0 << 8)
}

// 4 FP8 codes in a dword -> 4 fp16 (2 dwords), element order preserved.
template <int FMT>
__device__ __forceinline__ u32x2 fp8x4_to_h4(uint32_t w) {
  u32x2 r;
  if constexpr (FMT == KV_E5M2) {
    r.x = e5m2x2_to_h2(w, 0x010c000cu);  // bytes 0,1
    r.y = e5m2x2_to_h2(w, 0x030c020cu);  // bytes 2,3
  } else {
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  return r;
}

// 8 FP8 codes (2 dwords) -> half8 MFMA operand.
template <int FMT>
__device__ __forceinline__ half8 fp8x8_to_half8(uint32_t w0, uint32_t w1) {
  u32x2 a = fp8x4_to_h4<FMT>(w0);
  u32x2 b = fp8x4_to_h4<FMT>(w1);
  u32x4 r;
  r.x = a.x; r.y = a.y; r.z = b.x; r.w = b.y;
  return __builtin_bit_cast(half8, r);
}

// Two fp16 bit patterns -> two bf16 bit patterns. Exact for every value an
// FP8 code produces (at most 4 significant bits, exponents far inside bf16's
// range): fp16 -> fp32 is exact and the low 16 bits of the fp32 are zero.
__device__ __forceinline__ uint32_t h2_to_bf2(uint32_t h2) {
  _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(h2 & 0xFFFFu));
  _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(h2 >> 16));
  uint32_t flo = __builtin_bit_cast(uint32_t, (float)lo);
  uint32_t fhi = __builtin_bit_cast(uint32_t, (float)hi);
  return __builtin_amdgcn_perm(fhi, flo, 0x07060302u);  // high halves
}

template <int FMT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf2(uint32_t w) {
  if constexpr (FMT == KV_E4M3) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  } else {
    return h2_to_bf2(e5m2x2_to_h2(w, HI ? 0x030c020cu : 0x010c000cu));
  }
}

template <int FMT>
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r.x = fp8x2_to_bf2<FMT, false>(w0); r.y = fp8x2_to_bf2<FMT, true>(w0);
  r.z = fp8x2_to_bf2<FMT, false>(w1); r.w = fp8x2_to_bf2<FMT, true>(w1);
  return __builtin_bit_cast(bf16x8, r);
}

// Factor that turns the 16-bit operand value back into the code's value
// (1: both conversions above are value-exact).
template <int FMT>
__device__ __forceinline__ constexpr float kv_fold() {
  return 1.0f;
}

// Four fp32 values -> four FP8 codes (bytes 0..3), round to nearest even,
// saturating, sign kept, by gfx950's packed conversions. The values are first
// clamped to the format's largest finite value (NaN passes through), so the
// result never depends on how the conversion treats overflow.
template <int FMT>
__device__ __forceinline__ uint32_t fp8x4_from_f32(float y0, float y1, float y2, float y3) {
  constexpr float kMax = FMT == KV_E4M3 ? 448.0f : 57344.0f;
  auto sat = [](float y) { return y != y ? y : fminf(fmaxf(y, -kMax), kMax); };
  y0 = sat(y0); y1 = sat(y1); y2 = sat(y2); y3 = sat(y3);
  if constexpr (FMT == KV_E4M3) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)lo, true);
  } else {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, (int)lo, true);
  }
}

// 16-bit source element -> fp32 (exact).
template <int ST>
__device__ __forceinline__ float src_to_f32(uint16_t bits) {
  if constexpr (ST == Q_BF16) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
}

// y[i] = x[i] / s, correctly rounded, for N elements: the three-operation
// quotient for all of them, and the division itself only in the (rare) lanes
// where some element lies outside the shortcut's range -- one branch per N
// elements instead of one per element.
template <int N>
__device__ __forceinline__ void divide_n(float (&y)[N], const float (&x)[N], const Divisor& d) {
  bool ok = true;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    y[i] = div_fast(x[i], d);
    ok = ok & div_fast_ok(x[i], d);
  }
  if (!ok) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!div_fast_ok(x[i], d)) y[i] = x[i] / d.s;
  }
}

// 8 source elements (one 16-byte chunk) -> 8 cache codes: FP8 in the low 8
// bytes, or the fp16 elements unchanged.
template <int ST, int FMT>
__device__ __forceinline__ u32x4 encode8(u32x4 w, bool scaled, const Divisor& div) {
  if constexpr (FMT == KV_F16) {
    return w;
  } else {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float x[8], y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = src_to_f32<ST>((uint16_t)(ww[i >> 1] >> ((i & 1) * 16)));
      y[i] = x[i];
    }
    if (scaled) divide_n<8>(y, x, div);   // x / scale, correctly rounded
    return u32x4{fp8x4_from_f32<FMT>(y[0], y[1], y[2], y[3]),
                 fp8x4_from_f32<FMT>(y[4], y[5], y[6], y[7]), 0u, 0u};
  }
}

// ---------------------------------------------------------------------------
// Output stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int OT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (OT == O_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if constexpr (OT == O_F16) {
    reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lane_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Reductions between lanes l and l ^ 32 (permlane32 swap) or l and l ^ 16
// (permlane16 swap) of a wave64: one VALU instruction, no LDS round trip.
// With the same value in both operands, a swap leaves one member of each lane
// pair's values in one output and the other member's in the other output, so
// combining the two outputs with a symmetric operation reduces each lane with
// its partner. (The outputs are copied to scalars before the bit casts: this
// compiler reads element 0 when a bit cast takes a vector element.)
template <int XOR>
__device__ __forceinline__ float swap_max(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  uint32_t r0, r1;
  if constexpr (XOR == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r0 = r[0]; r1 = r[1];
  } else {
    static_assert(XOR == 16, "lane distance 16 or 32");
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r0 = r[0]; r1 = r[1];
  }
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

template <int XOR>
__device__ __forceinline__ float swap_sum(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  uint32_t r0, r1;
  if constexpr (XOR == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r0 = r[0]; r1 = r[1];
  } else {
    static_assert(XOR == 16, "lane distance 16 or 32");
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r0 = r[0]; r1 = r[1];
  }
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// Global loads of 16 bytes with no alias assumptions.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Load of a value the kernel never writes (block tables, context lengths,
// scales), through the constant address space. Where the address is
// wave-uniform this is a scalar load, counted apart from the vector loads:
// a kernel that also stores to global memory otherwise gets a vector load plus
// a move to a scalar register, and its wait for that load also waits for every
// vector load issued before it.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

}  // namespace pa

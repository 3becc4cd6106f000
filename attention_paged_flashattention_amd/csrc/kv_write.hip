// Quantize-on-write of new K/V tokens into the block-paged cache.
//
// FP8 KV cache formats: "1Cat-vLLM 1.0.0" README, "Optional experimental
// feature: FP8 KV cache" (E5M2) and "SM70 release profile and acceleration
// status" (E4M3 for the release profile). Reused pages are never assumed to be
// clean ("1Cat-vLLM 1.5.0" notes, "Reliability and correctness fixes": newly
// reused KV blocks are zeroed before attention): every slot a token maps to is
// overwritten in full, and the attention kernels never read a slot past the
// context.
//
// Quantization: x / scale as the correctly rounded fp32 quotient (from the
// scale's reciprocal and one fma correction where that is exact, a division
// elsewhere: pa_divide.h), then the fp32 value to
// FP8 by gfx950's packed conversion after a clamp to the largest finite value
// (round to nearest even, saturating, sign kept).
//
// Large writes (prefill chunks) with head_dim 64 or 128: a work-group per 64
// tokens of one head, reading whole source rows and transposing the value
// codes through LDS (the row kernel). Other head sizes: each thread quantizes
// 16 consecutive dimensions of one token. Small writes (a decode or verify
// step): each thread quantizes 4 dimensions.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// 4 source elements (8 bytes) -> 4 FP8 codes.
template <int ST, int FMT>
__device__ __forceinline__ uint32_t encode4(u32x2 w, bool scaled, const Divisor& div) {
  float x[4], y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = src_to_f32<ST>((uint16_t)((i < 2 ? w.x : w.y) >> ((i & 1) * 16)));
    y[i] = x[i];
  }
  if (scaled) divide_n<4>(y, x, div);   // x / scale, correctly rounded
  return fp8x4_from_f32<FMT>(y[0], y[1], y[2], y[3]);
}

// One 16-element chunk c of token t, head h: K row (16 contiguous codes) and
// 16 value codes (one per dimension row of the page).
template <int ST, int FMT>
__device__ __forceinline__ void write_chunk(const WriteArgs& a, int64_t t, int h, int c) {
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  const int D = a.head_dim;
  const uint16_t* ksrc = a.key + (t * a.num_kv_heads + h) * D + c * 16;
  const uint16_t* vsrc = a.value + (t * a.num_kv_heads + h) * D + c * 16;
  // source and scale loads first: they do not depend on the slot
  u32x4 kr0 = ld16(ksrc), kr1 = ld16(ksrc + 8);
  u32x4 vr0 = ld16(vsrc), vr1 = ld16(vsrc + 8);
  const bool ksc = a.k_scale != nullptr, vsc = a.v_scale != nullptr;
  const float kdiv = ksc ? a.k_scale[h] : 1.0f;
  const float vdiv = vsc ? a.v_scale[h] : 1.0f;
  const Divisor kd = make_divisor(kdiv), vd = make_divisor(vdiv);
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t page = slot >> a.bs_log2;
  const int64_t off = slot & ((1 << a.bs_log2) - 1);
  const int64_t bs = (int64_t)1 << a.bs_log2;
  const int64_t ph = page * a.num_kv_heads + h;
  uint8_t* kdst = a.key_cache + ((ph * bs + off) * D + c * 16) * ES;   // token row, contiguous
  // values: dimension-major inside groups of T = min(bs, 64) tokens
  const int vg_log2 = a.bs_log2 < 6 ? a.bs_log2 : 6;
  const int64_t T = (int64_t)1 << vg_log2;
  uint8_t* vdst = a.value_cache +
      ((((ph << (a.bs_log2 - vg_log2)) + (off >> vg_log2)) * D + c * 16) * T + (off & (T - 1))) * ES;

  if constexpr (FMT == KV_F16) {
    // plain copy of fp16 sources
    *reinterpret_cast<u32x4*>(kdst) = kr0;
    *reinterpret_cast<u32x4*>(kdst + 16) = kr1;
    const uint32_t vw[8] = {vr0.x, vr0.y, vr0.z, vr0.w, vr1.x, vr1.y, vr1.z, vr1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      reinterpret_cast<uint16_t*>(vdst)[(int64_t)i * T] = (uint16_t)(vw[i >> 1] >> ((i & 1) * 16));
  } else {
    const u32x4 k0 = encode8<ST, FMT>(kr0, ksc, kd), k1 = encode8<ST, FMT>(kr1, ksc, kd);
    *reinterpret_cast<u32x4*>(kdst) = u32x4{k0.x, k0.y, k1.x, k1.y};
    const u32x4 v0 = encode8<ST, FMT>(vr0, vsc, vd), v1 = encode8<ST, FMT>(vr1, vsc, vd);
    const uint32_t vw[4] = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
    for (int i = 0; i < 16; ++i) vdst[(int64_t)i * T] = (uint8_t)(vw[i >> 2] >> ((i & 3) * 8));
  }
}

// Many tokens: work-group = 64 consecutive tokens of one head, lane i owns
// token t0 + i, so a wave's value stores for one dimension hit consecutive slots.
template <int ST, int FMT>
__global__ __launch_bounds__(256) void kv_write_tokens_kernel(const WriteArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  if (t >= a.num_tokens) return;
  for (int c = threadIdx.x >> 6; c < a.head_dim / 16; c += 4) write_chunk<ST, FMT>(a, t, blockIdx.y, c);
}

// Many tokens, the row form: work-group = 64 consecutive tokens of one KV
// head. Source rows are read whole (16 bytes per thread, consecutive threads
// on consecutive bytes) and key codes go straight to their rows. Value codes
// are transposed through LDS: when the 64 slots are consecutive and start a
// 64-token value group (a prefill chunk's usual case) the group's D x 64 codes
// are one contiguous block and leave with 16-byte stores; otherwise each code
// goes to its own slot.
constexpr int kRowTokens = 64;

// Element index of (dimension d, token tok) in the LDS transpose: [D][64],
// each row rotated by 4 (d / 8) tokens. A chunk's writes put the 8 dimensions
// ch*8 .. ch*8+7 of one token, and the lanes of a wave hold 16 (or 8) chunks
// ch of the same token: unrotated, those land 512 bytes apart, all in one LDS
// bank; the rotation spreads them over 16 banks. Rotations are whole dwords,
// so a dword of the row still holds consecutive tokens.
__device__ __forceinline__ int vt_pos(int d, int tok) {
  return d * kRowTokens + ((tok + 4 * (d >> 3)) & (kRowTokens - 1));
}

template <int ST, int FMT, int D>
__global__ __launch_bounds__(256) void kv_write_rows_kernel(const WriteArgs a) {
  constexpr int cpt = D / 8;                        // 16-byte source chunks per token
  constexpr int kRowIters = kRowTokens * cpt / 256;  // chunks per thread
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t vt[];   // [D][64] value codes
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kRowTokens;
  const int ntok = (int)min<int64_t>(kRowTokens, a.num_tokens - t0);
  const bool ksc = a.k_scale != nullptr, vsc = a.v_scale != nullptr;
  const float kdiv = ksc ? ld_const(a.k_scale, h) : 1.0f;
  const float vdiv = vsc ? ld_const(a.v_scale, h) : 1.0f;
  const Divisor kd = make_divisor(kdiv), vd = make_divisor(vdiv);
  const int bs_mask = (1 << a.bs_log2) - 1;

  // Every load of the work-group first, unconditionally: a chunk of a token
  // past the end re-reads the last token (its codes are not stored), and the
  // slots the contiguity check below needs come with them. One wait then
  // covers all loads, and no load waits behind a store (the stores could
  // alias the sources as far as the compiler knows).
  constexpr int nf = kRowTokens * cpt;
  static_assert(nf % 256 == 0, "whole chunks per thread");
  const int i = threadIdx.x;
  u32x4 kr[kRowIters], vr[kRowIters];
  int64_t sl[kRowIters];
#pragma unroll
  for (int it = 0; it < kRowIters; ++it) {
    const int f = i + 256 * it;
    const int tok = f / cpt, ch = f - tok * cpt;
    const int64_t t = t0 + min(tok, ntok - 1);
    const int64_t src = (t * a.num_kv_heads + h) * D + ch * 8;
    kr[it] = ld16(a.key + src);
    vr[it] = ld16(a.value + src);
    sl[it] = a.slots[t];
  }
  const int64_t s0 = ld_const(a.slots, t0);
  // the slot of token i % 64: the one token whose value codes this thread
  // stores when the slots are not one contiguous group (256 threads, 64 tokens)
  const int64_t my_slot = a.slots[t0 + min(i & (kRowTokens - 1), ntok - 1)];
  // All loaded values are consumed here (an empty asm statement), so the
  // compiler waits for them once and cannot sink a load into the conditional
  // key store that alone uses it. Then all conversions, then the stores.
#pragma unroll
  for (int it = 0; it < kRowIters; ++it) asm volatile("" ::"v"(kr[it]), "v"(vr[it]), "v"(sl[it]));
  asm volatile("" ::"v"(my_slot));
  u32x4 kc[kRowIters], vc[kRowIters];
#pragma unroll
  for (int it = 0; it < kRowIters; ++it) {
    kc[it] = encode8<ST, FMT>(kr[it], ksc, kd);
    vc[it] = encode8<ST, FMT>(vr[it], vsc, vd);
  }
#pragma unroll
  for (int it = 0; it < kRowIters; ++it) {
    const int f = i + 256 * it;
    const int tok = f / cpt, ch = f - tok * cpt;
    const int64_t slot = sl[it];
    if (tok < ntok && slot >= 0) {
      const int64_t ph = (slot >> a.bs_log2) * a.num_kv_heads + h;
      uint8_t* kdst = a.key_cache + (((ph << a.bs_log2) + (slot & bs_mask)) * D + ch * 8) * ES;
      if constexpr (ES == 2) *reinterpret_cast<u32x4*>(kdst) = kc[it];
      else *reinterpret_cast<u32x2*>(kdst) = u32x2{kc[it].x, kc[it].y};
    }
    // value codes to the LDS transpose (cells of tokens past the end are
    // never read)
    const uint32_t vw[4] = {vc[it].x, vc[it].y, vc[it].z, vc[it].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint8_t* cell = vt + vt_pos(ch * 8 + e, tok) * ES;
      if constexpr (ES == 2) *reinterpret_cast<uint16_t*>(cell) = (uint16_t)(vw[e >> 1] >> ((e & 1) * 16));
      else *cell = (uint8_t)(vw[e >> 2] >> ((e & 3) * 8));
    }
  }
  // one contiguous value block when the 64 slots are consecutive from the
  // start of a value group
  const bool mine = i >= kRowTokens || (i < ntok && my_slot == s0 + i);
  const bool block = __syncthreads_and(mine) && ntok == kRowTokens && a.bs_log2 >= 6 &&
                     s0 >= 0 && (s0 & (kRowTokens - 1)) == 0;
  if (block) {
    const int64_t ph = (s0 >> a.bs_log2) * a.num_kv_heads + h;
    uint8_t* vdst = a.value_cache +
        (((ph << (a.bs_log2 - 6)) + ((s0 & bs_mask) >> 6)) * D) * kRowTokens * ES;
    constexpr int per_row = kRowTokens * ES / 16;   // 16-byte chunks per dimension row
    constexpr int tpd = 4 / ES;                      // tokens per dword
    const int n16 = D * per_row;
    for (int f = threadIdx.x; f < n16; f += 256) {
      const int d = f / per_row, tok = (f - d * per_row) * (16 / ES);
      uint32_t w4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w4[q] = *reinterpret_cast<const uint32_t*>(vt + vt_pos(d, tok + q * tpd) * ES);
      reinterpret_cast<u32x4*>(vdst)[f] = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
  } else {
    const int vg_log2 = a.bs_log2 < 6 ? a.bs_log2 : 6;
    const int T = 1 << vg_log2;
    static_assert(256 % kRowTokens == 0, "a thread keeps one token");
    const int tok = i & (kRowTokens - 1);
    if (tok < ntok && my_slot >= 0) {
      const int64_t ph = (my_slot >> a.bs_log2) * a.num_kv_heads + h;
      const int off = (int)(my_slot & bs_mask);
      uint8_t* vbase = a.value_cache +
          (((ph << (a.bs_log2 - vg_log2)) + (off >> vg_log2)) * D * T + (off & (T - 1))) * ES;
      for (int d = i / kRowTokens; d < D; d += 256 / kRowTokens) {
        const int idx = vt_pos(d, tok);
        uint8_t* vdst = vbase + (int64_t)d * T * ES;
        if constexpr (ES == 2) *reinterpret_cast<uint16_t*>(vdst) = *reinterpret_cast<const uint16_t*>(vt + idx * 2);
        else *vdst = vt[idx];
      }
    }
  }
}

// Slot of new token t when the slots come from the block table: token
// t % q_len of sequence t / q_len sits at position ctx - q_len + t % q_len
// (-1, not written, before the sequence start).
__device__ __forceinline__ int64_t derived_slot(const WriteArgs& a, int t) {
  const int b = t / a.q_len;
  const int pos = a.context_lens[b] - a.q_len + (t - b * a.q_len);
  if (pos < 0) return -1;
  const int64_t page = a.block_tables[(int64_t)b * a.max_blocks + (pos >> a.bs_log2)];
  return (page << a.bs_log2) | (pos & ((1 << a.bs_log2) - 1));
}

// Four dimensions [4q, 4q + 4) of token t, head h: 4 key codes (one store)
// and 4 value codes (one per dimension row of the value group). DERIVED: the
// slot comes from the block table instead of the slot mapping.
template <int ST, int FMT, bool DERIVED = false>
__device__ __forceinline__ void write_quad(const WriteArgs& a, int t, int h, int q) {
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  // The source values and the scale do not depend on the slot: their loads
  // are issued together with the slot's, so the write costs one round trip.
  const int D = a.head_dim;
  const int64_t src = ((int64_t)t * a.num_kv_heads + h) * D + 4 * q;
  const u32x2 kr = *reinterpret_cast<const u32x2*>(a.key + src);
  const u32x2 vr = *reinterpret_cast<const u32x2*>(a.value + src);
  const bool ksc = a.k_scale != nullptr, vsc = a.v_scale != nullptr;
  const float kdiv = ksc ? a.k_scale[h] : 1.0f;
  const float vdiv = vsc ? a.v_scale[h] : 1.0f;
  const Divisor kd = make_divisor(kdiv), vd = make_divisor(vdiv);
  const int64_t slot = DERIVED ? derived_slot(a, t) : a.slots[t];
  if (slot < 0) return;
  const int64_t page = slot >> a.bs_log2;
  const int off = (int)(slot & ((1 << a.bs_log2) - 1));
  const int64_t ph = page * a.num_kv_heads + h;
  uint8_t* kdst = a.key_cache + ((ph << a.bs_log2) + off) * D * ES + 4 * q * ES;
  const int vg_log2 = a.bs_log2 < 6 ? a.bs_log2 : 6;
  const int T = 1 << vg_log2;
  uint8_t* vdst = a.value_cache +
      ((((ph << (a.bs_log2 - vg_log2)) + (off >> vg_log2)) * D + 4 * q) * T + (off & (T - 1))) * ES;
  if constexpr (FMT == KV_F16) {
    *reinterpret_cast<u32x2*>(kdst) = kr;
    uint16_t* vd = reinterpret_cast<uint16_t*>(vdst);
    vd[0] = (uint16_t)vr.x;
    vd[T] = (uint16_t)(vr.x >> 16);
    vd[2 * T] = (uint16_t)vr.y;
    vd[3 * T] = (uint16_t)(vr.y >> 16);
  } else {
    *reinterpret_cast<uint32_t*>(kdst) = encode4<ST, FMT>(kr, ksc, kd);
    const uint32_t vcode = encode4<ST, FMT>(vr, vsc, vd);
#pragma unroll
    for (int i = 0; i < 4; ++i) vdst[i * T] = (uint8_t)(vcode >> (i * 8));
  }
}

// Few tokens (a decode or verify step): one thread per four dimensions of one
// token and head, so all of a step's conversions run side by side.
template <int ST, int FMT>
__global__ __launch_bounds__(256) void kv_write_chunks_kernel(const WriteArgs a) {
  const int nq = a.head_dim / 4;
  const int id = blockIdx.x * 256 + threadIdx.x;
  const int per_token = nq * a.num_kv_heads;
  if (id >= (int)a.num_tokens * per_token) return;
  const int t = id / per_token;
  const int r = id - t * per_token;
  write_quad<ST, FMT>(a, t, r / nq, r % nq);
}

// The append form of the same kernel: slots from the block table.
template <int ST, int FMT>
__global__ __launch_bounds__(256) void kv_append_kernel(const WriteArgs a) {
  const int nq = a.head_dim / 4;
  const int id = blockIdx.x * 256 + threadIdx.x;
  const int per_token = nq * a.num_kv_heads;
  if (id >= (int)a.num_tokens * per_token) return;
  const int t = id / per_token;
  const int r = id - t * per_token;
  write_quad<ST, FMT, true>(a, t, r / nq, r % nq);
}

constexpr int64_t kFewTokens = 64;

template <int ST, int FMT>
static hipError_t launch_write(const WriteArgs& a, hipStream_t s, const ProfileEvents& ev) {
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  const size_t rows_lds = (size_t)a.head_dim * kRowTokens * ES;
  if (a.num_tokens < kFewTokens) {
    const int64_t total = a.num_tokens * a.num_kv_heads * (a.head_dim / 4);
    return launch_kernel(kv_write_chunks_kernel<ST, FMT>, dim3((unsigned)((total + 255) / 256)),
                         dim3(256), 0, s, ev, a);
  } else if (a.head_dim == 64 || a.head_dim == 128) {
    dim3 grid((unsigned)((a.num_tokens + kRowTokens - 1) / kRowTokens), (unsigned)a.num_kv_heads);
    if (a.head_dim == 64)
      return launch_kernel(kv_write_rows_kernel<ST, FMT, 64>, grid, dim3(256), (uint32_t)rows_lds,
                           s, ev, a);
    return launch_kernel(kv_write_rows_kernel<ST, FMT, 128>, grid, dim3(256), (uint32_t)rows_lds,
                         s, ev, a);
  }
  dim3 grid((unsigned)((a.num_tokens + 63) / 64), (unsigned)a.num_kv_heads);
  return launch_kernel(kv_write_tokens_kernel<ST, FMT>, grid, dim3(256), 0, s, ev, a);
}

hipError_t launch_kv_write(const WriteArgs& a, int src_is_bf16, int fmt, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const ProfileEvents ev = take_profile_events();
  if (fmt == KV_F16) return launch_write<Q_F16, KV_F16>(a, stream, ev);
  if (fmt == KV_E4M3)
    return src_is_bf16 ? launch_write<Q_BF16, KV_E4M3>(a, stream, ev)
                       : launch_write<Q_F16, KV_E4M3>(a, stream, ev);
  return src_is_bf16 ? launch_write<Q_BF16, KV_E5M2>(a, stream, ev)
                     : launch_write<Q_F16, KV_E5M2>(a, stream, ev);
}

template <int ST, int FMT>
static hipError_t launch_append(const WriteArgs& a, hipStream_t s) {
  const int64_t total = a.num_tokens * a.num_kv_heads * (a.head_dim / 4);
  return launch_kernel(kv_append_kernel<ST, FMT>, dim3((unsigned)((total + 255) / 256)),
                       dim3(256), 0, s, ProfileEvents{}, a);
}

hipError_t launch_kv_append(const WriteArgs& a, int src_is_bf16, int fmt, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  if (fmt == KV_F16) return launch_append<Q_F16, KV_F16>(a, stream);
  if (fmt == KV_E4M3)
    return src_is_bf16 ? launch_append<Q_BF16, KV_E4M3>(a, stream)
                       : launch_append<Q_F16, KV_E4M3>(a, stream);
  return src_is_bf16 ? launch_append<Q_BF16, KV_E5M2>(a, stream)
                     : launch_append<Q_F16, KV_E5M2>(a, stream);
}

}  // namespace pa

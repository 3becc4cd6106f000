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
// Large writes (prefill chunks): each thread quantizes 16 consecutive head
// dimensions of one token's K and V, consecutive tokens on consecutive lanes.
// Small writes (a decode or verify step): each thread quantizes 4 dimensions.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

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
    const uint32_t kw[8] = {kr0.x, kr0.y, kr0.z, kr0.w, kr1.x, kr1.y, kr1.z, kr1.w};
    const uint32_t vw[8] = {vr0.x, vr0.y, vr0.z, vr0.w, vr1.x, vr1.y, vr1.z, vr1.w};
    uint32_t kout[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = src_to_f32<ST>((uint16_t)(kw[i >> 1] >> ((i & 1) * 16)));
      const float y = ksc ? x / kdiv : x;   // IEEE fp32 division (correctly rounded)
      const uint32_t code = FMT == KV_E4M3 ? f32_to_e4m3(y) : f32_to_e5m2(y);
      kout[i >> 2] |= code << ((i & 3) * 8);
    }
    *reinterpret_cast<u32x4*>(kdst) = u32x4{kout[0], kout[1], kout[2], kout[3]};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = src_to_f32<ST>((uint16_t)(vw[i >> 1] >> ((i & 1) * 16)));
      const float y = vsc ? x / vdiv : x;
      const uint32_t code = FMT == KV_E4M3 ? f32_to_e4m3(y) : f32_to_e5m2(y);
      vdst[(int64_t)i * T] = (uint8_t)code;
    }
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

// Four dimensions [4q, 4q + 4) of token t, head h: 4 key codes (one store)
// and 4 value codes (one per dimension row of the value group).
template <int ST, int FMT>
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
  const int64_t slot = a.slots[t];
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
    const uint32_t kw[2] = {kr.x, kr.y}, vw[2] = {vr.x, vr.y};
    uint32_t kout = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = src_to_f32<ST>((uint16_t)(kw[i >> 1] >> ((i & 1) * 16)));
      const float y = ksc ? x / kdiv : x;   // IEEE fp32 division (correctly rounded)
      kout |= (FMT == KV_E4M3 ? f32_to_e4m3(y) : f32_to_e5m2(y)) << (i * 8);
    }
    *reinterpret_cast<uint32_t*>(kdst) = kout;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = src_to_f32<ST>((uint16_t)(vw[i >> 1] >> ((i & 1) * 16)));
      const float y = vsc ? x / vdiv : x;
      vdst[i * T] = (uint8_t)(FMT == KV_E4M3 ? f32_to_e4m3(y) : f32_to_e5m2(y));
    }
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

constexpr int64_t kFewTokens = 64;

template <int ST, int FMT>
static void launch_write(const WriteArgs& a, hipStream_t s) {
  if (a.num_tokens < kFewTokens) {
    const int64_t total = a.num_tokens * a.num_kv_heads * (a.head_dim / 4);
    hipLaunchKernelGGL((kv_write_chunks_kernel<ST, FMT>), dim3((unsigned)((total + 255) / 256)),
                       dim3(256), 0, s, a);
  } else {
    dim3 grid((unsigned)((a.num_tokens + 63) / 64), (unsigned)a.num_kv_heads);
    hipLaunchKernelGGL((kv_write_tokens_kernel<ST, FMT>), grid, dim3(256), 0, s, a);
  }
}

hipError_t launch_kv_write(const WriteArgs& a, int src_is_bf16, int fmt, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const ProfileEvents ev = take_profile_events();
  record_if(ev.start, stream);
  if (fmt == KV_F16) launch_write<Q_F16, KV_F16>(a, stream);
  else if (fmt == KV_E4M3) {
    if (src_is_bf16) launch_write<Q_BF16, KV_E4M3>(a, stream);
    else launch_write<Q_F16, KV_E4M3>(a, stream);
  } else {
    if (src_is_bf16) launch_write<Q_BF16, KV_E5M2>(a, stream);
    else launch_write<Q_F16, KV_E5M2>(a, stream);
  }
  record_if(ev.stop, stream);
  return hipGetLastError();
}

}  // namespace pa

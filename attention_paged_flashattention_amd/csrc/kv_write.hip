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
// Each thread quantizes 16 consecutive head dimensions of one token's K and V.
// Large writes (prefill chunks) put consecutive tokens on consecutive lanes;
// small writes (a decode step) put every chunk of every head on its own thread.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// One 16-element chunk c of token t, head h: K row (16 contiguous codes) and
// 16 value codes (one per dimension row of the page).
template <int ST, int FMT>
__device__ __forceinline__ void write_chunk(const WriteArgs& a, int64_t t, int h, int c) {
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t page = slot >> a.bs_log2;
  const int64_t off = slot & ((1 << a.bs_log2) - 1);
  const int D = a.head_dim;
  const int64_t bs = (int64_t)1 << a.bs_log2;
  const uint16_t* ksrc = a.key + (t * a.num_kv_heads + h) * D + c * 16;
  const uint16_t* vsrc = a.value + (t * a.num_kv_heads + h) * D + c * 16;
  const int64_t ph = page * a.num_kv_heads + h;
  uint8_t* kdst = a.key_cache + ((ph * bs + off) * D + c * 16) * ES;   // token row, contiguous
  // values: dimension-major inside groups of T = min(bs, 64) tokens
  const int vg_log2 = a.bs_log2 < 6 ? a.bs_log2 : 6;
  const int64_t T = (int64_t)1 << vg_log2;
  uint8_t* vdst = a.value_cache +
      ((((ph << (a.bs_log2 - vg_log2)) + (off >> vg_log2)) * D + c * 16) * T + (off & (T - 1))) * ES;

  u32x4 kr0 = ld16(ksrc), kr1 = ld16(ksrc + 8);
  u32x4 vr0 = ld16(vsrc), vr1 = ld16(vsrc + 8);
  if constexpr (FMT == KV_F16) {
    // plain copy of fp16 sources
    *reinterpret_cast<u32x4*>(kdst) = kr0;
    *reinterpret_cast<u32x4*>(kdst + 16) = kr1;
    const uint32_t vw[8] = {vr0.x, vr0.y, vr0.z, vr0.w, vr1.x, vr1.y, vr1.z, vr1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      reinterpret_cast<uint16_t*>(vdst)[(int64_t)i * T] = (uint16_t)(vw[i >> 1] >> ((i & 1) * 16));
  } else {
    const bool ksc = a.k_scale != nullptr, vsc = a.v_scale != nullptr;
    const float kdiv = ksc ? a.k_scale[h] : 1.0f;
    const float vdiv = vsc ? a.v_scale[h] : 1.0f;
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

// Few tokens (a decode or verify step): one thread per 16-element chunk, all
// chunks of all heads in flight at once.
template <int ST, int FMT>
__global__ __launch_bounds__(256) void kv_write_chunks_kernel(const WriteArgs a) {
  const int nc = a.head_dim / 16;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = a.num_tokens * a.num_kv_heads * nc;
  if (id >= total) return;
  const int c = (int)(id % nc);
  const int h = (int)((id / nc) % a.num_kv_heads);
  const int64_t t = id / ((int64_t)nc * a.num_kv_heads);
  write_chunk<ST, FMT>(a, t, h, c);
}

constexpr int64_t kFewTokens = 64;

template <int ST, int FMT>
static void launch_write(const WriteArgs& a, hipStream_t s) {
  if (a.num_tokens < kFewTokens) {
    const int64_t total = a.num_tokens * a.num_kv_heads * (a.head_dim / 16);
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

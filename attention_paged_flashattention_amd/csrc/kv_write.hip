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
// One work-group covers 64 consecutive tokens of one KV head; lane i of each
// wave owns token t0 + i and 16 consecutive head dimensions per step, so a
// wave's value-cache byte stores for one dimension land on consecutive slots.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int ST, int FMT>
__global__ __launch_bounds__(256) void kv_write_kernel(const WriteArgs a) {
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int h = blockIdx.y;
  if (t >= a.num_tokens) return;
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t page = slot >> a.bs_log2;
  const int64_t off = slot & ((1 << a.bs_log2) - 1);
  const int D = a.head_dim;
  const int64_t bs = (int64_t)1 << a.bs_log2;

  const uint16_t* ksrc = a.key + (t * a.num_kv_heads + h) * D;
  const uint16_t* vsrc = a.value + (t * a.num_kv_heads + h) * D;
  const int64_t ph = page * a.num_kv_heads + h;
  uint8_t* kdst = a.key_cache + ((ph * bs + off) * D) * ES;   // token row, contiguous D
  uint8_t* vdst = a.value_cache + ((ph * D) * bs + off) * ES;  // column: stride bs per dim

  const bool ksc = a.k_scale != nullptr, vsc = a.v_scale != nullptr;
  const float kdiv = ksc ? a.k_scale[h] : 1.0f;
  const float vdiv = vsc ? a.v_scale[h] : 1.0f;

  for (int c = threadIdx.x >> 6; c < D / 16; c += 4) {
    u32x4 kr0 = ld16(ksrc + c * 16), kr1 = ld16(ksrc + c * 16 + 8);
    u32x4 vr0 = ld16(vsrc + c * 16), vr1 = ld16(vsrc + c * 16 + 8);
    uint32_t kw[8] = {kr0.x, kr0.y, kr0.z, kr0.w, kr1.x, kr1.y, kr1.z, kr1.w};
    uint32_t vw[8] = {vr0.x, vr0.y, vr0.z, vr0.w, vr1.x, vr1.y, vr1.z, vr1.w};
    if constexpr (FMT == KV_F16) {
      // plain copy of fp16 sources
      *reinterpret_cast<u32x4*>(kdst + (c * 16) * ES) = kr0;
      *reinterpret_cast<u32x4*>(kdst + (c * 16 + 8) * ES) = kr1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint16_t e = (uint16_t)(vw[i >> 1] >> ((i & 1) * 16));
        reinterpret_cast<uint16_t*>(vdst)[(int64_t)(c * 16 + i) * bs] = e;
      }
    } else {
      uint32_t kout[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = src_to_f32<ST>((uint16_t)(kw[i >> 1] >> ((i & 1) * 16)));
        float y = ksc ? x / kdiv : x;   // IEEE fp32 division (correctly rounded)
        uint32_t code = FMT == KV_E4M3 ? f32_to_e4m3(y) : f32_to_e5m2(y);
        kout[i >> 2] |= code << ((i & 3) * 8);
      }
      *reinterpret_cast<u32x4*>(kdst + c * 16) = u32x4{kout[0], kout[1], kout[2], kout[3]};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = src_to_f32<ST>((uint16_t)(vw[i >> 1] >> ((i & 1) * 16)));
        float y = vsc ? x / vdiv : x;
        uint32_t code = FMT == KV_E4M3 ? f32_to_e4m3(y) : f32_to_e5m2(y);
        vdst[(int64_t)(c * 16 + i) * bs] = (uint8_t)code;
      }
    }
  }
}

hipError_t launch_kv_write(const WriteArgs& a, int src_is_bf16, int fmt, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const ProfileEvents ev = take_profile_events();
  record_if(ev.start, stream);
  dim3 grid((unsigned)((a.num_tokens + 63) / 64), (unsigned)a.num_kv_heads);
  dim3 block(256);
  if (fmt == KV_F16) {
    hipLaunchKernelGGL((kv_write_kernel<Q_F16, KV_F16>), grid, block, 0, stream, a);
  } else if (fmt == KV_E4M3) {
    if (src_is_bf16)
      hipLaunchKernelGGL((kv_write_kernel<Q_BF16, KV_E4M3>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((kv_write_kernel<Q_F16, KV_E4M3>), grid, block, 0, stream, a);
  } else {
    if (src_is_bf16)
      hipLaunchKernelGGL((kv_write_kernel<Q_BF16, KV_E5M2>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((kv_write_kernel<Q_F16, KV_E5M2>), grid, block, 0, stream, a);
  }
  record_if(ev.stop, stream);
  return hipGetLastError();
}

}  // namespace pa

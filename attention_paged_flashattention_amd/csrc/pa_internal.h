// Host-side internal interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct WriteArgs {
  const uint16_t* key;
  const uint16_t* value;
  const int64_t* slots;
  int64_t num_tokens;
  uint8_t* key_cache;
  uint8_t* value_cache;
  const float* k_scale;  // may be null (E5M2 without scales, F16)
  const float* v_scale;
  int num_kv_heads;
  int head_dim;
  int bs_log2;
  // Slots derived from the block table (kv_append_kernel only): token t is
  // new token t % q_len of sequence t / q_len, at position ctx - q_len + i.
  const int32_t* block_tables;
  const int32_t* context_lens;
  int max_blocks;
  int q_len;
};

// Split-KV decode / grouped verify.
struct DecodeArgs {
  const uint16_t* q;        // [batch][q_len][Hq][D]
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  float* ws_ml;             // [rows][P][2]  (running max in log2 units, sum)
  float* ws_o;              // [rows][P][D]  (unnormalised partial output)
  void* out;                // [rows][D]
  int max_blocks;
  int q_len;
  int num_q_heads;
  int num_kv_heads;
  int bs_log2;
  int part_len;             // tokens per partition, a multiple of 64
  int num_parts;
  int window;               // -1: causal rows; W >= 0: non-causal window of W keys
  float softmax_scale;
  // Fused quantize-on-write (null k_new: none): the q_len new tokens of each
  // sequence, [batch][q_len][Hkv][D] in the query dtype, are written at their
  // positions ctx - q_len + i before they are attended.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* key_cache_w;     // the caches above, for the fused write
  uint8_t* value_cache_w;
  int out_type;             // OType of out (stored by the split kernel when num_parts == 1)
};

struct PrefillArgs {
  const uint16_t* q;        // [total_q][Hq][D]
  const int32_t* cu_seqlens;
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  void* out;                // [total_q][Hq][D]
  int batch;
  int max_blocks;
  int num_q_heads;
  int num_kv_heads;
  int bs_log2;
  int q_blocks;             // query tiles per sequence in the grid
  float softmax_scale;
};

// Events to record around the next main-kernel launch on this thread (the
// profiling hook); both null when none is pending.
struct ProfileEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
ProfileEvents take_profile_events();

// Launches kernel(a) on stream s and returns the launch's own status (the
// caller stops at the first failure; no error state left over from earlier
// HIP calls is read). With profiling events pending they are attached to this
// kernel's own dispatch (hipExtLaunchKernel), so the pair times the kernel
// alone, without the latency of separate marker packets.
template <typename Arg>
[[nodiscard]] inline hipError_t launch_kernel(void (*kernel)(Arg), dim3 grid, dim3 block,
                                              uint32_t shmem, hipStream_t s,
                                              const ProfileEvents& ev, const Arg& a) {
  void* args[] = {const_cast<Arg*>(&a)};
  const void* fn = reinterpret_cast<const void*>(kernel);
  if (ev.start && ev.stop)
    return hipExtLaunchKernel(fn, grid, block, args, shmem, s, ev.start, ev.stop, 0);
  return hipLaunchKernel(fn, grid, block, args, shmem, s);
}

hipError_t launch_kv_write(const WriteArgs& a, int src_is_bf16, int fmt, hipStream_t stream);

// The newest q_len tokens of each sequence written at their own positions
// (slots from the block table); records no profiling events.
hipError_t launch_kv_append(const WriteArgs& a, int src_is_bf16, int fmt, hipStream_t stream);

// fmt: KvFmt, qt: QType, ot: OType. nqb: number of 16-row query blocks.
hipError_t launch_decode(const DecodeArgs& a, int batch, int head_dim, int fmt, int qt,
                         int ot, int nqb, hipStream_t stream);

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int fmt, int qt, int ot,
                          hipStream_t stream);

// Rows of the prefill work-group tile (query tokens x heads of one KV group)
// and its threads (8 waves of 32 rows).
constexpr int kPrefillRows = 256;
constexpr int kPrefillThreads = 512;

}  // namespace pa

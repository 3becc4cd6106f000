// C ABI of the paged-attention library: argument checks, capability table,
// workspace sizing and dispatch to the HIP kernels.
//
// Each entry point checks its own contract -- dtypes, head shape, KV format,
// batch shape -- before launching anything, and reports an unsupported
// combination as PA_ERR_UNSUPPORTED so the caller can fall back for that one
// operator ("1Cat-vLLM 1.5.0" RELEASE notes: each verifier operator checks its
// own dtype, TP shape, KV format and live batch shape and falls back
// independently; capability is checked before dispatch instead of failing in
// the engine). Nothing here synchronizes, allocates or reads device memory,
// except the explicit debug check pa_validate_tables.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pagedattn.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local pa::ProfileEvents g_profile;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

int cache_fmt(pa_dtype d) {
  switch (d) {
    case PA_F16: return pa::KV_F16;
    case PA_FP8_E4M3: return pa::KV_E4M3;
    case PA_FP8_E5M2: return pa::KV_E5M2;
    default: return -1;
  }
}

int q_type(pa_dtype d) {
  switch (d) {
    case PA_F16: return pa::Q_F16;
    case PA_BF16: return pa::Q_BF16;
    default: return -1;
  }
}

int out_type(pa_dtype d) {
  switch (d) {
    case PA_F32: return pa::O_F32;
    case PA_F16: return pa::O_F16;
    case PA_BF16: return pa::O_BF16;
    default: return -1;
  }
}

constexpr int kMinBlock = 16;
constexpr int kMaxBlock = 1 << 16;
constexpr int kMaxRows = 64;       // q_len * G of one decode/verify group
// Query heads per KV head in prefill: a work-group's 256 rows hold
// floor(256 / G) whole tokens (the last 256 mod G rows idle), at least 4.
constexpr int kMaxPrefillGroup = 64;
constexpr int kTile = 64;          // keys per decode tile
constexpr int kMaxParts = 4096;

// Checks shared by the three attention calls. Returns PA_OK or the failure.
pa_status check_common(const void* q, pa_dtype q_dtype, const void* kc, const void* vc,
                       pa_dtype cache_dtype, int block_size, int64_t num_blocks,
                       const int32_t* block_tables, int max_blocks,
                       const int32_t* context_lens, int max_context_len, int hq, int hkv,
                       int head_dim, const float* k_scale, const float* v_scale,
                       float softmax_scale, const void* out, pa_dtype out_dtype) {
  if (!q || !kc || !vc || !block_tables || !context_lens || !out)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (hq <= 0 || hkv <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must be positive");
  if (hq % hkv != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                hq, hkv);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len %d outside [0, max_blocks_per_seq * block_size]",
                max_context_len);
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(PA_ERR_INVALID_ARG, "softmax_scale must be finite and positive");
  if (q_type(q_dtype) < 0) return fail(PA_ERR_UNSUPPORTED, "query dtype %d unsupported", q_dtype);
  if (cache_fmt(cache_dtype) < 0)
    return fail(PA_ERR_UNSUPPORTED, "cache dtype %d unsupported", cache_dtype);
  if (out_type(out_dtype) < 0) return fail(PA_ERR_UNSUPPORTED, "output dtype %d unsupported", out_dtype);
  if (cache_dtype == PA_F16 && q_dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "an fp16 cache needs fp16 queries");
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARG, "E4M3 cache needs k_scale and v_scale");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d unsupported (64, 128)", head_dim);
  if (!is_pow2(block_size) || block_size < kMinBlock || block_size > kMaxBlock)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d unsupported (power of two in [16, 65536])",
                block_size);
  if ((int64_t)num_blocks * hkv * block_size * head_dim * 2 > (int64_t(1) << 46))
    return fail(PA_ERR_INVALID_ARG, "cache too large");
  return PA_OK;
}

int auto_partitions(int batch, int q_len, int hkv, int max_ctx) {
  (void)q_len;
  const int64_t groups = (int64_t)std::max(batch, 1) * hkv;
  // Aim for one work-group per CU: fewer, longer partitions stream each
  // (page, head) run in order, which reads faster from HBM than two
  // work-groups per CU on half-length runs.
  int64_t p = (256 + groups - 1) / groups;
  const int64_t max_p = std::max<int64_t>(1, (max_ctx + 255) / 256);  // >= 256 keys each
  p = std::min(p, max_p);
  p = std::max<int64_t>(1, std::min<int64_t>(p, kMaxParts));
  return (int)p;
}

// Partition length (multiple of the tile) and the count actually launched.
void partition_shape(int requested, int max_ctx, int* part_len, int* parts) {
  int64_t len = (max_ctx + requested - 1) / std::max(requested, 1);
  len = std::max<int64_t>(kTile, (len + kTile - 1) / kTile * kTile);
  *part_len = (int)len;
  *parts = (int)std::max<int64_t>(1, (max_ctx + len - 1) / len);
}

// Keys a sequence's partitions must cover: the whole context, or with a
// window of W keys the W + q_len keys of the widest row set, plus one tile for
// rounding the start down to a tile boundary.
int key_span(int max_ctx, int q_len, int window) {
  if (window < 0) return max_ctx;
  return (int)std::min<int64_t>(max_ctx, (int64_t)window + q_len + kTile);
}

size_t ws_bytes(int64_t rows, int parts, int head_dim) {
  const size_t ml = (size_t)rows * parts * 2 * sizeof(float);
  const size_t ml_al = (ml + 255) / 256 * 256;
  return ml_al + (size_t)rows * parts * head_dim * sizeof(float);
}

// ---------------------------------------------------------------------------
// Scratch of attn_verify_paged_noalloc: the split-KV partials live in this
// file-scope device array instead of a caller's workspace. Each GPU holds its
// own copy (at its own address) until the process ends. In host code the name
// `scratch` is only a host-side stand-in: every use goes through the device
// address that hipGetSymbolAddress returns for the current device, looked up
// once per device and kept in g_scratch.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device (set-up on first use).
pa_status scratch_ptr(const char* name, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device index %d out of range", name, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", name, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PA_OK;
}

pa_status decode_like(const char* name, const void* q, pa_dtype q_dtype, int batch, int q_len,
                      const void* kc, const void* vc, pa_dtype cache_dtype, int block_size,
                      int64_t num_blocks, const int32_t* block_tables, int max_blocks,
                      const int32_t* context_lens, int max_context_len, int hq, int hkv,
                      int head_dim, const float* k_scale, const float* v_scale,
                      float softmax_scale, int num_partitions, void* workspace,
                      size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream,
                      int window = -1, const void* k_new = nullptr, const void* v_new = nullptr,
                      bool use_scratch = false) {
  if (batch < 0) return fail(PA_ERR_INVALID_ARG, "%s: batch must be >= 0", name);
  if (q_len <= 0) return fail(PA_ERR_INVALID_ARG, "%s: q_len must be positive", name);
  if (num_partitions < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_partitions must be >= 0", name);
  pa_status st = check_common(q, q_dtype, kc, vc, cache_dtype, block_size, num_blocks,
                              block_tables, max_blocks, context_lens, max_context_len, hq, hkv,
                              head_dim, k_scale, v_scale, softmax_scale, out, out_dtype);
  if (st != PA_OK) return st;
  const int G = hq / hkv;
  if ((int64_t)q_len * G > kMaxRows)
    return fail(PA_ERR_UNSUPPORTED, "%s: q_len * (num_q_heads / num_kv_heads) = %d exceeds %d",
                name, q_len * G, kMaxRows);
  if (num_partitions > kMaxParts)
    return fail(PA_ERR_UNSUPPORTED, "%s: at most %d partitions", name, kMaxParts);
  if (batch > 65535)   // a grid dimension
    return fail(PA_ERR_UNSUPPORTED, "%s: at most 65535 sequences per call", name);
  if (k_new && (int64_t)batch * q_len * hkv * (head_dim / 4) > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: too many new tokens for one call", name);
  if (batch == 0) return ok();
  const int span = key_span(max_context_len, q_len, window);
  const int req = num_partitions ? num_partitions : auto_partitions(batch, q_len, hkv, span);
  int part_len = 0, parts = 0;
  partition_shape(req, span, &part_len, &parts);
  const int64_t rows = (int64_t)batch * q_len * hq;
  const size_t need = ws_bytes(rows, parts, head_dim);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(PA_ERR_UNSUPPORTED,
                  "%s: needs %zu bytes of partials, more than the %zu-byte static scratch "
                  "(use attn_verify_paged with a workspace)", name, need, kScratchBytes);
    pa_status sst = scratch_ptr(name, &workspace);
    if (sst != PA_OK) return sst;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "%s: workspace is null", name);
  if (workspace_bytes < need)
    return fail(PA_ERR_INVALID_ARG, "%s: workspace of %zu bytes is smaller than the %zu needed",
                name, workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", name);

  pa::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.key_cache = static_cast<const uint8_t*>(kc);
  a.value_cache = static_cast<const uint8_t*>(vc);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const bool scaled = cache_dtype != PA_F16;
  a.k_scale = scaled ? k_scale : nullptr;
  a.v_scale = scaled ? v_scale : nullptr;
  const size_t ml = (size_t)rows * parts * 2 * sizeof(float);
  a.ws_ml = static_cast<float*>(workspace);
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + (ml + 255) / 256 * 256);
  a.out = out;
  a.max_blocks = max_blocks;
  a.q_len = q_len;
  a.num_q_heads = hq;
  a.num_kv_heads = hkv;
  a.bs_log2 = log2i(block_size);
  a.part_len = part_len;
  a.num_parts = parts;
  a.window = window < 0 ? -1 : std::min(window, max_context_len);
  a.out_type = out_type(out_dtype);
  a.softmax_scale = softmax_scale;
  const int nrows = q_len * G;
  const int nqb = nrows <= 16 ? 1 : (nrows <= 32 ? 2 : 4);
  hipError_t e = hipSuccess;
  if (k_new && nqb > 1) {
    // With more than one 16-row block the fused kernel's main loop compiles
    // measurably slower than the plain one, so the new tokens are written by a
    // small kernel first (same encoding, slots from the block table) and the
    // plain kernel attends.
    pa::WriteArgs w{};
    w.key = static_cast<const uint16_t*>(k_new);
    w.value = static_cast<const uint16_t*>(v_new);
    w.slots = nullptr;
    w.num_tokens = (int64_t)batch * q_len;
    w.key_cache = static_cast<uint8_t*>(const_cast<void*>(kc));
    w.value_cache = static_cast<uint8_t*>(const_cast<void*>(vc));
    w.k_scale = a.k_scale;
    w.v_scale = a.v_scale;
    w.num_kv_heads = hkv;
    w.head_dim = head_dim;
    w.bs_log2 = a.bs_log2;
    w.block_tables = block_tables;
    w.context_lens = context_lens;
    w.max_blocks = max_blocks;
    w.q_len = q_len;
    e = pa::launch_kv_append(w, q_dtype == PA_BF16, cache_fmt(cache_dtype),
                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e, name);
  } else if (k_new) {
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.key_cache_w = static_cast<uint8_t*>(const_cast<void*>(kc));
    a.value_cache_w = static_cast<uint8_t*>(const_cast<void*>(vc));
  }
  e = pa::launch_decode(a, batch, head_dim, cache_fmt(cache_dtype), q_type(q_dtype),
                        out_type(out_dtype), nqb, static_cast<hipStream_t>(stream));
  return hip_status(e, name);
}

}  // namespace

namespace pa {
ProfileEvents take_profile_events() {
  ProfileEvents e = g_profile;
  g_profile = ProfileEvents{};
  return e;
}
}  // namespace pa

extern "C" {

PA_API void pa_profile_next_call(void* start_event, void* stop_event) {
  if (!start_event || !stop_event) {
    g_profile = pa::ProfileEvents{};
    return;
  }
  g_profile.start = static_cast<hipEvent_t>(start_event);
  g_profile.stop = static_cast<hipEvent_t>(stop_event);
}

PA_API const char* pa_last_error(void) { return g_last_error.c_str(); }

PA_API const char* pa_version(void) { return "pagedattn 0.1.0 (gfx950)"; }

PA_API pa_status kv_cache_write_fp8(const void* key, const void* value, pa_dtype src_dtype,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    void* key_cache, void* value_cache, pa_dtype cache_dtype,
                                    int64_t num_blocks, int block_size, int num_kv_heads,
                                    int head_dim, const float* k_scale, const float* v_scale,
                                    void* stream) {
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "kv_cache_write_fp8: num_tokens < 0");
  if (!key || !value || !slot_mapping || !key_cache || !value_cache)
    return fail(PA_ERR_INVALID_ARG, "kv_cache_write_fp8: null pointer argument");
  if (num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PA_ERR_INVALID_ARG, "kv_cache_write_fp8: sizes must be positive");
  if (src_dtype != PA_F16 && src_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "kv_cache_write_fp8: source dtype %d unsupported", src_dtype);
  const int fmt = cache_fmt(cache_dtype);
  if (fmt < 0)
    return fail(PA_ERR_UNSUPPORTED, "kv_cache_write_fp8: cache dtype %d unsupported", cache_dtype);
  if (cache_dtype == PA_F16 && src_dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "kv_cache_write_fp8: an fp16 cache takes fp16 sources");
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARG, "kv_cache_write_fp8: E4M3 needs k_scale and v_scale");
  if (head_dim % 16 != 0 || head_dim > 1024)
    return fail(PA_ERR_UNSUPPORTED, "kv_cache_write_fp8: head_dim %d unsupported (multiple of 16)",
                head_dim);
  if (!is_pow2(block_size) || block_size < kMinBlock || block_size > kMaxBlock)
    return fail(PA_ERR_UNSUPPORTED, "kv_cache_write_fp8: block_size %d unsupported", block_size);
  if (num_kv_heads > 65535)
    return fail(PA_ERR_UNSUPPORTED, "kv_cache_write_fp8: too many KV heads");
  if (num_tokens == 0) return ok();
  pa::WriteArgs a{};
  a.key = static_cast<const uint16_t*>(key);
  a.value = static_cast<const uint16_t*>(value);
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.key_cache = static_cast<uint8_t*>(key_cache);
  a.value_cache = static_cast<uint8_t*>(value_cache);
  const bool scaled = cache_dtype != PA_F16;
  a.k_scale = scaled ? k_scale : nullptr;
  a.v_scale = scaled ? v_scale : nullptr;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.bs_log2 = log2i(block_size);
  hipError_t e = pa::launch_kv_write(a, src_dtype == PA_BF16, fmt, static_cast<hipStream_t>(stream));
  return hip_status(e, "kv_cache_write_fp8");
}

PA_API pa_status attn_prefill_paged(const void* q, pa_dtype q_dtype, const int32_t* cu_seqlens_q,
                                    int batch, int max_q_len, int64_t total_q,
                                    const void* key_cache, const void* value_cache,
                                    pa_dtype cache_dtype, int block_size, int64_t num_blocks,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len,
                                    int num_q_heads, int num_kv_heads, int head_dim,
                                    const float* k_scale, const float* v_scale,
                                    float softmax_scale, void* out, pa_dtype out_dtype,
                                    void* stream) {
  if (batch < 0 || max_q_len < 0 || total_q < 0)
    return fail(PA_ERR_INVALID_ARG, "attn_prefill_paged: negative size");
  if (!cu_seqlens_q) return fail(PA_ERR_INVALID_ARG, "attn_prefill_paged: null cu_seqlens_q");
  pa_status st = check_common(q, q_dtype, key_cache, value_cache, cache_dtype, block_size,
                              num_blocks, block_tables, max_blocks_per_seq, context_lens,
                              max_context_len, num_q_heads, num_kv_heads, head_dim, k_scale,
                              v_scale, softmax_scale, out, out_dtype);
  if (st != PA_OK) return st;
  if (max_q_len > max_context_len)
    return fail(PA_ERR_INVALID_ARG, "attn_prefill_paged: max_q_len exceeds max_context_len");
  const int G = num_q_heads / num_kv_heads;
  if (G > kMaxPrefillGroup)
    return fail(PA_ERR_UNSUPPORTED,
                "attn_prefill_paged: num_q_heads / num_kv_heads = %d unsupported (at most %d)", G,
                kMaxPrefillGroup);
  if (batch == 0 || max_q_len == 0 || total_q == 0) return ok();
  pa::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.cu_seqlens = cu_seqlens_q;
  a.key_cache = static_cast<const uint8_t*>(key_cache);
  a.value_cache = static_cast<const uint8_t*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const bool scaled = cache_dtype != PA_F16;
  a.k_scale = scaled ? k_scale : nullptr;
  a.v_scale = scaled ? v_scale : nullptr;
  a.out = out;
  a.batch = batch;
  a.max_blocks = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.bs_log2 = log2i(block_size);
  const int tok_per_tile = pa::kPrefillRows / G;
  a.q_blocks = (max_q_len + tok_per_tile - 1) / tok_per_tile;
  a.softmax_scale = softmax_scale;
  hipError_t e = pa::launch_prefill(a, head_dim, cache_fmt(cache_dtype), q_type(q_dtype),
                                    out_type(out_dtype), static_cast<hipStream_t>(stream));
  return hip_status(e, "attn_prefill_paged");
}

PA_API pa_status attn_decode_paged(const void* q, pa_dtype q_dtype, int batch,
                                   const void* key_cache, const void* value_cache,
                                   pa_dtype cache_dtype, int block_size, int64_t num_blocks,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int max_context_len,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   const float* k_scale, const float* v_scale,
                                   float softmax_scale, int num_partitions, void* workspace,
                                   size_t workspace_bytes, void* out, pa_dtype out_dtype,
                                   void* stream) {
  return decode_like("attn_decode_paged", q, q_dtype, batch, 1, key_cache, value_cache,
                     cache_dtype, block_size, num_blocks, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, num_q_heads, num_kv_heads, head_dim, k_scale,
                     v_scale, softmax_scale, num_partitions, workspace, workspace_bytes, out,
                     out_dtype, stream);
}

PA_API pa_status attn_verify_paged(const void* q, pa_dtype q_dtype, int batch, int q_len,
                                   const void* key_cache, const void* value_cache,
                                   pa_dtype cache_dtype, int block_size, int64_t num_blocks,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int max_context_len,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   const float* k_scale, const float* v_scale,
                                   float softmax_scale, int num_partitions, void* workspace,
                                   size_t workspace_bytes, void* out, pa_dtype out_dtype,
                                   void* stream) {
  return decode_like("attn_verify_paged", q, q_dtype, batch, q_len, key_cache, value_cache,
                     cache_dtype, block_size, num_blocks, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, num_q_heads, num_kv_heads, head_dim, k_scale,
                     v_scale, softmax_scale, num_partitions, workspace, workspace_bytes, out,
                     out_dtype, stream);
}

PA_API pa_status attn_verify_paged_noalloc(const void* q, pa_dtype q_dtype, int batch, int q_len,
                                           const void* key_cache, const void* value_cache,
                                           pa_dtype cache_dtype, int block_size,
                                           int64_t num_blocks, const int32_t* block_tables,
                                           int max_blocks_per_seq, const int32_t* context_lens,
                                           int max_context_len, int num_q_heads,
                                           int num_kv_heads, int head_dim, const float* k_scale,
                                           const float* v_scale, float softmax_scale,
                                           int num_partitions, void* out, pa_dtype out_dtype,
                                           void* stream) {
  return decode_like("attn_verify_paged_noalloc", q, q_dtype, batch, q_len, key_cache,
                     value_cache, cache_dtype, block_size, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_q_heads, num_kv_heads,
                     head_dim, k_scale, v_scale, softmax_scale, num_partitions, nullptr, 0, out,
                     out_dtype, stream, -1, nullptr, nullptr, true);
}

PA_API pa_status attn_window_paged(const void* q, pa_dtype q_dtype, int batch, int q_len,
                                   int window_left, const void* key_cache,
                                   const void* value_cache, pa_dtype cache_dtype, int block_size,
                                   int64_t num_blocks, const int32_t* block_tables,
                                   int max_blocks_per_seq, const int32_t* context_lens,
                                   int max_context_len, int num_q_heads, int num_kv_heads,
                                   int head_dim, const float* k_scale, const float* v_scale,
                                   float softmax_scale, int num_partitions, void* workspace,
                                   size_t workspace_bytes, void* out, pa_dtype out_dtype,
                                   void* stream) {
  if (window_left < 0) return fail(PA_ERR_INVALID_ARG, "attn_window_paged: window_left must be >= 0");
  return decode_like("attn_window_paged", q, q_dtype, batch, q_len, key_cache, value_cache,
                     cache_dtype, block_size, num_blocks, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, num_q_heads, num_kv_heads, head_dim, k_scale,
                     v_scale, softmax_scale, num_partitions, workspace, workspace_bytes, out,
                     out_dtype, stream, window_left);
}

PA_API pa_status attn_decode_append_paged(const void* q, pa_dtype q_dtype, int batch, int q_len,
                                          const void* key_new, const void* value_new,
                                          void* key_cache, void* value_cache,
                                          pa_dtype cache_dtype, int block_size,
                                          int64_t num_blocks, const int32_t* block_tables,
                                          int max_blocks_per_seq, const int32_t* context_lens,
                                          int max_context_len, int num_q_heads, int num_kv_heads,
                                          int head_dim, const float* k_scale,
                                          const float* v_scale, float softmax_scale,
                                          int num_partitions, void* workspace,
                                          size_t workspace_bytes, void* out, pa_dtype out_dtype,
                                          void* stream) {
  if (!key_new || !value_new)
    return fail(PA_ERR_INVALID_ARG, "attn_decode_append_paged: null key_new or value_new");
  return decode_like("attn_decode_append_paged", q, q_dtype, batch, q_len, key_cache, value_cache,
                     cache_dtype, block_size, num_blocks, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, num_q_heads, num_kv_heads, head_dim, k_scale,
                     v_scale, softmax_scale, num_partitions, workspace, workspace_bytes, out,
                     out_dtype, stream, -1, key_new, value_new);
}

PA_API int pa_decode_partitions(int batch, int q_len, int num_q_heads, int num_kv_heads,
                                int head_dim, int max_context_len) {
  (void)num_q_heads;
  (void)head_dim;
  if (batch <= 0 || q_len <= 0 || num_kv_heads <= 0 || max_context_len < 0) return 0;
  int part_len = 0, parts = 0;
  partition_shape(auto_partitions(batch, q_len, num_kv_heads, max_context_len), max_context_len,
                  &part_len, &parts);
  return parts;
}

PA_API size_t pa_workspace_bytes(int op, int batch, int q_len, int num_q_heads, int num_kv_heads,
                                 int head_dim, int num_partitions, int max_context_len) {
  if (op == PA_OP_WRITE || op == PA_OP_PREFILL) return 0;
  if (op != PA_OP_DECODE && op != PA_OP_VERIFY) return 0;
  if (batch <= 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_partitions < 0 || max_context_len < 0)
    return 0;
  if (op == PA_OP_DECODE) q_len = 1;
  const int req = num_partitions ? num_partitions
                                 : auto_partitions(batch, q_len, num_kv_heads, max_context_len);
  int part_len = 0, parts = 0;
  partition_shape(req, max_context_len, &part_len, &parts);
  return ws_bytes((int64_t)batch * q_len * num_q_heads, parts, head_dim);
}

PA_API size_t pa_window_workspace_bytes(int batch, int q_len, int num_q_heads, int num_kv_heads,
                                        int head_dim, int num_partitions, int max_context_len,
                                        int window_left) {
  if (batch <= 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_partitions < 0 || max_context_len < 0 || window_left < 0)
    return 0;
  const int span = key_span(max_context_len, q_len, window_left);
  const int req = num_partitions ? num_partitions
                                 : auto_partitions(batch, q_len, num_kv_heads, span);
  int part_len = 0, parts = 0;
  partition_shape(req, span, &part_len, &parts);
  return ws_bytes((int64_t)batch * q_len * num_q_heads, parts, head_dim);
}

PA_API int pa_supports(int op, pa_dtype q_dtype, pa_dtype cache_dtype, int head_dim,
                       int num_q_heads, int num_kv_heads, int block_size, int q_len) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return 0;
  if (!is_pow2(block_size) || block_size < kMinBlock || block_size > kMaxBlock) return 0;
  const int G = num_q_heads / num_kv_heads;
  if (op == PA_OP_WRITE) {
    if (q_dtype != PA_F16 && q_dtype != PA_BF16) return 0;
    if (cache_fmt(cache_dtype) < 0) return 0;
    if (cache_dtype == PA_F16 && q_dtype != PA_F16) return 0;
    return head_dim > 0 && head_dim % 16 == 0 && head_dim <= 1024;
  }
  if (q_type(q_dtype) < 0 || cache_fmt(cache_dtype) < 0) return 0;
  if (cache_dtype == PA_F16 && q_dtype != PA_F16) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  if (op == PA_OP_PREFILL) return q_len >= 0 && G <= kMaxPrefillGroup;
  if (op == PA_OP_DECODE) return q_len == 1 && G <= kMaxRows;
  if (op == PA_OP_VERIFY || op == PA_OP_WINDOW) return q_len >= 1 && (int64_t)q_len * G <= kMaxRows;
  return 0;
}

PA_API pa_status pa_validate_tables(const int32_t* block_tables, int batch, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len,
                                    int block_size, int64_t num_blocks,
                                    const int32_t* cu_seqlens_q, void* stream) {
  if (!block_tables || !context_lens || batch < 0 || max_blocks_per_seq <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: bad arguments");
  if (batch == 0) return ok();
  std::vector<int32_t> bt((size_t)batch * max_blocks_per_seq), cl((size_t)batch);
  std::vector<int32_t> cu(cu_seqlens_q ? (size_t)batch + 1 : 0);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = hipMemcpy(bt.data(), block_tables, bt.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess)
    e = hipMemcpy(cl.data(), context_lens, cl.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess && cu_seqlens_q)
    e = hipMemcpy(cu.data(), cu_seqlens_q, cu.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e, "pa_validate_tables");
  const int64_t cap = std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size);
  for (int b = 0; b < batch; ++b) {
    if (cl[b] < 0 || cl[b] > cap)
      return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: context_lens[%d] = %d outside [0, %lld]",
                  b, cl[b], (long long)cap);
    const int used = (int)(((int64_t)cl[b] + block_size - 1) / block_size);
    for (int k = 0; k < used; ++k) {
      const int32_t id = bt[(size_t)b * max_blocks_per_seq + k];
      if (id < 0 || id >= num_blocks)
        return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: block_tables[%d][%d] = %d outside [0, %lld)",
                    b, k, id, (long long)num_blocks);
    }
  }
  if (cu_seqlens_q) {
    if (cu[0] != 0)
      return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: cu_seqlens_q[0] = %d, not 0", cu[0]);
    for (int b = 0; b < batch; ++b) {
      const int64_t q_len = (int64_t)cu[b + 1] - cu[b];
      if (q_len < 0)
        return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: cu_seqlens_q decreases at %d", b + 1);
      if (q_len > cl[b])
        return fail(PA_ERR_INVALID_ARG,
                    "pa_validate_tables: sequence %d has %lld new queries but context_lens %d",
                    b, (long long)q_len, cl[b]);
    }
  }
  return ok();
}

}  // extern "C"

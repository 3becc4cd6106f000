/*
 * pagedattn.h -- C ABI of the paged-attention library (libpagedattn.so, gfx950).
 *
 * Operations (all from "1Cat-vLLM 1.5.0" RELEASE notes, section "Flash-V100
 * long-context improvements", and "SM70 release profile and acceleration
 * status"):
 *   kv_cache_write_fp8  -- quantize new K/V tokens into the block-paged cache
 *                          (FP8 E4M3 with per-head scales, FP8 E5M2, or fp16);
 *   attn_prefill_paged  -- causal prefill of a chunk of new tokens that attends
 *                          to its whole paged prefix (chunked prefill);
 *   attn_decode_paged   -- one new token per sequence, split-KV partitions
 *                          plus a log-sum-exp combine (long-context decode);
 *   attn_verify_paged   -- the grouped speculative-verify step: q_len new
 *                          causal tokens per sequence (q_len = 8 is the q8
 *                          verifier: seven drafts plus one);
 *   attn_decode_append_paged -- decode / verify and the new tokens'
 *                          quantize-on-write in one call (inside the attention
 *                          kernel when one 16-row block holds a KV head's rows).
 *
 * Semantics shared by the attention calls. Sequence b has context_lens[b]
 * keys, counting its new tokens (which must already be in the cache: write,
 * then attend). Its i-th new query sits at position
 * pos = context_lens[b] - q_len_b + i and attends keys 0..pos. Query head h
 * reads KV head h / (num_q_heads / num_kv_heads). With K, V the dequantized
 * cache values:
 *     out = sum_j softmax_j(softmax_scale * q.K_j) V_j     over j <= pos.
 * A row with no visible key (context_lens[b] == 0) is written as zeros.
 *
 * Cache layout (caller-owned device memory; the pages do not fix one):
 *   key_cache   [num_blocks][num_kv_heads][block_size][head_dim]
 *   value_cache [num_blocks][num_kv_heads][block_size / T][head_dim][T],
 *               T = min(block_size, 64)
 * i.e. keys are token-major inside one page of one head, and values are
 * dimension-major inside each group of T consecutive tokens of a page, so the
 * 64 keys' values a kernel tile needs are one contiguous run. Elements are
 * uint8 FP8 codes (OCP E4M3FN or E5M2) or fp16. Token o of a page (offset
 * o = j % block_size) has its value for dimension d at
 * value_cache[page][h][o / T][d][o % T].
 * Token j of sequence b lives in physical page block_tables[b][j / block_size]
 * at offset j % block_size ("block tables consistently use physical page
 * units", 1.5.0 notes, "Reliability and correctness fixes").
 * FP8 value = decoded code * scale[kv_head] (E4M3: scales required; E5M2:
 * scales optional, NULL means 1).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked (host). Tensors are dense,
 *     row-major, in the shapes stated; attention outputs (out) start on a
 *     16-byte boundary (rows leave as 16-byte runs). The library never allocates or frees
 *     device memory and keeps no pointer after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously. No call synchronizes, reads device memory from the
 *     host or allocates, so the calls may be captured into a HIP graph.
 *   - Arguments the host can check are checked before anything is launched:
 *     PA_ERR_INVALID_ARG for null pointers, non-positive sizes, num_q_heads not
 *     a multiple of num_kv_heads, missing E4M3 scales, too small a workspace,
 *     a misaligned workspace or output;
 *     PA_ERR_UNSUPPORTED for well-formed shapes no kernel covers (see
 *     pa_supports), so the caller can fall back. PA_ERR_HIP reports a launch
 *     error. pa_last_error() describes the last failure on the calling thread.
 *   - Device-resident values (context_lens, block table entries, slots) are
 *     preconditions, not checked on the hot path: context_lens[b] <=
 *     max_context_len, every block-table entry for a visible token in
 *     [0, num_blocks). pa_validate_tables() checks them synchronously.
 *   - Cache slots past a sequence's context, spare pages and block-table
 *     padding are never read, whatever they hold (NaN included).
 *   - Results are bitwise reproducible for identical inputs and arguments.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_API __attribute__((visibility("default")))

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,
  PA_ERR_UNSUPPORTED = 2,
  PA_ERR_HIP = 3
} pa_status;

typedef enum pa_dtype {
  PA_F16 = 0,
  PA_BF16 = 1,
  PA_F32 = 2,
  PA_FP8_E4M3 = 3, /* OCP E4M3FN: max 448, no infinities */
  PA_FP8_E5M2 = 4  /* OCP E5M2: max 57344 */
} pa_dtype;

typedef enum pa_op {
  PA_OP_WRITE = 0,
  PA_OP_PREFILL = 1,
  PA_OP_DECODE = 2,
  PA_OP_VERIFY = 3,
  PA_OP_WINDOW = 4
} pa_op;

/*
 * Quantize-on-write of new K/V tokens into the paged cache.
 * (FP8 KV cache: "1Cat-vLLM 1.0.0" README, "Optional experimental feature: FP8
 * KV cache"; E4M3 release KV: "SM70 release profile and acceleration status".)
 *
 *   key, value     [num_tokens][num_kv_heads][head_dim], src_dtype F16 or BF16
 *   slot_mapping   [num_tokens] int64: slot = page * block_size + offset;
 *                  a negative slot skips the token
 *   key_cache, value_cache  layout above, element type cache_dtype
 *                  (PA_FP8_E4M3, PA_FP8_E5M2, or PA_F16 for a plain copy of
 *                  F16 sources)
 *   k_scale, v_scale [num_kv_heads] float32 per-head scales; required for
 *                  E4M3, optional for E5M2 (NULL = 1), ignored for F16
 *
 * FP8 encoding of element x of head h: y = float32(x) / scale[h] (IEEE
 * float32 division, correctly rounded), saturate |y| to the largest finite
 * value, round to nearest with ties to even; the sign is kept (-0 -> 0x80).
 * Bit-exact. num_tokens == 0 is a no-op. Slots must be distinct and below
 * num_blocks * block_size.
 */
PA_API pa_status kv_cache_write_fp8(
    const void* key, const void* value, pa_dtype src_dtype,
    const int64_t* slot_mapping, int64_t num_tokens,
    void* key_cache, void* value_cache, pa_dtype cache_dtype,
    int64_t num_blocks, int block_size, int num_kv_heads, int head_dim,
    const float* k_scale, const float* v_scale, void* stream);

/*
 * Causal prefill of one chunk per sequence over the paged prefix ("SM70 release
 * profile": prompts prefilled in 4096-token chunks; "1Cat-vLLM 1.5.0" notes:
 * long-prefill GQA attention with FP32 accumulation and several query heads
 * packed onto one KV head).
 *
 *   q            [total_q][num_q_heads][head_dim], q_dtype F16 or BF16;
 *                sequence b owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   cu_seqlens_q [batch + 1] int32, cu_seqlens_q[0] = 0, non-decreasing;
 *                each q_len_b <= max_q_len (host) and <= context_lens[b]
 *                (the chunk is written before it is attended; a longer chunk
 *                is outside the contract, yet its rows before position 0 are
 *                written as zeros and nothing outside the sequence's pages is
 *                read; pa_validate_tables checks these bounds)
 *   block_tables [batch][max_blocks_per_seq] int32 physical page ids
 *   context_lens [batch] int32, keys of sequence b including its new chunk
 *   k_scale, v_scale [num_kv_heads] float32 (see kv_cache_write_fp8)
 *   out          [total_q][num_q_heads][head_dim], out_dtype F32, F16 or BF16
 * num_q_heads / num_kv_heads may be any value up to 64 (PA_ERR_UNSUPPORTED
 * above).
 */
PA_API pa_status attn_prefill_paged(
    const void* q, pa_dtype q_dtype, const int32_t* cu_seqlens_q, int batch,
    int max_q_len, int64_t total_q,
    const void* key_cache, const void* value_cache, pa_dtype cache_dtype,
    int block_size, int64_t num_blocks,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int max_context_len,
    int num_q_heads, int num_kv_heads, int head_dim,
    const float* k_scale, const float* v_scale, float softmax_scale,
    void* out, pa_dtype out_dtype, void* stream);

/*
 * Single-token decode, split-KV ("1Cat-vLLM 1.5.0" notes: batched FP8 decode
 * that reuses page ids and widens cache loads to 128 bits; long-context E4M3
 * decode routing at 128K/256K). Keys are cut into num_partitions equal ranges;
 * each range yields (max, sum, partial output) per row, and a second kernel
 * merges them by log-sum-exp in a fixed order.
 *
 *   q              [batch][num_q_heads][head_dim], F16 or BF16
 *   batch          at most 65535 (PA_ERR_UNSUPPORTED above: a launch dimension;
 *                  the same holds for the verify, window and append calls)
 *   num_partitions 0 = automatic (pa_decode_partitions), else >= 1
 *   workspace      device scratch of at least pa_workspace_bytes(PA_OP_DECODE,
 *                  ...) bytes, 256-byte aligned; contents need no
 *                  initialisation and are clobbered
 *   out            [batch][num_q_heads][head_dim], F32, F16 or BF16
 * Other arguments as in attn_prefill_paged (q_len = 1).
 */
PA_API pa_status attn_decode_paged(
    const void* q, pa_dtype q_dtype, int batch,
    const void* key_cache, const void* value_cache, pa_dtype cache_dtype,
    int block_size, int64_t num_blocks,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int max_context_len,
    int num_q_heads, int num_kv_heads, int head_dim,
    const float* k_scale, const float* v_scale, float softmax_scale,
    int num_partitions, void* workspace, size_t workspace_bytes,
    void* out, pa_dtype out_dtype, void* stream);

/*
 * Grouped speculative verify ("1Cat-vLLM 1.5.0" notes: exact grouped q8
 * verification over FP8 E5M2 KV, seven drafts plus one): q_len new tokens per
 * sequence, all G query heads of a KV head and all q_len tokens processed as
 * one group over one pass of the KV stream. Exact: row i equals a decode at
 * context context_lens[b] - q_len + 1 + i.
 *
 *   q     [batch][q_len][num_q_heads][head_dim]
 *   out   [batch][q_len][num_q_heads][head_dim]
 *   q_len 1 <= q_len, q_len * (num_q_heads / num_kv_heads) <= 64
 * Other arguments as in attn_decode_paged (workspace op PA_OP_VERIFY).
 */
PA_API pa_status attn_verify_paged(
    const void* q, pa_dtype q_dtype, int batch, int q_len,
    const void* key_cache, const void* value_cache, pa_dtype cache_dtype,
    int block_size, int64_t num_blocks,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int max_context_len,
    int num_q_heads, int num_kv_heads, int head_dim,
    const float* k_scale, const float* v_scale, float softmax_scale,
    int num_partitions, void* workspace, size_t workspace_bytes,
    void* out, pa_dtype out_dtype, void* stream);

/*
 * attn_verify_paged without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid allocation. Same arguments, kernels and
 * results as attn_verify_paged (bit for bit, q_len = 1 is decode), but the
 * split-KV partials go to a static device array of 16 MiB that the library
 * holds on each GPU it runs on until the process ends. This call allocates
 * nothing and frees nothing (the array's device address is looked up once per
 * device, on the first call with that device current).
 *
 *   Limit: the partials need pa_workspace_bytes(PA_OP_VERIFY, batch, q_len,
 *          num_q_heads, num_kv_heads, head_dim, num_partitions,
 *          max_context_len) bytes; a call needing more than 16 MiB (16777216)
 *          returns PA_ERR_UNSUPPORTED before launching anything (the 128K
 *          headline decode needs 0.5 MiB, 4 x 128K q16 verify 8.5 MiB).
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *          last call's partials (every value read is written first by the same
 *          call, so nothing needs clearing). Calls that overlap on one GPU --
 *          on different streams, or from several threads without ordering --
 *          race on the array and may return wrong results; order them.
 */
PA_API pa_status attn_verify_paged_noalloc(
    const void* q, pa_dtype q_dtype, int batch, int q_len,
    const void* key_cache, const void* value_cache, pa_dtype cache_dtype,
    int block_size, int64_t num_blocks,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int max_context_len,
    int num_q_heads, int num_kv_heads, int head_dim,
    const float* k_scale, const float* v_scale, float softmax_scale,
    int num_partitions, void* out, pa_dtype out_dtype, void* stream);

/*
 * Write-then-attend in one call: the quantize-on-write of the q_len newest
 * tokens of every sequence fused into the decode / verify kernel. The pages
 * write each step's new K/V into the FP8 cache ("1Cat-vLLM 1.0.0" README,
 * "Optional experimental feature: FP8 KV cache") and then attend over it
 * (decode, or the grouped q8 verify of the 1.5.0 notes). When the rows of one
 * KV head (q_len * num_q_heads / num_kv_heads) fit one 16-row block, as in
 * decode, the work-group that will read a new token's keys writes them first,
 * inside the attention kernel, which saves the write kernel's launch; wider
 * row groups get a small write kernel (slots from the block table) before the
 * attention kernel, in the same call.
 *
 * Result (cache bytes and out) identical to
 *     kv_cache_write_fp8(key_new, value_new, q_dtype, slots, batch * q_len, ...)
 *     attn_verify_paged(q, ..., q_len, ...)      (attn_decode_paged if q_len = 1)
 * with slots[b * q_len + i] = block_tables[b][pos / block_size] * block_size
 * + pos % block_size at pos = context_lens[b] - q_len + i, i.e. each new token
 * goes to its own position in the sequence's pages (tokens with pos < 0 are
 * not written). The encoding is the one of kv_cache_write_fp8, bit for bit.
 *
 *   key_new, value_new  [batch][q_len][num_kv_heads][head_dim], in q_dtype
 *                       (the write's source dtype)
 *   key_cache, value_cache  written at the new tokens' slots only
 * Other arguments as in attn_verify_paged (workspace op PA_OP_VERIFY). The
 * pages holding the new tokens must not be read by another sequence of the
 * same call (a shared prefix page is fine; the page being appended to is the
 * sequence's own).
 */
PA_API pa_status attn_decode_append_paged(
    const void* q, pa_dtype q_dtype, int batch, int q_len,
    const void* key_new, const void* value_new,
    void* key_cache, void* value_cache, pa_dtype cache_dtype,
    int block_size, int64_t num_blocks,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int max_context_len,
    int num_q_heads, int num_kv_heads, int head_dim,
    const float* k_scale, const float* v_scale, float softmax_scale,
    int num_partitions, void* workspace, size_t workspace_bytes,
    void* out, pa_dtype out_dtype, void* stream);

/*
 * Non-causal sliding-window attention over the paged cache: the draft model's
 * attention of the "1Cat-vLLM 1.5.0" notes ("Production DFlash2 on V100":
 * non-causal sliding-window draft attention; "Flash-V100 long-context
 * improvements": prefix tiles outside the window are skipped). The pages give
 * no formula; the reading implemented is the usual left window without a
 * causal mask: query i of sequence b sits at pos = context_lens[b] - q_len + i
 * and attends every key j with
 *
 *     pos - window_left <= j < context_lens[b]
 *
 * (window_left keys before its own position, itself, and every later key of
 * its block). Pages holding only keys before the window are never read.
 *
 *   q            [batch][q_len][num_q_heads][head_dim]
 *   out          [batch][q_len][num_q_heads][head_dim]
 *   window_left  >= 0 (PA_ERR_INVALID_ARG otherwise); a window at least as
 *                long as the context is full non-causal attention
 *   q_len        1 <= q_len, q_len * (num_q_heads / num_kv_heads) <= 64
 *   workspace    at least pa_window_workspace_bytes(...) bytes
 * Other arguments as in attn_decode_paged.
 */
PA_API pa_status attn_window_paged(
    const void* q, pa_dtype q_dtype, int batch, int q_len, int window_left,
    const void* key_cache, const void* value_cache, pa_dtype cache_dtype,
    int block_size, int64_t num_blocks,
    const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int max_context_len,
    int num_q_heads, int num_kv_heads, int head_dim,
    const float* k_scale, const float* v_scale, float softmax_scale,
    int num_partitions, void* workspace, size_t workspace_bytes,
    void* out, pa_dtype out_dtype, void* stream);

/* Bytes of workspace attn_window_paged needs for these arguments
 * (num_partitions = 0 means automatic); 0 for invalid arguments. Host-only
 * arithmetic, no device access. The caller owns the workspace, as the engine
 * of the pages owns and releases its attention workspaces ("1Cat-vLLM 1.5.0"
 * RELEASE notes, "Reliability and correctness fixes", "Runtime and API
 * stability": shutdown releases the SM70 global workspaces); the partitions
 * cover only the keys the window can see ("Flash-V100 long-context
 * improvements": prefix tiles outside the window are skipped). */
PA_API size_t pa_window_workspace_bytes(int batch, int q_len, int num_q_heads,
                                        int num_kv_heads, int head_dim, int num_partitions,
                                        int max_context_len, int window_left);

/* Partition count that num_partitions = 0 selects for decode/verify (host
 * arithmetic, no device access): the split of the long-context decode route
 * ("1Cat-vLLM 1.5.0" RELEASE notes, "Flash-V100 long-context improvements":
 * long E4M3 decode routing at 128K/256K), here one work-group per compute
 * unit and at least 256 keys per partition. Returns 0 for invalid
 * arguments. */
PA_API int pa_decode_partitions(int batch, int q_len, int num_q_heads, int num_kv_heads,
                                int head_dim, int max_context_len);

/* Bytes of workspace attn_decode_paged / attn_verify_paged need (0 for the
 * write and prefill ops): one (max, sum) pair and one partial output row per
 * (query row, partition) of the split-KV decode ("1Cat-vLLM 1.5.0" RELEASE
 * notes, "Flash-V100 long-context improvements": long-context decode routing).
 * num_partitions = 0 means automatic. Host-only arithmetic; the caller owns
 * the workspace ("Reliability and correctness fixes", "Runtime and API
 * stability": the engine releases its attention workspaces itself). Returns 0
 * for invalid arguments. */
PA_API size_t pa_workspace_bytes(int op, int batch, int q_len, int num_q_heads,
                                 int num_kv_heads, int head_dim, int num_partitions,
                                 int max_context_len);

/* 1 if a kernel covers this combination, else 0: the capability check a
 * caller makes before dispatch so that it can fall back for this one operator
 * ("1Cat-vLLM 1.5.0" RELEASE notes, "Reliability and correctness fixes",
 * "Runtime and API stability": q16 verification checks the grouped
 * verifier's capability before dispatch and q8-only builds fall back safely;
 * "Production DFlash2 on V100": each verifier operator checks its dtype, KV
 * format and live batch shape and falls back independently). The attention
 * calls make the same check and return PA_ERR_UNSUPPORTED when it fails.
 * q_len is the per-sequence query count (1 for decode, the verify or window
 * block width, the chunk for prefill). Host-only. */
PA_API int pa_supports(int op, pa_dtype q_dtype, pa_dtype cache_dtype, int head_dim,
                       int num_q_heads, int num_kv_heads, int block_size, int q_len);

/* Description of the last error on the calling thread ("" after success):
 * the reason behind a PA_ERR_* status, so that a caller that falls back for
 * one operator can report why ("Production DFlash2 on V100": operators fall
 * back independently when their local contract is not met; "SM70 release
 * profile and acceleration status": disabled paths are reported with a
 * reason). The string is owned by the library and valid until the thread's
 * next call. */
PA_API const char* pa_last_error(void);

/* Library version string. */
PA_API const char* pa_version(void);

/*
 * Profiling hook (in the spirit of the pages' per-route performance counters,
 * "SM70 release profile and acceleration status"): start_event and stop_event
 * are hipEvent_t handles owned by the caller. The next write or attention call
 * made on the calling thread attaches both to the dispatch of its main kernel
 * (the write kernel, the prefill kernel, or the split kernel of decode /
 * verify; hipExtLaunchKernel), so they record that kernel's start and end,
 * then forgets both. Passing NULL for either clears a pending request. No
 * effect on results.
 */
PA_API void pa_profile_next_call(void* start_event, void* stop_event);

/*
 * Debug check, synchronous, never on the hot path: copies context_lens,
 * block_tables and (when not NULL) cu_seqlens_q to the host (after
 * synchronizing `stream`) and verifies 0 <= context_lens[b] <=
 * min(max_context_len, max_blocks_per_seq * block_size), that every block id
 * a visible token uses is a physical page id in [0, num_blocks) ("1Cat-vLLM
 * 1.5.0" RELEASE notes, "Reliability and correctness fixes": block tables use
 * physical page units), and, for a prefill batch, that cu_seqlens_q starts at
 * 0, never decreases and gives each chunk q_len_b <= context_lens[b] (a chunk
 * is written before it is attended). The device-resident values the
 * attention calls take as preconditions are exactly these. Returns
 * PA_ERR_INVALID_ARG naming the first violation, PA_ERR_HIP if a copy fails.
 *
 *   cu_seqlens_q  [batch + 1] int32 (device) or NULL to skip that check
 */
PA_API pa_status pa_validate_tables(const int32_t* block_tables, int batch,
                                    int max_blocks_per_seq, const int32_t* context_lens,
                                    int max_context_len, int block_size,
                                    int64_t num_blocks, const int32_t* cu_seqlens_q,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */

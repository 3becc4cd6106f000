"""Seeded synthetic inputs for the paged-attention workloads.

This module only draws random numbers and lays out block tables; it holds no
attention and no FP8 arithmetic, so both the HIP path and the CPU oracle can
take their inputs from it.

Recipe (the same for every workload). ``rng = numpy.random.Generator(
PCG64(seed))`` draws, in this order:

1. structure: per-sequence context lengths where they are random (uniform
   integers, both ends inclusive);
2. Q, then K, then V: ``standard_normal(dtype=float32) * sigma``, rounded to
   the source dtype with round-to-nearest-even (numpy for fp16, torch's CPU
   cast for bf16);
3. the outlier mask where the workload has one: every (token, KV head) pair
   independently with probability ``outlier_frac``; its whole K vector is
   multiplied by ``outlier_mult`` (a power of two, so exact) before the scales
   are taken;
4. a permutation of the page pool: sequence b takes the next
   ``ceil(ctx_b / block_size)`` physical pages of the permutation; the rest
   (at least 10% of the pool, at least one page) stay spare.

Per-KV-head FP8 scales (E4M3): ``float32(amax_g) / float32(448)``, amax over
all tokens and dims of head g of the workload's K (resp. V) tensor; an all-zero
head gets scale 1. E5M2 workloads take no scales.

Cache contents that the workload never writes -- spare pages, the unused
tail of each sequence's last page -- are meant to be filled with NaN patterns
(``POISON``) before the writes, and block-table padding is ``INT32_MAX``, so a
kernel that reads outside the visible context is caught.
"""

from dataclasses import dataclass, field
import math

import numpy as np

INT32_MAX = np.iinfo(np.int32).max
# byte (FP8) or 16-bit (fp16) NaN pattern used to poison unwritten cache slots
POISON = {"e4m3": 0x7F, "e5m2": 0x7F, "f16": 0x7E00}
FP8_E4M3_MAX = 448.0


def rng_for(seed):
    return np.random.Generator(np.random.PCG64(seed))


def round_to(x32, dtype):
    """float32 -> 16-bit storage: np.float16 array, or uint16 bf16 bits."""
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def to_f32(arr, dtype):
    """Exact float32 values of a 16-bit storage array."""
    if dtype == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(arr, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def normal16(rng, shape, sigma, dtype, chunk=1 << 26):
    """sigma * N(0,1) rounded to dtype, drawn in row order in bounded chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16 if dtype == "f16" else np.uint16)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        x = rng.standard_normal(m, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[i:i + m] = round_to(x, dtype)
    return out.reshape(shape)


def head_scales(x16, dtype):
    """Per-KV-head scale float32(amax) / 448 for x16 [T, Hkv, D]."""
    Hkv = x16.shape[1]
    s = np.empty(Hkv, dtype=np.float32)
    for g in range(Hkv):
        amax = np.float32(np.abs(to_f32(x16[:, g, :], dtype)).max()) if x16.shape[0] else np.float32(0)
        s[g] = np.float32(1.0) if amax == 0 else amax / np.float32(FP8_E4M3_MAX)
    return s


@dataclass
class Case:
    """One workload: the whole token content of every sequence plus paging.

    q      [total_q, Hq, D]  16-bit storage (np.float16 or bf16 bits)
    k, v   [total_tokens, Hkv, D] source dtype storage, sequences back to back
    """
    name: str
    q_dtype: str
    kv_dtype: str            # dtype of the new K/V tokens before the write
    cache_fmt: str           # "f16", "e4m3" or "e5m2"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    softmax_scale: float
    q: np.ndarray
    q_lens: np.ndarray       # [B] queries per sequence in ``q``
    k: np.ndarray
    v: np.ndarray
    ctx_lens: np.ndarray     # [B] int32, keys visible to each sequence's last query
    tok_start: np.ndarray    # [B] int64, first row of sequence b in k/v
    block_tables: np.ndarray  # [B, max_blocks] int32, padded with INT32_MAX
    slot_mapping: np.ndarray  # [total_tokens] int64
    num_blocks: int
    k_scale: np.ndarray = None
    v_scale: np.ndarray = None
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.ctx_lens)

    @property
    def gqa(self):
        return self.num_q_heads // self.num_kv_heads


def make_case(name, seed, ctx_lens, q_lens, num_q_heads, num_kv_heads, head_dim,
              block_size, q_dtype, kv_dtype, cache_fmt, softmax_scale=None,
              sigma_q=1.0, sigma_kv=1.0, outlier_frac=0.0, outlier_mult=8.0,
              ctx_range=None, batch=None, spare_frac=0.10, meta=None):
    """Build a workload. ``ctx_lens`` may be None with ``ctx_range=(lo, hi)``
    and ``batch``: lengths are then drawn uniformly from lo..hi inclusive.
    ``q_lens`` is an int (same for all sequences) or a list."""
    rng = rng_for(seed)
    if ctx_lens is None:
        lo, hi = ctx_range
        ctx_lens = rng.integers(lo, hi, size=batch, endpoint=True)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    B = len(ctx_lens)
    if np.isscalar(q_lens):
        q_lens = [int(q_lens)] * B
    q_lens = np.asarray(q_lens, dtype=np.int64)
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / math.sqrt(D)))

    q = normal16(rng, (int(q_lens.sum()), Hq, D), sigma_q, q_dtype)
    T = int(ctx_lens.sum())
    k = normal16(rng, (T, Hkv, D), sigma_kv, kv_dtype)
    v = normal16(rng, (T, Hkv, D), sigma_kv, kv_dtype)
    if outlier_frac > 0:
        mask = rng.random((T, Hkv)) < outlier_frac
        kf = to_f32(k[mask], kv_dtype) * np.float32(outlier_mult)
        k[mask] = round_to(kf, kv_dtype)

    bs = int(block_size)
    pages_per_seq = [-(-int(c) // bs) for c in ctx_lens]
    used = sum(pages_per_seq)
    spare = max(1, int(math.ceil(spare_frac * used)))
    num_blocks = used + spare
    perm = rng.permutation(num_blocks).astype(np.int64)
    max_blocks = max(1, max(pages_per_seq))
    bt = np.full((B, max_blocks), INT32_MAX, dtype=np.int32)
    tok_start = np.zeros(B, dtype=np.int64)
    slots = np.empty(T, dtype=np.int64)
    p0 = 0
    t0 = 0
    for b in range(B):
        n = pages_per_seq[b]
        bt[b, :n] = perm[p0:p0 + n]
        p0 += n
        tok_start[b] = t0
        c = int(ctx_lens[b])
        j = np.arange(c)
        slots[t0:t0 + c] = bt[b, j // bs].astype(np.int64) * bs + j % bs
        t0 += c

    k_scale = v_scale = None
    if cache_fmt == "e4m3":
        k_scale = head_scales(k, kv_dtype)
        v_scale = head_scales(v, kv_dtype)
    return Case(name=name, q_dtype=q_dtype, kv_dtype=kv_dtype, cache_fmt=cache_fmt,
                num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                softmax_scale=float(np.float32(softmax_scale)), q=q, q_lens=q_lens,
                k=k, v=v, ctx_lens=ctx_lens.astype(np.int32), tok_start=tok_start,
                block_tables=bt, slot_mapping=slots, num_blocks=num_blocks,
                k_scale=k_scale, v_scale=v_scale, seed=seed, meta=dict(meta or {}))


# --------------------------------------------------------------------------
# The five workloads and the 128K decode headline.
# Seeds: 1000 + workload number (the headline uses 1006).
# --------------------------------------------------------------------------

def prefill_decode_small(seed=1001):
    """1 sequence: causal prefill of 64 tokens, then one decode step at
    position 64. Hq=4, Hkv=1, D=64, fp16 Q/K/V ~ N(0,1), fp16 KV cache in
    16-token pages, shuffled block table, softmax scale 1/8. ``q`` holds the
    65 queries (64 prefill + 1 decode); the cache holds 65 tokens."""
    return make_case("prefill64_decode_fp16_d64", seed, [65], [65], 4, 1, 64, 16,
                     "f16", "f16", "f16", softmax_scale=0.125,
                     meta=dict(prefill_len=64))


def batched_decode_e4m3(seed=1002):
    """8 sequences, context lengths uniform in [1024, 4096], decode (one query
    each). Hq=32, Hkv=8, D=128, fp16 Q ~ N(0,1), K/V ~ N(0,1) written as E4M3
    with per-head amax scales, 16-token pages, random page permutation."""
    return make_case("decode_b8_1k4k_e4m3_bs16", seed, None, 1, 32, 8, 128, 16,
                     "f16", "f16", "e4m3", ctx_range=(1024, 4096), batch=8)


def chunked_prefill_32k(seed=1003, total=32768, chunk=4096):
    """1 sequence prefilled to 32768 tokens in 4096-token chunks; chunk c
    writes its tokens and then attends to its paged prefix (ctx = 4096 (c+1)).
    Hq=32, Hkv=8, D=128, bf16 Q/K/V ~ N(0,1), E4M3 KV with per-head scales
    (amax over all 32768 tokens), 2048-token pages (16, permuted)."""
    return make_case("prefill32k_chunk4k_bf16_e4m3_bs2048", seed, [total], [total],
                     32, 8, 128, 2048, "bf16", "bf16", "e4m3",
                     meta=dict(chunk=chunk))


def verify_q8_128k(seed=1004, ctx=131072):
    """Speculative verify: 4 sequences, 8 new causal queries each against
    131072-token contexts (the 8 queries at positions 131064..131071), FP8
    E5M2 KV with no scales, Hq=32, Hkv=8, D=128, 2048-token pages (64 per
    sequence, 256-page pool permuted), K/V ~ N(0, 0.5), fp16 Q ~ N(0,1)."""
    return make_case("verify_q8_b4_128k_e5m2_bs2048", seed, [ctx] * 4, 8, 32, 8, 128,
                     2048, "f16", "f16", "e5m2", sigma_kv=0.5)


def long_decode_256k(seed=1005, ctx=262144, partitions=64):
    """1 sequence, decode at 262144 tokens, Hq=32, Hkv=8, D=128, E4M3 KV with
    per-head scales, 2048-token pages (128 permuted), split-KV into 64
    partitions; values ~ N(0,1), 1% of (token, head) K vectors scaled x8."""
    return make_case("decode_256k_e4m3_bs2048_p64", seed, [ctx], 1, 32, 8, 128, 2048,
                     "f16", "f16", "e4m3", outlier_frac=0.01, outlier_mult=8.0,
                     meta=dict(partitions=partitions))


def headline_decode_128k(seed=1006, ctx=131072, partitions=32):
    """The 128K FP8 decode headline: the 256K recipe at 131072 tokens
    (E4M3 per-head scales, 1% x8 K outliers), split into 32 partitions of
    4096 tokens (one work-group per CU)."""
    return make_case("decode_128k_e4m3_bs2048_p32", seed, [ctx], 1, 32, 8, 128, 2048,
                     "f16", "f16", "e4m3", outlier_frac=0.01, outlier_mult=8.0,
                     meta=dict(partitions=partitions))


# --------------------------------------------------------------------------
# Second workloads on the same kernels (seeds 1007..1009).
# --------------------------------------------------------------------------

def batched_decode_e5m2_16k(seed=1007, batch=16, ctx=16384):
    """16 sequences at 16384 tokens each, decode (one query each). Hq=32,
    Hkv=8, D=128, fp16 Q/K/V ~ N(0,1), E5M2 KV (no scales), 16-token pages,
    random page permutation."""
    return make_case("decode_b16_16k_e5m2_bs16", seed, [ctx] * batch, 1, 32, 8, 128, 16,
                     "f16", "f16", "e5m2")


def verify_q16_128k(seed=1008, ctx=131072):
    """The q8 verify recipe with 16 new causal queries per sequence (the
    wider lookup verification): 4 sequences at 131072 tokens (queries at
    131056..131071), E5M2 KV, K/V ~ N(0, 0.5), 2048-token pages."""
    return make_case("verify_q16_b4_128k_e5m2_bs2048", seed, [ctx] * 4, 16, 32, 8, 128,
                     2048, "f16", "f16", "e5m2", sigma_kv=0.5)


def chunked_prefill_64k(seed=1009, total=65536, chunk=4096):
    """The 32K chunked-prefill recipe to 65536 tokens (32 pages of 2048);
    run in 4096- or 8192-token chunks."""
    return make_case(f"prefill64k_chunk{chunk // 1024}k_bf16_e4m3_bs2048", seed, [total], [total],
                     32, 8, 128, 2048, "bf16", "bf16", "e4m3", meta=dict(chunk=chunk))


def chunked_prefill_long(total=131072, chunk=4096, seed=None):
    """The 32K chunked-prefill recipe to 131072 (seed 1011) or 262144 (seed
    1012) tokens, 2048-token pages (64 or 128), run in 4096- or 8192-token
    chunks (the 4096 / 8192 prefill budgets of the long-context profile)."""
    if seed is None:
        seed = {131072: 1011, 262144: 1012}[total]
    return make_case(f"prefill{total // 1024}k_chunk{chunk // 1024}k_bf16_e4m3_bs2048", seed,
                     [total], [total], 32, 8, 128, 2048, "bf16", "bf16", "e4m3",
                     meta=dict(chunk=chunk))


def window_draft_q8(seed=1010, ctx=131072, window=4096, batch=4):
    """Draft attention: 4 sequences, blocks of 8 new queries each attending
    non-causally to a 4096-key sliding window (plus the later keys of their
    block) at the given context, E5M2 KV (no scales), fp16 Q ~ N(0,1), K/V ~
    N(0, 0.5), 2048-token pages. The window length and the block width are
    readings (the pages give neither); the block is the verifier's q8."""
    return make_case(f"window{window // 1024}k_q8_b{batch}_{ctx // 1024}k_e5m2_bs2048", seed,
                     [ctx] * batch, 8, 32, 8, 128, 2048, "f16", "f16", "e5m2", sigma_kv=0.5,
                     meta=dict(window=window))


WORKLOADS = {
    1: prefill_decode_small,
    2: batched_decode_e4m3,
    3: chunked_prefill_32k,
    4: verify_q8_128k,
    5: long_decode_256k,
    "H": headline_decode_128k,
    "b16": batched_decode_e5m2_16k,
    "q16": verify_q16_128k,
    "64k": chunked_prefill_64k,
    "128k": lambda chunk=4096: chunked_prefill_long(131072, chunk),
    "256k": lambda chunk=4096: chunked_prefill_long(262144, chunk),
    "win": window_draft_q8,
}

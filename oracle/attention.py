"""Naive float64 causal attention over the block-paged KV cache.

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ("1Cat-vLLM 1.5.0" RELEASE notes, "Flash-V100 long-context
improvements": paged prefill, decode and the grouped q8 verifier are all the
same attention over the paged prefix; "SM70 release profile": prompts are
prefilled in chunks that attend to the pages already written):

For sequence b with ``ctx_b`` keys (every key visible to its last query,
including the new tokens) and ``q_len_b`` new queries, query i sits at
position ``pos = ctx_b - q_len_b + i`` and attends keys ``0..pos``. For query
head h the KV head is ``g = h // G`` with ``G = Hq / Hkv`` (contiguous head
groups). With K, V the dequantized keys and values of head g:

    s_j = softmax_scale * (q . K_j)            for j <= pos
    m   = max_j s_j,   p_j = exp(s_j - m),   l = sum_j p_j
    o   = sum_j p_j V_j / l

A row with no visible key (pos < 0, e.g. ``ctx_b == 0``) has o = 0,
m = -inf, l = 0.

``softmax_scale`` is a float32 and is widened to float64. Decode is
``q_len = 1``, verify ``q_len = 8`` (any q_len works), prefill one chunk of
``q_len`` tokens. Splitting keys into partitions is not part of the
definition; ``attend_partitioned`` exists only to self-test the log-sum-exp
combine algebra.

Sliding-window attention ("1Cat-vLLM 1.5.0" RELEASE notes, "Production
DFlash2 on V100": the draft model's non-causal sliding-window attention;
"Flash-V100 long-context improvements": that attention skips the prefix tiles
outside the window). The pages give no formula; the reading taken is the usual
one for a left window of ``W`` keys with no causal mask: query i of a block of
``q_len`` sits at ``pos = ctx_b - q_len_b + i`` and attends every key j with

    pos - W <= j < ctx_b

-- the W keys before its own position, its own key, and every later key of
its block. The arithmetic per row is the same as above over that key set;
``W >= ctx_b`` gives plain non-causal attention over the whole context.

Rows are processed a block at a time purely to bound memory; each row's
arithmetic is the definition above.
"""

import numpy as np

from . import paged


def _rows_attend(qrows, pos, K, V, scale, probs=True):
    """Causal rows: row r sees keys 0..pos[r]."""
    pos = np.asarray(pos)
    return _rows_attend_range(qrows, np.zeros_like(pos), pos, K, V, scale, probs)


def _rows_attend_range(qrows, lo, hi, K, V, scale, probs=True):
    """qrows [R, D] float64; row r sees keys lo[r]..hi[r] (inclusive) of the
    ctx keys in K, V. Returns o [R, D], m [R], l [R], and P [R, ctx] (None
    when ``probs`` is false)."""
    R, D = qrows.shape
    ctx = K.shape[0]
    o = np.zeros((R, D))
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    P = np.zeros((R, ctx)) if probs else None
    if ctx == 0:
        return o, m, l, P
    s = scale * (qrows @ K.T)                       # [R, ctx]
    j = np.arange(ctx)
    visible = (j[None, :] >= np.asarray(lo)[:, None]) & (j[None, :] <= np.asarray(hi)[:, None])
    has = visible.any(axis=1)
    s = np.where(visible, s, -np.inf)
    m_h = s[has].max(axis=1)
    p = np.exp(s[has] - m_h[:, None])              # masked keys -> exp(-inf) = 0
    l_h = p.sum(axis=1)
    o[has] = (p @ V) / l_h[:, None]
    m[has] = m_h
    l[has] = l_h
    if probs:
        P[has] = p / l_h[:, None]
    return o, m, l, P


def _row_keys(pos, ctx, window):
    """Visible key range (inclusive) of rows at positions pos: causal 0..pos,
    or pos - window .. ctx - 1 for the non-causal sliding window."""
    pos = np.asarray(pos)
    if window is None:
        return np.zeros_like(pos), pos
    return pos - int(window), np.full_like(pos, ctx - 1)


def attend(q, q_lens, ctx_lens, k_cache, v_cache, block_tables, fmt,
           num_kv_heads, softmax_scale, k_scale=None, v_scale=None,
           return_probs=False, row_block=256, window=None):
    """q: [total_q, Hq, D] (sequences concatenated, seq b owns q_lens[b] rows).
    Returns o [total_q, Hq, D] float64, m and l [total_q, Hq]
    (m in natural-log units), and the probabilities when asked (tiny inputs).
    ``window=None`` is causal attention; an integer W >= 0 is the non-causal
    sliding window of W keys."""
    q = np.asarray(q)
    total_q, Hq, D = q.shape
    Hkv = int(num_kv_heads)
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    scale = np.float64(np.float32(softmax_scale))
    o = np.zeros((total_q, Hq, D))
    m = np.full((total_q, Hq), -np.inf)
    l = np.zeros((total_q, Hq))
    probs = {} if return_probs else None
    start = 0
    for b, (qlen, ctx) in enumerate(zip(q_lens, ctx_lens)):
        qlen, ctx = int(qlen), int(ctx)
        for g in range(Hkv):
            K, V = paged.gather(k_cache, v_cache, block_tables[b], ctx, g, fmt,
                                k_scale, v_scale)
            for i0 in range(0, qlen, row_block):
                i1 = min(qlen, i0 + row_block)
                for gh in range(G):
                    h = g * G + gh
                    rows = q[start + i0:start + i1, h, :].astype(np.float64)
                    pos = ctx - qlen + np.arange(i0, i1)
                    if window is None:
                        ob, mb, lb, Pb = _rows_attend(rows, pos, K, V, scale)
                    else:
                        lo, hi = _row_keys(pos, ctx, window)
                        ob, mb, lb, Pb = _rows_attend_range(rows, lo, hi, K, V, scale)
                    o[start + i0:start + i1, h] = ob
                    m[start + i0:start + i1, h] = mb
                    l[start + i0:start + i1, h] = lb
                    if return_probs:
                        for r in range(i1 - i0):
                            probs[(start + i0 + r, h)] = Pb[r]
        start += qlen
    if return_probs:
        return o, m, l, probs
    return o, m, l


def attend_rows(q_rows, heads, positions, seq_ctx, k_cache, v_cache, block_table,
                fmt, num_q_heads, num_kv_heads, softmax_scale, k_scale=None, v_scale=None,
                window=None, row_block=256):
    """The same definition for selected rows of one sequence: q_rows [R, D],
    heads [R] (the query head of each row), positions [R]. Each row's result
    depends only on its own query, head and position, so any subset of rows
    can be computed on its own; rows of one KV head share that head's gather
    and are taken ``row_block`` at a time. Returns o [R, D]."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    heads = np.asarray(heads, dtype=np.int64).reshape(-1)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    G = num_q_heads // num_kv_heads
    scale = np.float64(np.float32(softmax_scale))
    out = np.zeros((len(heads), q_rows.shape[1]))
    kv = heads // G
    for g in np.unique(kv):
        idx = np.nonzero(kv == g)[0]
        K, V = paged.gather(k_cache, v_cache, block_table, seq_ctx, int(g), fmt,
                            k_scale, v_scale)
        for i0 in range(0, len(idx), row_block):
            sel = idx[i0:i0 + row_block]
            pos = positions[sel]
            if window is None:
                ob, _, _, _ = _rows_attend(q_rows[sel], pos, K, V, scale, probs=False)
            else:
                lo, hi = _row_keys(pos, seq_ctx, window)
                ob, _, _, _ = _rows_attend_range(q_rows[sel], lo, hi, K, V, scale, probs=False)
            out[sel] = ob
    return out


def decode(q, ctx_lens, k_cache, v_cache, block_tables, fmt, num_kv_heads,
           softmax_scale, k_scale=None, v_scale=None):
    """q [B, Hq, D]: one query per sequence at position ctx_b - 1."""
    B = q.shape[0]
    o, m, l = attend(q, [1] * B, ctx_lens, k_cache, v_cache, block_tables, fmt,
                     num_kv_heads, softmax_scale, k_scale, v_scale)
    return o


def verify(q, ctx_lens, k_cache, v_cache, block_tables, fmt, num_kv_heads,
           softmax_scale, k_scale=None, v_scale=None):
    """q [B, q_len, Hq, D]: the q_len newest positions of each sequence, each
    attending causally (the grouped speculative-verify step)."""
    B, qlen, Hq, D = q.shape
    o, m, l = attend(q.reshape(B * qlen, Hq, D), [qlen] * B, ctx_lens, k_cache,
                     v_cache, block_tables, fmt, num_kv_heads, softmax_scale,
                     k_scale, v_scale)
    return o.reshape(B, qlen, Hq, D)


def attend_partitioned(q, q_lens, ctx_lens, k_cache, v_cache, block_tables, fmt,
                       num_kv_heads, softmax_scale, partition_len,
                       k_scale=None, v_scale=None):
    """Split-KV form: keys [p*L, (p+1)*L) form partition p. Each partition
    yields (m_p, l_p, O_p = sum_j exp(s_j - m_p) V_j); partitions are merged by
    M = max_p m_p, w_p = exp(m_p - M), o = sum_p w_p O_p / sum_p w_p l_p.
    Partitions with no visible key (m_p = -inf, l_p = 0) are left out."""
    q = np.asarray(q)
    total_q, Hq, D = q.shape
    Hkv = int(num_kv_heads)
    G = Hq // Hkv
    scale = np.float64(np.float32(softmax_scale))
    L = int(partition_len)
    o = np.zeros((total_q, Hq, D))
    start = 0
    for b, (qlen, ctx) in enumerate(zip(q_lens, ctx_lens)):
        qlen, ctx = int(qlen), int(ctx)
        for g in range(Hkv):
            K, V = paged.gather(k_cache, v_cache, block_tables[b], ctx, g, fmt,
                                k_scale, v_scale)
            for i in range(qlen):
                pos = ctx - qlen + i
                for gh in range(G):
                    h = g * G + gh
                    qv = q[start + i, h].astype(np.float64)
                    parts = []
                    for p0 in range(0, max(ctx, 1), L):
                        hi = min(p0 + L, pos + 1)
                        if hi <= p0:
                            continue
                        s = scale * (K[p0:hi] @ qv)
                        mp = s.max()
                        e = np.exp(s - mp)
                        parts.append((mp, e.sum(), e @ V[p0:hi]))
                    if not parts:
                        continue
                    M = max(mp for mp, _, _ in parts)
                    w = [np.exp(mp - M) for mp, _, _ in parts]
                    num = sum(wp * Op for wp, (_, _, Op) in zip(w, parts))
                    den = sum(wp * lp for wp, (_, lp, _) in zip(w, parts))
                    o[start + i, h] = num / den
        start += qlen
    return o


def useful_flops(q_lens, ctx_lens, num_q_heads, head_dim):
    """"Useful causal" FLOPs (counting only unmasked work, as the 1.5.0 notes
    do for the long-prefill kernel): 4 * D per visible (query head, key) pair,
    2 * D for q.k and 2 * D for p * v."""
    pairs = 0
    for qlen, ctx in zip(q_lens, ctx_lens):
        qlen, ctx = int(qlen), int(ctx)
        for i in range(qlen):
            pairs += max(0, ctx - qlen + i + 1)
    return 4 * head_dim * num_q_heads * pairs

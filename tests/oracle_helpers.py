"""Test-side glue: build the oracle's paged cache for a synthetic workload.

Test infrastructure only: this module calls ``oracle`` and the seeded
generators in ``attention_paged_flashattention_amd.synth``; it never touches
the HIP library. Every cache byte is written by the oracle's own
``paged.write_tokens`` (pinned against the per-token ``paged.write``).
"""

import numpy as np

from attention_paged_flashattention_amd import synth
from oracle import paged


def poison_fill(fmt):
    """NaN pattern of unwritten cache slots (a code, or an fp16 NaN)."""
    return {"f16": np.float16(np.nan), "e4m3": synth.POISON["e4m3"],
            "e5m2": synth.POISON["e5m2"]}[fmt]


def new_oracle_caches(case):
    return paged.new_caches(case.num_blocks, case.num_kv_heads, case.block_size,
                            case.head_dim, case.cache_fmt, fill=poison_fill(case.cache_fmt))


def oracle_cache(case, tokens=None):
    """The oracle's own cache for ``case``: poisoned everywhere, then every
    token (or the given token indices) written through its slot."""
    kc, vc = new_oracle_caches(case)
    k32 = synth.to_f32(case.k, case.kv_dtype)
    v32 = synth.to_f32(case.v, case.kv_dtype)
    idx = np.arange(len(case.slot_mapping)) if tokens is None else np.asarray(tokens)
    paged.write_tokens(k32[idx], v32[idx], case.slot_mapping[idx], kc, vc, case.cache_fmt,
                       case.k_scale, case.v_scale)
    return kc, vc


def oracle_cache_heads(case, seqs_heads):
    """Oracle cache holding only the listed (sequence, KV head) pairs, every
    other slot poisoned; enough for rows that read those heads."""
    kc, vc = new_oracle_caches(case)
    for b, g in seqs_heads:
        t0, c = int(case.tok_start[b]), int(case.ctx_lens[b])
        k32 = synth.to_f32(case.k[t0:t0 + c, g:g + 1, :], case.kv_dtype)
        v32 = synth.to_f32(case.v[t0:t0 + c, g:g + 1, :], case.kv_dtype)
        paged.write_tokens(k32, v32, case.slot_mapping[t0:t0 + c], kc, vc, case.cache_fmt,
                           case.k_scale, case.v_scale, heads=[g])
    return kc, vc


def q_f32(case):
    return synth.to_f32(case.q, case.q_dtype)

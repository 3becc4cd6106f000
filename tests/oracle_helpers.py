"""Test-side glue: build the oracle's paged cache for a synthetic workload.

Test infrastructure only: this module calls ``oracle`` and the seeded
generators in ``attention_paged_flashattention_amd.synth``; it never touches
the HIP library.
"""

import numpy as np

from attention_paged_flashattention_amd import synth
from oracle import paged


def oracle_cache(case, tokens=None):
    """The oracle's own cache for ``case``: poisoned everywhere, then every
    token (or the given token indices) written through its slot."""
    fill = {"f16": np.float16(np.nan), "e4m3": synth.POISON["e4m3"],
            "e5m2": synth.POISON["e5m2"]}[case.cache_fmt]
    kc, vc = paged.new_caches(case.num_blocks, case.num_kv_heads, case.block_size,
                              case.head_dim, case.cache_fmt, fill=fill)
    k32 = synth.to_f32(case.k, case.kv_dtype)
    v32 = synth.to_f32(case.v, case.kv_dtype)
    idx = np.arange(len(case.slot_mapping)) if tokens is None else np.asarray(tokens)
    write_tokens(case, kc, vc, k32[idx], v32[idx], case.slot_mapping[idx])
    return kc, vc


def write_tokens(case, kc, vc, k32, v32, slots):
    """Vectorised form of oracle.paged.write for many tokens at once (the
    per-element arithmetic is oracle.paged.quantize, unchanged)."""
    bs = case.block_size
    T = paged.value_group(bs)
    keep = slots >= 0
    slots = slots[keep]
    page, off = slots // bs, slots % bs
    kq = paged.quantize(k32[keep], case.cache_fmt, None if case.k_scale is None else case.k_scale[None, :, None])
    vq = paged.quantize(v32[keep], case.cache_fmt, None if case.v_scale is None else case.v_scale[None, :, None])
    for h in range(case.num_kv_heads):
        kc[page, h, off, :] = kq[:, h, :]
        vc[page, h, off // T, :, off % T] = vq[:, h, :]


def q_f32(case):
    return synth.to_f32(case.q, case.q_dtype)

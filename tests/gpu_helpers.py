"""Shared pieces of the GPU parity tests: tolerances and oracle references.

Tolerances (max-abs, against the float64 oracle fed the same dequantized
values): 2e-3 for an fp16 KV cache, 8e-3 for an FP8 cache, with outputs
stored as float32. When the output is stored in the query dtype the store
itself may add half an ulp of that dtype at the reference's magnitude.
"""

import sys

import numpy as np
import torch

from attention_paged_flashattention_amd import synth
from oracle import attention
from tests.oracle_helpers import oracle_cache, oracle_cache_heads, q_f32  # noqa: F401

TOL = {"f16": 2e-3, "e4m3": 8e-3, "e5m2": 8e-3}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def half_ulp(ref, dtype):
    a = np.abs(ref)
    if dtype == torch.float16:
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
        return 0.5 * 2.0 ** (e - 10)
    if dtype == torch.bfloat16:
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
        return 0.5 * 2.0 ** (e - 7)
    return np.zeros_like(a)


def check_close(got, ref, fmt, what, out_dtype=torch.float32):
    got = got.detach().float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = TOL[fmt] + half_ulp(ref, out_dtype)
    worst = float(np.max(err - bound)) if err.size else -1.0
    log(f"  {what}: max|err| = {float(err.max()) if err.size else 0:.3e} (tol {TOL[fmt]:.0e})")
    assert worst <= 0.0, f"{what}: max abs error {float(err.max()):.3e} exceeds tolerance"
    return float(err.max()) if err.size else 0.0


def oracle_full(case, kc=None, vc=None):
    """Oracle output for every query row of the case, [total_q, Hq, D]."""
    if kc is None:
        kc, vc = oracle_cache(case)
    o, _, _ = attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                               case.block_tables, case.cache_fmt, case.num_kv_heads,
                               case.softmax_scale, case.k_scale, case.v_scale)
    return o


def oracle_rows(case, kc, vc, b, q_rows_f32, heads, positions, window=None):
    return attention.attend_rows(q_rows_f32, heads, positions, int(case.ctx_lens[b]), kc, vc,
                                 case.block_tables[b], case.cache_fmt, case.num_q_heads,
                                 case.num_kv_heads, case.softmax_scale, case.k_scale, case.v_scale,
                                 window=window)

"""Pins for the oracle's row sampler and its cache builders (CPU only).

The full-size GPU checks compare against ``oracle.attention.attend_rows``
(selected rows of one sequence) over caches built by
``oracle.paged.write_tokens`` (``tests.oracle_helpers.oracle_cache`` and
``oracle_cache_heads``). These tests tie each of them to a function pinned
elsewhere:

* ``attend_rows`` equals ``attend`` (itself pinned against torch's float64
  SDPA, closed forms and invariants) row for row, for causal and
  sliding-window rows, GQA ratios 1, 4 and 6, rows on chunk and page edges,
  rows given in any order, and a sequence shorter than its query block
  (rows with no visible key are zeros);
* planted mistakes in the oracle (a wrong KV head, a position off by one)
  make that comparison fail;
* ``write_tokens`` over a subset of KV heads, and ``oracle_cache_heads``,
  write exactly the bytes the per-token ``paged.write`` writes for those heads
  and leave every other slot poisoned.
"""

import numpy as np
import pytest

from attention_paged_flashattention_amd import synth
from oracle import attention, paged
from tests.oracle_helpers import (new_oracle_caches, oracle_cache, oracle_cache_heads, q_f32)


def _case(fmt, ctx, q_len, Hq, Hkv, D=32, bs=16, q_dtype="f16", seed=5, sigma_kv=1.0):
    kv_dtype = "bf16" if q_dtype == "bf16" and fmt != "f16" else "f16"
    return synth.make_case("rows", seed, list(ctx), q_len, Hq, Hkv, D, bs, q_dtype, kv_dtype,
                           fmt, sigma_kv=sigma_kv)


def _rows_vs_attend(case, window=None, kc=None, vc=None, ref=None, seed=0):
    """max |attend_rows - attend| over every row of every sequence, the rows
    handed to attend_rows in a shuffled order."""
    if kc is None:
        kc, vc = oracle_cache(case)
    q = q_f32(case)
    if ref is None:
        ref, _, _ = attention.attend(q, case.q_lens, case.ctx_lens, kc, vc, case.block_tables,
                                     case.cache_fmt, case.num_kv_heads, case.softmax_scale,
                                     case.k_scale, case.v_scale, window=window)
    rng = np.random.default_rng(seed)
    err = 0.0
    start = 0
    for b in range(case.batch):
        ql, c = int(case.q_lens[b]), int(case.ctx_lens[b])
        ii, hh = np.meshgrid(np.arange(ql), np.arange(case.num_q_heads), indexing="ij")
        ii, hh = ii.reshape(-1), hh.reshape(-1)
        order = rng.permutation(len(ii))
        ii, hh = ii[order], hh[order]
        got = attention.attend_rows(q[start + ii, hh], hh, c - ql + ii, c, kc, vc,
                                    case.block_tables[b], case.cache_fmt, case.num_q_heads,
                                    case.num_kv_heads, case.softmax_scale, case.k_scale,
                                    case.v_scale, window=window, row_block=7)
        err = max(err, float(np.max(np.abs(got - ref[start + ii, hh]))))
        start += ql
    return err


ROW_CASES = [
    # fmt, ctx, q_len, Hq, Hkv, bs, q_dtype, window
    ("e4m3", (37, 70), 5, 8, 2, 16, "f16", None),           # G 4, decode-like block
    ("e5m2", (20, 90), 8, 4, 4, 16, "f16", 7),              # G 1, sliding window
    ("f16", (40, 100), 40, 12, 2, 16, "f16", None),         # G 6, chunk over page edges
    ("e4m3", (3, 5), 8, 8, 2, 16, "f16", None),             # ctx < q_len: leading rows empty
    ("e4m3", (65, 129), 33, 8, 2, 32, "bf16", 0),           # window 0, bf16 queries
    ("e5m2", (64, 128), 64, 6, 1, 64, "f16", None),         # G 6, chunk = whole pages
]


@pytest.mark.parametrize("fmt,ctx,q_len,Hq,Hkv,bs,q_dtype,window", ROW_CASES,
                         ids=[str(i) for i in range(len(ROW_CASES))])
def test_attend_rows_equals_attend(fmt, ctx, q_len, Hq, Hkv, bs, q_dtype, window):
    case = _case(fmt, ctx, q_len, Hq, Hkv, bs=bs, q_dtype=q_dtype,
                 sigma_kv=0.5 if fmt == "e5m2" else 1.0)
    assert _rows_vs_attend(case, window) < 1e-13


def test_rows_without_a_visible_key_are_zero():
    case = _case("e4m3", (3,), 8, 8, 2)
    kc, vc = oracle_cache(case)
    q = q_f32(case)
    heads = np.arange(8)
    got = attention.attend_rows(q[0, heads], heads, np.full(8, -5), 3, kc, vc,
                                case.block_tables[0], "e4m3", 8, 2, case.softmax_scale,
                                case.k_scale, case.v_scale)
    assert np.all(got == 0)


@pytest.mark.parametrize("mutant", ["head_map", "position_off_by_one", "window_shift"])
def test_planted_row_sampler_mistakes_fail(monkeypatch, mutant):
    case = _case("e4m3", (37, 70), 5, 8, 2)
    kc, vc = oracle_cache(case)
    window = 6 if mutant == "window_shift" else None
    ref, _, _ = attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                                 case.block_tables, "e4m3", case.num_kv_heads,
                                 case.softmax_scale, case.k_scale, case.v_scale, window=window)
    if mutant == "head_map":
        orig = paged.gather

        def gather_wrong_head(kc_, vc_, bt, ctx, g, *a, **k):
            return orig(kc_, vc_, bt, ctx, (g + 1) % case.num_kv_heads, *a, **k)
        monkeypatch.setattr(paged, "gather", gather_wrong_head)
    elif mutant == "position_off_by_one":
        orig = attention._rows_attend
        monkeypatch.setattr(attention, "_rows_attend",
                            lambda qr, pos, K, V, s, probs=True: orig(qr, pos - 1, K, V, s, probs))
    else:
        orig = attention._row_keys
        monkeypatch.setattr(attention, "_row_keys",
                            lambda pos, ctx, w: orig(pos + 1, ctx, w))
    assert _rows_vs_attend(case, window, kc, vc, ref) > 1e-6


@pytest.mark.parametrize("fmt,bs", [("e4m3", 16), ("e5m2", 64), ("f16", 32)])
def test_write_tokens_subset_matches_per_token_write(fmt, bs):
    case = _case(fmt, (45, 77, 3), 1, 8, 4, bs=bs)
    k32 = synth.to_f32(case.k, case.kv_dtype)
    v32 = synth.to_f32(case.v, case.kv_dtype)
    slots = case.slot_mapping.copy()
    slots[::5] = -1                                  # skipped tokens
    full_k, full_v = new_oracle_caches(case)
    paged.write(k32, v32, slots, full_k, full_v, fmt, case.k_scale, case.v_scale)
    heads = [3, 1]
    kc, vc = new_oracle_caches(case)
    paged.write_tokens(k32[:, heads], v32[:, heads], slots, kc, vc, fmt, case.k_scale,
                       case.v_scale, heads=heads)
    pk, pv = new_oracle_caches(case)
    for h in range(case.num_kv_heads):
        ek, ev = (full_k, full_v) if h in heads else (pk, pv)
        assert np.array_equal(kc[:, h].view(np.uint8), ek[:, h].view(np.uint8)), h
        assert np.array_equal(vc[:, h].view(np.uint8), ev[:, h].view(np.uint8)), h
    # all heads at once equals the per-token write everywhere
    ka, va = new_oracle_caches(case)
    paged.write_tokens(k32, v32, slots, ka, va, fmt, case.k_scale, case.v_scale)
    assert np.array_equal(ka.view(np.uint8), full_k.view(np.uint8))
    assert np.array_equal(va.view(np.uint8), full_v.view(np.uint8))


def test_oracle_cache_heads_matches_per_token_write():
    case = _case("e4m3", (45, 77), 1, 8, 4, bs=16)
    pairs = [(0, 2), (1, 0), (1, 3)]
    kc, vc = oracle_cache_heads(case, pairs)
    # expected: the per-token write of sequence b's tokens, copied for head g
    full_k, full_v = new_oracle_caches(case)
    paged.write(synth.to_f32(case.k, "f16"), synth.to_f32(case.v, "f16"), case.slot_mapping,
                full_k, full_v, "e4m3", case.k_scale, case.v_scale)
    ek, ev = new_oracle_caches(case)
    bs, T = case.block_size, paged.value_group(case.block_size)
    for b, g in pairs:
        t0, c = int(case.tok_start[b]), int(case.ctx_lens[b])
        for t in range(t0, t0 + c):
            page, off = divmod(int(case.slot_mapping[t]), bs)
            ek[page, g, off] = full_k[page, g, off]
            ev[page, g, off // T, :, off % T] = full_v[page, g, off // T, :, off % T]
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    # and rows of those heads agree with the oracle on the whole cache
    kf, vf = oracle_cache(case)
    q = q_f32(case)
    for b, g in pairs:
        c = int(case.ctx_lens[b])
        heads = np.arange(g * 2, g * 2 + 2)
        qr = q[b][heads]
        a = attention.attend_rows(qr, heads, [c - 1] * 2, c, kc, vc, case.block_tables[b],
                                  "e4m3", 8, 4, case.softmax_scale, case.k_scale, case.v_scale)
        f = attention.attend_rows(qr, heads, [c - 1] * 2, c, kf, vf, case.block_tables[b],
                                  "e4m3", 8, 4, case.softmax_scale, case.k_scale, case.v_scale)
        assert np.array_equal(a, f)


def test_oracle_pool_matches_attend():
    """The worker pool (shared memory-mapped cache, one process per piece of
    (sequence, KV head) work) returns exactly the oracle's rows: the cache it
    builds is byte-identical to oracle_cache, and its rows equal attend."""
    from tests.oracle_pool import OraclePool, row_tasks
    case = _case("e4m3", (45, 77), 5, 8, 2, bs=16)
    kc, vc = oracle_cache(case)
    ref, _, _ = attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                                 case.block_tables, "e4m3", 2, case.softmax_scale,
                                 case.k_scale, case.v_scale)
    with OraclePool(case, workers=2, tmp_root=None) as pool:
        pairs = [(b, g) for b in range(2) for g in range(2)]
        pool.build(pairs, pieces=3)
        built_k = np.load(pool.dir + "/kc.npy")
        built_v = np.load(pool.dir + "/vc.npy")
        assert np.array_equal(built_k, kc) and np.array_equal(built_v, vc)
        got = np.full_like(ref, np.nan)
        for b, g in pairs:
            tasks, index = row_tasks(case, b, g, np.arange(5), split=2)
            for rows, (t, h) in zip(pool.run(tasks), index):
                got[b * 5 + t, h] = rows
    assert np.array_equal(got, ref) or np.max(np.abs(got - ref)) < 1e-13

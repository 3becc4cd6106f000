"""Pins for the oracle's non-causal sliding-window attention (CPU only).

Reading pinned here: query i of a block of q_len at position
pos = ctx - q_len + i attends the keys j with pos - W <= j < ctx (a left
window of W keys, no causal mask inside the block). It is checked against
things other than itself:

* a library routine: torch's scaled_dot_product_attention in float64 on
  unpaged K/V with that window written out as an explicit boolean mask;
* closed forms: W = 0 at q_len 1 returns the last value; Q = 0 returns the
  mean of the values in the window (a cumulative-sum formula);
* invariants: W >= ctx makes every row of the block equal the causal
  oracle's last-position row for the same query; shifting the block by
  unrelated prefix keys outside every window changes nothing;
* planted mistakes (a window one key too short, a causal mask inside the
  block, the window anchored at the block end instead of each row) must fail
  the library cross-check.
"""

import numpy as np
import pytest
import torch

from oracle import attention
from tests.oracle_helpers import oracle_cache, q_f32
from tests.test_oracle_attention import _case, _contig_kv


def _window_oracle(case, W, kc=None, vc=None):
    if kc is None:
        kc, vc = oracle_cache(case)
    o, _, _ = attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                               case.block_tables, case.cache_fmt, case.num_kv_heads,
                               case.softmax_scale, case.k_scale, case.v_scale, window=W)
    return o


def _window_sdpa(case, W):
    q = q_f32(case).astype(np.float64)
    outs, start, G = [], 0, case.gqa
    for b in range(case.batch):
        ql, c = int(case.q_lens[b]), int(case.ctx_lens[b])
        K, V = _contig_kv(case, b)
        qt = torch.from_numpy(q[start:start + ql]).permute(1, 0, 2)
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
        pos = c - ql + torch.arange(ql)
        j = torch.arange(c)[None, :]
        mask = (j >= pos[:, None] - W) & (j < c)
        o = torch.nn.functional.scaled_dot_product_attention(
            qt.contiguous(), kt.contiguous(), vt.contiguous(), attn_mask=mask,
            scale=float(np.float64(np.float32(case.softmax_scale))))
        outs.append(o.permute(1, 0, 2).numpy())
        start += ql
    return np.concatenate(outs, 0)


@pytest.mark.parametrize("fmt,W,q_len,ctx,bs", [
    ("e4m3", 0, 1, (37, 70), 16),
    ("e4m3", 5, 8, (37, 70), 16),
    ("e5m2", 17, 4, (90, 33), 32),
    ("f16", 40, 8, (64, 130), 16),
    ("e4m3", 1000, 8, (37, 70), 16),
    ("e5m2", 63, 16, (200, 65), 64),
])
def test_window_matches_sdpa_with_explicit_mask(fmt, W, q_len, ctx, bs):
    case = _case(fmt=fmt, B=2, ctx=ctx, q_len=q_len, bs=bs)
    o = _window_oracle(case, W)
    ref = _window_sdpa(case, W)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_window_zero_decode_returns_last_value():
    case = _case(fmt="e4m3", B=2, ctx=(37, 70), q_len=1)
    kc, vc = oracle_cache(case)
    o = _window_oracle(case, 0, kc, vc)
    for b in range(2):
        K, V = _contig_kv(case, b)
        c = int(case.ctx_lens[b])
        for h in range(case.num_q_heads):
            assert np.array_equal(o[b, h], V[c - 1, h // case.gqa])


@pytest.mark.parametrize("W", [0, 3, 12, 500])
def test_window_zero_query_is_window_mean(W):
    case = _case(fmt="e5m2", B=2, ctx=(37, 70), q_len=6)
    case.q[:] = 0
    o = _window_oracle(case, W)
    start = 0
    for b in range(2):
        K, V = _contig_kv(case, b)
        c, ql = int(case.ctx_lens[b]), int(case.q_lens[b])
        cs = np.concatenate([np.zeros((1,) + V.shape[1:]), np.cumsum(V, axis=0)])
        for i in range(ql):
            pos = c - ql + i
            lo = max(0, pos - W)
            mean = (cs[c] - cs[lo]) / (c - lo)           # [Hkv, D]
            for h in range(case.num_q_heads):
                np.testing.assert_allclose(o[start + i, h], mean[h // case.gqa], atol=1e-12)
        start += ql


def test_window_covering_everything_equals_causal_last_row():
    """W >= ctx: every query of the block sees all ctx keys, which is what the
    causal oracle gives a query placed at the last position."""
    case = _case(fmt="e4m3", B=2, ctx=(37, 70), q_len=5)
    kc, vc = oracle_cache(case)
    o = _window_oracle(case, 10**6, kc, vc)
    q = q_f32(case)
    start = 0
    for b in range(2):
        ql, c = int(case.q_lens[b]), int(case.ctx_lens[b])
        for i in range(ql):
            oc, _, _ = attention.attend(q[start + i:start + i + 1], [1], [c], kc, vc,
                                        case.block_tables[b:b + 1], "e4m3", case.num_kv_heads,
                                        case.softmax_scale, case.k_scale, case.v_scale)
            np.testing.assert_allclose(o[start + i], oc[0], atol=1e-13)
        start += ql


def test_window_ignores_keys_outside_every_window():
    """Overwriting the cached values of keys older than every row's window
    (positions < ctx - q_len - W) changes no output."""
    case = _case(fmt="f16", B=1, ctx=(90,), q_len=4, bs=16)
    W = 20
    kc, vc = oracle_cache(case)
    o1 = _window_oracle(case, W, kc, vc)
    kc2, vc2 = kc.copy(), vc.copy()
    bs = case.block_size
    T = vc.shape[-1]
    for j in range(90 - 4 - W):
        page = int(case.block_tables[0][j // bs])
        kc2[page, :, j % bs, :] = np.float16(7.0)
        vc2[page, :, (j % bs) // T, :, (j % bs) % T] = np.float16(-9.0)
    o2 = _window_oracle(case, W, kc2, vc2)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("mutant", ["short_by_one", "causal_inside", "anchored_at_end"])
def test_planted_window_mistakes_fail_the_library_check(monkeypatch, mutant):
    case = _case(fmt="e4m3", B=2, ctx=(37, 70), q_len=8)
    W = 9
    orig = attention._row_keys
    if mutant == "short_by_one":
        monkeypatch.setattr(attention, "_row_keys",
                            lambda pos, ctx, w: (lambda lo, hi: (lo + 1, hi))(*orig(pos, ctx, w)))
    elif mutant == "causal_inside":
        monkeypatch.setattr(attention, "_row_keys",
                            lambda pos, ctx, w: (orig(pos, ctx, w)[0], np.asarray(pos)))
    elif mutant == "anchored_at_end":
        monkeypatch.setattr(attention, "_row_keys",
                            lambda pos, ctx, w: (np.full_like(np.asarray(pos), ctx - 1 - w),
                                                 orig(pos, ctx, w)[1]))
    o = _window_oracle(case, W)
    ref = _window_sdpa(case, W)
    assert not (np.max(np.abs(o - ref)) < 1e-6), mutant

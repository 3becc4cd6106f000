"""Pins for the oracle's paged attention (CPU only).

The oracle is checked against things other than itself:

* a library routine: torch's scaled_dot_product_attention on the CPU in
  float64, fed K/V that were quantized and dequantized in token order with no
  paging at all, GQA expanded with repeat_interleave and an explicit
  causal-with-offset boolean mask;
* a hand-worked example (tests/golden/attention_worked_example.json);
* closed forms: one visible key returns its value, constant V returns the
  constant, Q = 0 gives the causal prefix mean, a dominant score returns its
  value;
* invariants: probabilities sum to 1, paged == contiguous, invariance to the
  physical page permutation, decode == last prefill row, verify row i ==
  decode at ctx - q_len + 1 + i, chunked == unchunked prefill, GQA == MHA
  with repeated KV heads, split-KV log-sum-exp == unsplit, o(2V) = 2 o(V);
* planted mistakes (a wrong head mapping, an off-by-one causal mask, a dropped
  softmax scale, the V layout read as the K layout) must fail the library
  cross-check.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from attention_paged_flashattention_amd import synth
from oracle import attention, fp8, paged
from tests.oracle_helpers import oracle_cache, q_f32


def _case(fmt="e4m3", B=2, ctx=(37, 70), q_len=5, Hq=8, Hkv=2, D=32, bs=16, seed=7,
          q_dtype="f16", sigma_kv=1.0):
    kv_dtype = "bf16" if q_dtype == "bf16" and fmt != "f16" else "f16"
    return synth.make_case("t", seed, list(ctx)[:B], q_len, Hq, Hkv, D, bs, q_dtype,
                           kv_dtype, fmt, sigma_kv=sigma_kv)


def _contig_kv(case, b):
    """Dequantized K/V of sequence b in token order, never paged: quantize then
    dequantize each token directly (independent of slots and block tables)."""
    t0, c = int(case.tok_start[b]), int(case.ctx_lens[b])
    k32 = synth.to_f32(case.k[t0:t0 + c], case.kv_dtype)
    v32 = synth.to_f32(case.v[t0:t0 + c], case.kv_dtype)
    if case.cache_fmt == "f16":
        return k32.astype(np.float16).astype(np.float64), v32.astype(np.float16).astype(np.float64)
    ks = None if case.k_scale is None else case.k_scale[None, :, None]
    vs = None if case.v_scale is None else case.v_scale[None, :, None]
    K = fp8.dequant(fp8.encode(k32, case.cache_fmt, ks), case.cache_fmt, ks)
    V = fp8.dequant(fp8.encode(v32, case.cache_fmt, vs), case.cache_fmt, vs)
    return K, V


def _sdpa(case):
    """torch float64 SDPA per sequence on unpaged K/V."""
    q = q_f32(case).astype(np.float64)
    outs = []
    start = 0
    G = case.gqa
    for b in range(case.batch):
        ql, c = int(case.q_lens[b]), int(case.ctx_lens[b])
        K, V = _contig_kv(case, b)                         # [c, Hkv, D]
        qt = torch.from_numpy(q[start:start + ql]).permute(1, 0, 2)          # [Hq, ql, D]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)    # [Hq, c, D]
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
        pos = c - ql + torch.arange(ql)
        mask = torch.arange(c)[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt.contiguous(), kt.contiguous(), vt.contiguous(), attn_mask=mask,
            scale=float(np.float64(np.float32(case.softmax_scale))))
        outs.append(o.permute(1, 0, 2).numpy())
        start += ql
    return np.concatenate(outs, 0)


def _oracle(case, kc=None, vc=None, **kw):
    if kc is None:
        kc, vc = oracle_cache(case)
    return attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                            case.block_tables, case.cache_fmt, case.num_kv_heads,
                            case.softmax_scale, case.k_scale, case.v_scale, **kw)


CASES = [
    dict(fmt="e4m3"),
    dict(fmt="e5m2", sigma_kv=0.5),
    dict(fmt="f16"),
    dict(fmt="e4m3", q_dtype="bf16", bs=32, D=64),
    dict(fmt="e4m3", Hq=4, Hkv=4, q_len=1),
    dict(fmt="e5m2", Hq=8, Hkv=1, q_len=8, ctx=(9, 130), bs=64),
    dict(fmt="f16", Hq=4, Hkv=1, D=64, q_len=17, ctx=(17, 64)),
]


@pytest.mark.parametrize("kw", CASES, ids=[str(i) for i in range(len(CASES))])
def test_oracle_matches_torch_sdpa_float64(kw):
    case = _case(**kw)
    o, m, l = _oracle(case)
    ref = _sdpa(case)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_vectorised_write_matches_plain_write():
    case = _case(fmt="e4m3")
    kc1, vc1 = oracle_cache(case)
    kc2, vc2 = paged.new_caches(case.num_blocks, case.num_kv_heads, case.block_size,
                                case.head_dim, "e4m3", fill=synth.POISON["e4m3"])
    paged.write(synth.to_f32(case.k, "f16"), synth.to_f32(case.v, "f16"),
                case.slot_mapping, kc2, vc2, "e4m3", case.k_scale, case.v_scale)
    assert np.array_equal(kc1, kc2) and np.array_equal(vc1, vc2)


def test_golden_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "attention_worked_example.json")))
    D = ex["head_dim"]
    keys = np.array(ex["keys"], dtype=np.float16)
    vals = np.array(ex["values"], dtype=np.float16)
    n = len(keys)
    bs = ex["block_size"]
    kc, vc = paged.new_caches(2, 1, bs, D, "f16", fill=np.float16(np.nan))
    bt = np.array([[1, synth.INT32_MAX]], dtype=np.int32)   # physical page 1
    slots = np.arange(n) + 1 * bs
    paged.write(keys[:, None, :], vals[:, None, :], slots, kc, vc, "f16")
    q = np.tile(np.array(ex["q"], dtype=np.float16), (n, 1))[:, None, :]
    o, m, l, P = attention.attend(q, [n], [n], kc, vc, bt, "f16", 1,
                                  ex["softmax_scale"], return_probs=True)
    tol = ex["tolerance"]
    assert np.max(np.abs(o[:, 0, :] - np.array(ex["prefill_expected"]))) < tol
    for i, w in enumerate(ex["prefill_weights_expected"]):
        assert np.max(np.abs(P[(i, 0)][:len(w)] - np.array(w))) < tol
    od = attention.decode(q[-1:], [n], kc, vc, bt, "f16", 1, ex["softmax_scale"])
    assert np.max(np.abs(od[0, 0] - np.array(ex["decode_expected"]))) < tol
    # the same example through E4M3 pages with a per-head scale of 0.5 is exact
    kc8, vc8 = paged.new_caches(2, 1, bs, D, "e4m3", fill=0x7F)
    s = np.array([0.5], dtype=np.float32)
    paged.write(keys[:, None, :], vals[:, None, :], slots, kc8, vc8, "e4m3", s, s)
    o8, _, _ = attention.attend(q, [n], [n], kc8, vc8, bt, "e4m3", 1, ex["softmax_scale"], s, s)
    assert np.max(np.abs(o8[:, 0, :] - np.array(ex["prefill_expected"]))) < tol


def test_probabilities_sum_to_one():
    case = _case(fmt="e4m3", B=1, ctx=(40,), q_len=6)
    o, m, l, P = _oracle(case, return_probs=True)
    for (r, h), p in P.items():
        assert abs(p.sum() - 1.0) < 1e-12
        pos = int(case.ctx_lens[0]) - 6 + r
        assert np.all(p[pos + 1:] == 0)


def test_single_visible_key_returns_its_value():
    case = _case(fmt="e4m3", B=1, ctx=(20,), q_len=20)     # row 0 sees only key 0
    kc, vc = oracle_cache(case)
    o, _, _ = _oracle(case, kc, vc)
    K, V = paged.gather(kc, vc, case.block_tables[0], 20, 0, "e4m3", case.k_scale, case.v_scale)
    for h in range(case.gqa):                               # heads of KV head 0
        assert np.array_equal(o[0, h], V[0])


def test_constant_v_gives_constant_output():
    case = _case(fmt="f16", B=2, ctx=(33, 50), q_len=4)
    case.v[:] = np.float16(-1.375)
    o, _, _ = _oracle(case)
    assert np.max(np.abs(o + 1.375)) < 1e-14


def test_zero_query_gives_causal_prefix_mean():
    case = _case(fmt="e5m2", B=1, ctx=(48,), q_len=48, Hq=2, Hkv=1)
    case.q[:] = 0
    kc, vc = oracle_cache(case)
    o, _, _ = _oracle(case, kc, vc)
    _, V = paged.gather(kc, vc, case.block_tables[0], 48, 0, "e5m2")
    mean = np.cumsum(V, axis=0) / np.arange(1, 49)[:, None]
    assert np.max(np.abs(o[:, 0] - mean)) < 1e-13
    assert np.max(np.abs(o[:, 1] - mean)) < 1e-13


def test_dominant_score_returns_its_value():
    case = _case(fmt="f16", B=1, ctx=(30,), q_len=1, Hq=1, Hkv=1, D=16)
    case.k[:] = 0
    case.q[:] = np.float16(1.0)
    case.k[11, 0, :] = np.float16(4.0)
    case.softmax_scale = 1.0                     # s_11 = 16 * 4 = 64, others 0: gap > 50
    o, _, _ = _oracle(case)
    _, V = _contig_kv(case, 0)
    assert np.max(np.abs(o[0, 0] - V[11, 0])) < 1e-20


def test_paged_equals_contiguous_and_permutation_invariance():
    case = _case(fmt="e4m3", B=2, ctx=(45, 77), bs=16)
    kc, vc = oracle_cache(case)
    for b in range(2):
        for g in range(case.num_kv_heads):
            K, V = paged.gather(kc, vc, case.block_tables[b], int(case.ctx_lens[b]), g,
                                "e4m3", case.k_scale, case.v_scale)
            Kc, Vc = _contig_kv(case, b)
            assert np.array_equal(K, Kc[:, g]) and np.array_equal(V, Vc[:, g])
    o1, _, _ = _oracle(case, kc, vc)
    # re-page: a new physical permutation of the pool, same logical content
    perm = np.random.default_rng(3).permutation(case.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = case.block_tables.copy()
    valid = bt2 != synth.INT32_MAX
    bt2[valid] = perm[bt2[valid]]
    o2, _, _ = attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc2, vc2, bt2,
                                "e4m3", case.num_kv_heads, case.softmax_scale,
                                case.k_scale, case.v_scale)
    assert np.array_equal(o1, o2)


def test_decode_equals_last_prefill_row():
    case = _case(fmt="e4m3", B=1, ctx=(57,), q_len=57)
    kc, vc = oracle_cache(case)
    o, _, _ = _oracle(case, kc, vc)
    q = q_f32(case)
    for i in [0, 13, 56]:
        od = attention.decode(q[i:i + 1], [i + 1], kc, vc, case.block_tables, "e4m3",
                              case.num_kv_heads, case.softmax_scale, case.k_scale, case.v_scale)
        assert np.max(np.abs(od[0] - o[i])) < 1e-14


def test_verify_rows_equal_decode():
    case = _case(fmt="e5m2", B=2, ctx=(40, 90), q_len=8)
    kc, vc = oracle_cache(case)
    q = q_f32(case).reshape(2, 8, case.num_q_heads, case.head_dim)
    ov = attention.verify(q, case.ctx_lens, kc, vc, case.block_tables, "e5m2",
                          case.num_kv_heads, case.softmax_scale)
    for b in range(2):
        c = int(case.ctx_lens[b])
        for i in range(8):
            od = attention.decode(q[b, i][None], [c - 7 + i], kc, vc, case.block_tables[b:b + 1],
                                  "e5m2", case.num_kv_heads, case.softmax_scale)
            assert np.max(np.abs(od[0] - ov[b, i])) < 1e-14


def test_chunked_equals_unchunked_prefill():
    case = _case(fmt="e4m3", B=1, ctx=(96,), q_len=96, bs=16)
    kc, vc = oracle_cache(case)
    o, _, _ = _oracle(case, kc, vc)
    q = q_f32(case)
    for c0, c1 in [(0, 32), (32, 64), (64, 96)]:
        # chunk [c0, c1) sees only the tokens written so far
        kcc, vcc = oracle_cache(case, tokens=np.arange(c1))
        oc, _, _ = attention.attend(q[c0:c1], [c1 - c0], [c1], kcc, vcc, case.block_tables,
                                    "e4m3", case.num_kv_heads, case.softmax_scale,
                                    case.k_scale, case.v_scale)
        assert np.max(np.abs(oc - o[c0:c1])) < 1e-14


def test_gqa_equals_mha_with_repeated_kv():
    case = _case(fmt="f16", B=1, ctx=(50,), q_len=3, Hq=8, Hkv=2)
    o, _, _ = _oracle(case)
    G = case.gqa
    mha = synth.make_case("m", 1, [50], 3, 8, 8, case.head_dim, case.block_size, "f16", "f16", "f16")
    mha.q = case.q
    mha.k = np.repeat(case.k, G, axis=1)
    mha.v = np.repeat(case.v, G, axis=1)
    mha.softmax_scale = case.softmax_scale
    mha.block_tables, mha.slot_mapping, mha.num_blocks = case.block_tables, case.slot_mapping, case.num_blocks
    o2, _, _ = _oracle(mha)
    assert np.max(np.abs(o - o2)) < 1e-15


@pytest.mark.parametrize("L", [1, 7, 16, 64, 1000])
def test_partitioned_lse_equals_unpartitioned(L):
    case = _case(fmt="e4m3", B=2, ctx=(45, 77), q_len=3)
    kc, vc = oracle_cache(case)
    o, _, _ = _oracle(case, kc, vc)
    op = attention.attend_partitioned(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                                      case.block_tables, "e4m3", case.num_kv_heads,
                                      case.softmax_scale, L, case.k_scale, case.v_scale)
    assert np.max(np.abs(o - op)) < 1e-12


def test_output_is_linear_in_v_scale():
    case = _case(fmt="e4m3")
    kc, vc = oracle_cache(case)
    o1, _, _ = _oracle(case, kc, vc)
    o2, _, _ = attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                                case.block_tables, "e4m3", case.num_kv_heads,
                                case.softmax_scale, case.k_scale, case.v_scale * 2)
    assert np.array_equal(o2, 2 * o1)


def test_empty_context_gives_zeros():
    case = _case(fmt="e4m3", B=2, ctx=(10, 20), q_len=1)
    kc, vc = oracle_cache(case)
    o, m, l = attention.attend(q_f32(case), [1, 1], [0, 20], kc, vc, case.block_tables,
                               "e4m3", case.num_kv_heads, case.softmax_scale,
                               case.k_scale, case.v_scale)
    assert np.all(o[0] == 0) and np.all(np.isneginf(m[0])) and np.all(l[0] == 0)
    assert np.all(np.isfinite(o[1]))


def test_poisoned_slots_never_reach_the_output():
    # every unwritten slot holds NaN codes; outputs must stay finite
    case = _case(fmt="e4m3", B=2, ctx=(33, 47), bs=16)
    o, _, _ = _oracle(case)
    assert np.all(np.isfinite(o))


def test_useful_flops_closed_form():
    # 32768 tokens in 8 chunks of 4096, Hq=32, D=128: per chunk c the visible
    # pairs are 4096 * 4096 c + 4096 * 4097 / 2
    total = 0
    for c in range(8):
        f = attention.useful_flops([4096], [4096 * (c + 1)], 32, 128)
        assert f == 4 * 128 * 32 * (4096 * 4096 * c + 4096 * 4097 // 2)
        total += f
    assert abs(total / 8.796e12 - 1) < 1e-3


# ------------------------- planted mistakes -------------------------------

@pytest.mark.parametrize("mutant", ["head_map", "causal_off_by_one", "no_scale", "v_layout"])
def test_planted_attention_mistakes_fail_the_library_check(monkeypatch, mutant):
    case = _case(fmt="e4m3", B=2, ctx=(37, 70), q_len=5, Hq=8, Hkv=2, D=32)
    orig_rows = attention._rows_attend
    orig_gather = paged.gather
    if mutant == "causal_off_by_one":
        monkeypatch.setattr(attention, "_rows_attend",
                            lambda qr, pos, K, V, s: orig_rows(qr, pos - 1, K, V, s))
    elif mutant == "no_scale":
        monkeypatch.setattr(attention, "_rows_attend",
                            lambda qr, pos, K, V, s: orig_rows(qr, pos, K, V, 1.0))
    elif mutant == "head_map":
        # g = h % Hkv instead of h // G
        def gather_swapped(kc, vc, bt, ctx, g, *a, **k):
            return orig_gather(kc, vc, bt, ctx, (g + 1) % case.num_kv_heads, *a, **k)
        monkeypatch.setattr(paged, "gather", gather_swapped)
    elif mutant == "v_layout":
        def gather_vt(kc, vc, bt, ctx, g, fmt, ks=None, vs=None):
            K, _ = orig_gather(kc, vc, bt, ctx, g, fmt, ks, vs)
            bs = kc.shape[2]
            j = np.arange(ctx)
            pages = np.asarray(bt[:-(-ctx // bs)], dtype=np.int64)[j // bs]
            raw = vc.reshape(vc.shape[0], vc.shape[1], bs, -1)[pages, g, j % bs, :]   # token-major reading
            return K, paged.dequant(raw, fmt, None if vs is None else vs[g])
        monkeypatch.setattr(paged, "gather", gather_vt)
    o, _, _ = _oracle(case)
    ref = _sdpa(case)
    err = np.nanmax(np.abs(o - ref)) if np.any(np.isfinite(o)) else np.inf
    assert not (err < 1e-6), mutant

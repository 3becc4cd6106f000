"""The largest shapes the entry points accept, against the float64 oracle:
the largest page size (65536 tokens), the most partitions a decode can have
(4096), and the widest row group (64 query heads on one KV head)."""

import numpy as np
import pytest
import torch

from attention_paged_flashattention_amd import synth
from tests.gpu_helpers import check_close, log, oracle_cache_heads, oracle_full, oracle_rows
from tests.oracle_helpers import oracle_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def runner():
    from attention_paged_flashattention_amd import runner as r
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return r


@pytest.mark.parametrize("q_len", [1, 8])
def test_largest_page_size(runner, q_len):
    """65536-token pages: the write is bit-exact and decode / verify match the
    oracle across the page boundary (70000 keys span two pages)."""
    case = synth.make_case(f"bs65536-q{q_len}", 41, [70000, 3000], q_len, 8, 2, 128, 65536,
                           "f16", "f16", "e4m3")
    log(f"{case.name}: {case.num_blocks} pages of 65536")
    dc = runner.DeviceCase(case)
    dc.write_all()
    kc, vc = oracle_cache(case)
    torch.cuda.synchronize()
    assert np.array_equal(dc.key_cache.cpu().numpy(), kc), "key cache not bit-exact"
    assert np.array_equal(dc.value_cache.cpu().numpy(), vc), "value cache not bit-exact"
    out = dc.verify(q_len, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close(out.reshape(-1, 8, 128), oracle_full(case, kc, vc), "e4m3", "bs 65536")


def test_most_partitions(runner):
    """4096 partitions of 64 keys over a 262144-key decode (the most the
    combine takes): every query head of two KV heads against the oracle."""
    case = synth.long_decode_256k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.decode(num_partitions=4096, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    kv_heads = [1, 6]
    kc, vc = oracle_cache_heads(case, [(0, g) for g in kv_heads])
    q32 = synth.to_f32(case.q, case.q_dtype)
    G = case.gqa
    heads = [g * G + i for g in kv_heads for i in range(G)]
    ref = oracle_rows(case, kc, vc, 0, q32[0, heads], heads, [int(case.ctx_lens[0]) - 1] * len(heads))
    check_close(out[0, heads], ref, "e4m3", "4096 partitions")


@pytest.mark.parametrize("fmt,q_len", [("e4m3", 1), ("e5m2", 2)])
def test_widest_row_group(runner, fmt, q_len):
    """64 query heads on one KV head at q_len 1 (64 rows), and 32 heads at
    q_len 2: four 16-row MFMA blocks per work-group."""
    hq = 64 // q_len
    case = synth.make_case(f"rows64-{fmt}-q{q_len}", 43, [900, 2500], q_len, hq, 1, 128, 16,
                           "f16", "f16", fmt)
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(q_len, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close(out.reshape(-1, hq, 128), oracle_full(case), fmt, "64-row group")


def test_prefill_largest_page_size(runner):
    """A 1000-token prefill chunk straddling the boundary of two 65536-token
    pages (positions 65000..65999), bf16 Q and E4M3 cache: sampled rows of
    every query head against the oracle."""
    case = synth.make_case("bs65536-prefill", 44, [66000], [66000], 8, 2, 128, 65536, "bf16",
                           "bf16", "e4m3")
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_tokens(0, 65000)
    out = dc.prefill_chunk(65000, 66000, out_dtype=torch.float32)
    torch.cuda.synchronize()
    kc, vc = oracle_cache_heads(case, [(0, 0), (0, 1)])
    q32 = synth.to_f32(case.q, "bf16")
    rng = np.random.default_rng(5)
    pos = np.unique(np.concatenate([[65000, 65535, 65536, 65999], rng.integers(65000, 66000, 8)]))
    rows_q, rows_h, rows_p = [], [], []
    for p in pos:
        for h in range(8):
            rows_q.append(q32[p, h])
            rows_h.append(h)
            rows_p.append(int(p))
    ref = oracle_rows(case, kc, vc, 0, np.array(rows_q), rows_h, rows_p)
    got = out.cpu()[torch.tensor(np.array(rows_p) - 65000), torch.tensor(rows_h)]
    check_close(got, ref, "e4m3", "prefill across 65536-token pages")

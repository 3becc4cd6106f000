"""The five workloads, the 128K decode headline and the second workloads
(batched E5M2 decode, q16 verify, 64K / 128K / 256K chunked prefill, the
draft's sliding window) at full size, in the launch configuration bench.py
times (automatic partitions unless the workload states a split).

Element-by-element comparison with the float64 oracle:

* decode, verify and window workloads: every output row -- every (sequence,
  KV head) pair -- against the oracle, run per (sequence, KV head) in a pool
  of worker processes (tests/oracle_pool.py);
* the 32K chunked prefill: every row of the first and the last chunk (all 32
  query heads) and sampled positions of the chunks between;
* the 64K / 128K / 256K chunked prefills: sampled positions (all heads) of the
  first, a middle and the last chunk.

Every output is also checked for properties that hold at any size: finite,
and inside the convex hull bound |o| <= max |V| of its KV head.
"""

import dataclasses
import functools
import time

import numpy as np
import pytest
import torch

from attention_paged_flashattention_amd import synth
from tests.gpu_helpers import check_close, log, oracle_full
from tests.oracle_pool import OraclePool, row_tasks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def runner():
    from attention_paged_flashattention_amd import runner as r
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return r


def _vmax_per_head(dc):
    """max |V| per KV head over the written cache (dequantized on the host
    from the bytes; a property bound, not a reference value)."""
    from oracle import fp8
    c = dc.case
    out = []
    for g in range(c.num_kv_heads):
        if c.cache_fmt == "f16":
            vals = dc.value_cache[:, g].float().abs()
            vals = torch.nan_to_num(vals, nan=0.0)
            out.append(float(vals.max()))
        else:
            codes = torch.unique(dc.value_cache[:, g]).cpu().numpy()
            tab = np.abs(fp8.decode_table(c.cache_fmt)[codes])
            tab = tab[np.isfinite(tab)]
            s = 1.0 if c.v_scale is None else float(c.v_scale[g])
            out.append(float(tab.max()) * s)
    return np.array(out)


def _hull_check(out, dc):
    c = dc.case
    o = out.float()
    assert torch.isfinite(o).all().item(), "non-finite output"
    G = c.gqa
    vmax = _vmax_per_head(dc)
    amax = o.abs().amax(dim=-1)                     # [..., Hq]
    amax = amax.reshape(-1, c.num_q_heads).amax(dim=0).cpu().numpy()
    bound = np.repeat(vmax, G) * (1 + 1e-3) + 1e-3
    assert np.all(amax <= bound), (amax, bound)


def _pool_log(pool, what):
    log(f"  oracle {what}: {pool.last_wall:.1f} s wall, {pool.last_cpu:.1f} s of work on "
        f"{pool.workers} worker processes")


def _oracle_all_rows(case, window=None):
    """Oracle output for every row of a decode / verify / window workload,
    [B * q_len, Hq, D], computed per (sequence, KV head) in worker processes."""
    B, Hkv = case.batch, case.num_kv_heads
    qlen = int(case.q_lens[0])
    pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    ref = np.full((B * qlen, case.num_q_heads, case.head_dim), np.nan)
    with OraclePool(case) as pool:
        pool.build(pairs, pieces=max(1, 32 // len(pairs)))
        _pool_log(pool, f"cache of {len(pairs)} (sequence, KV head) pairs")
        tasks, index, owner = [], [], []
        for b, g in pairs:
            t, ix = row_tasks(case, b, g, np.arange(qlen), window=window)
            tasks += t
            index += ix
            owner += [b] * len(t)
        rows = pool.run(tasks)
        _pool_log(pool, f"{B * qlen * case.num_q_heads} rows")
    for r, (t, h), b in zip(rows, index, owner):
        ref[b * qlen + t, h] = r
    assert not np.isnan(ref).any()
    return ref


def test_workload1_prefill64_then_decode(runner):
    case = synth.prefill_decode_small()
    log(f"{case.name}")
    dc = runner.DeviceCase(case)
    o_pf = dc.prefill_chunk(0, 64, out_dtype=torch.float32)
    dc.write_tokens(64, 65)
    o_dec = dc.decode(q=dc.q[64:65].contiguous(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle_full(case)          # 65 rows: 64 prefill positions + the decode position
    check_close(o_pf, ref[:64], "f16", "prefill 64")
    check_close(o_dec, ref[64:65], "f16", "decode @64")


def test_workload2_batched_decode_e4m3(runner):
    case = synth.batched_decode_e4m3()
    log(f"{case.name} ctx={case.ctx_lens.tolist()}")
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.decode(out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close(out, _oracle_all_rows(case).reshape(out.shape), "e4m3", "decode B=8, every row")
    _hull_check(out, dc)


def _chunked_prefill_check(runner, case, full_chunks, sampled_chunks, n_sampled, seed):
    """Run every chunk of a single-sequence chunked prefill (write, then
    attend to the paged prefix) and compare with the oracle: every row of
    ``full_chunks``, ``n_sampled`` random positions (all heads) of
    ``sampled_chunks``. The oracle runs in worker processes while the GPU
    works."""
    chunk = case.meta["chunk"]
    total = int(case.ctx_lens[0])
    n = total // chunk
    Hkv, G, Hq, D = case.num_kv_heads, case.gqa, case.num_q_heads, case.head_dim
    rng = np.random.default_rng(seed)
    plan = {}
    for c in sorted(set(full_chunks) | set(sampled_chunks)):
        s, e = c * chunk, (c + 1) * chunk
        if c in full_chunks:
            toks = np.arange(s, e)
        else:
            toks = np.unique(np.concatenate([[s, s + 1, e - 2, e - 1],
                                             rng.integers(s, e, size=n_sampled - 4)]))
        plan[c] = toks
    with OraclePool(case) as pool:
        t0 = time.perf_counter()
        pool.build([(0, g) for g in range(Hkv)], pieces=8)
        _pool_log(pool, f"cache of {total} tokens x {Hkv} KV heads")
        tasks, index, owner = [], [], []
        for c, toks in plan.items():
            e = (c + 1) * chunk
            split = max(1, len(toks) * G // 2048)
            for g in range(Hkv):
                t, ix = row_tasks(case, 0, g, toks, keys=e, split=split)
                tasks += t
                index += ix
                owner += [c] * len(t)
        handle = pool.submit(tasks)            # oracle rows while the GPU runs
        dc = runner.DeviceCase(case)
        got = {}
        for c in range(n):
            s, e = c * chunk, (c + 1) * chunk
            out = dc.prefill_chunk(s, e, out_dtype=torch.float32)
            torch.cuda.synchronize()
            _hull_check(out, dc)
            if c in plan:
                got[c] = out.cpu().numpy()
        del dc
        torch.cuda.empty_cache()
        rows = pool.collect(handle)
        log(f"  oracle rows: {time.perf_counter() - t0:.1f} s since the pool started, "
            f"{pool.last_cpu:.1f} s of work on {pool.workers} worker processes")
    refs = {c: np.full((len(plan[c]), Hq, D), np.nan) for c in plan}
    slot = {c: {int(t): i for i, t in enumerate(plan[c])} for c in plan}
    for r, (t, h), c in zip(rows, index, owner):
        ii = np.array([slot[c][int(x)] for x in t])
        refs[c][ii, h] = r
    for c in plan:
        assert not np.isnan(refs[c]).any()
        s = c * chunk
        sel = torch.from_numpy(got[c][plan[c] - s])
        what = "every row" if c in full_chunks else f"{len(plan[c])} sampled positions"
        check_close(sel, refs[c], "e4m3", f"chunk {c} ({what}, all {Hq} heads)")


def test_workload3_chunked_prefill_32k(runner):
    case = synth.chunked_prefill_32k()
    log(case.name)
    n = 32768 // case.meta["chunk"]
    _chunked_prefill_check(runner, case, full_chunks=[0, n - 1],
                           sampled_chunks=list(range(1, n - 1)), n_sampled=16, seed=3)


def test_workload4_verify_q8_128k(runner):
    case = synth.verify_q8_128k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(8, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    out = out.reshape(-1, case.num_q_heads, case.head_dim)
    del dc
    check_close(out, _oracle_all_rows(case), "e5m2", "verify q8 4 x 128K, every row")


def test_workload5_decode_256k(runner):
    case = synth.long_decode_256k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    from attention_paged_flashattention_amd import pagedattn as pa
    assert case.meta["partitions"] == 64     # the workload's stated split
    out = dc.decode(num_partitions=case.meta["partitions"], out_dtype=torch.float32)
    # the library's own choice (one work-group per CU: 32 partitions) agrees
    # to the rounding of P against each launch's running maximum
    assert pa.pa_decode_partitions(1, 1, 32, 8, 128, 262144) == 32
    auto = dc.decode(num_partitions=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    assert torch.max(torch.abs(auto - out)).item() < 1e-4
    del dc
    ref = _oracle_all_rows(case).reshape(out.shape)
    check_close(out, ref, "e4m3", "decode 256K, 64 partitions, every row")
    check_close(auto, ref, "e4m3", "decode 256K, 32 partitions, every row")


def test_headline_decode_128k(runner):
    case = synth.headline_decode_128k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.decode(num_partitions=case.meta["partitions"], out_dtype=torch.float32)
    out16 = dc.decode(num_partitions=case.meta["partitions"])
    a = dc.decode(num_partitions=case.meta["partitions"])
    torch.cuda.synchronize()
    _hull_check(out, dc)
    assert torch.equal(out16, a)
    del dc
    ref = _oracle_all_rows(case).reshape(out.shape)
    check_close(out, ref, "e4m3", "decode 128K, every row")
    check_close(out16, ref, "e4m3", "decode 128K fp16 out, every row", out_dtype=torch.float16)


# ---------------------------------------------------------------------------
# Second workloads on the same kernels
# ---------------------------------------------------------------------------

def test_batched_decode_e5m2_b16_16k(runner):
    case = synth.batched_decode_e5m2_16k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.decode(out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    del dc
    check_close(out, _oracle_all_rows(case).reshape(out.shape), "e5m2", "decode B16 x 16K, every row")


def test_verify_q16_128k(runner):
    case = synth.verify_q16_128k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(16, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    del dc
    check_close(out.reshape(-1, case.num_q_heads, case.head_dim), _oracle_all_rows(case), "e5m2",
                "verify q16 4 x 128K, every row")


@pytest.mark.parametrize("chunk", [4096, 8192])
def test_chunked_prefill_64k(runner, chunk):
    """64K prefill in 16 chunks of 4096 or 8 of 8192."""
    case = synth.chunked_prefill_64k(chunk=chunk)
    log(case.name)
    n = 65536 // chunk
    _chunked_prefill_check(runner, case, full_chunks=[], sampled_chunks=[0, n // 2, n - 1],
                           n_sampled=12, seed=4)


@functools.lru_cache(maxsize=1)
def _long_prefill_inputs(total):
    return synth.chunked_prefill_long(total, 4096)


@pytest.mark.parametrize("total,chunk", [(131072, 4096), (131072, 8192), (262144, 4096),
                                         (262144, 8192)])
def test_chunked_prefill_long(runner, total, chunk):
    """128K / 256K prefill in chunks of 4096 or 8192 (the long-context prefill
    budgets); sampled positions of the first, a middle and the last chunk.
    Both chunk sizes run over the same seeded inputs."""
    base = _long_prefill_inputs(total)
    case = dataclasses.replace(base, meta=dict(base.meta, chunk=chunk),
                               name=base.name.replace("chunk4k", f"chunk{chunk // 1024}k"))
    log(case.name)
    n = total // chunk
    _chunked_prefill_check(runner, case, full_chunks=[], sampled_chunks=[0, n // 2, n - 1],
                           n_sampled=8, seed=6)


@pytest.mark.parametrize("ctx", [32768, 131072])
def test_window_draft_q8(runner, ctx):
    case = synth.window_draft_q8(ctx=ctx)
    W = case.meta["window"]
    log(f"{case.name} window {W}")
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.window(8, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    del dc
    check_close(out.reshape(-1, case.num_q_heads, case.head_dim),
                _oracle_all_rows(case, window=W), "e5m2", f"window {W} q8, every row")

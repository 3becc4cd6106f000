"""The five workloads, the 128K decode headline and the second workloads
(batched E5M2 decode, q16 verify, 64K prefill, the draft's sliding window) at
full size, in the launch configuration bench.py times (automatic partitions). Rows the oracle can afford
are compared element by element (whole heads of sampled sequences); every row
is checked for properties that hold at any size: finite, and inside the convex
hull bound |o| <= max |V| of its KV head."""

import numpy as np
import pytest
import torch

from attention_paged_flashattention_amd import synth
from tests.gpu_helpers import check_close, log, oracle_cache_heads, oracle_full, oracle_rows

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


def _hull_check(out, dc, qrows_heads_axis=-2):
    c = dc.case
    o = out.float()
    assert torch.isfinite(o).all().item(), "non-finite output"
    G = c.gqa
    vmax = _vmax_per_head(dc)
    amax = o.abs().amax(dim=-1)                     # [..., Hq]
    amax = amax.reshape(-1, c.num_q_heads).amax(dim=0).cpu().numpy()
    bound = np.repeat(vmax, G) * (1 + 1e-3) + 1e-3
    assert np.all(amax <= bound), (amax, bound)


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
    check_close(out, oracle_full(case), "e4m3", "decode B=8")
    _hull_check(out, dc)


def test_workload3_chunked_prefill_32k(runner):
    case = synth.chunked_prefill_32k()
    log(case.name)
    dc = runner.DeviceCase(case)
    chunk = case.meta["chunk"]
    heads = np.array([0, 9, 18, 31])
    kv_heads = sorted(set(int(h) // case.gqa for h in heads))
    kc, vc = oracle_cache_heads(case, [(0, g) for g in kv_heads])
    q32 = synth.to_f32(case.q, "bf16")
    rng = np.random.default_rng(3)
    for c in range(32768 // chunk):
        s, e = c * chunk, (c + 1) * chunk
        out = dc.prefill_chunk(s, e, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _hull_check(out, dc)
        pos = np.unique(np.concatenate([[s, s + 1, e - 2, e - 1],
                                        rng.integers(s, e, size=6)]))
        rows_q, rows_h, rows_p = [], [], []
        for p in pos:
            for h in heads:
                rows_q.append(q32[p, h])
                rows_h.append(h)
                rows_p.append(p)
        ref = oracle_rows(case, kc, vc, 0, np.array(rows_q), rows_h, rows_p)
        got = out.cpu()[torch.tensor(np.array(rows_p) - s), torch.tensor(rows_h)]
        check_close(got, ref, "e4m3", f"chunk {c} sampled rows")


def _sampled_decode_check(case, dc, out, pairs, window=None):
    """Compare every row of the sampled (sequence, KV head) pairs."""
    kc, vc = oracle_cache_heads(case, pairs)
    q32 = synth.to_f32(case.q, case.q_dtype)
    G = case.gqa
    qlen = int(case.q_lens[0])
    for b, g in pairs:
        heads, positions, rows = [], [], []
        for i in range(qlen):
            for gh in range(G):
                h = g * G + gh
                heads.append(h)
                positions.append(int(case.ctx_lens[b]) - qlen + i)
                rows.append(q32[b * qlen + i, h])
        ref = oracle_rows(case, kc, vc, b, np.array(rows), heads, positions, window=window)
        got = out.reshape(-1, case.num_q_heads, case.head_dim)[b * qlen:(b + 1) * qlen][:, g * G:(g + 1) * G]
        check_close(got.reshape(-1, case.head_dim), ref, case.cache_fmt, f"seq {b} kv head {g}")


def test_workload4_verify_q8_128k(runner):
    case = synth.verify_q8_128k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(8, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    _sampled_decode_check(case, dc, out, [(0, 0), (1, 3), (2, 5), (3, 7)])


def test_workload5_decode_256k(runner):
    case = synth.long_decode_256k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    from attention_paged_flashattention_amd import pagedattn as pa
    assert case.meta["partitions"] == 64     # the workload's stated split
    out = dc.decode(num_partitions=case.meta["partitions"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    _sampled_decode_check(case, dc, out, [(0, 0), (0, 3), (0, 6)])
    # the library's own choice (one work-group per CU: 32 partitions) agrees
    # to the rounding of P against each launch's running maximum
    assert pa.pa_decode_partitions(1, 1, 32, 8, 128, 262144) == 32
    auto = dc.decode(num_partitions=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(auto - out)).item() < 1e-4


def test_headline_decode_128k(runner):
    case = synth.headline_decode_128k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.decode(num_partitions=case.meta["partitions"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    _sampled_decode_check(case, dc, out, [(0, 1), (0, 7)])
    out16 = dc.decode(num_partitions=case.meta["partitions"])
    a = dc.decode(num_partitions=case.meta["partitions"])
    torch.cuda.synchronize()
    assert torch.equal(out16, a)


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
    _sampled_decode_check(case, dc, out, [(0, 0), (5, 2), (11, 7), (15, 4)])


def test_verify_q16_128k(runner):
    case = synth.verify_q16_128k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(16, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _hull_check(out, dc)
    _sampled_decode_check(case, dc, out, [(0, 2), (3, 6)])


@pytest.mark.parametrize("chunk", [4096, 8192])
def test_chunked_prefill_64k(runner, chunk):
    """64K prefill in 16 chunks of 4096 or 8 of 8192; sampled rows of the
    first, a middle and the last chunk against the oracle, every chunk for
    the hull property."""
    case = synth.chunked_prefill_64k(chunk=chunk)
    log(case.name)
    dc = runner.DeviceCase(case)
    heads = np.array([3, 20])
    kv_heads = sorted(set(int(h) // case.gqa for h in heads))
    kc, vc = oracle_cache_heads(case, [(0, g) for g in kv_heads])
    q32 = synth.to_f32(case.q, "bf16")
    rng = np.random.default_rng(4)
    n = 65536 // chunk
    for c in range(n):
        s, e = c * chunk, (c + 1) * chunk
        out = dc.prefill_chunk(s, e, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _hull_check(out, dc)
        if c not in (0, n // 2, n - 1):
            continue
        pos = np.unique(np.concatenate([[s, e - 1], rng.integers(s, e, size=4)]))
        rows_q, rows_h, rows_p = [], [], []
        for p in pos:
            for h in heads:
                rows_q.append(q32[p, h])
                rows_h.append(h)
                rows_p.append(p)
        ref = oracle_rows(case, kc, vc, 0, np.array(rows_q), rows_h, rows_p)
        got = out.cpu()[torch.tensor(np.array(rows_p) - s), torch.tensor(rows_h)]
        check_close(got, ref, "e4m3", f"chunk {c} sampled rows")


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
    _sampled_decode_check(case, dc, out, [(0, 1), (3, 6)], window=W)

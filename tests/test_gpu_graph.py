"""HIP-graph capture of the hot path through the C ABI.

The calls take a stream, never synchronize and never allocate, so a serving
loop can capture them (the "1Cat-vLLM" README, "What this branch adds", lists
CUDA-graph compatibility; the "1Cat-vLLM 1.5.0" release notes, "Production
DFlash2 on V100", run the target and draft models under graphs). Each
test captures one step (quantize-on-write of the newest tokens, then the
attention call) into a graph on torch's capture stream, then replays it
several times. Between replays the captured query buffer is refilled with new
values and the output is poisoned with NaN in eager work, and every replay
must equal an eager call on the same inputs bit for bit (same kernels, same
launch shapes) -- so the replays recompute from live inputs rather than
returning what the capture left behind. The first replay is also checked
against the float64 oracle.
"""

import pytest
import torch

from attention_paged_flashattention_amd import synth
from tests.gpu_helpers import check_close, log, oracle_full

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def runner():
    from attention_paged_flashattention_amd import runner as r
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return r


def _capture(step):
    """Capture step() into a graph (after one warm-up run on a side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _replay_and_compare(g, q, out_g, eager, fresh_q):
    for r in range(REPLAYS):
        if r > 0:
            q.copy_(fresh_q(r))
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager()
        torch.cuda.synchronize()
        assert torch.isfinite(out_g).all().item(), f"replay {r}: output not fully written"
        assert torch.equal(out_g, ref), f"replay {r}: graph and eager results differ"
        log(f"  replay {r}: bitwise equal to the eager call")


@pytest.mark.parametrize("fmt,q_len,ctx,bs", [("e4m3", 1, (3000, 5000), 2048),
                                             ("e5m2", 8, (200, 4100), 64),
                                             ("e4m3", 1, (70, 900), 16)])
def test_decode_verify_step_graph(runner, fmt, q_len, ctx, bs):
    from attention_paged_flashattention_amd import pagedattn as pa
    log(f"graph {fmt} q_len={q_len} ctx={ctx} bs={bs}")
    B = len(ctx)
    case = synth.make_case(f"graph-{fmt}-q{q_len}", 21, list(ctx), q_len, 32, 8, 128, bs, "f16",
                           "f16", fmt, sigma_kv=0.5)
    dc = runner.DeviceCase(case)
    newest = dc.last_token_rows(q_len)
    older = torch.ones(dc.k.shape[0], dtype=torch.bool, device=dc.device)
    older[newest] = False
    idx = torch.nonzero(older).flatten()
    pa.kv_cache_write_fp8(dc.k[idx].contiguous(), dc.v[idx].contiguous(), dc.slots[idx].contiguous(),
                          dc.key_cache, dc.value_cache, fmt, dc.k_scale, dc.v_scale)
    k_new, v_new, s_new = (dc.k[newest].contiguous(), dc.v[newest].contiguous(),
                           dc.slots[newest].contiguous())
    op = pa.PA_OP_DECODE if q_len == 1 else pa.PA_OP_VERIFY
    wsb = pa.pa_workspace_bytes(op, B, q_len, 32, 8, 128, 0, dc.max_ctx)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dc.device)
    q = dc.q.clone() if q_len == 1 else dc.q.view(B, q_len, 32, 128).clone()
    out_g = torch.empty(q.shape, dtype=torch.float32, device=dc.device)
    out_e = torch.empty_like(out_g)
    attn = pa.attn_decode_paged if q_len == 1 else pa.attn_verify_paged

    def call(out):
        return attn(q, dc.key_cache, dc.value_cache, fmt, dc.block_tables, dc.ctx_lens, dc.max_ctx,
                    case.softmax_scale, dc.k_scale, dc.v_scale, workspace=ws, out=out)

    def step():
        pa.kv_cache_write_fp8(k_new, v_new, s_new, dc.key_cache, dc.value_cache, fmt, dc.k_scale,
                              dc.v_scale)
        call(out_g)

    g = _capture(step)
    # the captured write filled the newest slots: the first replay must match the oracle
    out_g.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    ref = oracle_full(case)
    check_close(out_g.reshape(ref.shape), ref, fmt, "graph replay vs oracle")

    gen = torch.Generator(device="cpu").manual_seed(5)

    def fresh_q(r):
        return torch.randn(q.shape, generator=gen).to(q.dtype).to(q.device)

    _replay_and_compare(g, q, out_g, lambda: call(out_e), fresh_q)


def test_prefill_chunk_graph(runner):
    """One chunk of a chunked prefill (write its K/V, attend to the paged
    prefix) captured and replayed."""
    from attention_paged_flashattention_amd import pagedattn as pa
    case = synth.make_case("graph-prefill", 22, [640], [640], 32, 8, 128, 64, "bf16", "bf16",
                           "e4m3")
    dc = runner.DeviceCase(case)
    dc.write_tokens(0, 384)
    s, e = 384, 640
    cu = torch.tensor([0, e - s], dtype=torch.int32, device=dc.device)
    ctx = torch.tensor([e], dtype=torch.int32, device=dc.device)
    q = dc.q[s:e].clone()
    k_new, v_new, s_new = dc.k[s:e].contiguous(), dc.v[s:e].contiguous(), dc.slots[s:e].contiguous()
    out_g = torch.empty(q.shape, dtype=torch.float32, device=dc.device)
    out_e = torch.empty_like(out_g)

    def call(out):
        return pa.attn_prefill_paged(q, cu, e - s, dc.key_cache, dc.value_cache, "e4m3",
                                     dc.block_tables, ctx, e, case.softmax_scale, dc.k_scale,
                                     dc.v_scale, out=out)

    def step():
        pa.kv_cache_write_fp8(k_new, v_new, s_new, dc.key_cache, dc.value_cache, "e4m3",
                              dc.k_scale, dc.v_scale)
        call(out_g)

    g = _capture(step)
    out_g.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    ref = oracle_full(case)[s:e]
    check_close(out_g, ref, "e4m3", "graph prefill replay vs oracle")
    gen = torch.Generator(device="cpu").manual_seed(6)

    def fresh_q(r):
        return torch.randn(q.shape, generator=gen).to(q.dtype).to(q.device)

    _replay_and_compare(g, q, out_g, lambda: call(out_e), fresh_q)


@pytest.mark.parametrize("fmt,q_len,ctx,bs", [("e4m3", 1, (3000, 5000), 2048),
                                             ("e5m2", 8, (200, 4100), 64)])
def test_fused_append_step_graph(runner, fmt, q_len, ctx, bs):
    """The write-then-attend step as one call (attn_decode_append_paged)
    captured and replayed: the capture's own run and every replay rewrite the
    newest slots from the captured new-token buffers, so a replay after the
    slots were poisoned must restore them and match the oracle."""
    from attention_paged_flashattention_amd import pagedattn as pa
    log(f"graph fused {fmt} q_len={q_len} ctx={ctx} bs={bs}")
    B = len(ctx)
    case = synth.make_case(f"graph-fused-{fmt}-q{q_len}", 23, list(ctx), q_len, 32, 8, 128, bs,
                           "f16", "f16", fmt, sigma_kv=0.5)
    dc = runner.DeviceCase(case)
    dc.write_all()
    newest = dc.last_token_rows(q_len)
    shape = (B, q_len, 8, 128)
    k_new = dc.k[newest].contiguous().view(shape)
    v_new = dc.v[newest].contiguous().view(shape)
    kc_ref, vc_ref = dc.key_cache.clone(), dc.value_cache.clone()
    wsb = pa.pa_workspace_bytes(pa.PA_OP_VERIFY, B, q_len, 32, 8, 128, 0, dc.max_ctx)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dc.device)
    q = dc.q.view(B, q_len, 32, 128).clone()
    out_g = torch.empty(q.shape, dtype=torch.float32, device=dc.device)
    out_e = torch.empty_like(out_g)

    def call(out):
        return pa.attn_decode_append_paged(q, k_new, v_new, dc.key_cache, dc.value_cache, fmt,
                                           dc.block_tables, dc.ctx_lens, dc.max_ctx,
                                           case.softmax_scale, dc.k_scale, dc.v_scale,
                                           workspace=ws, out=out)

    g = _capture(lambda: call(out_g))
    # poison the newest slots: the replay's fused write must put them back
    for b in range(B):
        for i in range(q_len):
            pos = int(case.ctx_lens[b]) - q_len + i
            page = int(case.block_tables[b, pos // bs])
            off = pos % bs
            dc.key_cache[page, :, off, :] = synth.POISON[fmt]
            dc.value_cache[page, :, off // min(bs, 64), :, off % min(bs, 64)] = synth.POISON[fmt]
    out_g.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(dc.key_cache, kc_ref) and torch.equal(dc.value_cache, vc_ref)
    ref = oracle_full(case)
    check_close(out_g.reshape(ref.shape), ref, fmt, "fused graph replay vs oracle")
    gen = torch.Generator(device="cpu").manual_seed(7)

    def fresh_q(r):
        return torch.randn(q.shape, generator=gen).to(q.dtype).to(q.device)

    _replay_and_compare(g, q, out_g, lambda: call(out_e), fresh_q)

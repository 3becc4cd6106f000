"""The allocation-free verify/decode entry point (attn_verify_paged_noalloc)
against attn_verify_paged with a caller workspace, through the C ABI: two
calls in a row on the static scratch, the second with a smaller input, each
bitwise equal to the workspace call (same kernels, same partition split) and
within the oracle tolerance; a call that needs more partials than the
scratch holds is rejected before any launch."""

import numpy as np
import pytest
import torch

from attention_paged_flashattention_amd import synth
from tests.gpu_helpers import check_close, log, oracle_full

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def runner():
    from attention_paged_flashattention_amd import runner as r
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return r


def _run_both(dc, q_len, parts, out_dtype):
    from attention_paged_flashattention_amd import pagedattn as pa
    c = dc.case
    q = dc.q.view(c.batch, q_len, c.num_q_heads, c.head_dim)
    ref = pa.attn_verify_paged(q, dc.key_cache, dc.value_cache, c.cache_fmt, dc.block_tables,
                               dc.ctx_lens, dc.max_ctx, c.softmax_scale, dc.k_scale, dc.v_scale,
                               num_partitions=parts, out_dtype=out_dtype)
    out = torch.empty_like(ref)
    pa.attn_verify_paged_noalloc(q, dc.key_cache, dc.value_cache, c.cache_fmt, dc.block_tables,
                                 dc.ctx_lens, dc.max_ctx, c.softmax_scale, out, dc.k_scale,
                                 dc.v_scale, num_partitions=parts)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_two_calls_second_smaller(runner):
    from attention_paged_flashattention_amd import pagedattn as pa
    # first: 4 sequences, q8 verify up to 20K keys, E5M2 2048-token pages,
    # 16 partitions (4 * 8 * 32 rows x 16 partitions: 8.5 MB of partials)
    big = synth.make_case("noalloc-big", 61, [20000, 9000, 17000, 12345], 8, 32, 8, 128, 2048,
                          "f16", "f16", "e5m2", sigma_kv=0.5)
    need = pa.pa_workspace_bytes(pa.PA_OP_VERIFY, 4, 8, 32, 8, 128, 16, 20000)
    assert 4 << 20 < need <= pa.NOALLOC_SCRATCH_BYTES
    log(f"noalloc call 1: {big.name}, {need} bytes of partials")
    d1 = runner.DeviceCase(big)
    d1.write_all()
    out1, ref1 = _run_both(d1, 8, 16, torch.float32)
    assert torch.equal(out1, ref1)
    check_close(out1.reshape(-1, 32, 128), oracle_full(big), "e5m2", "noalloc q8 verify")
    # second, smaller: 2 sequences, decode, E4M3 16-token pages, automatic
    # partitions, fp16 output; the scratch still holds call 1's partials
    small = synth.make_case("noalloc-small", 62, [700, 1500], 1, 32, 8, 128, 16, "f16", "f16",
                            "e4m3")
    log(f"noalloc call 2: {small.name}")
    d2 = runner.DeviceCase(small)
    d2.write_all()
    out2, ref2 = _run_both(d2, 1, 0, torch.float16)
    assert torch.equal(out2, ref2)
    check_close(out2.reshape(-1, 32, 128), oracle_full(small), "e4m3", "noalloc decode",
                out_dtype=torch.float16)
    # and the first shape again after the second (no state carried over)
    out3, _ = _run_both(d1, 8, 16, torch.float32)
    assert torch.equal(out3, ref1)


def test_noalloc_rejects_more_partials_than_the_scratch(runner):
    from attention_paged_flashattention_amd import pagedattn as pa
    case = synth.make_case("noalloc-over", 63, [5000] * 2, 16, 32, 8, 128, 2048, "f16", "f16",
                           "e5m2")
    dc = runner.DeviceCase(case)
    q = dc.q.view(2, 16, 32, 128)
    out = torch.zeros(q.shape, dtype=torch.float32, device=dc.device)
    # 2 x 16 x 32 rows x 64 partitions x 130 floats > 16 MiB
    assert pa.pa_workspace_bytes(pa.PA_OP_VERIFY, 2, 16, 32, 8, 128, 64, 5000) > \
        pa.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pa.PagedAttnError) as e:
        pa.attn_verify_paged_noalloc(q, dc.key_cache, dc.value_cache, "e5m2", dc.block_tables,
                                     dc.ctx_lens, dc.max_ctx, case.softmax_scale, out,
                                     num_partitions=64)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item()

"""attn_decode_append_paged: the new tokens' quantize-on-write and the decode /
verify attention in one call.

Its definition is the two calls it replaces: kv_cache_write_fp8 of the q_len
newest tokens of every sequence at their own positions, then attn_verify_paged
(attn_decode_paged at q_len 1). Every case runs both on copies of the same
cache and requires the fused call's output and both caches to equal the
two-call result bit for bit, and the output to match the float64 oracle. The
cases cover every cache format and query dtype, pages below and above one
64-key tile, head_dim 64 and 128, q_len 1 to 16, sequences shorter than q_len
(their missing positions are not written), an empty context, new tokens that
straddle a partition boundary (two work-groups write one sequence's tokens),
and both forms of the call: the write inside the attention kernel (at most 16
rows per KV head) and the write kernel with block-table slots ahead of it.
"""

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


def _new_kv(dc, q_len):
    """[B, q_len, Hkv, D] sources: token i of sequence b is the case's token
    at position ctx_b - q_len + i; positions < 0 get a NaN pattern (the call
    must not write them)."""
    c = dc.case
    rows = []
    for b in range(c.batch):
        ctx = int(c.ctx_lens[b])
        for i in range(q_len):
            pos = ctx - q_len + i
            rows.append(int(c.tok_start[b]) + pos if pos >= 0 else -1)
    idx = torch.tensor([max(r, 0) for r in rows], dtype=torch.int64, device=dc.device)
    k, v = dc.k[idx].clone(), dc.v[idx].clone()
    bad = torch.tensor([r < 0 for r in rows], device=dc.device)
    k[bad] = float("nan")
    v[bad] = float("nan")
    shape = (c.batch, q_len, c.num_kv_heads, c.head_dim)
    return k.view(shape).contiguous(), v.view(shape).contiguous()


def _slots_match_positions(c):
    """The case's slot of token j of sequence b is its block-table position,
    which is what the fused call derives."""
    for b in range(c.batch):
        ctx = int(c.ctx_lens[b])
        j = np.arange(ctx)
        want = c.block_tables[b, j // c.block_size].astype(np.int64) * c.block_size + \
            j % c.block_size
        got = c.slot_mapping[int(c.tok_start[b]):int(c.tok_start[b]) + ctx]
        if not np.array_equal(want, got):
            return False
    return True


CASES = [
    # fmt, q dtype, q_len, ctx lens, block size, head_dim, Hq, Hkv, partitions
    ("e4m3", "bf16", 1, (3000, 5000, 1, 64, 65), 16, 128, 32, 8, 0),
    ("e4m3", "f16", 1, (4100, 2049), 2048, 128, 32, 8, 0),
    ("e4m3", "f16", 1, (0, 700), 64, 128, 32, 8, 0),
    ("e5m2", "bf16", 8, (4099, 3267, 5), 64, 128, 32, 8, 4),     # 3267: tokens straddle 3264
    ("e5m2", "f16", 8, (200, 4100), 2048, 128, 32, 8, 0),
    ("e4m3", "bf16", 16, (2100, 17), 2048, 128, 32, 8, 0),
    ("e4m3", "bf16", 3, (130, 63), 32, 64, 8, 2, 0),
    ("f16", "f16", 4, (100, 33), 32, 64, 8, 2, 0),
    ("f16", "f16", 1, (257, 1), 16, 128, 16, 2, 0),
    # one partition: the new token's tile is a wave's second, third or later tile, in the
    # register pipeline (FP8) and in the one-tile loop (fp16 cache); only that wave writes it
    ("f16", "f16", 1, (700, 1100), 16, 128, 32, 8, 1),
    ("e4m3", "f16", 1, (400, 600, 1030), 64, 128, 32, 8, 1),
    # more than 16 rows per KV head: the write kernel with block-table slots
    # runs before the plain kernel
    ("f16", "f16", 8, (100, 33), 32, 64, 8, 2, 0),
    ("e4m3", "bf16", 5, (300, 4), 16, 128, 32, 8, 0),
    ("e5m2", "f16", 16, (70, 1000, 16), 16, 64, 16, 4, 3),
]


@pytest.mark.parametrize("fmt,qdt,q_len,ctx,bs,d,hq,hkv,parts", CASES)
def test_append_equals_write_then_attend(runner, fmt, qdt, q_len, ctx, bs, d, hq, hkv, parts):
    from attention_paged_flashattention_amd import pagedattn as pa
    log(f"append {fmt} q={qdt} q_len={q_len} ctx={ctx} bs={bs} D={d} Hq={hq} Hkv={hkv} P={parts}")
    kv_dtype = "f16" if fmt == "f16" else qdt
    case = synth.make_case(f"append-{fmt}-q{q_len}", 31, list(ctx), q_len, hq, hkv, d, bs, qdt,
                           kv_dtype, fmt)
    assert _slots_match_positions(case)
    dc = runner.DeviceCase(case)
    newest = dc.last_token_rows(q_len)
    keep = torch.ones(dc.k.shape[0], dtype=torch.bool, device=dc.device)
    keep[newest] = False
    old = keep.nonzero().flatten()
    if old.numel():
        pa.kv_cache_write_fp8(dc.k[old].contiguous(), dc.v[old].contiguous(),
                              dc.slots[old].contiguous(), dc.key_cache, dc.value_cache, fmt,
                              dc.k_scale, dc.v_scale)
    kc2, vc2 = dc.key_cache.clone(), dc.value_cache.clone()
    q = dc.q.view(case.batch, q_len, hq, d)

    # two calls: write, then verify (decode at q_len 1)
    pa.kv_cache_write_fp8(dc.k[newest].contiguous(), dc.v[newest].contiguous(),
                          dc.slots[newest].contiguous(), dc.key_cache, dc.value_cache, fmt,
                          dc.k_scale, dc.v_scale)
    ref = pa.attn_verify_paged(q, dc.key_cache, dc.value_cache, fmt, dc.block_tables,
                               dc.ctx_lens, dc.max_ctx, case.softmax_scale, dc.k_scale,
                               dc.v_scale, num_partitions=parts, out_dtype=torch.float32)
    # one call
    k_new, v_new = _new_kv(dc, q_len)
    got = pa.attn_decode_append_paged(q, k_new, v_new, kc2, vc2, fmt, dc.block_tables,
                                      dc.ctx_lens, dc.max_ctx, case.softmax_scale, dc.k_scale,
                                      dc.v_scale, num_partitions=parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(kc2.view(torch.uint8), dc.key_cache.view(torch.uint8)), "key cache differs"
    assert torch.equal(vc2.view(torch.uint8), dc.value_cache.view(torch.uint8)), "value cache differs"
    assert torch.equal(got, ref), "output differs from write-then-attend"
    check_close(got.reshape(-1, hq, d), oracle_full(case), fmt, "append vs oracle")

    # a second identical call rewrites the same codes and returns the same output
    again = pa.attn_decode_append_paged(q, k_new, v_new, kc2, vc2, fmt, dc.block_tables,
                                        dc.ctx_lens, dc.max_ctx, case.softmax_scale, dc.k_scale,
                                        dc.v_scale, num_partitions=parts,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)
    assert torch.equal(kc2.view(torch.uint8), dc.key_cache.view(torch.uint8))


def test_append_headline_128k_step(runner):
    """The 128K decode step in the launch configuration the benchmark times
    (32 partitions of 4096 keys, 2048-token pages): fused call vs write +
    decode, bitwise."""
    from attention_paged_flashattention_amd import pagedattn as pa
    case = synth.headline_decode_128k()
    log(case.name)
    dc = runner.DeviceCase(case)
    dc.write_all()
    newest = dc.last_token_rows(1)
    # overwrite the newest token's slot with poison in the fused copy
    kc2, vc2 = dc.key_cache.clone(), dc.value_cache.clone()
    c = case
    pos = int(c.ctx_lens[0]) - 1
    page = int(c.block_tables[0, pos // c.block_size])
    off = pos % c.block_size
    kc2[page, :, off, :] = synth.POISON["e4m3"]
    vc2[page, :, off // 64, :, off % 64] = synth.POISON["e4m3"]
    parts = c.meta["partitions"]
    ref = dc.decode(num_partitions=parts, out_dtype=torch.float32)
    k_new, v_new = _new_kv(dc, 1)
    got = pa.attn_decode_append_paged(dc.q.view(1, 1, c.num_q_heads, c.head_dim), k_new, v_new,
                                      kc2, vc2, "e4m3", dc.block_tables, dc.ctx_lens, dc.max_ctx,
                                      c.softmax_scale, dc.k_scale, dc.v_scale,
                                      num_partitions=parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(kc2, dc.key_cache) and torch.equal(vc2, dc.value_cache)
    assert torch.equal(got.view_as(ref), ref)
    del newest

"""GPU parity of every entry point against the float64 CPU oracle, at sizes the
oracle finishes in seconds: several tiles, ragged tails, both page sizes, all
cache formats. Calls go through the C ABI (via the ctypes binding)."""

import numpy as np
import pytest
import torch

from attention_paged_flashattention_amd import synth
from oracle import fp8, paged
from tests.gpu_helpers import check_close, log, oracle_full
from tests.oracle_helpers import oracle_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def runner():
    from attention_paged_flashattention_amd import runner as r
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return r


def _mk(fmt, B, ctx, q_len, Hq=8, Hkv=2, D=128, bs=16, q_dtype="f16", seed=11, sigma_kv=1.0,
        outlier=0.0):
    kv_dtype = "bf16" if (q_dtype == "bf16" and fmt != "f16") else "f16"
    return synth.make_case(f"{fmt}-B{B}-q{q_len}-D{D}-bs{bs}", seed, list(ctx), q_len, Hq, Hkv, D,
                           bs, q_dtype, kv_dtype, fmt, sigma_kv=sigma_kv, outlier_frac=outlier)


def _cache_np(t):
    return t.cpu().numpy()


def _ramp_keys(case, ramp):
    """Scale each key row by ramp[position] (one sequence), keeping the cache
    format's per-head scales consistent with the new keys."""
    kf = synth.to_f32(case.k, case.kv_dtype) * ramp[:, None, None].astype(np.float32)
    case.k = synth.round_to(kf, case.kv_dtype)
    if case.cache_fmt == "e4m3":
        case.k_scale = synth.head_scales(case.k, case.kv_dtype)
    return case


# ---------------------------------------------------------------------------
# quantize-on-write: bit-exact against the oracle, whole caches compared
# ---------------------------------------------------------------------------

WRITE_CASES = [
    ("e4m3", "f16", 16, 128, (37, 100, 5)),
    ("e4m3", "bf16", 2048, 128, (3000,)),
    ("e5m2", "f16", 64, 64, (130, 17)),
    ("e5m2", "bf16", 32, 128, (77,)),
    ("f16", "f16", 16, 64, (65, 33)),
    # fewer than 64 tokens: one thread per 16-element chunk
    ("e4m3", "f16", 16, 128, (5, 17, 1)),
    ("e5m2", "bf16", 2048, 64, (3,)),
    ("f16", "f16", 32, 128, (2, 9)),
    ("e4m3", "bf16", 64, 128, (63,)),
    # head sizes the attention kernels do not take: the 16-dimension write path
    ("e4m3", "f16", 16, 32, (100, 7)),
    ("e5m2", "bf16", 64, 256, (70,)),
    ("e4m3", "bf16", 2048, 256, (130,)),
    ("f16", "f16", 32, 32, (66,)),
]


@pytest.mark.parametrize("fmt,src,bs,D,ctx", WRITE_CASES)
def test_write_bit_exact(runner, fmt, src, bs, D, ctx):
    log(f"write {fmt} src={src} bs={bs} D={D} ctx={ctx}")
    case = synth.make_case("w", 21, list(ctx), 1, 4, 2, D, bs, "f16", src, fmt,
                           outlier_frac=0.05)
    # skip some tokens with a negative slot: they must not be written
    case.slot_mapping = case.slot_mapping.copy()
    case.slot_mapping[::7] = -1
    dc = runner.DeviceCase(case)
    dc.write_all()
    torch.cuda.synchronize()
    kc, vc = oracle_cache(case)
    assert np.array_equal(_cache_np(dc.key_cache).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(_cache_np(dc.value_cache).view(np.uint8), vc.view(np.uint8))


WRITE_SCALES = [("e4m3", 1.0), ("e4m3", 0.0105), ("e4m3", 7.0), ("e4m3", 13.0),
                ("e4m3", 0.2987244725227356), ("e4m3", 3.1415927410125732e-3),
                ("e5m2", None), ("e5m2", 0.37),
                # scales at the ends of the float32 range: subnormal scales, a
                # reciprocal that overflows (2^-130, 2^-149) or is subnormal
                # (2^127): the quotient falls back to a plain division there
                ("e4m3", 2.0 ** -149), ("e4m3", 2.0 ** -130), ("e4m3", 2.0 ** -126),
                ("e4m3", 2.0 ** 100), ("e4m3", 2.0 ** 127), ("e4m3", 1.9 * 2.0 ** 127),
                ("e5m2", 2.0 ** -140), ("e5m2", 1.5 * 2.0 ** 126)]


def _all_patterns(src):
    """Every 16-bit pattern of the source dtype as [512, 1, 128] storage, NaN
    patterns replaced by 0 (NaN inputs are outside the contract: the sign of a
    NaN is unspecified)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if src == "f16":
        x = bits.view(np.float16).copy()
        x[np.isnan(x)] = 0
        return x.reshape(512, 1, 128)
    f = synth.to_f32(bits, "bf16")
    bits = bits.copy()
    bits[np.isnan(f)] = 0
    return bits.reshape(512, 1, 128)


@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("bs,per_call", [(16, 512), (64, 512), (64, 63)])
@pytest.mark.parametrize("fmt,scale", WRITE_SCALES)
def test_write_every_16bit_pattern(runner, fmt, scale, bs, per_call, src):
    """All 65536 fp16 or bf16 bit patterns (inf included) through the write,
    in calls of 512 tokens (the row kernel; with 64-token pages its
    contiguous value blocks) or of 63 tokens (the few-token kernel)."""
    from attention_paged_flashattention_amd import pagedattn as pa
    log(f"write all {src} patterns {fmt} scale={scale} bs={bs} tokens/call={per_call}")
    x = _all_patterns(src)
    T, D = 512, 128
    nb = T // bs
    slots = np.arange(T, dtype=np.int64)
    dev = "cuda:0"
    if src == "f16":
        k = torch.from_numpy(x.copy()).to(dev)
        v = torch.from_numpy(x[::-1].copy()).to(dev)
    else:
        k = torch.from_numpy(x.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        v = torch.from_numpy(x[::-1].view(np.int16).copy()).to(dev).view(torch.bfloat16)
    vg = min(bs, 64)
    kc = torch.full((nb, 1, bs, D), 0x7F, dtype=torch.uint8, device=dev)
    vc = torch.full((nb, 1, bs // vg, D, vg), 0x7F, dtype=torch.uint8, device=dev)
    sc = None if scale is None else torch.tensor([scale], dtype=torch.float32, device=dev)
    st = torch.from_numpy(slots).to(dev)
    for t0 in range(0, T, per_call):
        t1 = min(T, t0 + per_call)
        pa.kv_cache_write_fp8(k[t0:t1], v[t0:t1], st[t0:t1], kc, vc, fmt, sc, sc)
    torch.cuda.synchronize()
    okc, ovc = paged.new_caches(nb, 1, bs, D, fmt, fill=0x7F)
    s = None if scale is None else np.array([scale], dtype=np.float32)
    xf = synth.to_f32(x, src)
    paged.write(xf, xf[::-1].copy(), slots, okc, ovc, fmt, s, s)
    assert np.array_equal(kc.cpu().numpy(), okc)
    assert np.array_equal(vc.cpu().numpy(), ovc)


# ---------------------------------------------------------------------------
# decode and verify
# ---------------------------------------------------------------------------

DECODE_CASES = [
    # fmt, B, ctx, Hq, Hkv, D, bs, q_dtype, partitions
    ("e4m3", 3, (1, 700, 1500), 32, 8, 128, 16, "f16", 0),
    ("e4m3", 2, (64, 1000), 32, 8, 128, 16, "f16", 3),
    ("e4m3", 1, (4097,), 32, 8, 128, 2048, "f16", 1),
    ("e4m3", 1, (5000,), 32, 8, 128, 2048, "f16", 7),
    ("e5m2", 2, (300, 2049), 32, 8, 128, 2048, "f16", 0),
    ("e4m3", 2, (129, 777), 32, 8, 128, 32, "bf16", 0),
    ("e5m2", 2, (129, 777), 16, 1, 128, 64, "bf16", 5),
    ("f16", 2, (65, 300), 4, 1, 64, 16, "f16", 0),
    ("f16", 1, (1000,), 8, 8, 64, 16, "f16", 4),
    ("e4m3", 2, (100, 513), 8, 2, 64, 16, "f16", 2),
    # one partition: the split kernel stores the output (no combine), bf16 out
    ("e4m3", 2, (129, 300), 32, 8, 128, 32, "bf16", 1),
]


@pytest.mark.parametrize("fmt,B,ctx,Hq,Hkv,D,bs,q_dtype,parts", DECODE_CASES)
def test_decode_parity(runner, fmt, B, ctx, Hq, Hkv, D, bs, q_dtype, parts):
    log(f"decode {fmt} B={B} ctx={ctx} Hq={Hq} Hkv={Hkv} D={D} bs={bs} q={q_dtype} P={parts}")
    case = _mk(fmt, B, ctx, 1, Hq, Hkv, D, bs, q_dtype, outlier=0.01)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.decode(num_partitions=parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle_full(case)
    check_close(out, ref, fmt, "decode f32")
    qt = torch.float16 if q_dtype == "f16" else torch.bfloat16
    out16 = dc.decode(num_partitions=parts)
    check_close(out16, ref, fmt, "decode q-dtype", out_dtype=qt)


VERIFY_CASES = [
    ("e5m2", 2, (8, 1000), 8, 32, 8, 128, 2048, 0),
    ("e5m2", 3, (9, 100, 2050), 8, 32, 8, 128, 64, 3),
    ("e4m3", 2, (70, 4096), 8, 32, 8, 128, 16, 0),
    ("e4m3", 1, (1030,), 16, 32, 8, 128, 16, 2),
    ("e4m3", 2, (40, 600), 3, 32, 8, 128, 16, 0),
    ("f16", 2, (64, 300), 8, 4, 1, 64, 16, 0),
    ("e5m2", 1, (129,), 1, 32, 8, 128, 16, 0),
    ("e5m2", 2, (8, 200), 8, 32, 8, 128, 64, 1),      # 32 rows, one partition
    ("e4m3", 2, (16, 900), 16, 32, 8, 128, 2048, 1),  # 64 rows, one partition (combine kept)
]


@pytest.mark.parametrize("fmt,B,ctx,q_len,Hq,Hkv,D,bs,parts", VERIFY_CASES)
def test_verify_parity(runner, fmt, B, ctx, q_len, Hq, Hkv, D, bs, parts):
    log(f"verify {fmt} B={B} ctx={ctx} q_len={q_len} Hq={Hq} Hkv={Hkv} D={D} bs={bs} P={parts}")
    case = _mk(fmt, B, ctx, q_len, Hq, Hkv, D, bs, "f16", sigma_kv=0.5)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(q_len, num_partitions=parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle_full(case).reshape(B, q_len, Hq, D)
    check_close(out, ref, fmt, "verify f32")


# the verify groups' LDS pipeline (pages of >= 64 keys, 32-64 rows): partitions shorter than
# the 4 waves' share of tiles, empty partitions, a ragged last tile, bf16 queries
LDS_VERIFY_CASES = [
    # fmt, B, ctx, q_len, bs, parts, q_dtype
    ("e5m2", 2, (16, 3000), 16, 64, 4, "f16"),
    ("e4m3", 3, (8, 70, 1500), 8, 64, 8, "f16"),
    ("e4m3", 2, (300, 2000), 12, 128, 0, "bf16"),
    ("e5m2", 1, (4100,), 16, 2048, 3, "bf16"),
    # one partition: 5 and 10 tiles (waves with 1-3 tiles, so the last copy of a wave is
    # waited for with none after it) and a 3-tile context (a wave with no tile)
    ("e5m2", 3, (320, 593, 129), 16, 64, 1, "f16"),
    ("e4m3", 2, (449, 200), 8, 128, 1, "bf16"),
]


@pytest.mark.parametrize("fmt,B,ctx,q_len,bs,parts,q_dtype", LDS_VERIFY_CASES)
def test_verify_parity_lds_pipeline(runner, fmt, B, ctx, q_len, bs, parts, q_dtype):
    log(f"verify (LDS pipeline) {fmt} B={B} ctx={ctx} q_len={q_len} bs={bs} P={parts} q={q_dtype}")
    case = _mk(fmt, B, ctx, q_len, 32, 8, 128, bs, q_dtype, sigma_kv=0.5)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(q_len, num_partitions=parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle_full(case).reshape(B, q_len, 32, 128)
    check_close(out, ref, fmt, "verify f32")


@pytest.mark.parametrize("fmt,q_len,bs,parts,q_dtype", [
    ("e4m3", 1, 2048, 4, "f16"),     # decode, register pipeline
    ("e5m2", 4, 16, 3, "f16"),       # per-lane page ids
    ("e4m3", 16, 64, 4, "bf16"),     # four row blocks, LDS pipeline
    ("e5m2", 8, 2048, 0, "f16"),     # default partitioning
])
def test_verify_scores_that_jump(runner, fmt, q_len, bs, parts, q_dtype):
    """Keys whose scores keep rising along the context (by ~100 in log2
    units), jump in one run of keys and fall back: each wave's running
    reference is raised in the middle of its tiles (see the prefill test)."""
    ctx = 3000
    case = _mk(fmt, 1, (ctx,), q_len, 32, 8, 128, bs, q_dtype)
    ramp = 1.0 + np.arange(ctx) / 150.0
    ramp[1700:1760] = 40.0
    case = _ramp_keys(case, ramp)
    log(f"verify with rising scores: {fmt} q_len={q_len} bs={bs} P={parts} q={q_dtype}")
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(q_len, num_partitions=parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle_full(case).reshape(1, q_len, 32, 128)
    check_close(out, ref, fmt, "verify rising scores f32")


def test_verify_rows_equal_decodes(runner):
    """The grouped verifier is exact: row i equals a decode at ctx - q_len + 1 + i
    (same kernels, so compared within fp32 rounding of the partition merge)."""
    case = _mk("e5m2", 2, (300, 2100), 8, 32, 8, 128, 64, "f16", sigma_kv=0.5)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.verify(8, out_dtype=torch.float32)
    qv = dc.q.view(2, 8, 32, 128)
    for i in range(8):
        ctx_i = dc.ctx_lens - 7 + i
        od = dc.decode(q=qv[:, i].contiguous(), ctx_lens=ctx_i.contiguous(),
                       max_ctx=int(case.ctx_lens.max()), out_dtype=torch.float32)
        # same kernels; P is rounded to fp16 against each launch's own running
        # max, so the two agree to fp16 rounding of P, far inside the tolerance
        assert torch.max(torch.abs(od - out[:, i])).item() < 1e-4


def test_decode_empty_context_rows_are_zero(runner):
    case = _mk("e4m3", 3, (200, 300, 50), 1)
    dc = runner.DeviceCase(case)
    dc.write_all()
    ctx = dc.ctx_lens.clone()
    ctx[1] = 0
    out = dc.decode(ctx_lens=ctx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(out[1] == 0).item()
    c2 = case.ctx_lens.copy()
    c2[1] = 0
    from oracle import attention
    from tests.oracle_helpers import q_f32
    kc, vc = oracle_cache(case)
    ref, _, _ = attention.attend(q_f32(case), [1, 1, 1], c2, kc, vc, case.block_tables, "e4m3",
                                 case.num_kv_heads, case.softmax_scale, case.k_scale, case.v_scale)
    check_close(out, ref, "e4m3", "decode with an empty row")


def test_decode_is_bitwise_deterministic(runner):
    case = _mk("e4m3", 2, (3000, 5000), 1, bs=2048)
    dc = runner.DeviceCase(case)
    dc.write_all()
    a = dc.decode(out_dtype=torch.float32)
    b = dc.decode(out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_partition_count_invariance(runner):
    case = _mk("e4m3", 1, (6000,), 1, bs=2048)
    dc = runner.DeviceCase(case)
    dc.write_all()
    outs = [dc.decode(num_partitions=p, out_dtype=torch.float32) for p in (1, 2, 5, 16, 94)]
    # each partitioning rounds P to fp16 against its own running maxima, so
    # results agree to fp16 rounding of P (far inside the oracle tolerance)
    for o in outs[1:]:
        assert torch.max(torch.abs(o - outs[0])).item() < 1e-4


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

PREFILL_CASES = [
    # fmt, total, chunk, Hq, Hkv, D, bs, q_dtype
    ("f16", 64, 64, 4, 1, 64, 16, "f16"),
    ("e4m3", 300, 100, 32, 8, 128, 16, "bf16"),
    ("e4m3", 1000, 333, 32, 8, 128, 2048, "bf16"),
    ("e4m3", 700, 700, 32, 8, 128, 64, "f16"),
    ("e5m2", 513, 257, 16, 2, 128, 32, "f16"),
    ("e5m2", 200, 200, 8, 8, 64, 16, "bf16"),
    ("f16", 300, 128, 8, 4, 128, 16, "f16"),
    ("e4m3", 130, 65, 32, 1, 64, 16, "f16"),
    # GQA ratios that are not powers of two (six query heads per KV head, the
    # packing the pages' long-prefill kernel uses; three) and the largest (64)
    ("e4m3", 600, 300, 48, 8, 128, 2048, "bf16"),
    ("e5m2", 257, 129, 12, 4, 64, 16, "f16"),
    ("e4m3", 100, 50, 64, 1, 128, 64, "bf16"),
]


@pytest.mark.parametrize("fmt,total,chunk,Hq,Hkv,D,bs,q_dtype", PREFILL_CASES)
def test_prefill_chunked_parity(runner, fmt, total, chunk, Hq, Hkv, D, bs, q_dtype):
    log(f"prefill {fmt} total={total} chunk={chunk} Hq={Hq} Hkv={Hkv} D={D} bs={bs} q={q_dtype}")
    case = _mk(fmt, 1, (total,), total, Hq, Hkv, D, bs, q_dtype)
    dc = runner.DeviceCase(case)
    ref = oracle_full(case)      # unchunked: chunked == unchunked is an oracle invariant
    outs = []
    for s in range(0, total, chunk):
        e = min(total, s + chunk)
        outs.append(dc.prefill_chunk(s, e, out_dtype=torch.float32))
    out = torch.cat(outs, 0)
    torch.cuda.synchronize()
    check_close(out, ref, fmt, "prefill f32")


@pytest.mark.parametrize("fmt,bs,q_dtype", [("e4m3", 2048, "bf16"), ("e5m2", 16, "f16")])
def test_prefill_scores_that_jump(runner, fmt, bs, q_dtype):
    """Scores whose row max keeps rising along the keys (by ~100 in log2
    units over the sequence), jumps in one run of keys and falls back: the
    softmax's running reference must be raised in the middle of the walk,
    many times per row, and later tiles far below it must not disturb it."""
    total = 1200
    case = _mk(fmt, 1, (total,), total, 32, 8, 128, bs, q_dtype)
    ramp = 1.0 + np.arange(total) / 60.0
    ramp[700:760] = 40.0
    case = _ramp_keys(case, ramp)
    log(f"prefill with rising scores: {fmt} bs={bs} q={q_dtype}")
    dc = runner.DeviceCase(case)
    ref = oracle_full(case)
    outs = [dc.prefill_chunk(s, min(total, s + 400), out_dtype=torch.float32)
            for s in range(0, total, 400)]
    out = torch.cat(outs, 0)
    torch.cuda.synchronize()
    check_close(out, ref, fmt, "prefill rising scores f32")


def test_prefill_batched_varlen(runner):
    """Several sequences in one call, each with its own chunk length and prefix."""
    case = _mk("e4m3", 3, (50, 400, 1200), 1, 32, 8, 128, 16, "bf16")
    dc = runner.DeviceCase(case)
    dc.write_all()
    qlens = [50, 130, 257]
    # queries: the last q_len positions of each sequence, from a fresh draw
    rng = np.random.default_rng(5)
    q32 = rng.standard_normal((sum(qlens), 32, 128)).astype(np.float32)
    qb = synth.round_to(q32, "bf16")
    from attention_paged_flashattention_amd.runner import upload16
    qt = upload16(qb, "bf16", "cuda:0")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32, device="cuda:0")
    out = dc.prefill(qt, cu, max(qlens), dc.ctx_lens, int(case.ctx_lens.max()),
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    from oracle import attention
    kc, vc = oracle_cache(case)
    ref, _, _ = attention.attend(synth.to_f32(qb, "bf16"), qlens, case.ctx_lens, kc, vc,
                                 case.block_tables, "e4m3", 8, case.softmax_scale, case.k_scale,
                                 case.v_scale)
    check_close(out, ref, "e4m3", "prefill varlen f32")


@pytest.mark.parametrize("bs", [16, 2048])
def test_prefill_chunk_longer_than_context(runner, bs):
    """Chunks longer than their context (outside the contract): rows before
    position 0 see no key and come back as zeros, rows at position >= 0 match
    the oracle, and nothing outside the sequences' block-table rows is read
    (an empty context's row holds only padding). Tiles wholly before position
    0, tiles that straddle it, and a sequence with no key at all."""
    case = _mk("e4m3", 3, (40, 0, 600), 1, 32, 8, 128, bs, "bf16")
    dc = runner.DeviceCase(case)
    dc.write_all()
    qlens = [300, 100, 200]
    rng = np.random.default_rng(8)
    q32 = rng.standard_normal((sum(qlens), 32, 128)).astype(np.float32)
    qb = synth.round_to(q32, "bf16")
    from attention_paged_flashattention_amd.runner import upload16
    qt = upload16(qb, "bf16", "cuda:0")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32, device="cuda:0")
    log(f"prefill chunks longer than their context: bs={bs} q_lens={qlens} ctx={case.ctx_lens.tolist()}")
    out = dc.prefill(qt, cu, max(qlens), dc.ctx_lens, int(case.ctx_lens.max()),
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    from oracle import attention
    kc, vc = oracle_cache(case)
    ref, _, _ = attention.attend(synth.to_f32(qb, "bf16"), qlens, case.ctx_lens, kc, vc,
                                 case.block_tables, "e4m3", 8, case.softmax_scale, case.k_scale,
                                 case.v_scale)
    assert np.all(ref[:260] == 0) and np.all(ref[300:400] == 0)
    check_close(out, ref, "e4m3", "prefill q_len > ctx f32")
    assert torch.all(out[:260] == 0).item() and torch.all(out[300:400] == 0).item()


def test_prefill_output_dtypes(runner):
    case = _mk("e4m3", 1, (500,), 500, 32, 8, 128, 16, "bf16")
    dc = runner.DeviceCase(case)
    ref = oracle_full(case)
    dc.write_all()
    for odt in (torch.bfloat16, torch.float16):
        cu = torch.tensor([0, 500], dtype=torch.int32, device="cuda:0")
        out = dc.prefill(dc.q, cu, 500, dc.ctx_lens, 500, out_dtype=odt)
        torch.cuda.synchronize()
        check_close(out, ref, "e4m3", f"prefill out {odt}", out_dtype=odt)


def test_prefill_is_bitwise_deterministic(runner):
    case = _mk("e4m3", 1, (1500,), 1500, 32, 8, 128, 2048, "bf16")
    dc = runner.DeviceCase(case)
    dc.write_all()
    cu = torch.tensor([0, 1500], dtype=torch.int32, device="cuda:0")
    a = dc.prefill(dc.q, cu, 1500, dc.ctx_lens, 1500, out_dtype=torch.float32)
    b = dc.prefill(dc.q, cu, 1500, dc.ctx_lens, 1500, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# non-causal sliding window (the draft attention): rows see pos - W .. ctx - 1
# ---------------------------------------------------------------------------

WINDOW_CASES = [
    # fmt, B, ctx, q_len, W, Hq, Hkv, D, bs, q_dtype, partitions
    ("e5m2", 2, (300, 5000), 8, 1000, 32, 8, 128, 2048, "f16", 0),
    ("e4m3", 3, (50, 700, 1500), 4, 63, 32, 8, 128, 16, "f16", 0),
    ("f16", 2, (65, 300), 1, 0, 4, 1, 64, 16, "f16", 0),
    ("e4m3", 1, (4097,), 16, 200, 32, 8, 128, 64, "f16", 3),
    ("e4m3", 2, (100, 900), 8, 5000, 32, 8, 128, 16, "bf16", 0),
    ("e5m2", 2, (129, 2100), 8, 7, 16, 4, 64, 32, "f16", 2),
]


def _oracle_window(case, W):
    from oracle import attention
    from tests.oracle_helpers import q_f32
    kc, vc = oracle_cache(case)
    o, _, _ = attention.attend(q_f32(case), case.q_lens, case.ctx_lens, kc, vc,
                               case.block_tables, case.cache_fmt, case.num_kv_heads,
                               case.softmax_scale, case.k_scale, case.v_scale, window=W)
    return o


@pytest.mark.parametrize("fmt,B,ctx,q_len,W,Hq,Hkv,D,bs,q_dtype,parts", WINDOW_CASES)
def test_window_parity(runner, fmt, B, ctx, q_len, W, Hq, Hkv, D, bs, q_dtype, parts):
    log(f"window {fmt} B={B} ctx={ctx} q_len={q_len} W={W} Hq={Hq} Hkv={Hkv} D={D} bs={bs} "
        f"q={q_dtype} P={parts}")
    case = _mk(fmt, B, ctx, q_len, Hq, Hkv, D, bs, q_dtype, sigma_kv=0.5)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.window(q_len, W, num_partitions=parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = _oracle_window(case, W).reshape(B, q_len, Hq, D)
    check_close(out, ref, fmt, "window f32")
    qt = torch.float16 if q_dtype == "f16" else torch.bfloat16
    out16 = dc.window(q_len, W, num_partitions=parts)
    check_close(out16, ref, fmt, "window q-dtype", out_dtype=qt)


def test_window_never_reads_the_prefix(runner):
    """Pages that hold only keys older than every row's window are poisoned
    with NaN codes after the writes; a read of any of them would turn the
    output into NaN (masked keys still multiply their values by zero)."""
    W, q_len = 300, 8
    case = _mk("e4m3", 2, (6000, 9000), q_len, bs=64)
    dc = runner.DeviceCase(case)
    dc.write_all()
    clean = dc.window(q_len, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bs = case.block_size
    for b in range(2):
        ctx = int(case.ctx_lens[b])
        first_seen = ctx - q_len - W
        for blk in range(first_seen // bs - 1):   # pages wholly before the window's first tile
            page = int(case.block_tables[b][blk])
            dc.key_cache[page].fill_(synth.POISON["e4m3"])
            dc.value_cache[page].fill_(synth.POISON["e4m3"])
    out = dc.window(q_len, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    assert torch.equal(out, clean)


def test_window_covering_the_context_equals_last_position_decode(runner):
    """A window longer than the context makes every row of the block see all
    ctx keys: each row equals a decode of the same query at the last position
    (same kernels; compared within the fp16 rounding of P)."""
    case = _mk("e5m2", 2, (300, 2100), 8, 32, 8, 128, 64, "f16", sigma_kv=0.5)
    dc = runner.DeviceCase(case)
    dc.write_all()
    out = dc.window(8, 10 ** 6, out_dtype=torch.float32)
    qv = dc.q.view(2, 8, 32, 128)
    for i in range(8):
        od = dc.decode(q=qv[:, i].contiguous(), out_dtype=torch.float32)
        assert torch.max(torch.abs(od - out[:, i])).item() < 1e-4


# ---------------------------------------------------------------------------
# the synchronous table check
# ---------------------------------------------------------------------------

def test_validate_tables(runner):
    """pa_validate_tables accepts a workload's own tables (block-table padding
    past the used pages is not looked at) and names the first bad entry."""
    from attention_paged_flashattention_amd import pagedattn as pa
    case = _mk("e4m3", 3, (100, 17, 0), 1)
    dc = runner.DeviceCase(case)
    bs, nb = case.block_size, case.num_blocks
    pa.pa_validate_tables(dc.block_tables, dc.ctx_lens, dc.max_ctx, bs, nb)

    def rejects(bt, cl, max_ctx=dc.max_ctx, what=""):
        with pytest.raises(pa.PagedAttnError) as e:
            pa.pa_validate_tables(bt, cl, max_ctx, bs, nb)
        assert e.value.status == pa.PA_ERR_INVALID_ARG
        assert what in str(e.value), str(e.value)

    bt = dc.block_tables.clone()
    bt[1, 1] = nb                              # a used page id out of range
    rejects(bt, dc.ctx_lens, what="block_tables[1][1]")
    bt = dc.block_tables.clone()
    bt[0, 6] = -1                              # last used page of a 100-key sequence
    rejects(bt, dc.ctx_lens, what="block_tables[0][6]")
    cl = dc.ctx_lens.clone()
    cl[2] = dc.max_ctx + 1                     # longer than max_context_len
    rejects(dc.block_tables, cl, what="context_lens[2]")
    # prefill chunk bounds: each chunk no longer than its context
    dev = dc.block_tables.device

    def cu(*v):
        return torch.tensor(v, dtype=torch.int32, device=dev)
    pa.pa_validate_tables(dc.block_tables, dc.ctx_lens, dc.max_ctx, bs, nb,
                          cu_seqlens_q=cu(0, 100, 117, 117))

    def rejects_cu(c, what):
        with pytest.raises(pa.PagedAttnError) as e:
            pa.pa_validate_tables(dc.block_tables, dc.ctx_lens, dc.max_ctx, bs, nb, cu_seqlens_q=c)
        assert e.value.status == pa.PA_ERR_INVALID_ARG
        assert what in str(e.value), str(e.value)
    rejects_cu(cu(0, 101, 117, 117), "sequence 0 has 101 new queries")
    rejects_cu(cu(0, 10, 8, 8), "decreases")
    rejects_cu(cu(1, 10, 20, 20), "cu_seqlens_q[0]")
    rejects_cu(cu(0, 10, 20, 21), "sequence 2 has 1 new queries")
    cl = dc.ctx_lens.clone()
    cl[1] = -3
    rejects(dc.block_tables, cl, what="context_lens[1]")


def test_profiling_hook(runner):
    """pa_profile_next_call: the next call's main kernel carries the event pair
    (positive duration) and computes the same result as an unprofiled call."""
    import ctypes
    from attention_paged_flashattention_amd import pagedattn as pa
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]

    def event():
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed(a, b):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    case = _mk("e4m3", 2, (700, 3000), 1, bs=64)
    dc = runner.DeviceCase(case)
    a, b = event(), event()
    pa.pa_profile_next_call(a, b)
    dc.write_all()                                 # the write kernel carries the events
    torch.cuda.synchronize()
    assert elapsed(a, b) > 0.0
    ref = dc.decode(out_dtype=torch.float32)
    a, b = event(), event()
    pa.pa_profile_next_call(a, b)
    out = dc.decode(out_dtype=torch.float32)       # the split kernel carries them
    torch.cuda.synchronize()
    assert elapsed(a, b) > 0.0
    assert torch.equal(out, ref)
    pa.pa_profile_next_call(event(), event())
    pa.pa_profile_next_call(None, None)            # a pending request can be cleared
    assert torch.equal(dc.decode(out_dtype=torch.float32), ref)

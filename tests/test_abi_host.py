"""Host-side tests of the C ABI (no GPU): the library loads, exports every
symbol include/pagedattn.h declares, and rejects bad arguments with the exact
status code before anything is launched."""

import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pagedattn.h")


@pytest.fixture(scope="module")
def pa():
    from attention_paged_flashattention_amd import pagedattn
    return pagedattn


def _declared():
    src = open(HEADER).read()
    return re.findall(r"PA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declares_the_four_operations():
    names = _declared()
    for n in ["kv_cache_write_fp8", "attn_prefill_paged", "attn_decode_paged", "attn_verify_paged"]:
        assert n in names


def test_library_exports_every_declared_symbol(pa):
    names = _declared()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(pa.lib(), n)
    assert set(pa.EXPORTS) == set(names)


def test_version(pa):
    assert "gfx950" in pa.pa_version()


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation
NUL = None


def _decode_args(**kw):
    a = dict(q=FAKE, q_dtype=0, batch=2, kc=FAKE, vc=FAKE, cache_dtype=3, bs=16, nb=10, bt=FAKE,
             maxblk=4, ctx=FAKE, maxctx=64, hq=8, hkv=2, d=128, ks=FAKE, vs=FAKE, scale=0.125,
             parts=0, ws=FAKE, wsb=1 << 20, out=FAKE, out_dtype=2, stream=NUL)
    a.update(kw)
    return a


def _call_decode(pa, **kw):
    a = _decode_args(**kw)
    return pa.lib().attn_decode_paged(a["q"], a["q_dtype"], a["batch"], a["kc"], a["vc"],
                                      a["cache_dtype"], a["bs"], a["nb"], a["bt"], a["maxblk"],
                                      a["ctx"], a["maxctx"], a["hq"], a["hkv"], a["d"], a["ks"],
                                      a["vs"], a["scale"], a["parts"], a["ws"], a["wsb"], a["out"],
                                      a["out_dtype"], a["stream"])


def _call_verify(pa, q_len, **kw):
    a = _decode_args(**kw)
    return pa.lib().attn_verify_paged(a["q"], a["q_dtype"], a["batch"], q_len, a["kc"], a["vc"],
                                      a["cache_dtype"], a["bs"], a["nb"], a["bt"], a["maxblk"],
                                      a["ctx"], a["maxctx"], a["hq"], a["hkv"], a["d"], a["ks"],
                                      a["vs"], a["scale"], a["parts"], a["ws"], a["wsb"], a["out"],
                                      a["out_dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=NUL), 1),
    (dict(kc=NUL), 1),
    (dict(bt=NUL), 1),
    (dict(out=NUL), 1),
    (dict(hq=7, hkv=2), 1),
    (dict(hkv=0), 1),
    (dict(d=0), 1),
    (dict(d=96), 2),
    (dict(d=256), 2),
    (dict(bs=24), 2),
    (dict(bs=8, maxctx=32), 2),
    (dict(bs=0), 1),
    (dict(q_dtype=2), 2),
    (dict(cache_dtype=1), 2),
    (dict(cache_dtype=0, q_dtype=1), 2),
    (dict(out_dtype=3), 2),
    (dict(ks=NUL), 1),
    (dict(vs=NUL), 1),
    (dict(scale=0.0), 1),
    (dict(scale=-1.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(maxctx=65), 1),           # > max_blocks * block_size
    (dict(maxctx=-1), 1),
    (dict(batch=-1), 1),
    (dict(parts=-2), 1),
    (dict(parts=5000), 2),
    (dict(ws=NUL), 1),
    (dict(wsb=16), 1),
    (dict(ws=ctypes.c_void_p(0x1010)), 1),   # misaligned workspace
    (dict(out=ctypes.c_void_p(0x1008)), 1),  # output not on a 16-byte boundary
    (dict(hq=128, hkv=1), 2),                # G = 128 rows exceed one decode group
    (dict(batch=65536), 2),                  # a launch dimension
])
def test_decode_rejects_before_launch(pa, kw, status):
    assert _call_decode(pa, **kw) == status
    assert pa.pa_last_error() != ""


def test_e5m2_needs_no_scales_and_batch_zero_is_a_noop(pa):
    # passes validation and returns before any launch because batch == 0
    assert _call_decode(pa, batch=0, cache_dtype=4, ks=NUL, vs=NUL) == 0
    assert pa.pa_last_error() == ""


def test_verify_limits(pa):
    assert _call_verify(pa, 0) == 1
    assert _call_verify(pa, 17, hq=8, hkv=2) == 2        # 17 * 4 rows > 64
    assert _call_verify(pa, 8, batch=0) == 0


def test_write_rejects_before_launch(pa):
    L = pa.lib()

    def call(**kw):
        a = dict(k=FAKE, v=FAKE, src=0, slots=FAKE, T=10, kc=FAKE, vc=FAKE, cdt=3, nb=4, bs=16,
                 hkv=2, d=128, ks=FAKE, vs=FAKE, stream=NUL)
        a.update(kw)
        return L.kv_cache_write_fp8(a["k"], a["v"], a["src"], a["slots"], a["T"], a["kc"], a["vc"],
                                    a["cdt"], a["nb"], a["bs"], a["hkv"], a["d"], a["ks"], a["vs"],
                                    a["stream"])
    assert call(T=-1) == 1
    assert call(k=NUL) == 1
    assert call(slots=NUL) == 1
    assert call(src=2) == 2
    assert call(cdt=1) == 2
    assert call(cdt=0, src=1) == 2
    assert call(ks=NUL) == 1
    assert call(d=40) == 2
    assert call(bs=48) == 2
    assert call(nb=0) == 1
    assert call(T=0) == 0                       # no-op, nothing launched
    assert call(T=0, cdt=4, ks=NUL, vs=NUL) == 0


def test_prefill_rejects_before_launch(pa):
    L = pa.lib()

    def call(**kw):
        a = dict(q=FAKE, qdt=1, cu=FAKE, B=1, maxq=64, totq=64, kc=FAKE, vc=FAKE, cdt=3, bs=2048,
                 nb=4, bt=FAKE, maxblk=2, ctx=FAKE, maxctx=4096, hq=32, hkv=8, d=128, ks=FAKE,
                 vs=FAKE, scale=0.088, out=FAKE, odt=2, stream=NUL)
        a.update(kw)
        return L.attn_prefill_paged(a["q"], a["qdt"], a["cu"], a["B"], a["maxq"], a["totq"], a["kc"],
                                    a["vc"], a["cdt"], a["bs"], a["nb"], a["bt"], a["maxblk"],
                                    a["ctx"], a["maxctx"], a["hq"], a["hkv"], a["d"], a["ks"],
                                    a["vs"], a["scale"], a["out"], a["odt"], a["stream"])
    assert call(cu=NUL) == 1
    assert call(maxq=5000) == 1
    assert call(hq=65, hkv=1) == 2           # G = 65 > 64
    assert call(out=ctypes.c_void_p(0x1002)) == 1   # output not on a 16-byte boundary
    assert call(B=-1) == 1
    assert call(B=0) == 0
    assert call(totq=0) == 0


def test_supports_table(pa):
    s = pa.pa_supports
    E4, E5, F16, BF16 = pa.PA_FP8_E4M3, pa.PA_FP8_E5M2, pa.PA_F16, pa.PA_BF16
    assert s(pa.PA_OP_DECODE, F16, E4, 128, 32, 8, 16, 1)
    assert s(pa.PA_OP_DECODE, F16, E4, 128, 32, 8, 2048, 1)
    assert s(pa.PA_OP_VERIFY, F16, E5, 128, 32, 8, 2048, 8)
    assert s(pa.PA_OP_VERIFY, F16, E5, 128, 32, 8, 2048, 16)
    assert not s(pa.PA_OP_VERIFY, F16, E5, 128, 32, 8, 2048, 17)
    assert s(pa.PA_OP_PREFILL, BF16, E4, 128, 32, 8, 2048, 4096)
    assert s(pa.PA_OP_PREFILL, F16, F16, 64, 4, 1, 16, 64)
    assert not s(pa.PA_OP_PREFILL, BF16, F16, 64, 4, 1, 16, 64)
    assert s(pa.PA_OP_PREFILL, BF16, E4, 128, 48, 8, 2048, 4096)     # G = 6
    assert s(pa.PA_OP_PREFILL, F16, E5, 128, 64, 1, 16, 64)          # G = 64
    assert not s(pa.PA_OP_PREFILL, F16, E5, 128, 65, 1, 16, 64)
    assert not s(pa.PA_OP_DECODE, F16, E4, 96, 32, 8, 16, 1)
    assert not s(pa.PA_OP_DECODE, F16, E4, 128, 32, 8, 24, 1)
    assert s(pa.PA_OP_WRITE, BF16, E4, 128, 8, 8, 2048, 0)
    assert not s(pa.PA_OP_WRITE, BF16, F16, 128, 8, 8, 2048, 0)


def test_partitions_and_workspace(pa):
    # one work-group per CU: 128K and 256K single-sequence decode in 32
    # partitions of 4096 / 8192 keys
    assert pa.pa_decode_partitions(1, 1, 32, 8, 128, 131072) == 32
    assert pa.pa_decode_partitions(1, 1, 32, 8, 128, 262144) == 32
    assert pa.pa_decode_partitions(8, 1, 32, 8, 128, 4096) == 4
    assert pa.pa_decode_partitions(4, 8, 32, 8, 128, 131072) == 8
    assert pa.pa_decode_partitions(16, 1, 32, 8, 128, 16384) == 2
    assert pa.pa_decode_partitions(1, 1, 32, 8, 128, 100) == 1
    def want(rows, parts, d):
        ml = rows * parts * 2 * 4
        return (ml + 255) // 256 * 256 + rows * parts * d * 4
    assert pa.pa_workspace_bytes(pa.PA_OP_DECODE, 1, 1, 32, 8, 128, 64, 131072) == want(32, 64, 128)
    assert pa.pa_workspace_bytes(pa.PA_OP_DECODE, 1, 1, 32, 8, 128, 0, 131072) == want(32, 32, 128)
    assert pa.pa_workspace_bytes(pa.PA_OP_PREFILL, 1, 4096, 32, 8, 128, 0, 32768) == 0
    assert pa.pa_workspace_bytes(pa.PA_OP_VERIFY, 4, 8, 32, 8, 128, 16, 131072) == \
        (4 * 8 * 32 * 16 * 2 * 4 + 255) // 256 * 256 + 4 * 8 * 32 * 16 * 128 * 4


def _call_window(pa, q_len, window, **kw):
    a = _decode_args(**kw)
    return pa.lib().attn_window_paged(a["q"], a["q_dtype"], a["batch"], q_len, window, a["kc"],
                                      a["vc"], a["cache_dtype"], a["bs"], a["nb"], a["bt"],
                                      a["maxblk"], a["ctx"], a["maxctx"], a["hq"], a["hkv"], a["d"],
                                      a["ks"], a["vs"], a["scale"], a["parts"], a["ws"], a["wsb"],
                                      a["out"], a["out_dtype"], a["stream"])


@pytest.mark.parametrize("q_len,window,kw,status", [
    (8, -1, {}, 1),                       # negative window
    (8, 16, dict(q=NUL), 1),
    (0, 16, {}, 1),                       # q_len must be positive
    (17, 16, {}, 2),                      # 17 * G(4) rows exceed one group
    (8, 16, dict(d=96), 2),
    (8, 16, dict(wsb=16), 1),
    (8, 16, dict(maxctx=65), 1),
])
def test_window_rejects_before_launch(pa, q_len, window, kw, status):
    assert _call_window(pa, q_len, window, **kw) == status
    assert pa.pa_last_error() != ""


def test_window_batch_zero_is_a_noop(pa):
    assert _call_window(pa, 8, 16, batch=0) == 0


def test_window_workspace_covers_only_the_window(pa):
    """The partitions of the window call tile the W + q_len keys a sequence's
    rows can see (plus one tile of rounding), so a short window over a long
    context needs a short workspace; a window longer than the context needs
    what the verify call needs."""
    ctx = 131072
    for batch in (1, 4):
        full = pa.pa_workspace_bytes(pa.PA_OP_VERIFY, batch, 8, 32, 8, 128, 0, ctx)
        assert pa.pa_window_workspace_bytes(batch, 8, 32, 8, 128, 0, ctx, 10 ** 6) == full
        small = pa.pa_window_workspace_bytes(batch, 8, 32, 8, 128, 0, ctx, 4096)
        assert 0 < small <= full
    # one sequence: 32 partitions over the context, but at most one per 256
    # keys of the 4096 + 8 + 64 the window's rows span
    s1 = pa.pa_window_workspace_bytes(1, 8, 32, 8, 128, 0, ctx, 4096)
    assert s1 == pa.pa_workspace_bytes(pa.PA_OP_VERIFY, 1, 8, 32, 8, 128, 17, ctx)
    assert s1 < pa.pa_workspace_bytes(pa.PA_OP_VERIFY, 1, 8, 32, 8, 128, 0, ctx)
    # explicit partitions: the same count as verify over the window's span
    assert pa.pa_window_workspace_bytes(4, 8, 32, 8, 128, 2, ctx, 4096) == \
        pa.pa_workspace_bytes(pa.PA_OP_VERIFY, 4, 8, 32, 8, 128, 2, 4096 + 8 + 64)
    assert pa.pa_window_workspace_bytes(4, 8, 32, 8, 128, 0, ctx, -1) == 0


def test_supports_window(pa):
    assert pa.pa_supports(pa.PA_OP_WINDOW, 0, 4, 128, 32, 8, 2048, 8)
    assert pa.pa_supports(pa.PA_OP_WINDOW, 0, 3, 128, 32, 8, 16, 16)
    assert not pa.pa_supports(pa.PA_OP_WINDOW, 0, 3, 128, 32, 8, 16, 17)


def _call_append(pa, q_len, knew=FAKE, vnew=FAKE, **kw):
    a = _decode_args(**kw)
    return pa.lib().attn_decode_append_paged(a["q"], a["q_dtype"], a["batch"], q_len, knew, vnew,
                                             a["kc"], a["vc"], a["cache_dtype"], a["bs"], a["nb"],
                                             a["bt"], a["maxblk"], a["ctx"], a["maxctx"], a["hq"],
                                             a["hkv"], a["d"], a["ks"], a["vs"], a["scale"],
                                             a["parts"], a["ws"], a["wsb"], a["out"],
                                             a["out_dtype"], a["stream"])


@pytest.mark.parametrize("q_len,kw,status", [
    (1, dict(knew=NUL), 1),
    (8, dict(vnew=NUL), 1),
    (1, dict(q=NUL), 1),
    (0, {}, 1),                           # q_len must be positive
    (17, {}, 2),                          # 17 * G(4) rows exceed one group
    (1, dict(d=96), 2),
    (1, dict(cache_dtype=0, q_dtype=1), 2),   # an fp16 cache takes fp16 sources
    (8, dict(ks=NUL), 1),                 # E4M3 needs scales for the write too
    (1, dict(wsb=16), 1),
    (8, dict(maxctx=65), 1),
])
def test_append_rejects_before_launch(pa, q_len, kw, status):
    assert _call_append(pa, q_len, **kw) == status
    assert pa.pa_last_error() != ""


def test_append_batch_zero_is_a_noop(pa):
    assert _call_append(pa, 8, batch=0) == 0
    assert pa.pa_last_error() == ""


def _no_device():
    """True where no GPU is present (checked without initialising HIP):
    valid argument sets then reach the launch, which must fail cleanly."""
    import torch
    return not os.path.exists("/dev/kfd") and torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_device(), reason="launches with fake pointers need a GPU-less host")
def test_valid_calls_without_a_device_report_the_launch_error(pa):
    """Arguments that pass every host check reach the kernel launch; with no
    device the launch fails and the call returns PA_ERR_HIP with a message.
    The status is this call's own: an invalid call right after it reports
    PA_ERR_INVALID_ARG, and a no-op call reports PA_OK."""
    L = pa.lib()
    calls = {
        "decode": lambda: _call_decode(pa),
        "decode_e5m2_no_scales": lambda: _call_decode(pa, cache_dtype=4, ks=NUL, vs=NUL),
        "verify_q8": lambda: _call_verify(pa, 8),
        "verify_q16": lambda: _call_verify(pa, 16),
        "window": lambda: _call_window(pa, 8, 16),
        "append_q1": lambda: _call_append(pa, 1),
        "append_q8": lambda: _call_append(pa, 8),
        "write": lambda: L.kv_cache_write_fp8(FAKE, FAKE, 0, FAKE, 10, FAKE, FAKE, 3, 4, 16, 2, 128,
                                              FAKE, FAKE, NUL),
        "prefill": lambda: L.attn_prefill_paged(FAKE, 1, FAKE, 1, 64, 64, FAKE, FAKE, 3, 2048, 4,
                                                FAKE, 2, FAKE, 4096, 32, 8, 128, FAKE, FAKE, 0.088,
                                                FAKE, 2, NUL),
    }
    for name, call in calls.items():
        assert call() == pa.PA_ERR_HIP, name
        msg = pa.pa_last_error()
        assert msg != "", name
        assert _call_decode(pa, q=NUL) == pa.PA_ERR_INVALID_ARG, name
        assert _call_decode(pa, batch=0) == pa.PA_OK, name
        assert pa.pa_last_error() == "", name


def _call_noalloc(pa, q_len, **kw):
    a = _decode_args(**kw)
    return pa.lib().attn_verify_paged_noalloc(a["q"], a["q_dtype"], a["batch"], q_len, a["kc"],
                                              a["vc"], a["cache_dtype"], a["bs"], a["nb"],
                                              a["bt"], a["maxblk"], a["ctx"], a["maxctx"], a["hq"],
                                              a["hkv"], a["d"], a["ks"], a["vs"], a["scale"],
                                              a["parts"], a["out"], a["out_dtype"], a["stream"])


def test_noalloc_checks_before_launch(pa):
    assert _call_noalloc(pa, 8, q=NUL) == pa.PA_ERR_INVALID_ARG
    assert _call_noalloc(pa, 17) == pa.PA_ERR_UNSUPPORTED          # 17 * 4 rows > 64
    assert _call_noalloc(pa, 8, batch=0) == pa.PA_OK
    # more partials than the 16 MiB scratch: 64 x 16 x 32 rows x 4096 partitions
    big = dict(batch=64, hq=32, hkv=8, maxblk=4096, bs=2048, maxctx=1 << 20, parts=64)
    assert pa.pa_workspace_bytes(pa.PA_OP_VERIFY, 64, 16, 32, 8, 128, 64, 1 << 20) > 16 << 20
    assert _call_noalloc(pa, 16, **big) == pa.PA_ERR_UNSUPPORTED
    assert "scratch" in pa.pa_last_error()


@pytest.mark.skipif(not _no_device(), reason="launches with fake pointers need a GPU-less host")
def test_noalloc_without_a_device_reports_the_hip_error(pa):
    assert _call_noalloc(pa, 8) == pa.PA_ERR_HIP
    assert pa.pa_last_error() != ""

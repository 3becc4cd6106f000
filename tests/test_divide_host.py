"""CPU check of the write kernels' divide-by-scale arithmetic (pa_divide.h).

The FP8 write encodes y = x / scale with IEEE float32 division, correctly
rounded ("1Cat-vLLM 1.0.0" README, "Optional experimental feature: FP8 KV
cache"; the rounding is the reading the oracle takes). The kernels form the
quotient from the scale's reciprocal plus one fma correction where that is
exact, and divide otherwise. The helper is host+device code: here it is
compiled for the host (hipcc, no GPU needed) and compared bit for bit with
numpy's IEEE float32 division over every fp16 and every bf16 value at scales
across the whole float32 range -- subnormal scales, scales whose reciprocal
overflows or is subnormal, infinity -- plus random float32 pairs.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_paged_flashattention_amd", "csrc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("divide") / "divide_check")
    subprocess.run([hipcc, "-O2", "-std=c++17", "--offload-host-only", "-x", "hip", "-I", CSRC,
                    os.path.join(ROOT, "tests", "divide_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def _run(exe, x, s):
    pairs = np.empty(2 * len(x), dtype=np.float32)
    pairs[0::2] = x
    pairs[1::2] = s
    out = subprocess.run([exe], input=pairs.tobytes(), capture_output=True, check=True).stdout
    return np.frombuffer(out, dtype=np.float32)


def _same(a, b):
    """Bitwise equality, any NaN equal to any NaN."""
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))


def _all16():
    f16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    bf16 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    return np.concatenate([f16, bf16])


SCALES = [2.0 ** -149, 3 * 2.0 ** -149, 2.0 ** -140, 2.0 ** -130, 2.0 ** -128, 1.5 * 2.0 ** -127,
          2.0 ** -127, 2.0 ** -126, 1.25 * 2.0 ** -126, 2.0 ** -100, 3.1415927e-3, 0.0105,
          0.2987244725227356, 1.0, 7.0, 13.0, 2.0 ** 100, 1.7 * 2.0 ** 125, 2.0 ** 126,
          1.5 * 2.0 ** 126, 2.0 ** 127, 1.9 * 2.0 ** 127, float(np.finfo(np.float32).max),
          float("inf")]


def test_every_16bit_value_at_extreme_scales(harness):
    x = _all16()
    for s in SCALES:
        s32 = np.float32(s)
        got = _run(harness, x, np.full_like(x, s32))
        with np.errstate(all="ignore"):
            ref = x / s32
        bad = ~_same(got, ref)
        assert not bad.any(), (s, x[bad][:5], got[bad][:5], ref[bad][:5])


def test_random_float32_pairs(harness):
    rng = np.random.default_rng(17)
    n = 1 << 20
    x = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    s = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    # and scales of the usual size: amax / 448 for amax in [1e-3, 1e3]
    s[: n // 2] = (np.exp(rng.uniform(np.log(1e-3), np.log(1e3), n // 2)) / 448).astype(np.float32)
    got = _run(harness, x, s)
    with np.errstate(all="ignore"):
        ref = x / s
    bad = ~_same(got, ref)
    assert not bad.any(), (x[bad][:5], s[bad][:5], got[bad][:5], ref[bad][:5])


def test_zero_over_tiny_scale_is_a_signed_zero(harness):
    # the case a reciprocal-only method gets wrong: 1/s overflows, 0 * inf = NaN
    x = np.array([0.0, -0.0, 1e-3, -1e-3], dtype=np.float32)
    got = _run(harness, x, np.full(4, np.float32(1e-39)))
    assert got[0] == 0 and not np.signbit(got[0])
    assert got[1] == 0 and np.signbit(got[1])
    assert np.isfinite(got[2:]).all()

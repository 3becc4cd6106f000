"""Pins for the oracle's FP8 codec (CPU only).

Independent of the oracle's own code: hand-derived spot values
(tests/golden/fp8_spot_values.txt, from the OCP FP8 format definition) and
torch's CPU float8 casts, an independent library routine (RNE but
non-saturating, so inputs are pre-clamped to the largest finite value).
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
MAXF = {"e4m3": 448.0, "e5m2": 57344.0}


def _parse_val(s):
    s = s.strip()
    if s in ("nan", "inf", "-inf"):
        return float(s)
    return float(s)


def _golden(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "fp8_spot_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def test_decode_spot_values(golden_dir):
    n = 0
    for row in _golden(golden_dir):
        if row[0] != "decode":
            continue
        fmt, code, val = row[1], int(row[2], 16), _parse_val(row[3])
        got = fp8.decode_table(fmt)[code]
        if math.isnan(val):
            assert math.isnan(got), (fmt, hex(code))
        else:
            assert got == val, (fmt, hex(code), got, val)
            assert math.copysign(1.0, got) == math.copysign(1.0, val)
        n += 1
    assert n >= 25


def test_encode_spot_values(golden_dir):
    n = 0
    for row in _golden(golden_dir):
        if row[0] != "encode":
            continue
        fmt, x, scale, code = row[1], _parse_val(row[2]), row[3], int(row[4], 16)
        scale = None if scale == "-" else float(scale)
        got = int(fp8.encode(np.array([x], dtype=np.float64), fmt, scale)[0])
        assert got == code, (fmt, x, scale, hex(got), hex(code))
        n += 1
    assert n >= 20


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_table_matches_torch(fmt):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
    tab = fp8.decode_table(fmt)
    assert np.array_equal(np.isnan(ref), np.isnan(tab))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], tab[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(tab[fin]))


def _torch_encode(x32, fmt, scale):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    if scale is not None:
        t = t / torch.tensor(np.float32(scale))
    m = MAXF[fmt]
    t = torch.clamp(t, -m, m)
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


def _all_fp16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    return x[~np.isnan(x)]


@pytest.mark.parametrize("fmt,scale", [
    ("e5m2", None),
    ("e4m3", None),
    ("e4m3", 1.0),
    ("e4m3", float(np.float32(4.71875) / np.float32(448.0))),
    ("e4m3", float(np.float32(0.0123) / np.float32(448.0))),
    ("e4m3", float(np.float32(37.5) / np.float32(448.0))),
    ("e4m3", 7.0),
    ("e4m3", 13.0),
    ("e5m2", 0.37),
])
def test_encode_exhaustive_fp16(fmt, scale):
    x = _all_fp16()
    got = fp8.encode(x, fmt, scale)
    ref = _torch_encode(x.astype(np.float32), fmt, scale)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_encode_bf16_like_inputs():
    """bf16 inputs (8 significant bits, full float32 exponent range) over a
    dense sample of bit patterns, against torch."""
    bits = np.arange(0, 65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x)]
    for fmt, scale in [("e4m3", float(np.float32(5.25) / np.float32(448))), ("e5m2", None)]:
        got = fp8.encode(x, fmt, scale)
        ref = _torch_encode(x, fmt, scale)
        assert np.array_equal(got, ref), fmt


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_roundtrip_every_finite_code(fmt):
    tab = fp8.decode_table(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(tab[c])], dtype=np.uint8)
    back = fp8.encode(tab[codes], fmt)
    assert np.array_equal(back, codes)


def test_dequant_applies_scale_in_float64():
    codes = np.array([0x38, 0x7e, 0x01], dtype=np.uint8)
    s = np.float32(0.1)
    got = fp8.dequant(codes, "e4m3", s)
    assert np.array_equal(got, np.array([1.0, 448.0, 2.0 ** -9]) * np.float64(s))


# ---- planted mistakes: the pins above must reject plausible codec bugs ----

def _encode_variant(monkeypatch, which):
    if which == "truncate":
        monkeypatch.setattr(fp8.np, "rint", np.trunc, raising=True)
    elif which == "no_saturation":
        monkeypatch.setattr(fp8, "max_finite", lambda fmt: float("inf"))
    elif which == "round_half_up":
        monkeypatch.setattr(fp8.np, "rint", lambda a: np.floor(a + 0.5))
    elif which == "reciprocal_scale":
        orig = fp8.to_float32_scaled

        def recip(x, scale=None):
            y = np.asarray(x).astype(np.float32)
            if scale is not None:
                y = y * (np.float32(1.0) / np.float32(scale))
            return y
        monkeypatch.setattr(fp8, "to_float32_scaled", recip)
        del orig


@pytest.mark.parametrize("which", ["truncate", "no_saturation", "round_half_up", "reciprocal_scale"])
def test_planted_codec_mistakes_are_caught(monkeypatch, which, golden_dir):
    """Each planted mistake must fail the spot values or the exhaustive sweep."""
    _encode_variant(monkeypatch, which)
    failed = False
    try:
        test_encode_spot_values(golden_dir)
    except (AssertionError, Exception):
        failed = True
    if not failed:
        scale = float(np.float32(4.71875) / np.float32(448.0))
        x = _all_fp16()
        x = x[np.abs(x.astype(np.float64)) < 60000]
        got = fp8.encode(x, "e4m3", scale)
        failed = not np.array_equal(got, _torch_encode(x.astype(np.float32), "e4m3", scale))
    assert failed, which

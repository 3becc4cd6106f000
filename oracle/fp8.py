"""FP8 (E4M3FN, E5M2) codec, written from the format definitions.

Test infrastructure only (see ``oracle/__init__.py``).

The pages name the two KV-cache formats ("1Cat-vLLM 1.0.0" README, "Optional
experimental feature: FP8 KV cache"; "SM70 release profile", the E4M3 release
KV) but do not define them. The definitions below are those of the OCP 8-bit
floating point specification:

* E4M3 (the "FN" flavour): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
  Exponent field 0 is subnormal, value m * 2^-9. The all-ones pattern
  S.1111.111 is NaN; every other pattern with exponent 15 is a normal number,
  so the largest finite value is 1.75 * 2^8 = 448. There are no infinities.
* E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits. Exponent 0 is
  subnormal, value m * 2^-16. Exponent 31 is +-inf (m = 0) or NaN (m != 0).
  Largest finite value 1.75 * 2^15 = 57344.

Readings taken where the pages are silent (each is listed with its reason in
the design notes):

* Encoding divides by the per-head scale in IEEE float32 (correctly rounded),
  saturates to +-max finite, then rounds to nearest with ties to even. The
  sign is kept, so negative values that round to zero encode as 0x80.
* Without a scale (E5M2 "no scales") the float32 value is encoded directly.
* NaN input encodes as S.1111111 (a NaN in both formats); it is not exercised.
"""

import numpy as np

E4M3 = "e4m3"
E5M2 = "e5m2"

# (exponent bits, mantissa bits, bias)
_FORMATS = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}


def _check(fmt):
    if fmt not in _FORMATS:
        raise ValueError(f"unknown FP8 format {fmt!r}")
    return _FORMATS[fmt]


def decode_value(code, fmt):
    """Value of one FP8 byte, as a Python float, straight from the definition."""
    ebits, mbits, bias = _check(fmt)
    code = int(code) & 0xFF
    s = code >> 7
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    sign = -1.0 if s else 1.0
    emax_field = (1 << ebits) - 1
    if fmt == E4M3:
        if e == emax_field and m == (1 << mbits) - 1:
            return float("nan")
    else:
        if e == emax_field:
            return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        # subnormal: m / 2^mbits * 2^(1 - bias)
        return sign * (m / float(1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / float(1 << mbits)) * 2.0 ** (e - bias)


def decode_table(fmt):
    """float64[256]: the value of every code."""
    return np.array([decode_value(c, fmt) for c in range(256)], dtype=np.float64)


def max_finite(fmt):
    tab = decode_table(fmt)
    return float(np.nanmax(tab[np.isfinite(tab)]))


def min_normal(fmt):
    _, _, bias = _check(fmt)
    return 2.0 ** (1 - bias)


def quantum_subnormal(fmt):
    """Spacing of the grid below the smallest normal: 2^(1 - bias - mbits)."""
    _, mbits, bias = _check(fmt)
    return 2.0 ** (1 - bias - mbits)


def to_float32_scaled(x, scale=None):
    """y = float32(x) / float32(scale) in IEEE float32 (numpy divides with
    correct rounding); y = float32(x) when no scale is given."""
    y = np.asarray(x).astype(np.float32)
    if scale is not None:
        # a quotient beyond the float32 range is +-inf, as IEEE division gives
        # it; round_to_grid saturates it (numpy's overflow warning is muted)
        with np.errstate(over="ignore"):
            y = y / np.float32(scale)
    return y


def round_to_grid(y, fmt):
    """Saturate |y| to the largest finite value, then round to the nearest
    point of the FP8 grid with ties to even. Returns float64 magnitudes and
    the sign bits separately; NaN magnitudes stay NaN."""
    _, mbits, _ = _check(fmt)
    y = np.asarray(y, dtype=np.float64)          # float32 -> float64 is exact
    neg = np.signbit(y)
    a = np.abs(y)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    a = np.minimum(a, max_finite(fmt))           # saturate (also +-inf)
    # quantum: 2^(floor(log2 a) - mbits) for normals, fixed below min normal
    _, ex = np.frexp(np.where(a > 0, a, 1.0))    # a = f * 2^ex, f in [0.5, 1)
    q_norm = np.ldexp(1.0, ex - 1 - mbits)
    quantum = np.where(a >= min_normal(fmt), q_norm, quantum_subnormal(fmt))
    # a / quantum is exact in float64 (power-of-two scaling); rint is RNE
    r = np.rint(a / quantum) * quantum
    r = np.where(nan, np.nan, r)
    return r, neg


def encode(x, fmt, scale=None):
    """uint8 codes for x (any real dtype), optional float32 scale divisor."""
    y = to_float32_scaled(x, scale)
    mag, neg = round_to_grid(y, fmt)
    tab = decode_table(fmt)
    pos_codes = np.arange(0, 128)
    finite = np.isfinite(tab[pos_codes])
    pos_codes = pos_codes[finite]
    pos_vals = tab[pos_codes]                     # strictly increasing
    nan = np.isnan(mag)
    idx = np.searchsorted(pos_vals, np.where(nan, 0.0, mag))
    idx = np.minimum(idx, len(pos_vals) - 1)
    if not np.all(nan | (pos_vals[idx] == mag)):
        raise AssertionError("rounded value is not on the FP8 grid")
    codes = pos_codes[idx].astype(np.uint16)
    codes = np.where(nan, 0x7F, codes)
    codes = codes | np.where(neg, 0x80, 0)
    return codes.astype(np.uint8)


def dequant(codes, fmt, scale=None):
    """float64 values of codes times float64(scale) (scale defaults to 1)."""
    v = decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]
    if scale is not None:
        v = v * np.float64(np.float32(scale))
    return v

"""OCP FP8 E4M3FN: exact decode and round-to-nearest-even encode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Format (named as the required input type in "Route large SM90
row/column-scaled FP8 GEMMs to Torch", Summary; the gfx94x FNUZ variant with a
224 maximum is the other format PR #33533 warns about, Modifications 3 -- it is
not this one): one sign bit, a 4-bit exponent E with bias 7 and a 3-bit
mantissa T.

    E = 0           value = (-1)^s * T * 2^-9              (subnormal)
    E = 15, T = 7   NaN                                    (no infinities)
    otherwise       value = (-1)^s * (8 + T) * 2^(E - 10)

The largest finite magnitude is 448 (code 0x7E).

Encoding is written as a search over the 127 non-negative finite magnitudes,
not as bit manipulation: the nearest one wins, an exact midpoint goes to the
code with the even mantissa (round half to even), and the sign bit is copied
from the input, so -0.0 encodes as 0x80.  PR #33533 (Motivation) works one tie
through: 168.0 lies halfway between 160 and 176 and must give 160, while the
fp32 value one ulp above it must give 176.

Pins (tests/test_oracle_e4m3.py): all 256 codes decode equal to torch's
independent float8_e4m3fn CPU conversion; encode(decode(c)) == c for every
finite code; encode agrees with a brute-force nearest search over all codes and
with torch's fp32 -> float8_e4m3fn cast on every midpoint, its fp32 neighbours
and random samples; the worked example of PR #33533 (tests/golden).
"""
import numpy as np

E4M3_MAX = 448.0


def decode_code(c: int) -> float:
    """Exact value of one E4M3FN code (NaN for 0x7F / 0xFF)."""
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    t = c & 0x7
    if e == 15 and t == 7:
        return float("nan")
    if e == 0:
        mag = t * 2.0 ** -9
    else:
        mag = (8 + t) * 2.0 ** (e - 10)
    return -mag if s else mag


# 256-entry table of exact values (float64 holds every one exactly).
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes in code order 0x00..0x7E; they increase with
# the code, so the code of a magnitude is its index here.
_MAGS = DECODE_TABLE[:127].copy()
# Midpoints between neighbouring magnitudes.  Each has at most five
# significant bits, so float64 holds it exactly and comparisons against it are
# exact.
_MIDS = (_MAGS[:-1] + _MAGS[1:]) / 2.0


def decode(codes) -> np.ndarray:
    """uint8 codes (any shape) -> exact float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[codes]


def encode(y) -> np.ndarray:
    """Round finite values with |y| <= 448 to E4M3FN, ties to even.

    ``y`` is float32 or float64; it is widened exactly to float64.  Values
    outside [-448, 448] or non-finite values are rejected: the quantizers clamp
    before they encode, so such an input means a bug in the caller.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("encode: non-finite input")
    a = np.abs(y)
    if np.any(a > E4M3_MAX):
        raise ValueError("encode: |y| > 448 (clamp first)")
    # i = number of midpoints strictly below a, so _MIDS[i-1] < a <= _MIDS[i]:
    # a is nearest to magnitude i unless it sits exactly on _MIDS[i].
    i = np.searchsorted(_MIDS, a, side="left")
    code = i.astype(np.int64)
    inside = i < _MIDS.size
    on_mid = np.zeros(a.shape, dtype=bool)
    on_mid[inside] = a[inside] == _MIDS[i[inside]]
    # On a midpoint the candidates are i and i+1; take the even one.
    code[on_mid & (code % 2 == 1)] += 1
    sign = np.signbit(y).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def finite_codes() -> np.ndarray:
    """All 254 finite codes (both signs, both zeros)."""
    c = np.arange(256, dtype=np.uint8)
    return c[~np.isnan(DECODE_TABLE)]

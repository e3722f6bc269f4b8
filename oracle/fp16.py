"""Round float64 to IEEE binary16, nearest with ties to even.

TEST INFRASTRUCTURE ONLY (see the package docstring).

binary16 has 11 significant bits (10 stored), a 5-bit exponent and a largest
finite value of 65504.  The rounding is done with exact float64 operations:
for |x| in [2^e, 2^(e+1)) the fp16 spacing is 2^(e-10) (2^-24 below the normal
range, which starts at 2^-14), x / spacing is an exact float64, numpy's rint
rounds it half-to-even, and multiplying back is exact; a result above 65504
is an overflow to +-inf.  fp16 is one of the two output dtypes of the
deterministic FP8 linear (sglang PR #44861, Modifications: BF16/FP16 cases).

Pins (tests/test_oracle_fp16.py): on fp32 inputs it equals torch's fp32 ->
float16 cast; on random float64 inputs it equals a brute-force choice between
the neighbouring fp16 values made with Python fractions; the overflow
threshold 65520 (65504 plus half a spacing) and the subnormal spacing.
"""
import numpy as np

_F16_MAX = 65504.0


def round_to_fp16(x) -> np.ndarray:
    """float64 array -> float64 array of fp16 values (RNE).  Overflow -> inf."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(np.abs(xf))  # |x| = f * 2^e2 with f in [0.5, 1)
    e = np.maximum(e2 - 1, -14)   # subnormal fp16 share the 2^-24 spacing
    spacing = np.ldexp(1.0, e - 10)
    r = np.rint(xf / spacing) * spacing
    big = np.abs(r) > _F16_MAX
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def to_fp16_bits(x) -> np.ndarray:
    """float64 -> uint16 fp16 bit patterns (RNE)."""
    r = round_to_fp16(x).astype(np.float16)  # exact: r is an fp16 value
    return r.view(np.uint16)


def bits_to_f64(bits) -> np.ndarray:
    """uint16 fp16 bit patterns -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)

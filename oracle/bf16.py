"""Round float64 to bfloat16, nearest with ties to even.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bfloat16 keeps fp32's 8-bit exponent and 8 significant bits (7 stored).  The
rounding is done with exact float64 operations: for |x| in [2^e, 2^(e+1)) the
bf16 spacing is 2^(e-7) (2^-133 below the normal range), x / spacing is an
exact float64, numpy's rint rounds it half-to-even, and multiplying back is
exact.  The GEMM outputs of the pages' path are bf16 ("Route large SM90
row/column-scaled FP8 GEMMs to Torch", Summary).

Pins (tests/test_oracle_bf16.py): on fp32-representable inputs it equals
torch's fp32 -> bfloat16 cast; on random float64 inputs it equals a
brute-force choice between the two neighbouring bf16 values computed with
Python fractions.
"""
import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")


def round_to_bf16(x) -> np.ndarray:
    """float64 array -> float64 array of bf16 values (RNE).  Overflow -> inf."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(np.abs(xf))  # |x| = f * 2^e2 with f in [0.5, 1)
    e = e2 - 1                    # |x| in [2^e, 2^(e+1))
    e = np.maximum(e, -126)       # subnormal bf16 share the 2^-133 spacing
    spacing = np.ldexp(1.0, e - 7)
    r = np.rint(xf / spacing) * spacing
    r[np.abs(r) > _BF16_MAX] = np.copysign(np.inf, r[np.abs(r) > _BF16_MAX])
    out[fin] = r
    return out


def to_bf16_bits(x) -> np.ndarray:
    """float64 -> uint16 bf16 bit patterns (RNE)."""
    r = round_to_bf16(x).astype(np.float32)  # exact: r is a bf16 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)

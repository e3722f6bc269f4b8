"""Scaled E4M3FN GEMMs: exact accumulation, scales, one rounding to bf16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Rowwise / per-tensor ("Route large SM90 row/column-scaled FP8 GEMMs to Torch",
Summary: E4M3FN inputs, fp32 row and column scales, bf16 output, no bias; the
per-tensor form with two scalar scales is the one in the prhub digest of sglang
PR #33148, key source excerpts):

    acc[m, n] = sum_k dec(A[m, k]) * dec(B[n, k])          (exact)
    out[m, n] = bf16( acc[m, n] * (sa[m] * sb[n]) )

With the optional epilogue of the deterministic FP8 linear (sglang PR #44861,
Modifications: tests with bias and BF16/FP16 outputs; the linear's apply()
passes an optional bias, prhub digest of PR #33148, key source excerpts):

    out[m, n] = rnd( acc[m, n] * (sa[m] * sb[n]) + bias[n] )

with bias a vector of output-dtype values and rnd the round-to-nearest-even
conversion to bf16 or fp16 (fp16 overflows to +-inf) -- the pages print no
order of the epilogue operations; this is the plain reading, computed in
float64 and rounded once.

A is [M, K] row-major, B is [N, K] with K contiguous (the [K, N]
column-major weight of the digest's excerpt), sa/sb are fp32 vectors or
scalars.

Why the float64 matmul below is exact: every E4M3FN value is an integer
multiple of 2^-9 no larger than 448, so every product is a multiple of 2^-18
no larger than 448^2 < 2^17.7, and every partial sum of K <= 2^17 products is a
multiple of 2^-18 below 2^34.7; it needs at most 53 significant bits, so
float64 holds every partial sum exactly whatever the summation order or
blocking of the library routine.  sa * sb (two fp32 values) is exact in
float64 too, so the only roundings are acc * (sa * sb) to float64 and then to
bf16.

Blockwise (the 1x128-group activation x 128x128-block weight form; the pages
name the consumer -- a DeepGEMM blockwise GEMM fed by the 1x128 UE8M0 quant,
PR #33533 Modifications 3 -- but print no formula; this is the plain reading):

    P[kb][m, n] = sum_{k in block kb} dec(A[m, k]) * dec(B[n, k])     (exact)
    out[m, n]   = bf16( sum_kb  sa[m, kb] * sb[n // 128, kb] * P[kb][m, n] )

with the outer sum in float64 in ascending kb.

Pins (tests/test_oracle_gemm.py): the float64 accumulator equals exact int64
accumulation in units of 2^-18; one-hot products of all 254 x 254 finite codes
come out exactly; small-integer cases with closed-form sums; zero rows give
+0; power-of-two scale linearity; transposition symmetry; agreement with
torch's float64 matmul; blockwise with unit scales equals rowwise, and a
2^j block scale scales exactly that block's contribution.
"""
import numpy as np

from . import e4m3
from .bf16 import to_bf16_bits, bits_to_f64
from . import fp16 as _fp16

KMAX_EXACT = 1 << 17


def _as_vec(s, n):
    s = np.asarray(s, dtype=np.float32)
    if s.ndim == 0 or s.size == 1:
        return np.full(n, s.reshape(-1)[0] if s.size else 0.0, dtype=np.float32)
    if s.size != n:
        raise ValueError("scale vector has the wrong length")
    return s.reshape(n)


class MMResult:
    """bits: output [M, N] as uint16 (bf16, or fp16 when out == "fp16");
    value: float64 before the output rounding; acc: exact accumulator;
    sab: sa[m] * sb[n] (exact)."""

    def __init__(self, bits, value, acc, sab, out="bf16"):
        self.bits = bits
        self.value = value
        self.acc = acc
        self.sab = sab
        self.dtype = out

    @property
    def out(self):
        return _fp16.bits_to_f64(self.bits) if self.dtype == "fp16" else bits_to_f64(self.bits)


def accumulate(a_codes, b_codes, chunk=4096):
    """Exact sum_k dec(A[m,k]) * dec(B[n,k]) as float64 [M, N].

    B is decoded ``chunk`` rows at a time to bound memory; chunking the output
    columns does not touch any single output's sum.
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    b_codes = np.asarray(b_codes, dtype=np.uint8)
    M, K = a_codes.shape
    N, K2 = b_codes.shape
    if K != K2:
        raise ValueError("A and B disagree on K")
    if K > KMAX_EXACT:
        raise ValueError("K too large for exact float64 accumulation")
    a = e4m3.decode(a_codes)
    if np.isnan(a).any():
        raise ValueError("A holds NaN codes")
    acc = np.empty((M, N), dtype=np.float64)
    for j in range(0, N, chunk):
        b = e4m3.decode(b_codes[j:j + chunk])
        if np.isnan(b).any():
            raise ValueError("B holds NaN codes")
        acc[:, j:j + chunk] = a @ b.T
    return acc


def scaled_mm(a_codes, b_codes, sa, sb, bias=None, out="bf16"):
    """Rowwise (sa [M], sb [N]) or per-tensor (scalars) scaled GEMM; bias:
    None or [N] output-dtype values (as floats); out: "bf16" or "fp16"."""
    M = np.asarray(a_codes).shape[0]
    N = np.asarray(b_codes).shape[0]
    acc = accumulate(a_codes, b_codes)
    sa64 = _as_vec(sa, M).astype(np.float64)
    sb64 = _as_vec(sb, N).astype(np.float64)
    sab = sa64[:, None] * sb64[None, :]
    value = acc * sab
    if bias is not None:
        value = value + np.asarray(bias, dtype=np.float64).reshape(1, N)
    if out == "fp16":
        return MMResult(_fp16.to_fp16_bits(value), value, acc, sab, out)
    if out != "bf16":
        raise ValueError("out must be 'bf16' or 'fp16'")
    return MMResult(to_bf16_bits(value), value, acc, sab)


def ue8m0_values(e_bytes):
    """Scale values of UE8M0 exponent bytes: 2^(byte - 127), exact, as float64
    (the storage form 2^(e-127) of sglang PR #33533, Modifications 3).  Every
    byte 0..255 is taken as a power of two; bytes 0 and 255 give 2^-127 and
    2^128, outside the fp32 normal range (the latter beyond fp32 itself)."""
    e = np.asarray(e_bytes)
    if e.dtype != np.uint8:
        raise ValueError("UE8M0 scales are bytes")
    return np.ldexp(np.ones(e.shape), e.astype(np.int64) - 127)


def blockwise_mm(a_codes, a_scale, b_codes, b_scale, block=128):
    """Blockwise scaled GEMM.

    a_scale: [M, ceil(K/block)] scale values: float32 values, or float64 as
    given (ue8m0_values for UE8M0 bytes, which may lie beyond fp32);
    b_scale: [ceil(N/block), ceil(K/block)] float32.
    Returns (MMResult with sab = max_kb a_scale * b_scale, the per-output
    scale magnitude the tolerance uses).
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    b_codes = np.asarray(b_codes, dtype=np.uint8)
    M, K = a_codes.shape
    N = b_codes.shape[0]
    KB = -(-K // block)
    a_scale = np.asarray(a_scale)
    if a_scale.dtype != np.float64:
        a_scale = a_scale.astype(np.float32)
    a_scale = a_scale.reshape(M, KB).astype(np.float64)
    b_scale = np.asarray(b_scale, dtype=np.float32).reshape(-(-N // block), KB).astype(np.float64)
    nb_of_n = np.arange(N) // block
    total = np.zeros((M, N), dtype=np.float64)
    smax = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        ks = slice(kb * block, min(K, (kb + 1) * block))
        P = accumulate(a_codes[:, ks], b_codes[:, ks])
        s = a_scale[:, kb][:, None] * b_scale[nb_of_n, kb][None, :]
        total += s * P
        smax = np.maximum(smax, s)
    return MMResult(to_bf16_bits(total), total, None, smax)


def scaled_mm_entries(a_codes, b_codes, sa, sb, rows, cols, bias=None, out="bf16"):
    """The rowwise GEMM on the sub-grid rows x cols only (for sampled checks
    at full size).  Same definition as scaled_mm."""
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    b_codes = np.asarray(b_codes, dtype=np.uint8)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    M = a_codes.shape[0]
    N = b_codes.shape[0]
    sa_v = _as_vec(sa, M)[rows]
    sb_v = _as_vec(sb, N)[cols]
    b_v = None if bias is None else np.asarray(bias).reshape(-1)[cols]
    return scaled_mm(a_codes[rows], b_codes[cols], sa_v, sb_v, b_v, out)

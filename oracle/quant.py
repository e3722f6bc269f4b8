"""Activation and weight quantization to E4M3FN, step by step in fp32.

TEST INFRASTRUCTURE ONLY (see the package docstring).

All arithmetic below is IEEE binary32 with round-to-nearest-even (numpy float32
operations), written as RN32(.) in the comments.  Inputs arrive as float32
arrays holding bf16 or fp16 values widened exactly.

Group quant with an fp32 scale (PR #33533 "[JIT] per_token_group_quant: fix the
fp16 UE8M0 multiplier overflow ...", commit messages and Motivation), for each
group of ``group`` consecutive elements of a row (group == K: per token):

    a  = max |x|                       absolute maximum of the group
    a' = max(a, 1e-10)                 floor; a compile-time constant on the
                                       pages (Modifications 4), applied as a
                                       max() because 448/1e-10 = 4.5e12 is the
                                       multiplier's stated ceiling (Mod. 1)
    s  = RN32(a' / 448)                scale stored for the GEMM
    m  = RN32(448 / a')                multiplier: one correctly rounded
                                       divide per group (Motivation; the
                                       "plain divide" reading)
    q  = E4M3(clamp(RN32(x * m), -448, 448))

UE8M0 scales (same PR: Modifications 3 names the fp32 2^(e-127) storage; Mod. 1
the overflow this form must avoid): e = ceil(log2 s), read from the fp32 bits
(unbiased exponent, plus one unless the mantissa is zero), so that 2^e >= s and
no element is clipped.  The stored byte is e + 127, the scale value 2^e, and
q = E4M3(clamp(RN32(x * 2^-e))).  The multiplier 2^-e is a finite fp32 power of
two whatever the input dtype, so the fp16 failure the PR describes (an inf
multiplier turning whole groups into +-448 and zero rows into NaN -> +448)
cannot arise.

Fused SiLU-and-mul (Modifications 2: silu evaluated per element with a plain
divide): the row [g | u] is split in halves, gate first, and

    silu32(g) = RN32(g / RN32(1 + RN32(exp(-g))))
    y         = RN32(silu32(g) * u)

where RN32(exp(t)) is the correctly rounded fp32 exponential.  The pages do not
fix the exponential's accuracy; correctly rounded is the one choice both sides
can meet exactly.  It is computed here as float64 exp rounded to fp32, and
tests/test_oracle_quant.py checks, for every value a bf16 or fp16 gate can
take, that this equals the exponential evaluated with Python's decimal module
at 40 digits and rounded once.

Static per-tensor quant with a given scalar s (prhub digest of sglang
PR #33148, motivation and key source excerpts: one checkpoint activation
scale per layer):  q = E4M3(clamp(RN32(x * RN32(1 / s)))).

Weight quant: per output channel (rows of B [N, K], the a1 rule with
group == K), or per 128x128 block with the same fp32 rule over each block.

Pins: tests/test_oracle_quant.py (closed forms for zero groups and
power-of-two maxima, scale invariance under x * 2^j, sign symmetry,
permutation equivariance, every bf16 pattern through a group whose maximum is
448, the fp16 tiny-group regression, the exponential against decimal, and the
golden values in tests/golden/).
"""
import numpy as np

from . import e4m3

F32 = np.float32
AMAX_FLOOR = F32(1e-10)
Q_MAX = F32(448.0)


def _clamp(v):
    return np.minimum(np.maximum(v, -Q_MAX), Q_MAX).astype(F32)


def ue8m0_exponent(s):
    """ceil(log2 s) for positive normal float32 s, from its bit fields."""
    s = np.asarray(s, dtype=F32)
    bits = s.view(np.uint32)
    biased = ((bits >> 23) & 0xFF).astype(np.int32)
    if np.any(biased == 0) or np.any(biased == 255) or np.any(bits >> 31):
        raise ValueError("ue8m0_exponent: scale must be positive, normal, finite")
    mant = bits & 0x7FFFFF
    return biased - 127 + (mant != 0).astype(np.int32)


def pow2_f32(e):
    """2^e as float32 (exact for -126 <= e <= 127)."""
    e = np.asarray(e, dtype=np.int32)
    if np.any(e < -126) or np.any(e > 127):
        raise ValueError("pow2_f32: exponent out of the normal fp32 range")
    return np.ldexp(F32(1.0), e).astype(F32)


class GroupQuant:
    """Result of a group quant: codes [M, K] uint8, scale [M, G] float32 (the
    value the GEMM multiplies by), and for UE8M0 the exponent byte [M, G]."""

    def __init__(self, codes, scale, ue8m0_byte=None):
        self.codes = codes
        self.scale = scale
        self.ue8m0_byte = ue8m0_byte


def quant_group(x32, group, pow2=False):
    """Per-token (group == K) or per-group quant of an [M, K] float32 array."""
    x32 = np.asarray(x32, dtype=F32)
    M, K = x32.shape
    if group <= 0 or K % group:
        raise ValueError("group must divide K")
    G = K // group
    xg = x32.reshape(M, G, group)
    a = np.max(np.abs(xg), axis=2, initial=F32(0.0))
    a = np.maximum(a, AMAX_FLOOR).astype(F32)
    s = (a / Q_MAX).astype(F32)
    if pow2:
        e = ue8m0_exponent(s)
        scale = pow2_f32(e)
        mult = pow2_f32(-e)
        byte = (e + 127).astype(np.uint8)
    else:
        scale = s
        mult = (Q_MAX / a).astype(F32)
        byte = None
    y = (xg * mult[:, :, None]).astype(F32)
    codes = e4m3.encode(_clamp(y)).reshape(M, K)
    return GroupQuant(codes, scale, byte)


def exp_f32(t32):
    """Correctly rounded fp32 e^t (see the module docstring for the pin)."""
    t = np.asarray(t32, dtype=F32).astype(np.float64)
    with np.errstate(over="ignore"):
        return np.exp(t).astype(F32)


def silu_f32(g32):
    g = np.asarray(g32, dtype=F32)
    with np.errstate(over="ignore"):
        d = (F32(1.0) + exp_f32(-g)).astype(F32)
        return (g / d).astype(F32)


def silu_mul_f32(gu32):
    """[M, 2K] float32 rows [gate | up] -> y [M, K] float32."""
    gu32 = np.asarray(gu32, dtype=F32)
    M, K2 = gu32.shape
    if K2 % 2:
        raise ValueError("fused input must have an even number of columns")
    K = K2 // 2
    g = gu32[:, :K]
    u = gu32[:, K:]
    return (silu_f32(g) * u).astype(F32)


def quant_group_silu_mul(gu32, group, pow2=False):
    """Fused SiLU-and-mul followed by group quant of the [M, K] product."""
    return quant_group(silu_mul_f32(gu32), group, pow2)


def quant_static(x32, s):
    """Per-tensor quant with a given positive fp32 scale s."""
    x32 = np.asarray(x32, dtype=F32)
    inv = (F32(1.0) / F32(s)).astype(F32)
    return e4m3.encode(_clamp((x32 * inv).astype(F32)))


def quant_weight_block(w32, block=128):
    """Weight quant per block x block tile of an [N, K] float32 array.

    Returns codes [N, K] and fp32 scales [ceil(N/block), ceil(K/block)];
    partial edge blocks use their own maxima.
    """
    w32 = np.asarray(w32, dtype=F32)
    N, K = w32.shape
    nb = -(-N // block)
    kb = -(-K // block)
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((nb, kb), dtype=F32)
    for i in range(nb):
        for j in range(kb):
            blk = w32[i * block:(i + 1) * block, j * block:(j + 1) * block]
            a = max(F32(np.max(np.abs(blk))), AMAX_FLOOR)
            a = F32(a)
            s = F32(a / Q_MAX)
            m = F32(Q_MAX / a)
            codes[i * block:(i + 1) * block, j * block:(j + 1) * block] = \
                e4m3.encode(_clamp((blk * m).astype(F32)))
            scales[i, j] = s
    return codes, scales

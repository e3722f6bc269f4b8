"""Pins for oracle.fp16: torch's fp32 -> float16 cast (independent code), a
brute-force nearest choice made with exact rational arithmetic, and the
closed-form overflow and subnormal thresholds."""
from fractions import Fraction

import numpy as np
import torch

from oracle import fp16


def test_matches_torch_on_fp32_values():
    rng = np.random.Generator(np.random.PCG64(51))
    x = (rng.standard_normal(300000) * np.exp2(rng.integers(-30, 18, 300000))).astype(np.float32)
    # exact ties: fp16 values plus half an fp16 spacing (in fp32)
    h = rng.integers(0x0400, 0x7BFF, 20000, dtype=np.uint16).view(np.float16).astype(np.float32)
    sp = np.spacing(h.astype(np.float16)).astype(np.float32)
    ties = (h + sp / np.float32(2)).astype(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 65519.0, 65520.0, 1e-8])])
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fp16.to_fp16_bits(x.astype(np.float64)), ref)


def _exact_fp16(v):
    """Nearest fp16 to a float64 by exact search among fp16 magnitudes near |v|
    (zero included), ties to the even bit pattern; the sign is copied."""
    m = abs(v)
    b = int(np.array([np.float16(min(m, 65504.0))]).view(np.uint16)[0])
    cands = {0.0}
    for d in (-2, -1, 0, 1, 2):
        nb = b + d
        if 0 <= nb <= 0x7BFF:
            cands.add(float(np.array([nb], dtype=np.uint16).view(np.float16)[0]))
    fm = Fraction(m)
    best = min(abs(Fraction(c) - fm) for c in cands)
    near = sorted(c for c in cands if abs(Fraction(c) - fm) == best)
    pick = near[0] if len(near) == 1 else [
        c for c in near if int(np.array([c], dtype=np.float16).view(np.uint16)[0]) % 2 == 0][0]
    return -pick if v < 0 else pick


def test_matches_exact_rational_rounding_on_random_doubles():
    rng = np.random.Generator(np.random.PCG64(52))
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-26, 15, 3000))
    ours = fp16.round_to_fp16(x)
    for v, o in zip(x, ours):
        assert _exact_fp16(float(v)) == o


def test_overflow_and_subnormal_closed_forms():
    # 65504 + half a spacing (32) is the overflow tie: 65504 is odd -> rounds up to inf
    x = np.array([65504.0, 65519.999, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, -0.0])
    r = fp16.round_to_fp16(x)
    assert r[0] == 65504.0 and r[1] == 65504.0
    assert np.isinf(r[2]) and r[2] > 0 and np.isinf(r[3]) and r[3] < 0
    assert r[4] == 2.0 ** -24
    assert r[5] == 0.0                      # tie between 0 and 2^-24 -> even (0)
    assert r[6] == 2.0 ** -24               # 0.75 spacing -> up
    assert np.signbit(r[7])

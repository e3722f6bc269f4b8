"""Pins for oracle.bf16: torch's fp32 -> bf16 cast (independent code) and a
brute-force nearest choice made with exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import torch

from oracle import bf16


def test_matches_torch_on_fp32_values():
    rng = np.random.Generator(np.random.PCG64(21))
    bits = rng.integers(0, 0x7F7FFFFF, 300000, dtype=np.uint32)
    x = bits.view(np.float32)
    x = np.where(rng.integers(0, 2, x.size) == 1, -x, x).astype(np.float32)
    # exact ties: bf16 values plus half a bf16 spacing
    base = (rng.integers(0x00800000, 0x7F000000, 20000, dtype=np.uint32) & 0xFFFF0000)
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-45, -1e-45])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16.to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def _exact_bf16(v):
    """Nearest bf16 to a float64 by exact search over the two neighbours."""
    if v == 0:
        return v
    f32 = np.float32(v)  # some float32 near v; bf16 neighbours bracket it
    b = int(np.array([f32], dtype=np.float32).view(np.uint32)[0]) & 0xFFFF0000
    cands = []
    for d in (-0x10000, 0, 0x10000, 0x20000):
        nb = (b + d) & 0xFFFFFFFF
        c = float(np.array([nb], dtype=np.uint32).view(np.float32)[0])
        if np.isfinite(c):
            cands.append(c)
    fv = Fraction(v)
    best = min(abs(Fraction(c) - fv) for c in cands)
    near = sorted({c for c in cands if abs(Fraction(c) - fv) == best})
    if len(near) == 1:
        return near[0]
    even = [c for c in near
            if (int(np.array([c], dtype=np.float32).view(np.uint32)[0]) >> 16) % 2 == 0]
    return even[0]


def test_matches_exact_rational_rounding_on_random_doubles():
    rng = np.random.Generator(np.random.PCG64(22))
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    ours = bf16.round_to_bf16(x)
    for v, o in zip(x, ours):
        assert _exact_bf16(float(v)) == o


def test_subnormal_and_signed_zero():
    tiny = np.array([2.0 ** -133, -(2.0 ** -133), 2.0 ** -134, 3 * 2.0 ** -135, -0.0])
    out = bf16.round_to_bf16(tiny)
    assert out[0] == 2.0 ** -133 and out[1] == -(2.0 ** -133)
    assert out[2] == 0.0                      # tie between 0 and 2^-133 -> even (0)
    assert out[3] == 2.0 ** -133              # 0.75 spacing -> up
    assert np.signbit(out[4])

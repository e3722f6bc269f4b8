"""Pins for oracle.e4m3: decode and encode checked against things other than
themselves (torch's independent float8_e4m3fn conversion, brute force, and the
worked tie example of PR #33533's Motivation)."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import e4m3


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(y32):
    t = torch.from_numpy(np.asarray(y32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    c = np.arange(256, dtype=np.uint8)
    ours = e4m3.decode(c)
    ref = _torch_decode(c)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))
    assert list(np.flatnonzero(np.isnan(ours))) == [0x7F, 0xFF]
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_encode_decode_roundtrip_every_finite_code():
    c = e4m3.finite_codes()
    assert c.size == 254
    assert np.array_equal(e4m3.encode(e4m3.decode(c)), c)


def test_worked_tie_example_golden():
    rows = read_golden("e4m3_tie_example.txt")
    assert len(rows) == 4
    for bits_hex, _dec, code_hex in rows:
        y = np.array([int(bits_hex, 16)], dtype=np.uint32).view(np.float32)
        assert e4m3.encode(y)[0] == int(code_hex, 16), bits_hex


def _brute(y):
    """Nearest finite magnitude by exhaustive search, ties to even code."""
    mags = np.array([e4m3.decode_code(c) for c in range(127)])
    out = []
    for v in np.asarray(y, dtype=np.float64):
        d = np.abs(mags - abs(v))
        best = np.flatnonzero(d == d.min())
        code = best[0] if best.size == 1 else [b for b in best if b % 2 == 0][0]
        out.append(code | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def test_encode_matches_brute_force_on_random_values():
    rng = np.random.Generator(np.random.PCG64(11))
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), 4000)).astype(np.float32)
    mag = np.minimum(mag, np.float32(448))
    sign = rng.integers(0, 2, mag.size) * 2 - 1
    y = (mag * sign).astype(np.float32)
    y = np.concatenate([y, np.float32([0.0, -0.0, 448.0, -448.0, 2 ** -10, 3 * 2 ** -11])])
    assert np.array_equal(e4m3.encode(y), _brute(y))


def test_encode_matches_torch_at_every_midpoint_and_neighbours():
    mags = e4m3.decode(np.arange(127, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    vals = np.concatenate([mids, up, dn, mags.astype(np.float32)])
    vals = vals[np.abs(vals) <= 448]
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(e4m3.encode(vals), _torch_encode(vals))


def test_encode_matches_torch_on_dense_random_fp32():
    rng = np.random.Generator(np.random.PCG64(12))
    bits = rng.integers(0, 0x43E00001, 200000, dtype=np.uint32)  # |y| <= 448
    y = bits.view(np.float32)
    y = np.where(rng.integers(0, 2, y.size) == 1, -y, y).astype(np.float32)
    assert np.array_equal(e4m3.encode(y), _torch_encode(y))


def test_encode_rejects_out_of_range_and_nonfinite():
    with pytest.raises(ValueError):
        e4m3.encode(np.float32([448.01]))
    with pytest.raises(ValueError):
        e4m3.encode(np.float32([np.nan]))

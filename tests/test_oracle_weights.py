"""Pins of the load-time weight preparation oracle (oracle/weights.py)."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import inputs
from oracle import e4m3, weights as ow

F32 = np.float32


def _codes(shape, seed):
    return inputs.random_codes(shape, seed=seed)


def test_partition_at_the_max_scale_keeps_its_codes():
    # dec(q) * s rounds by at most half an fp32 ulp, then * RN32(1/s): the
    # value stays within a few fp32 ulps of dec(q), which is an E4M3 point far
    # from any E4M3 midpoint, so it rounds back to q
    q = _codes((40, 64), 1)
    s = np.array([0.013, 0.0071, 0.013], F32)
    s_max, out = ow.requantize_with_max_scale(q, s, [10, 20, 10])
    assert s_max == F32(0.013)
    assert np.array_equal(out[:10], q[:10]) and np.array_equal(out[30:], q[30:])
    # +-0 keep their sign
    z = np.array([[0x00, 0x80]], np.uint8)
    assert np.array_equal(ow.requantize_with_max_scale(z, [0.5], [1])[1], z)


def test_power_of_two_ratio_gives_the_scaled_codes():
    # s_i = s_max * 2^-j: w = dec(q) * s_i and w / s_max are exact, so
    # q' = E4M3(dec(q) * 2^-j), a pure re-encoding of exact values
    q = _codes((24, 48), 2)
    s_max = F32(0.75)
    for j in (0, 1, 3, 6):
        s = np.array([s_max, s_max * F32(2.0 ** -j)], F32)
        _, out = ow.requantize_with_max_scale(q, s, [12, 12])
        want = e4m3.encode((e4m3.decode(q[12:]) * 2.0 ** -j).astype(F32))
        assert np.array_equal(out[12:], want), j


def test_matches_torch_casts_on_random_scales():
    q = _codes((60, 96), 3)
    r = np.random.default_rng(4)
    widths = [25, 5, 30]
    s = r.uniform(1e-3, 5e-2, 3).astype(F32)
    s_max, out = ow.requantize_with_max_scale(q, s, widths)
    t = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    off = np.cumsum([0] + widths)
    inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(float(s_max), dtype=torch.float32)
    for i in range(3):
        w = t[off[i]:off[i + 1]] * torch.tensor(float(s[i]), dtype=torch.float32)
        ref = (w * inv).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(out[off[i]:off[i + 1]], ref), i
    assert s_max == F32(s.max())


def test_widths_are_checked():
    q = _codes((8, 16), 5)
    with pytest.raises(ValueError):
        ow.requantize_with_max_scale(q, [1.0, 1.0], [4, 3])
    with pytest.raises(ValueError):
        ow.requantize_with_max_scale(q, [1.0], [4, 4])


def test_channelwise_closed_form():
    got = ow.convert_to_channelwise([0.5, 0.25, 2.0], [2, 0, 3])
    assert got.dtype == F32 and list(got) == [0.5, 0.5, 2.0, 2.0, 2.0]
    assert list(ow.convert_to_channelwise([0.125], [1, 2])) == [0.125] * 3

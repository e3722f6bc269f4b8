"""The seeded generators are deterministic and follow their recipes."""
import numpy as np
import torch

from column_scaled_gemm_amd import inputs


def test_rowwise_is_deterministic_and_has_outlier_channels():
    a = inputs.rowwise(64, 32, 1000, seed=3)
    b = inputs.rowwise(64, 32, 1000, seed=3)
    assert torch.equal(a.x, b.x) and torch.equal(a.w, b.w)
    assert a.outlier_channels.size == 10
    x = a.x.float().abs()
    ch = a.outlier_channels
    rest = np.setdiff1d(np.arange(1000), ch)
    assert x[:, ch].mean() > 10 * x[:, rest].mean()
    assert abs(float(a.w.float().std()) - 0.02) < 0.002


def test_fused_recipe():
    f = inputs.fused(M=1024, K=512, N=128, seed=0)
    assert f.gu_bf16.shape == (1024, 1024) and f.gu_fp16.dtype == torch.float16
    assert torch.all(f.gu_bf16[7] == 0) and torch.all(f.gu_bf16[519] == 0)
    up = f.gu_bf16[:, 512:].float().reshape(1024, 4, 128).abs().amax(dim=2).numpy()
    live = ~f.zero_rows[:, None]
    assert np.all(up[f.tiny_groups & live] < 1e-3)
    assert np.all(up[~f.tiny_groups & live] > 1e-2)
    assert 0.03 < f.tiny_groups.mean() < 0.07


def test_random_codes_never_nan():
    c = inputs.random_codes((512, 512), seed=5)
    assert not np.isin(c, [0x7F, 0xFF]).any()
    assert np.unique(c).size == 254

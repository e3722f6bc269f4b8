"""GPU parity of the load-time weight preparation (requantization of a fused
weight to its largest partition scale, per-channel scale broadcast) against
the oracle: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import gemm as og, weights as ow
from gpu_util import assert_within_tolerance, bf16_bits, cuda, to_gpu_f32, to_gpu_u8

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.mark.parametrize("widths,K", [([96, 32, 48], 208), ([1], 16), ([0, 7, 0, 9], 64),
                                      ([4096, 512, 512], 5376)])
@pytest.mark.parametrize("in_place", [False, True])
def test_requantize_max_scale(widths, K, in_place):
    N = sum(widths)
    print(f"[case] requantize widths={widths} K={K} in_place={in_place}", flush=True)
    w = inputs.random_codes((N, K), seed=N + K)
    r = inputs.rng(K)
    s = r.uniform(1e-3, 4e-2, len(widths)).astype(F32)
    s[len(widths) // 2] = s.max() * F32(2.0)           # a clear maximum in the middle
    s_max, want = ow.requantize_with_max_scale(w, s, widths)
    wd = to_gpu_u8(w)
    m, q = fp8sm.requantize_max_scale(wd, to_gpu_f32(s), widths, q=wd if in_place else None)
    torch.cuda.synchronize()
    assert m.item() == float(s_max)
    assert np.array_equal(q.cpu().numpy(), want)
    if in_place:
        assert q.data_ptr() == wd.data_ptr()


def test_channelwise_and_gemm_with_requantized_weight():
    # the requantized weight with its broadcast scale in the rowwise GEMM
    widths = [64, 16, 48]
    N, K, M = sum(widths), 256, 24
    w = inputs.random_codes((N, K), seed=8) & 0x77     # finite, |v| <= 240
    s = np.array([0.01, 0.03, 0.02], F32)
    s_max, wq = ow.requantize_with_max_scale(w, s, widths)
    m, q = fp8sm.requantize_max_scale(to_gpu_u8(w), to_gpu_f32(s), widths)
    per_ch = fp8sm.scales_to_channelwise(m, [N])
    per_part = fp8sm.scales_to_channelwise(to_gpu_f32(s), widths)
    torch.cuda.synchronize()
    assert np.array_equal(per_ch.cpu().numpy(), ow.convert_to_channelwise([s_max], [N]))
    assert np.array_equal(per_part.cpu().numpy(), ow.convert_to_channelwise(s, widths))
    a = inputs.random_codes((M, K), seed=9) & 0x77
    sa = np.full(M, 0.5, F32)
    c = fp8sm.scaled_mm(to_gpu_u8(a), q, to_gpu_f32(sa), per_ch, fp8sm.KIND_ROW, fp8sm.KIND_COL)
    torch.cuda.synchronize()
    assert_within_tolerance(bf16_bits(c), og.scaled_mm(a, wq, sa, ow.convert_to_channelwise([s_max], [N])),
                            K, "requantized weight GEMM")

"""The matrix-pipe ceiling probe (fp8sm_rate_probe) behind bench.py --ceilings.

The probe reads no memory and its sink values depend only on the arithmetic,
so these tests check that it runs, fills every lane's value (finite without
the widen; with it the operands are arbitrary bit patterns), is deterministic,
and report the rate it reaches (no timing is asserted: a throttled box must not
fail the suite).
"""
import pytest
import torch

from column_scaled_gemm_amd import fp8sm
from gpu_util import progress

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("widen", [0, 1])
@pytest.mark.parametrize("wpb", [4, 8, 16])
def test_rate_probe_runs_and_is_deterministic(widen, wpb):
    progress(f"[case] rate probe widen={widen} waves_per_block={wpb}")
    a = fp8sm.rate_probe(widen, 8, wpb, 64)
    b = fp8sm.rate_probe(widen, 8, wpb, 64)
    torch.cuda.synchronize()
    assert a.numel() == 8 * 64 * wpb
    if not widen:  # widened operands are arbitrary bit patterns, NaN included
        assert torch.isfinite(a).all()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_rate_probe_full_grid_rate_is_reported():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4000
    fp8sm.rate_probe(0, cus, 8, iters)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    fp8sm.rate_probe(0, cus, 8, iters)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3
    tflops = 2.0 * 32 * 32 * 16 * 4 * iters * cus * 8 / us / 1e6
    progress(f"[rate] matrix pipe, 2 waves/SIMD: {tflops:.0f} TFLOP/s over {cus} CUs")
    assert tflops > 0

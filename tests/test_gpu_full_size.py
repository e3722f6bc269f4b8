"""Every output of the H3 rowwise workloads against the oracle.

The attention QKV projection (8320 x 5376 x 21504) and the three MLP
projections (gate/up 23216 and 15760 x 5376 x 28672, down 8320 x 14336 x 5376)
are the shapes of the pages' kernel benchmark ("Route large SM90
row/column-scaled FP8 GEMMs to Torch", Kernel results).  Each is run once at
full size through the library the way the bench runs it (per-token quant of
the bf16 activations and per-channel quant of the weights on the GPU, then the
rowwise GEMM picked by the shape dispatch), and checked completely: all codes
and scales bit-exact, all M x N outputs within |gpu - oracle| <= 2^-7 |oracle|
+ 1e-3 sa sb sqrt(K).  The oracle runs on row slabs of A (its rows are
independent by definition).
"""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import quant as oq
from gpu_util import bf16_bits, cuda, full_tolerance_report, progress

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
ROW, COL = fp8sm.KIND_ROW, fp8sm.KIND_COL


def _gpu_step(name):
    M, N, K = inputs.ROWWISE_SHAPES[name]
    w = inputs.workload(name)
    qa, sa = fp8sm.quant_group(w.x.to(cuda()), -1)
    qb, sb = fp8sm.quant_group(w.w.to(cuda()), -1)
    c = fp8sm.scaled_mm(qa, qb, sa.reshape(-1), sb.reshape(-1), ROW, COL)
    torch.cuda.synchronize()
    out = (w, qa.cpu().numpy(), sa.cpu().numpy(), qb.cpu().numpy(), sb.cpu().numpy(), bf16_bits(c))
    del qa, sa, qb, sb, c
    torch.cuda.empty_cache()
    return out


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["qkv", "mlp_down", "mlp_gateup_15760", "mlp_gateup_23216"])
def test_every_output_of_the_h3_workloads(name):
    M, N, K = inputs.ROWWISE_SHAPES[name]
    progress(f"[case] full-size {name} M={M} N={N} K={K} variant="
             f"{fp8sm.variant_name(fp8sm.pick_variant(M, N, K))}")
    w, ga, gsa, gb, gsb, bits = _gpu_step(name)
    oa = oq.quant_group(inputs.widen(w.x), K)
    assert np.array_equal(ga, oa.codes), f"{name}: activation codes differ"
    assert np.array_equal(gsa.view(np.uint32), oa.scale.view(np.uint32)), f"{name}: scales differ"
    del oa
    ob = oq.quant_group(inputs.widen(w.w), K)
    assert np.array_equal(gb, ob.codes), f"{name}: weight codes differ"
    assert np.array_equal(gsb.view(np.uint32), ob.scale.view(np.uint32))
    del w, ob
    progress(f"{name}: codes and scales bit-exact; comparing all {M * N} outputs")
    n, v, mx, at = full_tolerance_report(bits, ga, gb, gsa, gsb, K, name)
    progress(f"[tol] {name} full output: outputs={n} violations={v} max_err/tol={mx:.4f} at {at}")
    assert n == M * N
    assert v == 0, f"{name}: {v} outputs outside the bound (max err/tol {mx:.3f} at {at})"

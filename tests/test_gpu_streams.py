"""Concurrent use on two streams: the library keeps no state between calls
(no scratch memory, nothing cached on the device) and launches on the
caller's stream, so independent quant + GEMM steps enqueued on two streams at
once, interleaved and repeated, must give bitwise what the same calls give one
after another on one stream, and the oracle (codes bit-exact, GEMM within the
bound).  The row counts put decode and tile variants on the GPU together."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import gemm as og, quant as oq
from gpu_util import assert_within_tolerance, bf16_bits, cuda

pytestmark = pytest.mark.gpu
F32 = np.float32
ROW, COL = fp8sm.KIND_ROW, fp8sm.KIND_COL


def test_two_streams_equal_sequential_calls():
    N, K = 768, 1536
    Ms = (300, 17, 1, 129, 64, 5)
    print(f"[case] two streams N={N} K={K} M={Ms}", flush=True)
    d = cuda()
    r = inputs.rng(11)
    w = inputs.to_dtype(r.standard_normal((N, K), dtype=np.float32) * F32(0.02))
    xs = [inputs.to_dtype(r.standard_normal((M, K), dtype=np.float32)) for M in Ms]
    gs = [inputs.to_dtype(r.standard_normal((M, 2 * K), dtype=np.float32)) for M in Ms]
    qb, sb = fp8sm.quant_group(w.to(d), -1)
    sb = sb.reshape(-1)
    xd = [x.to(d) for x in xs]
    gd = [g.to(d) for g in gs]
    G = K // 128

    def outputs(M):
        return (torch.empty((M, K), dtype=torch.uint8, device=d),
                torch.empty((M, 1), dtype=torch.float32, device=d),
                torch.empty((M, N), dtype=torch.bfloat16, device=d),
                torch.empty((M, K), dtype=torch.uint8, device=d),
                torch.empty((M, G), dtype=torch.uint8, device=d))

    def step(i, out, stream=None):
        qa, sa, c, qf, sf = out
        fp8sm.quant_group(xd[i], -1, q=qa, scales=sa, stream=stream)
        fp8sm.scaled_mm(qa, qb, sa.reshape(-1), sb, ROW, COL, c=c, stream=stream)
        fp8sm.quant_group(gd[i], 128, fp8sm.SCALE_UE8M0_BYTE, fuse_silu_mul=True, q=qf,
                          scales=sf, stream=stream)

    ref = [outputs(M) for M in Ms]
    for i in range(len(Ms)):
        step(i, ref[i])
    got = [outputs(M) for M in Ms]
    for t in got:
        for u in t:
            u.zero_()
    torch.cuda.synchronize()
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    for _ in range(3):  # each job stays on its stream: repeats only overwrite in order
        for i in range(len(Ms)):
            s = streams[i % 2]
            with torch.cuda.stream(s):
                step(i, got[i], stream=s)
    torch.cuda.synchronize()
    for i, M in enumerate(Ms):
        for a, b in zip(ref[i], got[i]):
            if a.dtype == torch.bfloat16:
                assert np.array_equal(bf16_bits(a), bf16_bits(b)), f"M={M}"
            else:
                assert torch.equal(a, b), f"M={M}"
    # the sequential results against the oracle
    ob = oq.quant_group(inputs.widen(w), K)
    for i, M in enumerate(Ms):
        oa = oq.quant_group(inputs.widen(xs[i]), K)
        assert np.array_equal(ref[i][0].cpu().numpy(), oa.codes)
        res = og.scaled_mm(oa.codes, ob.codes, oa.scale.reshape(-1), ob.scale.reshape(-1))
        assert_within_tolerance(bf16_bits(ref[i][2]), res, K, f"two streams M={M}")
        of = oq.quant_group_silu_mul(inputs.widen(gs[i]), 128, pow2=True)
        assert np.array_equal(ref[i][3].cpu().numpy(), of.codes)
        assert np.array_equal(ref[i][4].cpu().numpy(), of.ue8m0_byte)

"""GPU parity of the scattered 1x128 group quant against the oracle: codes and
scales bit-exact at every destination row, untouched rows keep a sentinel,
out-of-range destinations are skipped."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import scatter as osc
from gpu_util import cuda

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("layout", [fp8sm.LAYOUT_MN_MAJOR, fp8sm.LAYOUT_ROW_MAJOR])
@pytest.mark.parametrize("fmt", [fp8sm.SCALE_UE8M0_BYTE, fp8sm.SCALE_FP32])
@pytest.mark.parametrize("T,K,topk", [(37, 512, 8), (1, 128, 1), (130, 7168, 4)])
def test_scatter_quant(dtype, layout, fmt, T, K, topk):
    print(f"[case] scatter T={T} K={K} topk={topk} {dtype} layout={layout} fmt={fmt}", flush=True)
    r = inputs.rng(T + K + topk)
    x = r.standard_normal((T, K), dtype=np.float32)
    x[0, :128] = 0.0                                      # a zero group
    xt = inputs.to_dtype(x, dtype)
    R = T * topk + 9                                      # some rows nobody names
    dst = r.permutation(R)[:T * topk].reshape(T, topk).astype(np.int32)
    dst[0, 0] = -1                                        # names no row
    if topk > 1:
        dst[-1, -1] = R + 3                               # past the end: skipped
    G = K // 128
    q = torch.full((R, K), 0x5A, dtype=torch.uint8, device=cuda())
    sdt = torch.uint8 if fmt == fp8sm.SCALE_UE8M0_BYTE else torch.float32
    s = torch.full(fp8sm.scale_shape(fmt, layout, R, K, 128), 7, dtype=sdt, device=cuda())
    fp8sm.quant_group_scatter(xt.to(cuda()), torch.from_numpy(dst).to(cuda()), R, fmt=fmt,
                              layout=layout, q=q, scales=s)
    torch.cuda.synchronize()
    codes, scale, byte, written = osc.quant_group_scatter(inputs.widen(xt), dst, R,
                                                          pow2=fmt == fp8sm.SCALE_UE8M0_BYTE)
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    got_s = sh[:, :R].T if layout == fp8sm.LAYOUT_MN_MAJOR else sh
    want_s = byte if fmt == fp8sm.SCALE_UE8M0_BYTE else scale
    assert np.array_equal(qh[written], codes[written])
    assert np.array_equal(got_s[written], want_s[written])
    assert np.all(qh[~written] == 0x5A) and np.all(got_s[~written] == 7)

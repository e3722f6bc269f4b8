"""Empty and degenerate inputs through the binding: every call with a zero-size
dimension (rows, columns, batches, tokens) returns without error and leaves
pre-filled outputs untouched; a GEMM with K = 0 from zero-width operands
writes the bias row (zeros without a bias); a masked call whose every count
is zero writes nothing."""
import pytest
import torch

from column_scaled_gemm_amd import fp8sm
from gpu_util import cuda

pytestmark = pytest.mark.gpu
U8, BF16, F16 = torch.uint8, torch.bfloat16, torch.float16
ROW, COL = fp8sm.KIND_ROW, fp8sm.KIND_COL
SENT_U8 = 0x5A


def _ones(n):
    return torch.ones(n, dtype=torch.float32, device=cuda())


@pytest.mark.parametrize("M,N", [(0, 256), (64, 0), (0, 0)])
def test_gemm_empty_rows_or_columns(M, N):
    print(f"[case] empty gemm M={M} N={N}", flush=True)
    d = cuda()
    a = torch.zeros((M, 512), dtype=U8, device=d)
    b = torch.zeros((N, 512), dtype=U8, device=d)
    c = fp8sm.scaled_mm(a, b, _ones(M), _ones(N), ROW, COL)
    assert c.shape == (M, N)
    bias = torch.zeros(N, dtype=F16, device=d)
    c = fp8sm.scaled_mm(a, b, _ones(M), _ones(N), ROW, COL, bias=bias, out_dtype=F16)
    assert c.shape == (M, N)
    B = 3
    c = fp8sm.scaled_mm_batched(torch.zeros((B, M, 512), dtype=U8, device=d), b, _ones(M),
                                _ones(N), ROW, COL)
    assert c.shape == (B, M, N)
    torch.cuda.synchronize()


def test_gemm_zero_width_operands_write_the_bias():
    print("[case] gemm K=0 from zero-width operands", flush=True)
    d = cuda()
    M, N = 5, 16
    a = torch.empty((M, 0), dtype=U8, device=d)
    b = torch.empty((N, 0), dtype=U8, device=d)
    c = torch.full((M, N), 7.0, dtype=BF16, device=d)
    fp8sm.scaled_mm(a, b, _ones(M), _ones(N), ROW, COL, c=c)
    bias = torch.arange(N, dtype=BF16, device=d)
    cb = fp8sm.scaled_mm(a, b, _ones(M), _ones(N), ROW, COL, bias=bias)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
    assert torch.equal(cb, bias.expand(M, N))


def test_gemm_no_batches():
    print("[case] gemm nbatch=0", flush=True)
    d = cuda()
    a = torch.zeros((0, 64, 512), dtype=U8, device=d)
    b = torch.zeros((256, 512), dtype=U8, device=d)
    c = fp8sm.scaled_mm_batched(a, b, _ones(64), _ones(256), ROW, COL)
    torch.cuda.synchronize()
    assert c.shape == (0, 64, 256)


def test_quant_empty_rows_batches_and_tokens():
    print("[case] empty quant", flush=True)
    d = cuda()
    x = torch.zeros((0, 512), dtype=BF16, device=d)
    for group, fmt, layout, fused in [(128, fp8sm.SCALE_FP32, fp8sm.LAYOUT_ROW_MAJOR, False),
                                      (-1, fp8sm.SCALE_FP32, fp8sm.LAYOUT_ROW_MAJOR, False),
                                      (128, fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_MN_MAJOR, True)]:
        q, s = fp8sm.quant_group(x, group, fmt, layout, fuse_silu_mul=fused)
        assert q.shape[0] == 0 and s.numel() == 0
    assert fp8sm.quant_static(x, _ones(1)).shape == (0, 512)
    assert fp8sm.silu_mul_f32(x).shape == (0, 256)
    q, s = fp8sm.quant_weight_block128(x)
    assert q.shape == (0, 512) and s.shape == (0, 4)
    for shape in [(0, 8, 512), (3, 0, 512)]:
        q, s = fp8sm.quant_group_batched(torch.zeros(shape, dtype=BF16, device=d), 128)
        assert q.shape == shape
    # scattered quant of no tokens leaves every destination row as it was
    R = 16
    q = torch.full((R, 512), SENT_U8, dtype=U8, device=d)
    sc = torch.full(fp8sm.scale_shape(fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_MN_MAJOR, R, 512, 128),
                    SENT_U8, dtype=U8, device=d)
    dst = torch.zeros((0, 4), dtype=torch.int32, device=d)
    fp8sm.quant_group_scatter(x, dst, R, q=q, scales=sc)
    torch.cuda.synchronize()
    assert torch.all(q == SENT_U8) and torch.all(sc == SENT_U8)


def test_masked_calls_with_every_count_zero_write_nothing():
    print("[case] masked, all counts zero", flush=True)
    d = cuda()
    B, M, K, N = 4, 96, 512, 256
    g = torch.Generator(device="cpu").manual_seed(3)
    x = torch.randn((B, M, 2 * K), generator=g).to(BF16).to(d)
    rows = torch.zeros(B, dtype=torch.int32, device=d)
    q = torch.full((B, M, K), SENT_U8, dtype=U8, device=d)
    s = torch.full((B,) + fp8sm.scale_shape(fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_MN_MAJOR, M, K,
                                            128), SENT_U8, dtype=U8, device=d)
    fp8sm.quant_group_batched(x, 128, fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_MN_MAJOR,
                              fuse_silu_mul=True, rows=rows, q=q, scales=s)
    a = torch.zeros((B, M, K), dtype=U8, device=d)
    w = torch.zeros((N, K), dtype=U8, device=d)
    c = torch.full((B, M, N), 3.0, dtype=BF16, device=d)
    fp8sm.scaled_mm_batched(a, w, _ones(M), _ones(N), ROW, COL, rows=rows, c=c)
    torch.cuda.synchronize()
    assert torch.all(q == SENT_U8) and torch.all(s == SENT_U8)
    assert torch.all(c == 3.0)

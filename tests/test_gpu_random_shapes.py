"""Seeded random shapes through the rowwise GEMM and the quant kernels: every
variant that accepts a shape against the oracle (accuracy bound) and against
the other variants (bitwise), and per-token / 1x128 quant against the oracle
(bit-exact).  Shapes are drawn across tile edges, K tails and decode sizes,
small enough for the oracle to finish in seconds."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import gemm as og, quant as oq
from gpu_util import assert_within_tolerance, bf16_bits, cuda, to_gpu_f32, to_gpu_u8

pytestmark = pytest.mark.gpu
F32 = np.float32


def _shapes(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(r.choice([1, 2, 3, 5, 17, 31, 33, 63, 65, 100, 127, 129, 200, 257, 300]))
        N = int(8 * r.integers(1, 70))             # multiples of 8 (bf16 rows of 16 bytes)
        K = int(16 * r.integers(1, 130))           # multiples of 16, tails of every size
        out.append((M, N, K))
    return out


def _quantized(M, N, K, seed):
    r = inputs.rng(seed)
    x = r.standard_normal((M, K), dtype=np.float32) * np.exp2(r.uniform(-6, 6, (M, 1))).astype(F32)
    w = r.standard_normal((N, K), dtype=np.float32) * F32(0.05)
    qa = oq.quant_group(inputs.widen(inputs.to_dtype(x)), K)
    qb = oq.quant_group(inputs.widen(inputs.to_dtype(w)), K)
    return qa.codes, qa.scale.reshape(-1), qb.codes, qb.scale.reshape(-1)


@pytest.mark.parametrize("idx,shape", list(enumerate(_shapes(24, 2024))))
def test_rowwise_random_shape_all_variants(idx, shape):
    M, N, K = shape
    print(f"[case] random shape {idx}: M={M} N={N} K={K}", flush=True)
    A, sa, B, sb = _quantized(M, N, K, 100 + idx)
    want = og.scaled_mm(A, B, sa, sb)
    first = None
    for v in range(fp8sm.variant_count()):
        if not fp8sm.variant_accepts(v, M, N, K):
            continue
        prev = fp8sm.force_variant(v)
        try:
            c = fp8sm.scaled_mm(to_gpu_u8(A), to_gpu_u8(B), to_gpu_f32(sa), to_gpu_f32(sb),
                                fp8sm.KIND_ROW, fp8sm.KIND_COL)
            torch.cuda.synchronize()
        finally:
            fp8sm.force_variant(prev)
        got = bf16_bits(c)
        assert_within_tolerance(got, want, K, f"{shape} {fp8sm.variant_name(v)}")
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), f"{shape}: {fp8sm.variant_name(v)} differs bitwise"


@pytest.mark.parametrize("idx", range(8))
def test_quant_random_shapes(idx):
    r = np.random.default_rng(500 + idx)
    M = int(r.integers(1, 400))
    K = int(128 * r.integers(1, 60))
    dtype = torch.bfloat16 if idx % 2 == 0 else torch.float16
    print(f"[case] random quant {idx}: M={M} K={K} {dtype}", flush=True)
    x = r.standard_normal((M, K)).astype(F32) * np.exp2(r.uniform(-12, 8, (M, 1))).astype(F32)
    xt = inputs.to_dtype(x, dtype)
    x32 = inputs.widen(xt)
    for group, fmt in ((-1, fp8sm.SCALE_FP32), (128, fp8sm.SCALE_UE8M0_BYTE), (128, fp8sm.SCALE_FP32)):
        q, s = fp8sm.quant_group(xt.to(cuda()), group, fmt)
        torch.cuda.synchronize()
        g = K if group == -1 else group
        ref = oq.quant_group(x32, g, fmt != fp8sm.SCALE_FP32)
        assert np.array_equal(q.cpu().numpy(), ref.codes), (group, fmt)
        sw = s.cpu().numpy().reshape(M, -1)
        if fmt == fp8sm.SCALE_UE8M0_BYTE:
            assert np.array_equal(sw, ref.ue8m0_byte.reshape(M, -1)), (group, fmt)
        else:
            assert np.array_equal(sw.view(np.uint32), ref.scale.reshape(M, -1).astype(F32).view(np.uint32)), (group, fmt)

"""GPU parity of the scaled GEMMs against the oracle: bit-exact where the
result is exactly representable, the accuracy bound 2^-7|ref| + 1e-3 sa sb sqrt(K) elsewhere, and bitwise
row invariance across M and across kernel variants."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import e4m3, gemm as og, quant as oq
from gpu_util import (assert_within_tolerance, bf16_bits, cuda, to_gpu_f32, to_gpu_u8)

pytestmark = pytest.mark.gpu
F32 = np.float32
T, ROW, COL = fp8sm.KIND_TENSOR, fp8sm.KIND_ROW, fp8sm.KIND_COL


def _mm(a, b, sa, sb, ka=ROW, kb=COL):
    c = fp8sm.scaled_mm(to_gpu_u8(a), to_gpu_u8(b), to_gpu_f32(sa), to_gpu_f32(sb), ka, kb)
    torch.cuda.synchronize()
    return bf16_bits(c)


def _variants_for(M, K):
    """Every rowwise kernel variant that computes an M-row call with this K."""
    return [v for v in range(fp8sm.variant_count()) if fp8sm.variant_accepts(v, M, 0, K)]


def _mm_variant(v, *args, **kw):
    prev = fp8sm.force_variant(v)
    try:
        return _mm(*args, **kw)
    finally:
        fp8sm.force_variant(prev)


def test_one_hot_products_of_all_finite_codes_are_exact():
    c = e4m3.finite_codes()
    n = 256
    for kpos, K in [(5, 16), (37, 384), (127, 384), (128, 384), (300, 384)]:
        A = np.zeros((254, K), np.uint8)
        B = np.zeros((n, K), np.uint8)
        A[:, kpos] = c
        B[:254, kpos] = c
        for v in _variants_for(254, K):
            got = _mm_variant(v, A, B, F32(1), F32(1), T, T)
            want = og.scaled_mm(A, B, 1.0, 1.0).bits
            assert np.array_equal(got, want), (kpos, fp8sm.variant_name(v))


def test_small_integer_sums_are_exact():
    # codes of the integers -16..16: every partial sum is an integer below
    # 2^24, so fp32 accumulation is exact and the bf16 rounding is the oracle's
    vals = np.arange(-16, 17, dtype=F32)
    codes = e4m3.encode(vals)
    r = inputs.rng(11)
    A = codes[r.integers(0, 33, (70, 1024))]
    B = codes[r.integers(0, 33, (136, 1024))]
    want = og.scaled_mm(A, B, 1.0, 1.0).bits
    for v in _variants_for(70, 1024):
        assert np.array_equal(_mm_variant(v, A, B, np.ones(70, F32), np.ones(136, F32)), want), v


def test_zero_rows_give_positive_zero():
    A = inputs.random_codes((40, 512), seed=12)
    B = inputs.random_codes((64, 512), seed=13)
    A[3] = 0
    A[17] = 0x80
    got = _mm(A, B, np.ones(40, F32), np.ones(64, F32))
    assert np.all(got[3] == 0) and np.all(got[17] == 0)


def _quantized_case(M, N, K, seed, outliers=True):
    w = inputs.rowwise(M, N, K, seed=seed, outliers=outliers)
    qa = oq.quant_group(inputs.widen(w.x), K)
    qb = oq.quant_group(inputs.widen(w.w), K)
    return qa.codes, qb.codes, qa.scale.reshape(-1), qb.scale.reshape(-1)


@pytest.mark.parametrize("shape", [(1, 8, 16), (37, 264, 80), (100, 136, 208), (130, 520, 1040),
                                   (64, 256, 512), (257, 128, 4096), (33, 1000, 2064),
                                   # K % 64 = 48 / 32 / 48, and K around the decode
                                   # kernels' prefetch depths (24 chunks for M <= 32,
                                   # 8 for M <= 64): below, exactly at, just past
                                   (5, 24, 48), (16, 40, 96), (3, 64, 176), (16, 48, 1472),
                                   (16, 48, 1536), (16, 48, 1552), (64, 72, 1552)])
def test_ragged_shapes_every_variant_bitwise_equal_and_within_bound(shape):
    M, N, K = shape
    print(f"[case] ragged M={M} N={N} K={K}", flush=True)
    A, B, sa, sb = _quantized_case(M, N, K, seed=M + N + K)
    res = og.scaled_mm(A, B, sa, sb)
    outs = {}
    for v in _variants_for(M, K):
        outs[v] = _mm_variant(v, A, B, sa, sb)
        assert_within_tolerance(outs[v], res, K, f"{shape} {fp8sm.variant_name(v)}")
    first = next(iter(outs.values()))
    for v, o in outs.items():
        assert np.array_equal(o, first), f"variant {fp8sm.variant_name(v)} differs bitwise"


def test_padded_leading_dimensions():
    # A, B and C as views into wider buffers: results equal the compact call
    # bitwise in every variant, and C's padding columns are left untouched
    M, N, K = 40, 72, 336
    A, B, sa, sb = _quantized_case(M, N, K, seed=91)
    Ab = torch.zeros((M, K + 32), dtype=torch.uint8)
    Bb = torch.zeros((N, K + 48), dtype=torch.uint8)
    Ab[:, :K] = torch.from_numpy(A)
    Bb[:, :K] = torch.from_numpy(B)
    Ag, Bg = Ab.to(cuda())[:, :K], Bb.to(cuda())[:, :K]
    sag, sbg = to_gpu_f32(sa), to_gpu_f32(sb)
    for v in _variants_for(M, K):
        prev = fp8sm.force_variant(v)
        try:
            Cb = torch.full((M, N + 8), 3.0, dtype=torch.bfloat16, device=cuda())
            fp8sm.scaled_mm(Ag, Bg, sag, sbg, fp8sm.KIND_ROW, fp8sm.KIND_COL, c=Cb[:, :N])
            ref = fp8sm.scaled_mm(to_gpu_u8(A), to_gpu_u8(B), sag, sbg, fp8sm.KIND_ROW,
                                  fp8sm.KIND_COL)
            torch.cuda.synchronize()
        finally:
            fp8sm.force_variant(prev)
        assert np.array_equal(bf16_bits(Cb[:, :N].contiguous()), bf16_bits(ref)), fp8sm.variant_name(v)
        assert torch.all(Cb[:, N:] == 3.0), fp8sm.variant_name(v)


@pytest.mark.parametrize("M", [9, 70])
def test_largest_row_strides_every_variant(M):
    # lda = ldb = 2^24 bytes, the largest the call accepts: 32-bit operand
    # offsets over a whole panel stay in range; K = 80 runs one whole chunk
    # (buffer copies) and a 16-byte tail (guarded copies)
    N, K, ld = 72, 80, 1 << 24
    A, B, sa, sb = _quantized_case(M, N, K, seed=97)
    Af = torch.zeros((M - 1) * ld + K, dtype=torch.uint8, device=cuda())
    Bf = torch.zeros((N - 1) * ld + K, dtype=torch.uint8, device=cuda())
    Ag = torch.as_strided(Af, (M, K), (ld, 1))
    Bg = torch.as_strided(Bf, (N, K), (ld, 1))
    Ag.copy_(torch.from_numpy(A).to(cuda()))
    Bg.copy_(torch.from_numpy(B).to(cuda()))
    sag, sbg = to_gpu_f32(sa), to_gpu_f32(sb)
    res = og.scaled_mm(A, B, sa, sb)
    first = None
    for v in _variants_for(M, K):
        prev = fp8sm.force_variant(v)
        try:
            c = fp8sm.scaled_mm(Ag, Bg, sag, sbg, ROW, COL)
            torch.cuda.synchronize()
        finally:
            fp8sm.force_variant(prev)
        bits = bf16_bits(c)
        assert_within_tolerance(bits, res, K, f"ld 2^24 {fp8sm.variant_name(v)} M={M}")
        if first is None:
            first = bits
        assert np.array_equal(bits, first), fp8sm.variant_name(v)


@pytest.mark.parametrize("shape", [(37, 264, 80), (100, 136, 208), (16, 48, 1552),
                                   (257, 128, 4096)])
@pytest.mark.parametrize("out,with_bias", [("fp16", False), ("bf16", True), ("fp16", True)])
def test_bias_and_fp16_epilogues_every_variant(shape, out, with_bias):
    # the epilogue of fp8sm_scaled_mm_ex against the oracle, bitwise equal
    # across every variant the shape admits (decode and tiles); the plain bf16
    # epilogue is the ragged-shape test above
    M, N, K = shape
    print(f"[case] epilogue M={M} N={N} K={K} out={out} bias={with_bias}", flush=True)
    A, B, sa, sb = _quantized_case(M, N, K, seed=M + 2 * N + K)
    tdt = torch.float16 if out == "fp16" else torch.bfloat16
    bias_t = None
    bias_v = None
    if with_bias:
        r = inputs.rng(M + N)
        bias_t = torch.from_numpy(r.standard_normal(N).astype(F32) * F32(0.5)).to(tdt)
        bias_v = bias_t.float().numpy().astype(np.float64)
        bias_t = bias_t.to(cuda())
    res = og.scaled_mm(A, B, sa, sb, bias=bias_v, out=out)
    outs = {}
    for v in _variants_for(M, K):
        prev = fp8sm.force_variant(v)
        try:
            c = fp8sm.scaled_mm(to_gpu_u8(A), to_gpu_u8(B), to_gpu_f32(sa), to_gpu_f32(sb),
                                fp8sm.KIND_ROW, fp8sm.KIND_COL, bias=bias_t, out_dtype=tdt)
            torch.cuda.synchronize()
        finally:
            fp8sm.force_variant(prev)
        outs[v] = bf16_bits(c)
        assert_within_tolerance(outs[v], res, K, f"{shape} {out} bias={with_bias} "
                                                 f"{fp8sm.variant_name(v)}")
    first = next(iter(outs.values()))
    for v, o in outs.items():
        assert np.array_equal(o, first), f"variant {fp8sm.variant_name(v)} differs bitwise"


def test_fp16_output_overflow_and_k0_bias():
    # outputs past 65504 are +-inf in fp16, as in the oracle; K == 0 writes the
    # bias row (C = rnd(0 + bias))
    big = e4m3.encode(np.float32([448.0]))[0]
    M, N, K = 5, 16, 64
    A = np.full((M, K), big, np.uint8)
    A[1] |= 0x80
    B = np.full((N, K), big, np.uint8)
    sb = np.full(N, 1.0, F32)
    sb[8:] = 2.0 ** -10                                  # 64 * 448^2 / 1024 = 12544: finite
    for v in _variants_for(M, K):
        prev = fp8sm.force_variant(v)
        try:
            c = fp8sm.scaled_mm(to_gpu_u8(A), to_gpu_u8(B), to_gpu_f32(np.ones(M, F32)),
                                to_gpu_f32(sb), fp8sm.KIND_ROW, fp8sm.KIND_COL,
                                out_dtype=torch.float16)
            torch.cuda.synchronize()
        finally:
            fp8sm.force_variant(prev)
        got = c.float().cpu().numpy()
        assert np.all(np.isposinf(got[0, :8])) and np.all(np.isneginf(got[1, :8]))
        assert np.all(got[0, 8:] == 12544.0) and np.all(got[1, 8:] == -12544.0)
    bias = torch.arange(16, dtype=torch.float16, device=cuda()) - 7.5
    c = torch.full((3, 16), 9.0, dtype=torch.float16, device=cuda())
    a0 = torch.zeros((3, 16), dtype=torch.uint8, device=cuda())
    b0 = torch.zeros((16, 16), dtype=torch.uint8, device=cuda())
    fp8sm.scaled_mm(a0[:, :0], b0[:, :0], to_gpu_f32(np.ones(3, F32)),
                    to_gpu_f32(np.ones(16, F32)), fp8sm.KIND_ROW, fp8sm.KIND_COL, c=c,
                    bias=bias, out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert torch.equal(c, bias.expand(3, 16))


def test_rows_do_not_depend_on_m():
    # sglang PR #44861 reviewers' check: rows of an M-row call against the same
    # rows inside a 101-row call, K = 6144, N = 5120
    M0, N, K = 101, 5120, 6144
    A, B, sa, sb = _quantized_case(M0, N, K, seed=21, outliers=False)
    full = _mm(A, B, sa, sb)
    for M in (1, 8, 16, 37, 64, 100):
        part = _mm(A[:M], B, sa[:M], sb)
        assert np.array_equal(part, full[:M]), M
    res = og.scaled_mm(A, B, sa, sb)
    assert_within_tolerance(full, res, K, "row-invariance case")


def test_power_of_two_scale_linearity_is_bitwise():
    A, B, sa, sb = _quantized_case(48, 256, 1024, seed=22)
    base = _mm(A, B, sa, sb)
    twice = _mm(A, B, (sa * F32(4)).astype(F32), (sb * F32(0.5)).astype(F32))
    b = base.astype(np.uint32) << 16
    t = twice.astype(np.uint32) << 16
    assert np.array_equal((b.view(F32) * F32(2)).view(np.uint32), t)


def test_per_tensor_equals_rowwise_with_broadcast_scales():
    A = inputs.random_codes((24, 768), seed=23)
    B = inputs.random_codes((96, 768), seed=24)
    s1, s2 = F32(0.0123), F32(0.000456)
    x = _mm(A, B, s1, s2, T, T)
    y = _mm(A, B, np.full(24, s1), np.full(96, s2), ROW, COL)
    assert np.array_equal(x, y)
    assert_within_tolerance(x, og.scaled_mm(A, B, s1, s2), 768, "per-tensor random codes")


def test_tiny_workload_pipeline():
    # quant of both operands on the GPU, compared bit-exactly, then the GEMM
    w = inputs.workload("tiny")
    M, N, K = inputs.ROWWISE_SHAPES["tiny"]
    qa, sa = fp8sm.quant_group(w.x.to(cuda()), -1)
    qb, sb = fp8sm.quant_group(w.w.to(cuda()), -1)
    c = fp8sm.scaled_mm(qa, qb, sa.reshape(-1), sb.reshape(-1), ROW, COL)
    torch.cuda.synchronize()
    oa = oq.quant_group(inputs.widen(w.x), K)
    ob = oq.quant_group(inputs.widen(w.w), K)
    assert np.array_equal(qa.cpu().numpy(), oa.codes)
    assert np.array_equal(qb.cpu().numpy(), ob.codes)
    res = og.scaled_mm(oa.codes, ob.codes, oa.scale.reshape(-1), ob.scale.reshape(-1))
    assert_within_tolerance(bf16_bits(c), res, K, "tiny 64x256x512")


@pytest.mark.parametrize("N", list(inputs.DECODE_NS))
def test_decode_workload_per_tensor(N):
    d = inputs.decode()
    xs = torch.tensor([d.x_scale], dtype=torch.float32, device=cuda())
    ws = torch.tensor([d.w_scale[N]], dtype=torch.float32, device=cuda())
    qx = fp8sm.quant_static(d.x.to(cuda()), xs)
    qw = fp8sm.quant_static(d.w[N].to(cuda()), ws)
    ox = oq.quant_static(inputs.widen(d.x), F32(d.x_scale))
    ow = oq.quant_static(inputs.widen(d.w[N]), F32(d.w_scale[N]))
    torch.cuda.synchronize()
    assert np.array_equal(qx.cpu().numpy(), ox)
    assert np.array_equal(qw.cpu().numpy(), ow)
    res = og.scaled_mm(ox, ow, F32(d.x_scale), F32(d.w_scale[N]))
    outs = {}
    for M in inputs.DECODE_MS:
        c = fp8sm.scaled_mm(qx[:M], qw, xs, ws, T, T)
        torch.cuda.synchronize()
        outs[M] = bf16_bits(c)
    assert_within_tolerance(outs[16], res, inputs.DECODE_K, f"decode N={N}")
    for M in inputs.DECODE_MS:
        assert np.array_equal(outs[M], outs[16][:M]), M
    # the weight stored at the padded row stride (K + 64) recommended for
    # small-M calls, quantized straight into that layout: codes and every
    # output bitwise equal to the compact layout's, padding bytes untouched
    K = inputs.DECODE_K
    wpad = torch.full((N, K + 64), 0x5A, dtype=torch.uint8, device=cuda())
    qwp = fp8sm.quant_static(d.w[N].to(cuda()), ws, q=wpad[:, :K])
    for M in inputs.DECODE_MS:
        c = fp8sm.scaled_mm(qx[:M], qwp, xs, ws, T, T)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(c), outs[M]), f"padded weight M={M}"
    assert np.array_equal(qwp.cpu().numpy(), ow)
    assert torch.all(wpad[:, K:] == 0x5A)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_fused_blockwise_workload(dtype):
    f = inputs.fused()
    x = f.gu_bf16 if dtype == torch.bfloat16 else f.gu_fp16
    qa, ea = fp8sm.quant_group(x.to(cuda()), 128, fp8sm.SCALE_UE8M0_BYTE, fuse_silu_mul=True)
    qb, sb = fp8sm.quant_weight_block128(f.w.to(cuda()))
    c = fp8sm.scaled_mm(qa, qb, ea, sb, fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_BLOCK128)
    torch.cuda.synchronize()
    oa = oq.quant_group_silu_mul(inputs.widen(x), 128, pow2=True)
    ob_codes, ob_scale = oq.quant_weight_block(inputs.widen(f.w))
    assert np.array_equal(qa.cpu().numpy(), oa.codes)
    assert np.array_equal(ea.cpu().numpy(), oa.ue8m0_byte)
    assert np.array_equal(qb.cpu().numpy(), ob_codes)
    res = og.blockwise_mm(oa.codes, oa.scale, ob_codes, ob_scale)
    got = bf16_bits(c)
    assert np.all(got[f.zero_rows] == 0)
    assert_within_tolerance(got, res, inputs.FUSED_K, f"fused blockwise {dtype}")


def test_blockwise_fp32_group_scales_ragged():
    r = inputs.rng(25)
    M, N, K = 70, 264, 400
    A = inputs.random_codes((M, K), seed=26)
    B = inputs.random_codes((N, K), seed=27)
    sa = np.exp2(r.uniform(-12, -4, (M, 4))).astype(F32)
    sb = np.exp2(r.uniform(-12, -4, (3, 4))).astype(F32)
    c = fp8sm.scaled_mm(to_gpu_u8(A), to_gpu_u8(B), to_gpu_f32(sa), to_gpu_f32(sb),
                        fp8sm.KIND_GROUP128_FP32, fp8sm.KIND_BLOCK128)
    torch.cuda.synchronize()
    assert_within_tolerance(bf16_bits(c), og.blockwise_mm(A, sa, B, sb), K, "blockwise fp32 ragged")


@pytest.mark.parametrize("shape", [(70, 264, 400), (5, 136, 1040), (33, 128, 128),
                                   (130, 520, 2064), (32, 384, 7168)])
def test_blockwise_ue8m0_ragged_and_row_invariant(shape):
    # ragged M / N / K (partial K blocks) against the oracle, and a row's bits
    # do not depend on M
    M, N, K = shape
    print(f"[case] blockwise ue8m0 M={M} N={N} K={K}", flush=True)
    r = inputs.rng(M + N + K)
    G = (K + 127) // 128
    A = inputs.random_codes((M, K), seed=M)
    B = inputs.random_codes((N, K), seed=N)
    e = r.integers(119, 131, size=(M, G)).astype(np.uint8)
    sb = np.exp2(r.uniform(-14, -6, ((N + 127) // 128, G))).astype(F32)

    def run(rows):
        c = fp8sm.scaled_mm(to_gpu_u8(A[:rows]), to_gpu_u8(B), torch.from_numpy(e[:rows]).to(cuda()),
                            to_gpu_f32(sb), fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_BLOCK128)
        torch.cuda.synchronize()
        return bf16_bits(c)
    full = run(M)
    assert np.array_equal(run(min(M, 5)), full[:5])
    a_vals = np.exp2(e.astype(np.float64) - 127).astype(F32)
    assert_within_tolerance(full, og.blockwise_mm(A, a_vals, B, sb), K, f"ue8m0 {shape}")


def test_k_zero_writes_zeros():
    c = torch.full((5, 16), 7.0, dtype=torch.bfloat16, device=cuda())
    a = torch.zeros((5, 16), dtype=torch.uint8, device=cuda())
    b = torch.zeros((16, 16), dtype=torch.uint8, device=cuda())
    s = torch.ones(16, dtype=torch.float32, device=cuda())
    st = fp8sm.lib().fp8sm_scaled_mm(a.data_ptr(), 16, b.data_ptr(), 16, c.data_ptr(), 16, 5, 16, 0,
                                     ROW, s.data_ptr(), COL, s.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == 0 and torch.all(c == 0)


def _sampled_full_size(name):
    M, N, K = inputs.ROWWISE_SHAPES[name]
    w = inputs.workload(name)
    qa, sa = fp8sm.quant_group(w.x.to(cuda()), -1)
    qb, sb = fp8sm.quant_group(w.w.to(cuda()), -1)
    c = fp8sm.scaled_mm(qa, qb, sa.reshape(-1), sb.reshape(-1), ROW, COL)
    torch.cuda.synchronize()
    r = inputs.rng(99)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), r.integers(0, M, 24)]))
    cols = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N), r.integers(0, N, 24)]))
    # the oracle quantizes only the sampled rows / channels (rows are independent)
    oa = oq.quant_group(inputs.widen(w.x[torch.from_numpy(rows)]), K)
    ga = qa[torch.from_numpy(rows).to(cuda())].cpu().numpy()
    assert np.array_equal(ga, oa.codes)
    ob_all = oq.quant_group(inputs.widen(w.w), K)
    assert np.array_equal(qb.cpu().numpy(), ob_all.codes)
    oa_cols = oq.quant_group(inputs.widen(w.x), K)
    gpu_bits = bf16_bits(c)
    res_r = og.scaled_mm(oa.codes, ob_all.codes, oa.scale.reshape(-1), ob_all.scale.reshape(-1))
    assert_within_tolerance(gpu_bits[rows], res_r, K, f"{name} sampled rows")
    res_c = og.scaled_mm(oa_cols.codes, ob_all.codes[cols], oa_cols.scale.reshape(-1),
                         ob_all.scale.reshape(-1)[cols])
    assert_within_tolerance(gpu_bits[:, cols], res_c, K, f"{name} sampled cols")


@pytest.mark.parametrize("name", ["qkv", "mlp_down"])
def test_full_size_rowwise_sampled(name):
    _sampled_full_size(name)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mlp_gateup_23216", "mlp_gateup_15760"])
def test_full_size_rowwise_sampled_large(name):
    _sampled_full_size(name)


def test_max_k_rowwise_every_variant():
    # K = 65536, the largest the boundary takes: every variant within the
    # bound and bitwise equal
    M, N, K = 37, 72, 65536
    print(f"[case] max K M={M} N={N} K={K}", flush=True)
    A, B, sa, sb = _quantized_case(M, N, K, seed=5)
    res = og.scaled_mm(A, B, sa, sb)
    outs = {}
    for v in _variants_for(M, K):
        outs[v] = _mm_variant(v, A, B, sa, sb)
        assert_within_tolerance(outs[v], res, K, f"max K {fp8sm.variant_name(v)}")
    first = next(iter(outs.values()))
    assert all(np.array_equal(o, first) for o in outs.values())


@pytest.mark.parametrize("shape", [(70, 264, 8320), (20, 128, 65536)])
def test_blockwise_ue8m0_long_k_restages_scales(shape):
    # more than 64 K blocks: the kernel re-stages the activation scale bytes
    # every 64 blocks; the last segment is partial
    M, N, K = shape
    print(f"[case] blockwise long K M={M} N={N} K={K}", flush=True)
    r = inputs.rng(K + M)
    G = (K + 127) // 128
    A = inputs.random_codes((M, K), seed=M + 1)
    B = inputs.random_codes((N, K), seed=N + 1)
    e = r.integers(119, 131, size=(M, G)).astype(np.uint8)
    sb = np.exp2(r.uniform(-14, -6, ((N + 127) // 128, G))).astype(F32)
    c = fp8sm.scaled_mm(to_gpu_u8(A), to_gpu_u8(B), torch.from_numpy(e).to(cuda()),
                        to_gpu_f32(sb), fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_BLOCK128)
    torch.cuda.synchronize()
    a_vals = np.exp2(e.astype(np.float64) - 127).astype(F32)
    assert_within_tolerance(bf16_bits(c), og.blockwise_mm(A, a_vals, B, sb), K, f"long K {shape}")


@pytest.mark.parametrize("M,variant", [(12, None), (300, None), (300, "tile128x256")])
def test_quant_and_rowwise_gemm_graph_replays(M, variant):
    # the hot path's step (per-token quant of the activations, rowwise GEMM
    # against per-channel weights) captured once in a HIP graph and replayed
    # with new activations, eager work and synchronizations between replays:
    # every replay equals the eager step bitwise and the oracle (codes
    # bit-exact, GEMM within the bound); K = 1040 has a 16-byte K tail
    N, K = 520, 1040
    print(f"[case] graph replay M={M} variant={variant}", flush=True)
    r = inputs.rng(M + 7)
    w = inputs.to_dtype(r.standard_normal((N, K), dtype=np.float32) * F32(0.02))
    xs = [inputs.to_dtype(r.standard_normal((M, K), dtype=np.float32)) for _ in range(3)]
    qb, sb = fp8sm.quant_group(w.to(cuda()), -1)
    ob = oq.quant_group(inputs.widen(w), K)
    x = torch.empty((M, K), dtype=torch.bfloat16, device=cuda())
    qa = torch.empty((M, K), dtype=torch.uint8, device=cuda())
    sa = torch.empty((M, 1), dtype=torch.float32, device=cuda())
    c = torch.empty((M, N), dtype=torch.bfloat16, device=cuda())
    names = {fp8sm.variant_name(v): v for v in range(fp8sm.variant_count())}
    prev = fp8sm.force_variant(names[variant] if variant else -1)
    try:
        def step():
            fp8sm.quant_group(x, -1, q=qa, scales=sa)
            fp8sm.scaled_mm(qa, qb, sa.reshape(-1), sb.reshape(-1), ROW, COL, c=c)

        x.copy_(xs[0].to(cuda()))
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            step()                        # warm up outside capture
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for xi in xs + xs[:1]:
            x.copy_(xi.to(cuda()))
            for t in (qa, sa, c):
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            qg, sg, cg = qa.clone(), sa.clone(), bf16_bits(c)
            for t in (qa, sa, c):
                t.zero_()
            step()
            torch.cuda.synchronize()
            assert torch.equal(qa, qg) and torch.equal(sa, sg)
            assert np.array_equal(bf16_bits(c), cg)
            oa = oq.quant_group(inputs.widen(xi), K)
            assert np.array_equal(qg.cpu().numpy(), oa.codes)
            res = og.scaled_mm(oa.codes, ob.codes, oa.scale.reshape(-1), ob.scale.reshape(-1))
            assert_within_tolerance(cg, res, K, f"graph replay M={M} {variant}")
    finally:
        fp8sm.force_variant(prev)


def test_blockwise_ue8m0_every_exponent_byte():
    # UE8M0 scales are 2^(byte - 127) for every byte 0..255.  Row r has one
    # live K block, with byte r, whose weight scale 2^s brings byte r's
    # power of two back near 1 (so every output is a normal, finite bf16);
    # its other blocks hold zero codes with random bytes (extremes
    # included).  Checked against the oracle with the bound's sa * sb taken
    # from the live block alone (stricter than the max over blocks).
    M, N, G = 256, 256, 5
    K = 128 * G
    print("[case] blockwise ue8m0 every byte M=256 N=256 K=640", flush=True)
    offs = np.array([110, 50, 0, -50, -110])
    r = inputs.rng(255)
    live = np.array([int(np.argmin(np.abs(b - 127 + offs))) for b in range(M)])
    A = np.zeros((M, K), np.uint8)
    codes = e4m3.finite_codes()
    for m in range(M):
        kb = live[m]
        A[m, 128 * kb:128 * (kb + 1)] = codes[r.integers(0, codes.size, 128)]
    B = codes[r.integers(0, codes.size, (N, K))]
    e = r.integers(0, 256, (M, G)).astype(np.uint8)
    e[np.arange(M), live] = np.arange(M)
    sb = np.tile(np.exp2(offs.astype(np.float64)).astype(F32), ((N + 127) // 128, 1))
    c = fp8sm.scaled_mm(to_gpu_u8(A), to_gpu_u8(B), torch.from_numpy(e).to(cuda()),
                        to_gpu_f32(sb), fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_BLOCK128)
    torch.cuda.synchronize()
    res = og.blockwise_mm(A, og.ue8m0_values(e), B, sb)
    res.sab = (og.ue8m0_values(e)[np.arange(M), live] * np.exp2(offs[live]))[:, None] * np.ones((1, N))
    assert np.all(np.isfinite(res.out)) and np.all(np.abs(res.out[res.out != 0]) >= 2.0 ** -126)
    assert_within_tolerance(bf16_bits(c), res, K, "ue8m0 every byte")

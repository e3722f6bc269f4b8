"""GPU parity of the batched and masked entry points.

Every live row must equal, bitwise, what the 2-D call gives for that batch's
operands (same forced kernel variant), and the oracle (bit-exact for quant,
within the GEMM bound); rows past a batch's count must keep the sentinel the
output held before the call.  Inputs are strided 3-D views (batch and row
strides that no dense 2-D matrix has)."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import batched as ob, gemm as og, quant as oq
from gpu_util import assert_within_tolerance, bf16_bits, cuda

pytestmark = pytest.mark.gpu
F32 = np.float32
ROW, COL, T = fp8sm.KIND_ROW, fp8sm.KIND_COL, fp8sm.KIND_TENSOR
SENT_U8 = 0x5A
SENT_U16 = 0x7FC1   # a NaN pattern in bf16 and in fp16: no kernel writes it


def _variants_for(M, K):
    """Every rowwise kernel variant that computes an M-row call with this K."""
    return [v for v in range(fp8sm.variant_count()) if fp8sm.variant_accepts(v, M, 0, K)]


def _strided_3d(t, B, M, pad_rows=1, pad_cols=64, dtype=None):
    """Copy t [B, M, C] into the middle of a larger buffer and return the view
    (row stride C + pad_cols, batch stride (M + 2 pad_rows) rows)."""
    C = t.shape[2]
    big = torch.zeros((B, M + 2 * pad_rows, C + pad_cols), dtype=dtype or t.dtype, device=cuda())
    view = big[:, pad_rows:pad_rows + M, :C]
    view.copy_(t.to(cuda()))
    assert view.stride(0) != M * view.stride(1)
    return view


def _live(rows, B, M):
    return ob.valid_rows(None if rows is None else rows, B, M)


def _rows_dev(rows):
    return None if rows is None else torch.tensor(rows, dtype=torch.int32, device=cuda())


# ---------------------------------------------------------------- quant

def _quant_case(B, M, K_in, dtype, seed):
    r = inputs.rng(seed)
    x = r.standard_normal((B, M, K_in), dtype=np.float32)
    x[0, 0] = 0.0                                    # a zero row
    return inputs.to_dtype(x, dtype)


@pytest.mark.parametrize("K", [384, 4224, 16384, 24592])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_per_token_quant_strided_masked(K, dtype):
    # K picks the kernel family: one chunk per lane, eleven with a partial
    # chunk, four wavefronts per row, two passes
    B, M = 3, 9
    rows = [9, 4, 0]
    print(f"[case] per-token batched K={K} {dtype}", flush=True)
    x = _quant_case(B, M, K, dtype, seed=K)
    xv = _strided_3d(x, B, M)
    for fmt in (fp8sm.SCALE_FP32, fp8sm.SCALE_UE8M0_BYTE):
        q = torch.full((B, M, K), SENT_U8, dtype=torch.uint8, device=cuda())
        sdt = torch.uint8 if fmt == fp8sm.SCALE_UE8M0_BYTE else torch.float32
        s = torch.full((B, M, 1), 7, dtype=sdt, device=cuda())
        fp8sm.quant_group_batched(xv, -1, fmt=fmt, rows=_rows_dev(rows), q=q, scales=s)
        torch.cuda.synchronize()
        ref = ob.quant_group_batched(inputs.widen(x), K, pow2=fmt != fp8sm.SCALE_FP32, rows=rows)
        qh, sh = q.cpu().numpy(), s.cpu().numpy()
        for b, mb in enumerate(_live(rows, B, M)):
            assert np.array_equal(qh[b, :mb], ref[b].codes), (b, fmt)
            want = ref[b].ue8m0_byte if fmt == fp8sm.SCALE_UE8M0_BYTE else ref[b].scale
            assert np.array_equal(sh[b, :mb], want.reshape(mb, 1)), (b, fmt)
            assert np.all(qh[b, mb:] == SENT_U8) and np.all(sh[b, mb:] == 7), (b, fmt)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("layout", [fp8sm.LAYOUT_ROW_MAJOR, fp8sm.LAYOUT_MN_MAJOR])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_group128_quant_strided_masked(fused, layout, dtype):
    B, M, K = 5, 37, 512
    rows = [37, 0, 12, 50, -3]
    print(f"[case] g128 batched fused={fused} layout={layout} {dtype}", flush=True)
    x = _quant_case(B, M, 2 * K if fused else K, dtype, seed=7 + fused)
    xv = _strided_3d(x, B, M)
    ref = ob.quant_group_batched(inputs.widen(x), 128, pow2=True, fused=fused, rows=rows)
    G, Mp = K // 128, ((M + 3) // 4) * 4
    q = torch.full((B, M, K), SENT_U8, dtype=torch.uint8, device=cuda())
    sshape = (B, G, Mp) if layout == fp8sm.LAYOUT_MN_MAJOR else (B, M, G)
    s = torch.full(sshape, 7, dtype=torch.uint8, device=cuda())
    fp8sm.quant_group_batched(xv, 128, fmt=fp8sm.SCALE_UE8M0_BYTE, layout=layout,
                              fuse_silu_mul=fused, rows=_rows_dev(rows), q=q, scales=s)
    torch.cuda.synchronize()
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    for b, mb in enumerate(_live(rows, B, M)):
        assert np.array_equal(qh[b, :mb], ref[b].codes), b
        assert np.all(qh[b, mb:] == SENT_U8), b
        got = sh[b, :, :mb].T if layout == fp8sm.LAYOUT_MN_MAJOR else sh[b, :mb]
        assert np.array_equal(got, ref[b].ue8m0_byte), b
        dead = sh[b, :, mb:] if layout == fp8sm.LAYOUT_MN_MAJOR else sh[b, mb:]
        assert np.all(dead == 7), b


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_fused_per_token_quant_masked(dtype):
    B, M, K = 3, 20, 1024
    rows = [20, 7, 1]
    x = _quant_case(B, M, 2 * K, dtype, seed=99)
    xv = _strided_3d(x, B, M)
    q = torch.full((B, M, K), SENT_U8, dtype=torch.uint8, device=cuda())
    s = torch.full((B, M, 1), -1.0, dtype=torch.float32, device=cuda())
    fp8sm.quant_group_batched(xv, -1, fuse_silu_mul=True, rows=_rows_dev(rows), q=q, scales=s)
    torch.cuda.synchronize()
    ref = ob.quant_group_batched(inputs.widen(x), K, fused=True, rows=rows)
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    for b, mb in enumerate(rows):
        assert np.array_equal(qh[b, :mb], ref[b].codes)
        assert np.array_equal(sh[b, :mb, 0], ref[b].scale[:, 0])
        assert np.all(qh[b, mb:] == SENT_U8) and np.all(sh[b, mb:] == -1.0)


def test_static_quant_strided():
    B, M, K = 4, 11, 264
    x = _quant_case(B, M, K, torch.bfloat16, seed=3)
    xv = _strided_3d(x, B, M)
    s = F32(inputs.static_scale(x))
    q = fp8sm.quant_static_batched(xv, torch.tensor([s], device=cuda()))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), ob.quant_static_batched(inputs.widen(x), s))


# ---------------------------------------------------------------- GEMM

def _gemm_case(B, M, N, K, per_batch_weight, seed):
    r = inputs.rng(seed)
    x = r.standard_normal((B, M, K), dtype=np.float32)
    nw = B if per_batch_weight else 1
    w = r.standard_normal((nw, N, K), dtype=np.float32) * F32(0.02)
    qa = [oq.quant_group(inputs.widen(inputs.to_dtype(x[b])), K) for b in range(B)]
    qw = [oq.quant_group(inputs.widen(inputs.to_dtype(w[b])), K) for b in range(nw)]
    A = np.stack([q.codes for q in qa])
    sa = np.stack([q.scale.reshape(-1) for q in qa])
    W = np.stack([q.codes for q in qw])
    sw = np.stack([q.scale.reshape(-1) for q in qw])
    if not per_batch_weight:
        W, sw = W[0], sw[0]
    return A, sa, W, sw


def _a_view(A):
    B, M, K = A.shape
    big = torch.zeros((B, M + 3, K + 32), dtype=torch.uint8, device=cuda())
    v = big[:, 2:2 + M, :K]
    v.copy_(torch.from_numpy(A).to(cuda()))
    return v


def _two_d(A, W, sa, sb, b, per_b, bias=None, out_dtype=torch.bfloat16):
    """Batch b through the 2-D call."""
    Wb = W[b] if per_b else W
    sbb = sb[b] if per_b else sb
    c = fp8sm.scaled_mm(torch.from_numpy(np.ascontiguousarray(A[b])).to(cuda()),
                        torch.from_numpy(np.ascontiguousarray(Wb)).to(cuda()),
                        torch.from_numpy(np.ascontiguousarray(sa[b])).to(cuda()),
                        torch.from_numpy(np.ascontiguousarray(sbb)).to(cuda()), ROW, COL,
                        bias=bias, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return bf16_bits(c)


@pytest.mark.parametrize("shape", [(3, 37, 264, 80), (2, 16, 48, 1552), (4, 5, 64, 176),
                                   (2, 130, 136, 208), (3, 64, 72, 384)])
@pytest.mark.parametrize("per_b", [False, True])
def test_batched_rowwise_strided_every_variant(shape, per_b):
    B, M, N, K = shape
    print(f"[case] batched rowwise {shape} per_batch_weight={per_b}", flush=True)
    A, sa, W, sb = _gemm_case(B, M, N, K, per_b, seed=M + N + K)
    av = _a_view(A)
    wd = torch.from_numpy(W).to(cuda())
    sad = torch.from_numpy(sa).to(cuda())
    sbd = torch.from_numpy(sb).to(cuda())
    res = ob.scaled_mm_batched(A, W, sa, sb if per_b else np.stack([sb] * B))
    first = None
    for v in _variants_for(M, K):
        prev = fp8sm.force_variant(v)
        try:
            c = fp8sm.scaled_mm_batched(av, wd, sad, sbd, ROW, COL)
            torch.cuda.synchronize()
            got = bf16_bits(c)
            for b in range(B):
                assert np.array_equal(got[b], _two_d(A, W, sa, sb, b, per_b)), (fp8sm.variant_name(v), b)
                assert_within_tolerance(got[b], res[b], K, f"{shape} {fp8sm.variant_name(v)} b={b}")
        finally:
            fp8sm.force_variant(prev)
        if first is None:
            first = got
        assert np.array_equal(got, first), fp8sm.variant_name(v)


@pytest.mark.parametrize("out", ["bf16", "fp16"])
def test_masked_rowwise_with_bias_leaves_dead_rows(out):
    B, M, N, K = 6, 40, 96, 256
    rows = [0, 3, 40, 49, -2, 17]
    tdt = torch.float16 if out == "fp16" else torch.bfloat16
    A, sa, W, sb = _gemm_case(B, M, N, K, True, seed=21)
    r = inputs.rng(4)
    bias = torch.from_numpy(r.standard_normal(N).astype(F32)).to(tdt)
    res = ob.scaled_mm_batched(A, W, sa, sb, rows=rows, bias=bias.float().numpy(), out=out)
    av = _a_view(A)
    for v in _variants_for(M, K):
        prev = fp8sm.force_variant(v)
        try:
            c = torch.full((B, M, N), SENT_U16, dtype=torch.int16, device=cuda()).view(tdt)
            fp8sm.scaled_mm_batched(av, torch.from_numpy(W).to(cuda()),
                                    torch.from_numpy(sa).to(cuda()), torch.from_numpy(sb).to(cuda()),
                                    ROW, COL, rows=_rows_dev(rows), c=c, bias=bias.to(cuda()),
                                    out_dtype=tdt)
            torch.cuda.synchronize()
            got = bf16_bits(c)
            for b, mb in enumerate(_live(rows, B, M)):
                assert np.all(got[b, mb:] == SENT_U16), (fp8sm.variant_name(v), b)
                want = _two_d(A, W, sa, sb, b, True, bias=bias.to(cuda()), out_dtype=tdt)[:mb]
                assert np.array_equal(got[b, :mb], want), (fp8sm.variant_name(v), b)
                assert_within_tolerance(got[b, :mb], res[b], K, f"masked {out} b={b}")
        finally:
            fp8sm.force_variant(prev)


def test_per_batch_tensor_scales():
    # one scalar scale per batch (TENSOR kind with a [B] tensor), shared weight
    B, M, N, K = 3, 8, 64, 128
    A = inputs.random_codes((B, M, K), seed=1) & 0x77      # |v| <= 240: finite, no NaN
    W = inputs.random_codes((N, K), seed=2) & 0x77
    sa = np.array([0.5, 0.25, 2.0], F32)
    sb = np.array([0.125], F32)
    c = fp8sm.scaled_mm_batched(_a_view(A), torch.from_numpy(W).to(cuda()),
                                torch.from_numpy(sa).to(cuda()), torch.from_numpy(sb).to(cuda()),
                                T, T)
    torch.cuda.synchronize()
    res = ob.scaled_mm_batched(A, W, sa, np.repeat(sb, B))
    got = bf16_bits(c)
    for b in range(B):
        assert_within_tolerance(got[b], res[b], K, f"tensor scales b={b}")


@pytest.mark.parametrize("kind", [fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_GROUP128_FP32])
def test_masked_grouped_blockwise(kind):
    B, M, N, K = 4, 70, 256, 384
    rows = [70, 0, 13, 129]
    print(f"[case] masked grouped blockwise kind={kind}", flush=True)
    r = inputs.rng(17)
    x = inputs.to_dtype(r.standard_normal((B, M, K), dtype=np.float32))
    w = inputs.to_dtype(r.standard_normal((B, N, K), dtype=np.float32) * F32(0.02))
    pow2 = kind == fp8sm.KIND_GROUP128_UE8M0
    qa = [oq.quant_group(inputs.widen(x[b]), 128, pow2=pow2) for b in range(B)]
    qw = [oq.quant_weight_block(inputs.widen(w[b])) for b in range(B)]
    A = np.stack([q.codes for q in qa])
    a_vals = np.stack([q.scale for q in qa])                       # [B, M, G] values
    a_dev = np.stack([q.ue8m0_byte for q in qa]) if pow2 else a_vals
    W = np.stack([c for c, _ in qw])
    ws = np.stack([s for _, s in qw])
    res = ob.blockwise_mm_batched(A, a_vals, W, ws, rows=rows)
    c = torch.full((B, M, N), SENT_U16, dtype=torch.int16, device=cuda()).view(torch.bfloat16)
    fp8sm.scaled_mm_batched(_a_view(A), torch.from_numpy(W).to(cuda()),
                            torch.from_numpy(a_dev).to(cuda()), torch.from_numpy(ws).to(cuda()),
                            kind, fp8sm.KIND_BLOCK128, rows=_rows_dev(rows), c=c)
    torch.cuda.synchronize()
    got = bf16_bits(c)
    for b, mb in enumerate(_live(rows, B, M)):
        assert np.all(got[b, mb:] == SENT_U16), b
        c2 = fp8sm.scaled_mm(torch.from_numpy(A[b]).to(cuda()), torch.from_numpy(W[b]).to(cuda()),
                             torch.from_numpy(a_dev[b]).to(cuda()), torch.from_numpy(ws[b]).to(cuda()),
                             kind, fp8sm.KIND_BLOCK128)
        torch.cuda.synchronize()
        assert np.array_equal(got[b, :mb], bf16_bits(c2)[:mb]), b
        assert_within_tolerance(got[b, :mb], res[b], K, f"grouped blockwise b={b}")


def test_batched_k0_masked_writes_bias():
    B, M, N = 3, 5, 32
    rows = [2, 0, 5]
    bias = torch.arange(N, dtype=torch.float32, device=cuda()).to(torch.bfloat16)
    c = torch.full((B, M, N), SENT_U16, dtype=torch.int16, device=cuda()).view(torch.bfloat16)
    a = torch.zeros((B, M, 16), dtype=torch.uint8, device=cuda())[:, :, :0]
    w = torch.zeros((N, 16), dtype=torch.uint8, device=cuda())[:, :0]
    one = torch.ones(1, dtype=torch.float32, device=cuda())
    fp8sm.scaled_mm_batched(a, w, one, one, T, T, rows=_rows_dev(rows), c=c, bias=bias)
    torch.cuda.synchronize()
    got = bf16_bits(c)
    want = bf16_bits(bias)
    for b, mb in enumerate(rows):
        assert np.all(got[b, :mb] == want[None, :]) and np.all(got[b, mb:] == SENT_U16)


def test_masked_moe_pipeline_graph_replays():
    # fused masked group quant -> grouped masked blockwise GEMM, captured once
    # in a graph and replayed with new per-expert counts written into the same
    # device tensor between replays; each replay must match the eager call
    E, Tm, inter, hidden = 6, 40, 256, 384
    r = inputs.rng(31)
    gu = inputs.to_dtype(r.standard_normal((E, Tm, 2 * inter), dtype=np.float32))
    w = inputs.to_dtype(r.standard_normal((E, hidden, inter), dtype=np.float32) * F32(0.02))
    qw = [oq.quant_weight_block(inputs.widen(w[e])) for e in range(E)]
    Wd = torch.from_numpy(np.stack([c for c, _ in qw])).to(cuda())
    ws = torch.from_numpy(np.stack([s for _, s in qw])).to(cuda())
    gud = gu.to(cuda())
    rows = torch.zeros(E, dtype=torch.int32, device=cuda())
    q = torch.zeros((E, Tm, inter), dtype=torch.uint8, device=cuda())
    s = torch.zeros((E, Tm, inter // 128), dtype=torch.uint8, device=cuda())
    c = torch.zeros((E, Tm, hidden), dtype=torch.bfloat16, device=cuda())

    def step(stream=None):
        fp8sm.quant_group_batched(gud, 128, fmt=fp8sm.SCALE_UE8M0_BYTE, fuse_silu_mul=True,
                                  rows=rows, q=q, scales=s, stream=stream)
        fp8sm.scaled_mm_batched(q, Wd, s, ws, fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_BLOCK128,
                                rows=rows, c=c, stream=stream)

    counts = [[40, 0, 3, 17, 1, 22], [5, 40, 0, 0, 39, 2], [0, 0, 0, 0, 0, 1]]
    rows.copy_(torch.tensor(counts[0], dtype=torch.int32))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step(cs)                          # warm up outside capture
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for cnt in counts:
        rows.copy_(torch.tensor(cnt, dtype=torch.int32))
        for t in (q, s, c):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        qg, sg, cg = q.clone(), s.clone(), bf16_bits(c)
        for t in (q, s, c):
            t.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(q, qg) and torch.equal(s, sg)
        assert np.array_equal(bf16_bits(c), cg)
        # and the oracle
        ref = ob.quant_group_batched(inputs.widen(gu), 128, pow2=True, fused=True, rows=cnt)
        res = ob.blockwise_mm_batched(
            np.stack([np.pad(ref[e].codes, ((0, Tm - cnt[e]), (0, 0))) for e in range(E)]),
            np.stack([np.pad(ref[e].scale, ((0, Tm - cnt[e]), (0, 0)), constant_values=1)
                      for e in range(E)]),
            np.stack([c_ for c_, _ in qw]), np.stack([s_ for _, s_ in qw]), rows=cnt)
        qh = q.cpu().numpy()
        for e in range(E):
            assert np.array_equal(qh[e, :cnt[e]], ref[e].codes), e
            assert_within_tolerance(cg[e, :cnt[e]], res[e], inter, f"replay {cnt} e={e}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_linear_graph_replays_strided_bias_k80(out_dtype):
    # the deterministic static-FP8 linear of sglang PR #44861 (Modifications:
    # graph replays with bias, strided 3-D inputs, BF16/FP16 and a K = 80 tail):
    # static quant of a strided [B, S, K] activation, then the batched GEMM
    # against one per-tensor weight with a bias, captured once and replayed
    # with new activations; every replay equals the eager call bitwise and the
    # oracle within the bound
    B, S, K, N = 3, 7, 80, 96
    r = inputs.rng(80)
    w = inputs.to_dtype(r.standard_normal((N, K), dtype=np.float32) * F32(0.02))
    ws = F32(inputs.static_scale(w))
    wq = ob.quant_static_batched(inputs.widen(w)[None], ws)[0]
    bias = inputs.to_dtype(r.standard_normal(N, dtype=np.float32), out_dtype)
    xs = [inputs.to_dtype(r.standard_normal((B, S, K), dtype=np.float32)) for _ in range(3)]
    xsc = F32(max(inputs.static_scale(x) for x in xs))
    xv = _strided_3d(xs[0], B, S)
    wd, sx, sw = torch.from_numpy(wq).to(cuda()), torch.tensor([xsc], device=cuda()), torch.tensor([ws], device=cuda())
    bd = bias.to(cuda())
    q = torch.empty((B, S, K), dtype=torch.uint8, device=cuda())
    c = torch.empty((B, S, N), dtype=out_dtype, device=cuda())

    def step(stream=None):
        fp8sm.quant_static_batched(xv, sx, q=q, stream=stream)
        fp8sm.scaled_mm_batched(q, wd, sx, sw, T, T, c=c, bias=bd, out_dtype=out_dtype, stream=stream)

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step(cs)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    out = "fp16" if out_dtype == torch.float16 else "bf16"
    for x in xs + xs[:1]:
        xv.copy_(x.to(cuda()))
        c.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        cg = bf16_bits(c)
        c.zero_()
        step()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(c), cg)
        qa = ob.quant_static_batched(inputs.widen(x), xsc)
        assert np.array_equal(q.cpu().numpy(), qa)
        res = ob.scaled_mm_batched(qa, wq, np.full(B, xsc, F32), np.full(B, ws, F32),
                                   bias=bias.float().numpy(), out=out)
        for b in range(B):
            assert_within_tolerance(cg[b], res[b], K, f"graph replay {out} b={b}")


def test_largest_batch_count_sampled():
    # 65535 batches (one grid row each), per-batch weights and scalar scales;
    # sampled batches against the oracle and the 2-D call
    B, M, N, K = 65535, 2, 16, 32
    A = inputs.random_codes((B, M, K), seed=11) & 0x77
    W = inputs.random_codes((B, N, K), seed=12) & 0x77
    r = inputs.rng(13)
    sa = np.exp2(r.integers(-4, 4, B)).astype(F32)
    sb = np.exp2(r.integers(-4, 4, B)).astype(F32)
    c = fp8sm.scaled_mm_batched(torch.from_numpy(A).to(cuda()), torch.from_numpy(W).to(cuda()),
                                torch.from_numpy(sa).to(cuda()), torch.from_numpy(sb).to(cuda()),
                                T, T)
    torch.cuda.synchronize()
    got = bf16_bits(c)
    pick = [0, 1, 255, 256, 32767, 65533, 65534]
    res = ob.scaled_mm_batched(A[pick], W[pick], sa[pick], sb[pick])
    for i, b in enumerate(pick):
        assert_within_tolerance(got[b], res[i], K, f"batch {b} of {B}")

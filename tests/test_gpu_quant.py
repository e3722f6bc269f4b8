"""GPU parity of the quant kernels against the oracle: codes and UE8M0 bytes
bit-exact, fp32 scales bit-exact."""
import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import quant as oq
from gpu_util import cuda, f32_bits

pytestmark = pytest.mark.gpu
F32 = np.float32


def _gpu_quant(x, group, fmt, layout, fused=False):
    q, s = fp8sm.quant_group(x.to(cuda()), group, fmt, layout, fuse_silu_mul=fused)
    torch.cuda.synchronize()
    M = x.shape[0]
    q = q.cpu().numpy()
    s = s.cpu().numpy()
    if layout == fp8sm.LAYOUT_MN_MAJOR:
        s = s[:, :M].T
    return q, s


def _oracle_quant(x, group, fmt, fused=False):
    x32 = inputs.widen(x)
    K = x32.shape[1] // 2 if fused else x32.shape[1]
    g = K if group == -1 else group
    pow2 = fmt != fp8sm.SCALE_FP32
    r = oq.quant_group_silu_mul(x32, g, pow2) if fused else oq.quant_group(x32, g, pow2)
    s = r.ue8m0_byte if fmt == fp8sm.SCALE_UE8M0_BYTE else r.scale
    return r.codes, s


def _check(x, group, fmt, layout, fused=False, what=""):
    print(f"[case] {what} M={x.shape[0]} Kin={x.shape[1]} group={group} fmt={fmt} "
          f"layout={layout} fused={fused} dtype={x.dtype}", flush=True)
    qg, sg = _gpu_quant(x, group, fmt, layout, fused)
    qo, so = _oracle_quant(x, group, fmt, fused)
    bad = qg != qo
    assert not bad.any(), f"{what}: {bad.sum()} codes differ, first at {np.argwhere(bad)[0]}"
    if fmt == fp8sm.SCALE_UE8M0_BYTE:
        assert np.array_equal(sg, so), what
    else:
        assert np.array_equal(sg.view(np.uint32), so.astype(F32).view(np.uint32)), what


def _mixed_rows(M, K, dtype, seed):
    """Normal rows with per-row magnitudes from 1e-6 to 1e3, a zero row, and
    rows with a single large outlier."""
    r = inputs.rng(seed)
    x = r.standard_normal((M, K), dtype=np.float32)
    x *= np.exp2(r.uniform(-20, 10, (M, 1))).astype(F32)
    if M > 3:
        x[1] = 0
        x[2, r.integers(0, K)] = 3000.0
    return inputs.to_dtype(x, dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("layout", [0, 1])
def test_group128_all_formats(dtype, fmt, layout):
    x = _mixed_rows(37, 896, dtype, seed=1)
    _check(x, 128, fmt, layout, what="group128")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("K", [8, 64, 384, 1008, 2000, 3056, 4096, 4224, 5376, 7168, 7184, 12288,
                               14336, 16384, 20480, 24592])
def test_per_token_fp32_many_widths(dtype, K):
    # widths cover every row-in-registers variant (one wavefront per row: 1, 2,
    # 4, 6, 8, 11 and 14 chunks per lane; four wavefronts per row: 4, 6, 8 and
    # 12 chunks per lane), each with a partial last chunk where K allows, and
    # the two-pass kernel
    x = _mixed_rows(9, K, dtype, seed=2)
    _check(x, -1, 0, 0, what="per-token")


@pytest.mark.parametrize("M,K", [(2600, 14336), (5000, 1024)])
def test_per_token_many_rows(M, K):
    # more rows than resident wavefronts / workgroups: every wavefront walks
    # several rows, alternating its two row buffers
    x = _mixed_rows(M, K, torch.bfloat16, seed=7)
    _check(x, -1, 0, 0, what="per-token many rows")


@pytest.mark.parametrize("fmt", [1, 2])
def test_per_token_ue8m0(fmt):
    x = _mixed_rows(21, 1024, torch.bfloat16, seed=3)
    _check(x, -1, fmt, 0, what="per-token ue8m0")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("group", [128, -1])
@pytest.mark.parametrize("fmt", [0, 2])
def test_fused_silu_mul(dtype, group, fmt):
    r = inputs.rng(4)
    x = r.standard_normal((19, 2 * 640), dtype=np.float32) * F32(3)
    x[5] = 0
    _check(inputs.to_dtype(x, dtype), group, fmt, 0, fused=True, what="fused")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_silu_mul_is_bit_exact_for_every_gate_value(dtype):
    # every finite bf16 / fp16 gate value, with up = 1 (y = silu(g) exactly)
    # and with random up values
    bits = np.arange(65536, dtype=np.uint32)
    if dtype == torch.bfloat16:
        g = (bits << 16).view(np.float32)
    else:
        g = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    g = g[np.isfinite(g)]
    n = -(-g.size // 512) * 512
    g = np.concatenate([g, np.zeros(n - g.size, F32)]).reshape(-1, 512)
    r = inputs.rng(5)
    for up in (np.ones_like(g), r.standard_normal(g.shape).astype(F32)):
        x = inputs.to_dtype(np.concatenate([g, up], axis=1), dtype)
        y = fp8sm.silu_mul_f32(x.to(cuda()))
        torch.cuda.synchronize()
        want = oq.silu_mul_f32(inputs.widen(x))
        got = y.cpu().numpy()
        bad = got.view(np.uint32) != want.view(np.uint32)
        assert not bad.any(), (g.reshape(-1)[bad.reshape(-1)][:8], got[bad][:8], want[bad][:8])


def test_fp16_tiny_groups_regression():
    # sglang PR #33533 Modifications 1: fp16 groups whose absmax is below
    # 448/65504 came out as +-448 (and zero rows as +448).  Here such groups
    # must match the oracle bit for bit in every scale format, and equal the
    # codes of the same values given as bf16 wherever both dtypes hold them.
    r = inputs.rng(6)
    x = (r.standard_normal((16, 1024)) * 6.8e-3 / 8).astype(F32)
    x[3] = 0
    x[7, :128] = 0
    x16 = inputs.to_dtype(x, torch.float16)
    xb = inputs.to_dtype(inputs.widen(x16), torch.bfloat16)
    same = inputs.widen(xb) == inputs.widen(x16)
    for fmt in (0, 1, 2):
        for group in (128, -1):
            _check(x16, group, fmt, 0, what="fp16 tiny")
            qa, _ = _gpu_quant(x16, group, fmt, 0)
            assert np.all(qa[3] == 0)
            assert np.mean((qa & 0x7F) == 0x7E) < 0.05
            rows = np.all(same, axis=1)
            qb, _ = _gpu_quant(xb, group, fmt, 0)
            assert np.array_equal(qa[rows], qb[rows])


def test_zero_rows_closed_form():
    x = torch.zeros((8, 256), dtype=torch.bfloat16)
    q, s = _gpu_quant(x, 128, 2, 0)
    assert np.all(q == 0) and np.all(s == 85)
    q, s = _gpu_quant(x, 128, 0, 0)
    assert np.all(q == 0) and np.all(s == F32(1e-10) / F32(448))


def test_static_quant():
    d = inputs.decode()
    for t, s in [(d.x, d.x_scale)] + [(d.w[n], d.w_scale[n]) for n in inputs.DECODE_NS]:
        sc = torch.tensor([s], dtype=torch.float32, device=cuda())
        q = fp8sm.quant_static(t.to(cuda()), sc)
        torch.cuda.synchronize()
        want = oq.quant_static(inputs.widen(t), F32(s))
        assert np.array_equal(q.cpu().numpy(), want)


def test_weight_block_quant_ragged():
    r = inputs.rng(7)
    w = inputs.to_dtype(r.standard_normal((300, 520), dtype=np.float32) * F32(0.02))
    q, s = fp8sm.quant_weight_block128(w.to(cuda()))
    torch.cuda.synchronize()
    qo, so = oq.quant_weight_block(inputs.widen(w))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_fused_workload_full_size(dtype):
    # gate|up [4096, 2 x 7168], SiLU-and-mul + 1x128 UE8M0 group quant
    f = inputs.fused()
    x = f.gu_bf16 if dtype == torch.bfloat16 else f.gu_fp16
    _check(x, 128, fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_ROW_MAJOR, fused=True, what="fused full")
    _check(x, 128, fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_MN_MAJOR, fused=True, what="fused full mn")


def test_qkv_activation_quant_full_size():
    w = inputs.workload("qkv")
    _check(w.x, -1, fp8sm.SCALE_FP32, fp8sm.LAYOUT_ROW_MAJOR, what="qkv per-token")


def test_per_token_quant_max_width():
    # the longest rows (K = 65536, two-pass kernel), fp32 and UE8M0 scales
    M, K = 3, 65536
    r = inputs.rng(65536)
    x = inputs.to_dtype(r.standard_normal((M, K), dtype=np.float32))
    for fmt, pow2 in ((fp8sm.SCALE_FP32, False), (fp8sm.SCALE_UE8M0_BYTE, True)):
        q, s = fp8sm.quant_group(x.to(cuda()), -1, fmt)
        torch.cuda.synchronize()
        ref = oq.quant_group(inputs.widen(x), K, pow2=pow2)
        assert np.array_equal(q.cpu().numpy(), ref.codes)
        want = ref.ue8m0_byte if pow2 else ref.scale
        assert np.array_equal(s.cpu().numpy().reshape(-1), want.reshape(-1))


def _boundary_rows(K, dtype):
    """Rows whose group maxima sit on the UE8M0 exponent boundary: exactly
    448 * 2^k and the next representable value of the input dtype below and
    above it (448 -+ 2 in bf16, 448 -+ 1/4 in fp16, times 2^k) for k across
    the dtype's normal range, plus a row below the 1e-10 absmax floor and a
    zero row.  The rest of each row is small noise, so the maximum decides
    the scale."""
    r = inputs.rng(11)
    u, ks = (2.0, range(-24, 25, 3)) if dtype == torch.bfloat16 else (0.25, range(-14, 8))
    rows = []
    for k in ks:
        for d in (-u, 0.0, u):
            v = (448.0 + d) * 2.0 ** k          # exact in fp64 and in the dtype
            row = r.standard_normal(K).astype(F32) * F32(v / 64)
            row[r.integers(0, K)] = F32(v) * (1 if r.random() < 0.5 else -1)
            rows.append(row)
    rows.append(np.full(K, 1e-12, dtype=F32))
    rows.append(np.zeros(K, dtype=F32))
    xt = inputs.to_dtype(np.stack(rows), dtype)
    # the planted maxima survive the conversion exactly
    got = np.abs(inputs.widen(xt)[:-2]).max(axis=1)
    want = np.array([(448.0 + d) * 2.0 ** k for k in ks for d in (-u, 0.0, u)])
    assert np.array_equal(got.astype(np.float64), want)
    return xt


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_ue8m0_exponent_boundary(dtype):
    # the kernels take e = ceil(log2 RN32(a/448)) from the bit fields of the
    # group maximum a, without a divide, and skip the clamp to +-448; these
    # rows put a on both sides of every carry the bit-field rule makes
    x = _boundary_rows(1024, dtype)
    _check(x, -1, fp8sm.SCALE_UE8M0_BYTE, 0, what="ue8m0 boundary per-token")
    _check(x, 128, fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_ROW_MAJOR, what="ue8m0 boundary g128")
    _check(x, 128, fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_MN_MAJOR, what="ue8m0 boundary g128 mn")
    _check(x, 128, fp8sm.SCALE_UE8M0_FP32, fp8sm.LAYOUT_ROW_MAJOR, what="ue8m0 fp32 value g128")

"""Pins of the batched / masked oracle (oracle/batched.py) against closed forms.

Every expected value below is written from the E4M3FN format and integer
arithmetic, not from the oracle: batch b's operands carry values that depend
on b, so reading another batch's slab, weight or scales changes the result."""
import numpy as np
import pytest

from oracle import batched as ob
from oracle import e4m3

F32 = np.float32
CODE_448 = 0x7E   # 0 1111 110: 1.75 * 2^8
CODE_256 = 0x78   # 0 1111 000: 2^8


def _enc(v):
    return e4m3.encode(np.atleast_1d(np.asarray(v, dtype=F32)))


def _grouped_case(B, M, N, K, per_batch_weight):
    # A[b, m]: (b+1) at k = 0, (m+1) at k = 1.  B[b', n]: (n+1) at k = 0,
    # 2 (b'+1) at k = 1 (or 2 when the weight is shared).
    A = np.zeros((B, M, K), np.uint8)
    for b in range(B):
        A[b, :, 0] = _enc(b + 1)
        A[b, :, 1] = _enc(np.arange(1, M + 1))
    if per_batch_weight:
        W = np.zeros((B, N, K), np.uint8)
        for b in range(B):
            W[b, :, 0] = _enc(np.arange(1, N + 1))
            W[b, :, 1] = _enc(2 * (b + 1))
    else:
        W = np.zeros((N, K), np.uint8)
        W[:, 0] = _enc(np.arange(1, N + 1))
        W[:, 1] = _enc(2)
    return A, W


def _grouped_expected(b, M, N, per_batch_weight):
    m = np.arange(M)[:, None]
    n = np.arange(N)[None, :]
    wk1 = 2 * (b + 1) if per_batch_weight else 2
    acc = (b + 1) * (n + 1) + (m + 1) * wk1
    return acc * 2.0 ** b * 2.0 ** -(n % 3)


@pytest.mark.parametrize("per_batch_weight", [False, True])
def test_grouped_rowwise_closed_form(per_batch_weight):
    B, M, N, K = 4, 5, 8, 32
    A, W = _grouped_case(B, M, N, K, per_batch_weight)
    sa = np.array([[2.0 ** b] * M for b in range(B)], F32)          # per row, per batch
    sb = np.array([[2.0 ** -(n % 3) for n in range(N)]] * B, F32)   # shared, repeated
    res = ob.scaled_mm_batched(A, W, sa, sb)
    for b in range(B):
        want = _grouped_expected(b, M, N, per_batch_weight)
        assert np.array_equal(res[b].out, want), b
    # per-batch scalar scales give the same values
    res2 = ob.scaled_mm_batched(A, W, np.array([2.0 ** b for b in range(B)], F32), sb)
    for b in range(B):
        assert np.array_equal(res2[b].out, res[b].out)


def test_row_counts_are_clamped_and_select_leading_rows():
    B, M, N, K = 4, 5, 8, 32
    A, W = _grouped_case(B, M, N, K, True)
    sa = np.array([2.0 ** b for b in range(B)], F32)
    sb = np.array([[2.0 ** -(n % 3) for n in range(N)]] * B, F32)
    rows = [3, 0, 99, -4]
    assert list(ob.valid_rows(rows, B, M)) == [3, 0, 5, 0]
    assert list(ob.valid_rows(None, B, M)) == [5] * 4
    res = ob.scaled_mm_batched(A, W, sa, sb, rows=rows)
    for b, mb in enumerate([3, 0, 5, 0]):
        assert res[b].bits.shape == (mb, N)
        assert np.array_equal(res[b].out, _grouped_expected(b, M, N, True)[:mb])
    with pytest.raises(ValueError):
        ob.valid_rows([1, 2], B, M)


def test_batch_permutation_equivariance():
    r = np.random.default_rng(5)
    B, M, N, K = 5, 7, 16, 64
    A = e4m3.encode((r.standard_normal((B, M, K)) * 3).astype(F32))
    W = e4m3.encode((r.standard_normal((B, N, K)) * 0.5).astype(F32))
    sa = r.uniform(0.5, 2, (B, M)).astype(F32)
    sb = r.uniform(0.5, 2, (B, N)).astype(F32)
    rows = np.array([7, 2, 0, 5, 3])
    p = np.array([3, 0, 4, 1, 2])
    res = ob.scaled_mm_batched(A, W, sa, sb, rows=rows)
    rp = ob.scaled_mm_batched(A[p], W[p], sa[p], sb[p], rows=rows[p])
    for i, b in enumerate(p):
        assert np.array_equal(rp[i].bits, res[b].bits)


def test_blockwise_grouped_closed_form():
    # A[b, m]: value (m+1) at k = 0 and 3 at k = 130 (second K block);
    # B[b, n]: 1 at k = 0 and (b+1) at k = 130.  Scales: a 2^-m in block 0 and
    # 2^b in block 1; weight block scales 2^(b+nb) / 2^-nb.
    B, M, N, K = 3, 4, 256, 256
    A = np.zeros((B, M, K), np.uint8)
    W = np.zeros((B, N, K), np.uint8)
    a_s = np.zeros((B, M, 2), F32)
    w_s = np.zeros((B, 2, 2), F32)
    for b in range(B):
        A[b, :, 0] = _enc(np.arange(1, M + 1))
        A[b, :, 130] = _enc(3)
        W[b, :, 0] = _enc(1)
        W[b, :, 130] = _enc(b + 1)
        a_s[b, :, 0] = 2.0 ** -np.arange(M)
        a_s[b, :, 1] = 2.0 ** b
        for nb in range(2):
            w_s[b, nb, 0] = 2.0 ** (b + nb)
            w_s[b, nb, 1] = 2.0 ** -nb
    res = ob.blockwise_mm_batched(A, a_s, W, w_s, rows=[4, 2, 9])
    for b, mb in enumerate([4, 2, 4]):
        m = np.arange(mb)[:, None]
        nb = (np.arange(N) // 128)[None, :]
        want = (m + 1) * 2.0 ** -m * 2.0 ** (b + nb) + 3 * (b + 1) * 2.0 ** b * 2.0 ** -nb
        assert np.array_equal(res[b].out, want), b


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("group", [128, 256])
def test_batched_quant_closed_form(pow2, group):
    # batch b is filled with +-2^j_b: a' = 2^j_b, so the fp32 scale is
    # 2^j_b * RN32(1/448) and every code is +-448; the UE8M0 exponent is
    # ceil(j_b - log2 448) = j_b - 8, every code +-256
    B, M, K = 4, 3, 256
    js = [-3, 0, 5, 11]
    x = np.empty((B, M, K), F32)
    for b, j in enumerate(js):
        x[b] = 2.0 ** j
        x[b, :, 1::2] *= -1
    out = ob.quant_group_batched(x, group, pow2=pow2, rows=[3, 1, 0, 7])
    for b, (j, mb) in enumerate(zip(js, [3, 1, 0, 3])):
        q = out[b]
        assert q.codes.shape == (mb, K)
        mag = CODE_256 if pow2 else CODE_448
        assert np.all(q.codes[:, 0::2] == mag) and np.all(q.codes[:, 1::2] == mag | 0x80)
        want = F32(2.0 ** (j - 8)) if pow2 else F32(2.0 ** j) * F32(1.0 / 448.0)
        assert q.scale.shape == (mb, K // group) and np.all(q.scale == want)
        if pow2:
            assert np.all(q.ue8m0_byte == j - 8 + 127)


def test_batched_fused_quant_closed_form():
    # gate 64: e^-64 vanishes next to 1 in fp32, so silu(64) = 64 exactly;
    # y = 64 * 2^j_b = 2^(j_b + 6)
    B, M, K = 3, 2, 128
    js = [-4, 1, 7]
    x = np.empty((B, M, 2 * K), F32)
    for b, j in enumerate(js):
        x[b, :, :K] = 64.0
        x[b, :, K:] = 2.0 ** j
    out = ob.quant_group_batched(x, 128, pow2=True, fused=True)
    for b, j in enumerate(js):
        assert np.all(out[b].codes == CODE_256)
        assert np.all(out[b].ue8m0_byte == j + 6 - 8 + 127)


def test_batched_static_quant_closed_form():
    B, M, K = 3, 2, 16
    x = np.empty((B, M, K), F32)
    for b in range(B):
        x[b] = 2.0 ** b
    q = ob.quant_static_batched(x, 2.0 ** -5)
    for b in range(B):
        # x / s = 2^(b+5) exactly: exponent field b + 5 + 7, mantissa 0
        assert np.all(q[b] == (b + 12) << 3)


def test_scales_must_be_per_batch():
    A = np.zeros((2, 3, 16), np.uint8)
    W = np.zeros((8, 16), np.uint8)
    with pytest.raises(ValueError):
        ob.scaled_mm_batched(A, W, np.ones(3, F32), np.ones((2, 8), F32))

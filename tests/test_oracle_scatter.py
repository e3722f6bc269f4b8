"""Pins of the scattered group quant oracle (oracle/scatter.py)."""
import numpy as np

from oracle import quant as oq, scatter as osc

F32 = np.float32
CODE_256 = 0x78   # 0 1111 000: 2^8


def _case(T=6, K=256, topk=3, R=24, seed=0):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((T, K)) * np.exp2(r.integers(-6, 6, (T, 1)))).astype(F32)
    dst = r.permutation(R)[:T * topk].reshape(T, topk).astype(np.int32)
    return x, dst


def test_scatter_equals_quantizing_the_replicated_rows():
    # replicate first (row d = x[t]), then the plain group quant: a different
    # order of the same steps through the independently pinned 2-D quant
    x, dst = _case()
    R = 24
    for pow2 in (False, True):
        codes, scale, byte, written = osc.quant_group_scatter(x, dst, R, pow2=pow2)
        rep = np.zeros((R, x.shape[1]), F32)
        for t in range(x.shape[0]):
            rep[dst[t]] = x[t]
        ref = oq.quant_group(rep, 128, pow2)
        assert np.array_equal(codes[written], ref.codes[written])
        assert np.array_equal(scale[written], ref.scale[written])
        if pow2:
            assert np.array_equal(byte[written], ref.ue8m0_byte[written])
        assert written.sum() == dst.size


def test_power_of_two_closed_form_per_token():
    # token t filled with +-2^j_t: UE8M0 exponent j_t - 8, every code +-256
    T, K, R = 4, 256, 16
    js = [-5, 0, 3, 9]
    x = np.empty((T, K), F32)
    for t, j in enumerate(js):
        x[t] = 2.0 ** j
        x[t, 1::2] *= -1
    dst = np.array([[3, 7], [0, 15], [8, -1], [16, 5]], np.int32)   # -1 and 16 name no row
    codes, scale, byte, written = osc.quant_group_scatter(x, dst, R)
    assert sorted(np.nonzero(written)[0]) == [0, 3, 5, 7, 8, 15]
    for t, j in enumerate(js):
        for d in dst[t]:
            if 0 <= d < R:
                assert np.all(codes[d, 0::2] == CODE_256) and np.all(codes[d, 1::2] == CODE_256 | 0x80)
                assert np.all(byte[d] == j - 8 + 127) and np.all(scale[d] == F32(2.0 ** (j - 8)))
    assert np.all(codes[~written] == 0)

"""Pins for oracle.quant: closed forms, invariants, torch's independent fp8
cast where the multiplier is a power of two, the exponential against decimal
arithmetic, and the facts PR #33533 states (tests/golden/)."""
import decimal

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import e4m3, quant

F32 = np.float32


def _torch_encode(y32):
    t = torch.from_numpy(np.asarray(y32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _all_bf16(max_abs=None):
    b = np.arange(65536, dtype=np.uint32) << 16
    v = b.view(np.float32)
    v = v[np.isfinite(v)]
    if max_abs is not None:
        v = v[np.abs(v) <= max_abs]
    return v


def _all_fp16():
    v = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    return v[np.isfinite(v)]


def _golden():
    return {k: v for k, v in read_golden("quant_closed_forms.txt")}


# ---------------------------------------------------------------- fp32 scales

def test_zero_group_closed_form_golden():
    g = _golden()
    x = np.zeros((3, 256), dtype=F32)
    r = quant.quant_group(x, 128)
    assert np.all(r.codes == int(g["zero_group_code"], 16))
    assert np.all(r.scale == F32(float(g["zero_group_scale_f32"])))
    r2 = quant.quant_group(x, 128, pow2=True)
    assert np.all(r2.ue8m0_byte == int(g["zero_group_ue8m0_byte"]))
    assert np.all(r2.codes == 0)
    # the multiplier of an all-zero group is the stated ceiling and is finite
    m = F32(448) / F32(float(g["amax_floor_f32"]))
    assert np.isfinite(m) and abs(float(m) / float(g["multiplier_ceiling"]) - 1) < 1e-6


def test_negative_zero_keeps_its_sign_bit():
    x = np.zeros((1, 128), dtype=F32)
    x[0, 1] = -0.0
    x[0, 2] = 1.0
    r = quant.quant_group(x, 128)
    assert r.codes[0, 0] == 0x00 and r.codes[0, 1] == 0x80


def test_every_bf16_value_with_unit_multiplier_matches_torch_cast():
    # A group whose maximum is exactly 448 has s = 1 and m = 1, so its codes
    # must be the plain fp32 -> E4M3FN conversion of its elements.
    v = _all_bf16(448.0)
    per = 127
    n = -(-v.size // per)
    pad = np.zeros(n * per - v.size, dtype=F32)
    body = np.concatenate([v, pad]).reshape(n, per)
    x = np.concatenate([np.full((n, 1), 448.0, dtype=F32), body], axis=1)
    r = quant.quant_group(x, 128)
    assert np.all(r.scale == 1.0)
    assert np.array_equal(r.codes[:, 1:].reshape(-1)[: v.size], _torch_encode(v))


@pytest.mark.parametrize("j", [-30, -7, -1, 1, 5, 20])
def test_power_of_two_maximum_gives_exact_scale_and_torch_codes(j):
    rng = np.random.Generator(np.random.PCG64(31))
    body = (rng.standard_normal((8, 127)) * 60).astype(F32)
    body = np.clip(body, -447, 447).astype(F32)
    x = np.concatenate([np.full((8, 1), 448.0, F32), body], axis=1)
    xs = (x * F32(2.0 ** j)).astype(F32)
    r = quant.quant_group(xs, 128)
    assert np.all(r.scale == F32(2.0 ** j))
    assert np.array_equal(r.codes, _torch_encode(x))
    ru = quant.quant_group(xs, 128, pow2=True)
    assert np.all(ru.ue8m0_byte == 127 + j)
    assert np.array_equal(ru.codes, r.codes)
    assert np.all(ru.codes[:, 0] == 0x7E)


def test_scale_invariance_under_power_of_two_scaling():
    rng = np.random.Generator(np.random.PCG64(32))
    x = rng.standard_normal((16, 512)).astype(F32)
    base = quant.quant_group(x, 128)
    baseu = quant.quant_group(x, 128, pow2=True)
    for j in (-20, -3, 4, 30):
        r = quant.quant_group((x * F32(2.0 ** j)).astype(F32), 128)
        assert np.array_equal(r.codes, base.codes)
        assert np.array_equal(r.scale, (base.scale * F32(2.0 ** j)).astype(F32))
        ru = quant.quant_group((x * F32(2.0 ** j)).astype(F32), 128, pow2=True)
        assert np.array_equal(ru.codes, baseu.codes)
        assert np.array_equal(ru.ue8m0_byte.astype(int), baseu.ue8m0_byte.astype(int) + j)


def test_negation_flips_only_the_sign_bit():
    rng = np.random.Generator(np.random.PCG64(33))
    x = rng.standard_normal((8, 384)).astype(F32)
    for pow2 in (False, True):
        a = quant.quant_group(x, 128, pow2)
        b = quant.quant_group(-x, 128, pow2)
        assert np.array_equal(a.scale, b.scale)
        assert np.array_equal(a.codes ^ 0x80, b.codes)


def test_groups_are_independent_and_permutation_equivariant():
    rng = np.random.Generator(np.random.PCG64(34))
    x = rng.standard_normal((4, 512)).astype(F32)
    r = quant.quant_group(x, 128)
    y = x.copy()
    y[:, 128:256] *= F32(37.0)             # only group 1 changes
    r2 = quant.quant_group(y, 128)
    keep = np.r_[0:128, 256:512]
    assert np.array_equal(r.codes[:, keep], r2.codes[:, keep])
    assert np.array_equal(r.scale[:, [0, 2, 3]], r2.scale[:, [0, 2, 3]])
    perm = rng.permutation(128)
    xp = x.copy()
    xp[:, 256:384] = x[:, 256:384][:, perm]
    rp = quant.quant_group(xp, 128)
    assert np.array_equal(rp.codes[:, 256:384], r.codes[:, 256:384][:, perm])


def test_multiplier_lands_products_on_the_tie_as_the_page_describes():
    # amax 8 -> m = 448/8 = 56 exactly, 3 * 56 = 168: a tie, rounds to 160.
    x = np.zeros((1, 128), F32)
    x[0, 0] = 8.0
    x[0, 1] = 3.0
    r = quant.quant_group(x, 128)
    assert r.codes[0, 0] == 0x7E and r.codes[0, 1] == 0x72
    # amax 3 -> m = RN32(448/3); 1.125 * m rounds to exactly 168.0 in fp32,
    # so the correctly rounded multiplier again gives the even code 0x72.
    x[0, 0] = 3.0
    x[0, 1] = 1.125
    r = quant.quant_group(x, 128)
    assert r.codes[0, 1] == 0x72
    # the same product with a multiplier one ulp high lands above the tie (176)
    m_hi = np.nextafter(F32(448) / F32(3), F32(np.inf))
    assert e4m3.encode(np.float32([F32(1.125) * m_hi]))[0] == 0x73


def test_one_ulp_high_multiplier_only_moves_codes_sitting_on_ties():
    # PR #33533 (Motivation): a multiplier one ulp too large changes a small
    # fraction of codes, all of them products that land on an E4M3 tie with the
    # correctly rounded multiplier.  Check that every code the oracle changes
    # under such a multiplier came from an exact midpoint (or from a product
    # within one fp32 ulp of one).
    rng = np.random.Generator(np.random.PCG64(35))
    x32 = rng.standard_normal((512, 4096), dtype=np.float32)
    x = torch.from_numpy(x32).to(torch.bfloat16).float().numpy()
    xg = x.reshape(512, 32, 128)
    a = np.maximum(np.abs(xg).max(axis=2), quant.AMAX_FLOOR).astype(F32)
    m = (F32(448) / a).astype(F32)
    m_hi = np.nextafter(m, F32(np.inf))
    c = quant.quant_group(x, 128).codes.reshape(512, 32, 128)
    p_hi = np.clip((xg * m_hi[:, :, None]).astype(F32), -448, 448)
    c_hi = e4m3.encode(p_hi)
    changed = c != c_hi
    assert 0 < changed.mean() < 0.01
    p = np.abs((xg * m[:, :, None]).astype(F32)[changed]).astype(np.float64)
    mags = e4m3.decode(np.arange(127, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    j = np.clip(np.searchsorted(mids, p), 0, mids.size - 1)
    near = np.minimum(np.abs(p - mids[j]), np.abs(p - mids[np.maximum(j - 1, 0)]))
    assert np.all(near <= np.spacing(p.astype(F32)).astype(np.float64))


def test_absmax_floor_is_a_max_not_an_addition():
    x = np.zeros((1, 128), F32)
    x[0, 0] = F32(1e-9)
    r = quant.quant_group(x, 128)
    assert r.scale[0, 0] == F32(F32(1e-9) / F32(448))
    assert r.codes[0, 0] == 0x7E


# ---------------------------------------------------------------- UE8M0

def test_ue8m0_rounds_the_exponent_up():
    # amax just above 448 * 2^j must give e = j + 1: the max element then lands
    # at ~224 (0x76), and nothing is clipped.
    for j in (-12, 0, 9):
        amax = F32(448.0 * 2.0 ** j * (1 + 2.0 ** -7))
        x = np.zeros((1, 128), F32)
        x[0, 0] = amax
        r = quant.quant_group(x, 128, pow2=True)
        assert r.ue8m0_byte[0, 0] == 128 + j
        assert r.codes[0, 0] == e4m3.encode(np.float32([amax / F32(2.0 ** (j + 1))]))[0]
        assert e4m3.decode(r.codes[0, 0]) <= 448


def test_ue8m0_exponent_matches_frexp_on_random_scales():
    rng = np.random.Generator(np.random.PCG64(36))
    s = np.exp2(rng.uniform(-100, 100, 20000)).astype(F32)
    s = np.concatenate([s, np.exp2(np.arange(-120, 120)).astype(F32)])
    e = quant.ue8m0_exponent(s)
    for v, ev in zip(s[::7], e[::7]):
        mant, ex = np.frexp(np.float64(v))  # v = mant * 2^ex, mant in [0.5, 1)
        want = ex - 1 if mant == 0.5 else ex
        assert ev == want


def test_fp16_tiny_groups_never_collapse_to_448():
    # PR #33533 Modifications 1: fp16 groups with absmax below 448/65504 used to
    # come out as +-448 everywhere and zero rows as +448.  The oracle scales in
    # fp32, so such groups quantize like any other: only the maximum sits at
    # the top of the range.
    g = _golden()
    thr = float(g["fp16_overflow_absmax_threshold"])
    rng = np.random.Generator(np.random.PCG64(37))
    x16 = (rng.standard_normal((8, 128)) * thr / 8).astype(np.float16)
    x16[3] = 0
    x = x16.astype(F32)
    assert np.abs(x).max() < thr
    for pow2 in (False, True):
        r = quant.quant_group(x, 128, pow2)
        mags = np.abs(e4m3.decode(r.codes))
        assert np.all(r.codes[3] == 0)
        assert np.mean(mags[[0, 1, 2, 4, 5, 6, 7]] >= 448) < 0.05
        # identical values given as bf16-widened floats give identical codes
        xb = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        same = xb == x
        rb = quant.quant_group(np.where(same, x, 0).astype(F32), 128, pow2)
        rows = np.all(same, axis=1)
        assert np.array_equal(rb.codes[rows], r.codes[rows])


# ---------------------------------------------------------------- exp / silu

def _cr_exp_f32(t):
    """Correctly rounded fp32 exp(t) via 40-digit decimal arithmetic."""
    if t > 100.0:
        return np.float32(np.inf)
    if t < -120.0:
        return np.float32(0.0)
    with decimal.localcontext() as ctx:
        ctx.prec = 40
        ex = decimal.Decimal(float(t)).exp()
        fmax = decimal.Decimal(float(np.finfo(np.float32).max))
        if ex >= fmax + decimal.Decimal(2) ** 103:   # max + half its ulp
            return np.float32(np.inf)
        c0 = np.float32(min(float(ex), float(np.finfo(np.float32).max)))
        cands = {c0, np.nextafter(c0, np.float32(np.inf)), np.nextafter(c0, np.float32(0))}
        cands = [c for c in cands if np.isfinite(c)]
        return min(cands, key=lambda c: abs(decimal.Decimal(float(c)) - ex))


@pytest.mark.parametrize("which", ["bf16", "fp16"])
def test_exp_is_correctly_rounded_for_every_gate_value(which):
    g = _all_bf16() if which == "bf16" else _all_fp16()
    t = (-g).astype(F32)
    ours = quant.exp_f32(t)
    ref = np.array([_cr_exp_f32(float(v)) for v in t], dtype=F32)
    bad = ~((ours == ref) | (np.isinf(ours) & np.isinf(ref)))
    assert not bad.any(), t[bad][:10]


def test_silu_special_values_and_gate_first_layout():
    g = np.float32([0.0, -0.0, 17.0, 30.0, 200.0, -90.0, -1e30, 1.0])
    s = quant.silu_f32(g)
    assert s[0] == 0 and not np.signbit(s[0])
    assert s[1] == 0 and np.signbit(s[1])
    assert s[2] == 17.0 and s[3] == 30.0 and s[4] == 200.0
    assert s[5] == 0 and np.signbit(s[5]) and s[6] == 0 and np.signbit(s[6])
    assert abs(s[7] - 1 / (1 + np.exp(-1.0))) < 1e-7
    gu = np.zeros((2, 4), F32)
    gu[0, :2] = [20.0, 0.0]    # gates
    gu[0, 2:] = [3.0, 5.0]     # ups
    y = quant.silu_mul_f32(gu)
    assert y[0, 0] == 60.0 and y[0, 1] == 0.0


def test_silu_within_three_roundings_of_float64_silu_for_every_bf16_gate():
    # three correctly rounded fp32 steps (exp, 1 + e, divide): the relative
    # error against the float64 silu is at most (1 + 2^-24)^3 - 1
    g = _all_bf16()
    g = g[np.abs(g) < 80]
    s = quant.silu_f32(g).astype(np.float64)
    g64 = g.astype(np.float64)
    ref = g64 / (1 + np.exp(-g64))
    ok = (np.abs(s - ref) <= 3.001 * 2.0 ** -24 * np.abs(ref)) | (np.abs(ref) < 1e-37)
    assert ok.all()


# ---------------------------------------------------------------- static / weights

def test_static_quant_unit_and_power_of_two_scale():
    rng = np.random.Generator(np.random.PCG64(38))
    x = (rng.standard_normal((4, 256)) * 100).astype(F32)
    c1 = quant.quant_static(x, 1.0)
    assert np.array_equal(c1, _torch_encode(np.clip(x, -448, 448)))
    c2 = quant.quant_static((x * F32(8)).astype(F32), 8.0)
    assert np.array_equal(c2, c1)


def test_weight_block_quant_matches_row_quant_on_single_row_blocks():
    rng = np.random.Generator(np.random.PCG64(39))
    w = np.zeros((128, 256), F32)
    w[0] = rng.standard_normal(256).astype(F32) * F32(0.02)
    codes, scales = quant.quant_weight_block(w)
    r = quant.quant_group(w[:1], 128)
    assert np.array_equal(codes[0], r.codes[0])
    assert np.array_equal(scales[0], r.scale[0])
    assert scales.shape == (1, 2)


# ------------------------------------------------------- 128 x 128 weight blocks
# Pins of the offline weight block quant that do not reuse its arithmetic:
# the hardware-independent torch cast where the multiplier is a power of two,
# the zero-block closed form, and invariants that catch a wrong block index,
# a transposed block or an edge block taking elements from outside itself.

def _blocks_with_power_of_two_maxima(nb, kb, js, rng, sign_flip=False):
    """[128 nb, 128 kb] array whose block (i, j) holds values in (-448, 448)
    times 2^js[i][j] with one element exactly +-448 * 2^js[i][j]."""
    w = np.clip(rng.standard_normal((128 * nb, 128 * kb)) * 80, -447, 447).astype(F32)
    base = w.copy()
    for i in range(nb):
        for j in range(kb):
            r, c = 128 * i + (7 * i + 3 * j) % 128, 128 * j + (11 * j + 5 * i) % 128
            base[r, c] = F32(-448.0 if (sign_flip and (i + j) % 2) else 448.0)
            w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] = \
                base[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] * F32(2.0 ** js[i][j])
    return w.astype(F32), base


def test_weight_block_unit_maximum_gives_torch_codes():
    rng = np.random.Generator(np.random.PCG64(40))
    w, base = _blocks_with_power_of_two_maxima(2, 3, [[0] * 3] * 2, rng, sign_flip=True)
    codes, scales = quant.quant_weight_block(w)
    assert np.all(scales == F32(1.0))
    assert np.array_equal(codes, _torch_encode(base))


def test_weight_block_power_of_two_maxima_give_exact_scales_per_block():
    # a different power of two in every block: a transposed or shifted block
    # index lands a wrong scale or wrongly scaled codes somewhere
    rng = np.random.Generator(np.random.PCG64(41))
    js = [[-9, 3, 0], [12, -20, 5]]
    w, base = _blocks_with_power_of_two_maxima(2, 3, js, rng)
    codes, scales = quant.quant_weight_block(w)
    assert np.array_equal(scales, np.array([[2.0 ** j for j in row] for row in js], F32))
    assert np.array_equal(codes, _torch_encode(base))


def test_weight_block_zero_block_closed_form():
    g = _golden()
    rng = np.random.Generator(np.random.PCG64(42))
    w = rng.standard_normal((256, 256)).astype(F32)
    w[128:, :128] = 0
    codes, scales = quant.quant_weight_block(w)
    assert scales[1, 0] == F32(float(g["zero_group_scale_f32"]))
    assert np.all(codes[128:, :128] == int(g["zero_group_code"], 16))


def test_weight_block_edges_equal_zero_padded_full_blocks():
    # a partial edge block takes its maximum from its own elements only: the
    # same values zero-padded to whole blocks (zeros never raise a maximum)
    # give the same scales and codes
    rng = np.random.Generator(np.random.PCG64(43))
    w = (rng.standard_normal((130, 200)) * 0.02).astype(F32)
    w[129, 150] = F32(5.0)                 # the largest value sits in edge block (1, 1)
    codes, scales = quant.quant_weight_block(w)
    pad = np.zeros((256, 256), F32)
    pad[:130, :200] = w
    cp, sp = quant.quant_weight_block(pad)
    assert scales.shape == (2, 2)
    assert np.array_equal(scales, sp)
    assert np.array_equal(codes, cp[:130, :200])
    assert scales[1, 1] > 20 * scales[0, 0]  # the planted maximum sets the edge block


def test_weight_block_blocks_are_independent_and_sign_symmetric():
    rng = np.random.Generator(np.random.PCG64(44))
    w = (rng.standard_normal((256, 384)) * 0.02).astype(F32)
    codes, scales = quant.quant_weight_block(w)
    y = w.copy()
    y[128:, 128:256] *= F32(1000.0)        # only block (1, 1) changes
    c2, s2 = quant.quant_weight_block(y)
    mask = np.ones((256, 384), bool)
    mask[128:, 128:256] = False
    assert np.array_equal(codes[mask], c2[mask])
    keep = np.ones((2, 3), bool)
    keep[1, 1] = False
    assert np.array_equal(scales[keep], s2[keep]) and s2[1, 1] != scales[1, 1]
    cn, sn = quant.quant_weight_block(-w)
    assert np.array_equal(sn, scales) and np.array_equal(cn, codes ^ 0x80)
    for j in (-12, 7):
        cj, sj = quant.quant_weight_block((w * F32(2.0 ** j)).astype(F32))
        assert np.array_equal(cj, codes)
        assert np.array_equal(sj, (scales * F32(2.0 ** j)).astype(F32))

"""Pins for oracle.gemm: exact int64 accumulation, exhaustive one-hot products,
closed-form integer sums, invariants and torch's float64 matmul."""
import numpy as np
import torch

from oracle import bf16, e4m3, gemm, quant

F32 = np.float32


def _rand_codes(rng, shape):
    c = e4m3.finite_codes()
    return c[rng.integers(0, c.size, shape)]


def _int_units(codes):
    """Each E4M3FN value times 2^9 is an integer; return it as int64."""
    v = e4m3.decode(codes) * 512.0
    iv = v.astype(np.int64)
    assert np.array_equal(iv.astype(np.float64), v)
    return iv


def test_accumulator_equals_exact_integer_sum():
    rng = np.random.Generator(np.random.PCG64(41))
    for (M, N, K) in [(37, 29, 300), (5, 7, 4096), (3, 2, 16384)]:
        a = _rand_codes(rng, (M, K))
        b = _rand_codes(rng, (N, K))
        acc = gemm.accumulate(a, b)
        exact = _int_units(a) @ _int_units(b).T          # units of 2^-18
        assert np.array_equal(acc * 2.0 ** 18, exact.astype(np.float64))
        assert np.array_equal((acc * 2.0 ** 18).astype(np.int64), exact)


def test_extreme_magnitudes_are_still_exact():
    # all-448 rows at K = 16384: the largest partial sums the configs can reach
    K = 16384
    a = np.full((2, K), 0x7E, np.uint8)
    b = np.full((3, K), 0x7E, np.uint8)
    b[1] = 0xFE
    b[2, ::2] = 0x01                                      # mix in 2^-9 values
    acc = gemm.accumulate(a, b)
    assert acc[0, 0] == 448.0 * 448.0 * K and acc[0, 1] == -448.0 * 448.0 * K
    assert acc[0, 2] == (K // 2) * 448.0 * 448.0 + (K // 2) * 448.0 * 2.0 ** -9


def test_one_hot_products_of_all_finite_codes_are_exact():
    c = e4m3.finite_codes()
    A = c[:, None].copy()            # [254, 1]
    B = c[:, None].copy()
    r = gemm.scaled_mm(A, B, 1.0, 1.0)
    prod = np.outer(e4m3.decode(c), e4m3.decode(c))       # exact in float64
    assert np.array_equal(r.out, prod)
    ref = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ref, prod)                       # exact in bf16 too
    # the one-hot may sit anywhere along K
    K = 300
    A2 = np.zeros((254, K), np.uint8)
    B2 = np.zeros((254, K), np.uint8)
    A2[:, 123] = c
    B2[:, 123] = c
    assert np.array_equal(gemm.scaled_mm(A2, B2, 1.0, 1.0).out, prod)


def test_small_integer_closed_forms():
    one = e4m3.encode(np.float32([1.0]))[0]
    two = e4m3.encode(np.float32([2.0]))[0]
    assert one == 0x38 and two == 0x40
    K = 200
    A = np.full((4, K), one, np.uint8)
    B = np.full((3, K), two, np.uint8)
    A[1, :100] = one | 0x80                               # row of +-1: sums to 0
    r = gemm.scaled_mm(A, B, np.float32([1, 1, 0.5, 3]), np.float32([1, 2, 0.25]))
    out = r.out
    assert out[0, 0] == 400 and out[0, 1] == 800 and out[0, 2] == 100
    assert out[1, 0] == 0 and not np.signbit(out[1, 0])
    assert out[2, 0] == 200 and out[3, 2] == 300


def test_zero_rows_give_positive_zero():
    rng = np.random.Generator(np.random.PCG64(42))
    A = _rand_codes(rng, (6, 256))
    B = _rand_codes(rng, (5, 256))
    A[2] = 0
    A[4] = 0x80
    r = gemm.scaled_mm(A, B, np.ones(6, F32), np.ones(5, F32))
    assert np.all(r.bits[2] == 0) and np.all(r.bits[4] == 0)


def test_power_of_two_scale_linearity_is_bitwise():
    rng = np.random.Generator(np.random.PCG64(43))
    A = _rand_codes(rng, (8, 512))
    B = _rand_codes(rng, (9, 512))
    sa = np.exp2(rng.uniform(-10, 0, 8)).astype(F32)
    sb = np.exp2(rng.uniform(-10, 0, 9)).astype(F32)
    base = gemm.scaled_mm(A, B, sa, sb).out
    for j in (-5, 3):
        r = gemm.scaled_mm(A, B, (sa * F32(2.0 ** j)).astype(F32), sb).out
        assert np.array_equal(r, base * 2.0 ** j)


def test_transposition_symmetry():
    rng = np.random.Generator(np.random.PCG64(44))
    A = _rand_codes(rng, (13, 640))
    B = _rand_codes(rng, (11, 640))
    sa = rng.uniform(0.001, 0.01, 13).astype(F32)
    sb = rng.uniform(0.001, 0.01, 11).astype(F32)
    r1 = gemm.scaled_mm(A, B, sa, sb)
    r2 = gemm.scaled_mm(B, A, sb, sa)
    assert np.array_equal(r1.bits, r2.bits.T)


def test_matches_torch_float64_matmul_and_bf16_cast():
    rng = np.random.Generator(np.random.PCG64(45))
    A = _rand_codes(rng, (33, 1000))
    B = _rand_codes(rng, (17, 1000))
    ta = torch.from_numpy(A).view(torch.float8_e4m3fn).double()
    tb = torch.from_numpy(B).view(torch.float8_e4m3fn).double()
    ref = (ta @ tb.T).numpy()
    r = gemm.scaled_mm(A, B, 1.0, 1.0)
    assert np.array_equal(r.acc, ref)
    # with unit scales every exact accumulator is a float64 whose bf16 rounding
    # torch computes directly when the value is also an fp32
    f32ok = ref.astype(F32).astype(np.float64) == ref
    tref = torch.from_numpy(ref[f32ok].astype(F32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(r.out[f32ok], tref)


def test_per_tensor_equals_rowwise_with_broadcast_scales():
    rng = np.random.Generator(np.random.PCG64(46))
    A = _rand_codes(rng, (9, 384))
    B = _rand_codes(rng, (7, 384))
    r1 = gemm.scaled_mm(A, B, F32(0.0123), F32(0.000456))
    r2 = gemm.scaled_mm(A, B, np.full(9, 0.0123, F32), np.full(7, 0.000456, F32))
    assert np.array_equal(r1.bits, r2.bits)


def test_blockwise_with_unit_scales_equals_rowwise():
    rng = np.random.Generator(np.random.PCG64(47))
    A = _rand_codes(rng, (10, 512))
    B = _rand_codes(rng, (260, 512))
    r1 = gemm.blockwise_mm(A, np.ones((10, 4), F32), B, np.ones((3, 4), F32))
    r2 = gemm.scaled_mm(A, B, 1.0, 1.0)
    assert np.array_equal(r1.bits, r2.bits)


def test_blockwise_block_scale_scales_exactly_its_own_block():
    rng = np.random.Generator(np.random.PCG64(48))
    A = _rand_codes(rng, (6, 384))
    B = _rand_codes(rng, (5, 384))
    A[:, :128] = 0
    A[:, 256:] = 0                                         # only block 1 is live
    ones_a = np.ones((6, 3), F32)
    ones_b = np.ones((1, 3), F32)
    base = gemm.blockwise_mm(A, ones_a, B, ones_b).out
    sa = ones_a.copy()
    sa[:, 1] = 2.0 ** -7
    sb = ones_b.copy()
    sb[0, 1] = 2.0 ** 3
    sb[0, 0] = 1000.0                                      # dead block: no effect
    r = gemm.blockwise_mm(A, sa, B, sb).out
    assert np.array_equal(r, base * 2.0 ** -4)


def test_blockwise_row_and_column_block_indexing():
    # a per-row UE8M0 scale on one k-block and a per-128-column weight scale
    # must land on exactly the outputs they belong to
    rng = np.random.Generator(np.random.PCG64(49))
    A = _rand_codes(rng, (4, 256))
    B = _rand_codes(rng, (256, 256))
    sa = np.ones((4, 2), F32)
    sb = np.ones((2, 2), F32)
    sa[2, 1] = 4.0
    sb[1, 0] = 0.5
    r = gemm.blockwise_mm(A, sa, B, sb).value
    P0 = gemm.accumulate(A[:, :128], B[:, :128])
    P1 = gemm.accumulate(A[:, 128:], B[:, 128:])
    want = P0 * np.where(np.arange(256) >= 128, 0.5, 1.0)[None, :] + P1 * np.array([1, 1, 4, 1.0])[:, None]
    assert np.array_equal(r, want)


def test_entries_equal_the_full_product_on_the_subgrid():
    rng = np.random.Generator(np.random.PCG64(50))
    A = _rand_codes(rng, (40, 256))
    B = _rand_codes(rng, (30, 256))
    sa = rng.uniform(0.001, 0.01, 40).astype(F32)
    sb = rng.uniform(0.001, 0.01, 30).astype(F32)
    full = gemm.scaled_mm(A, B, sa, sb).bits
    rows = np.array([0, 7, 39])
    cols = np.array([29, 3])
    sub = gemm.scaled_mm_entries(A, B, sa, sb, rows, cols).bits
    assert np.array_equal(sub, full[np.ix_(rows, cols)])


def test_rowwise_pipeline_from_bf16_inputs():
    # per-token activation quant + per-channel weight quant + GEMM on data whose
    # quantization is exact (powers of two and small integers), so the output
    # has a closed form
    x = np.zeros((2, 128), F32)
    x[0, :4] = [448, 224, 112, 56]
    x[1, :2] = [4, -2]
    w = np.zeros((3, 128), F32)
    w[0, :4] = [1, 1, 1, 1]
    w[1, :2] = [0.5, 0.5]
    w[2, 0] = 448
    qa = quant.quant_group(x, 128)
    qb = quant.quant_group(w, 128)
    r = gemm.scaled_mm(qa.codes, qb.codes, qa.scale.reshape(-1), qb.scale.reshape(-1))
    want = x.astype(np.float64) @ w.T.astype(np.float64)
    assert np.array_equal(r.out, bf16.round_to_bf16(want))


# ------------------------------------------------------------- bias / fp16 out

def test_bias_and_fp16_output_integer_closed_forms():
    # sums of +-1 * 2 products are small integers: acc * sa * sb + bias is an
    # exact small integer in both output dtypes
    one = e4m3.encode(np.float32([1.0]))[0]
    two = e4m3.encode(np.float32([2.0]))[0]
    K = 100
    A = np.full((2, K), one, np.uint8)
    A[1, :60] = one | 0x80                                # row 1: (40 - 60) * 2 = -40
    B = np.full((3, K), two, np.uint8)
    bias = np.array([3.0, -5.0, 0.5])
    # 200.5 needs 9 significant bits: a bf16 tie between 200 and 201 -> 200;
    # fp16 (11 bits) holds it
    want = {"bf16": [[203.0, 195.0, 200.0], [-37.0, -45.0, -39.5]],
            "fp16": [[203.0, 195.0, 200.5], [-37.0, -45.0, -39.5]]}
    for out in ("bf16", "fp16"):
        r = gemm.scaled_mm(A, B, 1.0, 1.0, bias=bias, out=out)
        assert r.dtype == out
        assert np.array_equal(r.out, np.array(want[out]))


def test_fp16_output_overflows_to_inf():
    big = e4m3.encode(np.float32([448.0]))[0]
    A = np.full((1, 16), big, np.uint8)
    B = np.full((2, 16), big, np.uint8)                   # 16 * 448^2 = 3.2e6
    r = gemm.scaled_mm(A, B, 1.0, np.float32([1.0, 2.0 ** -7]), out="fp16")
    assert np.isinf(r.out[0, 0]) and r.out[0, 0] > 0
    assert r.out[0, 1] == 25088.0                          # 3211264 / 128, exact in fp16


def test_zero_bias_is_no_bias_and_matches_torch_casts():
    rng = np.random.Generator(np.random.PCG64(61))
    A = _rand_codes(rng, (7, 96))
    B = _rand_codes(rng, (9, 96))
    sa = (rng.random(7) * 1e-2).astype(F32)
    sb = (rng.random(9) * 1e-2).astype(F32)
    base = gemm.scaled_mm(A, B, sa, sb)
    z = gemm.scaled_mm(A, B, sa, sb, bias=np.zeros(9))
    assert np.array_equal(base.bits, z.bits)
    # torch: float64 matmul of the decoded codes, scaled, plus bias, then the
    # library's float64 -> bf16 / fp16 conversions (via float32, where a double
    # rounding can differ: compare within one unit of the last place)
    bias = rng.standard_normal(9) * 4
    ta = torch.from_numpy(e4m3.decode(A))
    tb = torch.from_numpy(e4m3.decode(B))
    v = (ta @ tb.T) * torch.from_numpy(sa.astype(np.float64))[:, None] \
        * torch.from_numpy(sb.astype(np.float64))[None, :] + torch.from_numpy(bias)[None, :]
    for out, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        r = gemm.scaled_mm(A, B, sa, sb, bias=bias, out=out)
        ref = v.to(tdt).view(torch.int16).numpy().view(np.uint16).astype(np.int32)
        assert np.max(np.abs(r.bits.astype(np.int32) - ref)) <= 1


def test_ue8m0_values_follow_the_ieee_biased_exponent():
    # byte b in 1..254 is the biased exponent field of an fp32 power of two:
    # the float32 whose bit pattern is b << 23; byte 0 is 2^-127 (the fp32
    # subnormal with only bit 22 set), byte 255 is twice fp32's 2^127
    b = np.arange(256, dtype=np.uint8)
    v = gemm.ue8m0_values(b)
    assert v.dtype == np.float64
    ieee = (b[1:255].astype(np.uint32) << 23).view(np.float32).astype(np.float64)
    assert np.array_equal(v[1:255], ieee)
    assert v[0] == np.array([0x00400000], np.uint32).view(np.float32).astype(np.float64)[0]
    assert v[255] == 2.0 * np.array([254 << 23], np.uint32).view(np.float32).astype(np.float64)[0]
    assert v[127] == 1.0


def test_blockwise_extreme_ue8m0_scales_closed_forms():
    # one-hot products 1 x 1 in each of three K blocks with scales 2^128
    # (byte 255), 2^-127 (byte 0) and 1: out = sb * (2^128 + 2^-127 + 1) in
    # float64, rounded once to bf16; with sb = 2^-10, bf16(2^118 + ...) is
    # 2^118 (bits 245 << 7); a row with only the byte-0 block gives 2^-137,
    # below half the smallest bf16 subnormal 2^-133 (+0), and with sb = 1
    # 2^-127 = the subnormal 64 x 2^-133 (bits 0x0040); a row whose byte-255
    # block is the only live one overflows to +inf with sb = 1
    K = 384
    A = np.zeros((3, K), np.uint8)
    B = np.zeros((8, K), np.uint8)
    one = e4m3.encode(np.array([1.0], F32))[0]
    for kb in range(3):
        A[0, 128 * kb + 5] = one
        B[:, 128 * kb + 5] = one
    A[1, 128 * 1 + 5] = one
    A[2, 5] = one
    e = np.array([[255, 0, 127], [255, 0, 127], [255, 0, 127]], np.uint8)
    r = gemm.blockwise_mm(A, gemm.ue8m0_values(e), B, np.full((1, 3), 2.0 ** -10, F32))
    assert np.all(r.bits[0] == 245 << 7)
    assert np.all(r.bits[1] == 0)
    assert np.all(r.bits[2] == 245 << 7)
    r = gemm.blockwise_mm(A, gemm.ue8m0_values(e), B, np.ones((1, 3), F32))
    assert np.all(r.bits[1] == 0x0040)
    assert np.all(r.bits[2] == 0x7F80)                     # 2^128 > bf16 max: +inf

"""The quant kernels' UE8M0 exponent, taken from the bit fields of the group
absmax a without dividing, against the oracle's rule e = ceil(log2 RN32(a /
448)) ("[JIT] per_token_group_quant ...", Modifications 3: power-of-two
scales).  The kernels compute

    e = (((bits(a) + 0x1FFFFF) & 0xFF800000) >> 23) - 135

for every a >= 1e-10 (the absmax floor), which equals the rule because
RN32(a / 448) <= 2^k exactly when a <= 448 * 2^k.  This pins that identity on
every mantissa of the exponents around the floor, around 448 and at the top of
the range, and on the mantissas next to 1.75 (where the carry starts) for
every exponent a group can have; and it checks that the scaled values then
need no clamp: |a| * 2^-e <= 448.
"""
import numpy as np

from oracle import quant

F32 = np.float32


def kernel_exponent(a):
    bits = np.asarray(a, dtype=F32).view(np.uint32).astype(np.uint64)
    t = (bits + 0x1FFFFF) & 0xFF800000
    return (t >> 23).astype(np.int64) - 135


def oracle_exponent(a):
    s = (np.asarray(a, dtype=F32) / quant.Q_MAX).astype(F32)
    return quant.ue8m0_exponent(s).astype(np.int64)


def _values(biased, mant):
    bits = (np.uint32(biased) << np.uint32(23)) | np.asarray(mant, dtype=np.uint32)
    a = bits.view(F32)
    return a[a >= quant.AMAX_FLOOR]


def _check(a):
    e = kernel_exponent(a)
    assert np.array_equal(e, oracle_exponent(a))
    # the scaled group maximum stays within the E4M3FN range
    scaled = (a.astype(np.float64) * np.exp2(-e.astype(np.float64)))
    assert np.all(scaled <= 448.0)


def test_every_mantissa_of_selected_exponents():
    floor_exp = int((np.array([quant.AMAX_FLOOR], dtype=F32).view(np.uint32)[0] >> 23) & 0xFF)
    mant = np.arange(1 << 23, dtype=np.uint32)
    for biased in sorted({floor_exp, floor_exp + 1, 126, 127, 134, 135, 136, 200, 254}):
        _check(_values(biased, mant))


def test_mantissas_next_to_the_carry_for_every_exponent():
    floor_exp = int((np.array([quant.AMAX_FLOOR], dtype=F32).view(np.uint32)[0] >> 23) & 0xFF)
    mant = np.array([0, 1, 0x200000, 0x5FFFFF, 0x600000, 0x600001, 0x7FFFFE, 0x7FFFFF],
                    dtype=np.uint32)
    for biased in range(floor_exp, 255):
        _check(_values(biased, mant))


def test_floor_and_exact_powers():
    a = np.array([quant.AMAX_FLOOR, 448.0, 449.0, 447.0, 896.0, 1.0, 2.0 ** -20 * 448],
                 dtype=F32)
    _check(a)
    assert list(kernel_exponent(np.array([448.0, 449.0, 896.0], dtype=F32))) == [0, 1, 1]

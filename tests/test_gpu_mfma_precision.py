"""How gfx950's matrix instructions sum their products, and what that means
for the accuracy bound of the scaled FP8 GEMM.

The pages' GEMM accumulates E4M3FN products in fp32 ("Route large SM90
row/column-scaled FP8 GEMMs to Torch", Summary), and the accuracy bound
|gpu - oracle| <= 2^-7 |oracle| + 1e-3 sa sb sqrt(K) leaves outputs that nearly
cancel only an absolute error of ~0.07 code-product units at K = 5376.  These
tests measure, on crafted one-wavefront inputs through the fp8sm_mfma_probe
hook, whether a small product survives next to a large one inside one
instruction:

  * bf16 instructions (v_mfma_f32_16x16x32_bf16, v_mfma_f32_32x32x16_bf16):
    a product 2^-j next to a product 1 survives to fp32 precision;
  * fp8 instructions (v_mfma_f32_16x16x128_f8f6f4, v_mfma_f32_32x32x64_f8f6f4,
    v_mfma_f32_16x16x32_fp8_fp8): it is lost far earlier when the two products
    share a run of K, and kept when they do not;

and then run the rowwise GEMM on the fp8 instructions
(fp8sm_scaled_mm_fp8mfma) over the full QKV workload to count how many outputs
leave the bound, beside the bf16 path.  Layouts: operand element (row, k)
sits in lane row + R * (k // KL), register and byte / half within the lane as
given below; result element (i, j) of src0 row i and src1 row j sits where the
instructions' documented 16 x 16 / 32 x 32 output layouts put it (checked by
the exact small-integer test first).
"""
import time

import numpy as np
import pytest
import torch

from column_scaled_gemm_amd import fp8sm, inputs
from oracle import e4m3, quant as oq
from gpu_util import bf16_bits, cuda, full_tolerance_report, progress

pytestmark = pytest.mark.gpu
F32 = np.float32

# instr -> (rows R, instruction K, lane-group K width KL, bytes per element)
SHAPE = {
    fp8sm.MFMA_BF16_16x16x32: (16, 32, 8, 2),
    fp8sm.MFMA_BF16_32x32x16: (32, 16, 8, 2),
    fp8sm.MFMA_F8_16x16x128: (16, 128, 32, 1),
    fp8sm.MFMA_F8_32x32x64: (32, 64, 32, 1),
    fp8sm.MFMA_F8_16x16x32: (16, 32, 8, 1),
}
NAME = {0: "v_mfma_f32_16x16x32_bf16", 1: "v_mfma_f32_32x32x16_bf16",
        2: "v_mfma_f32_16x16x128_f8f6f4", 3: "v_mfma_f32_32x32x64_f8f6f4",
        4: "v_mfma_f32_16x16x32_fp8_fp8"}
BF16_INSTRS = (0, 1)
F8_INSTRS = (2, 3, 4)


def _bf16_bits_of(x):
    t = torch.from_numpy(np.asarray(x, dtype=F32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _regs(instr, elems):
    """Register images [64, 8] (int32) of an operand given as an element array
    [R, K]: bf16 bit patterns (uint16) or e4m3 codes (uint8)."""
    R, K, KL, nb = SHAPE[instr]
    img = np.zeros((64, 32), np.uint8)               # 32 bytes per lane
    raw = np.ascontiguousarray(elems).view(np.uint8).reshape(R, K * nb)
    for g in range(K // KL):
        img[g * R:(g + 1) * R, :KL * nb] = raw[:, g * KL * nb:(g + 1) * KL * nb]
    return torch.from_numpy(img.view(np.int32).copy()).to(cuda())


def _result(instr, d):
    """Result registers [64, 16] -> D [R, R], D[i, j] = sum_k X[i, k] Y[j, k]."""
    R = SHAPE[instr][0]
    d = d.cpu().numpy()
    out = np.zeros((R, R), np.float64)
    for i in range(R):
        for j in range(R):
            if R == 16:
                out[i, j] = d[j + 16 * (i // 4), i % 4]
            else:
                out[i, j] = d[j + 32 * ((i // 4) % 2), 4 * (i // 8) + i % 4]
    return out


def _run(instr, X, Y):
    """D = X Y^T through one instruction; X, Y [R, K] float values exactly
    representable in the operand format."""
    if instr in BF16_INSTRS:
        xa, ya = _bf16_bits_of(X), _bf16_bits_of(Y)
    else:
        xa, ya = e4m3.encode(np.asarray(X, F32)), e4m3.encode(np.asarray(Y, F32))
        assert np.array_equal(e4m3.decode(xa), np.asarray(X, np.float64))
        assert np.array_equal(e4m3.decode(ya), np.asarray(Y, np.float64))
    d = fp8sm.mfma_probe(instr, _regs(instr, xa), _regs(instr, ya))
    torch.cuda.synchronize()
    return _result(instr, d)


@pytest.mark.parametrize("instr", sorted(SHAPE))
def test_layouts_give_exact_small_integer_products(instr):
    # small integers: every product and partial sum is exact in any of the
    # instructions, so D must equal X Y^T exactly -- this pins the operand and
    # result layouts the precision tests below rely on
    R, K, _, _ = SHAPE[instr]
    r = inputs.rng(100 + instr)
    X = r.integers(-8, 9, (R, K)).astype(F32)
    Y = r.integers(-8, 9, (R, K)).astype(F32)
    D = _run(instr, X, Y)
    assert np.array_equal(D, X.astype(np.float64) @ Y.astype(np.float64).T), NAME[instr]


def _survival(instr, k_small):
    """Largest j (1..23) such that a product 2^-j at k = k_small survives next
    to a product 1 at k = 0 in output (0, 0): D[0, 0] == 1 + 2^-j exactly."""
    R, K, _, _ = SHAPE[instr]
    best = 0
    for j in range(1, 24):
        if instr in F8_INSTRS and j > 18:
            break                                  # 2^-9 * 2^-9 is the smallest e4m3 product
        X = np.zeros((R, K), F32)
        Y = np.zeros((R, K), F32)
        X[0, 0] = Y[0, 0] = 1.0
        ja = min(j, 9) if instr in F8_INSTRS else (j + 1) // 2
        X[0, k_small] = 2.0 ** -ja
        Y[0, k_small] = 2.0 ** -(j - ja)
        D = _run(instr, X, Y)
        if D[0, 0] == 1.0 + 2.0 ** -j:
            best = j
        else:
            break
    return best


def test_bf16_instructions_keep_small_products_to_fp32_precision():
    found = {}
    for instr in BF16_INSTRS:
        R, K, KL, _ = SHAPE[instr]
        for k_small in (1, 7, KL, K - 1):
            found[(instr, k_small)] = s = _survival(instr, k_small)
            progress(f"[mfma] {NAME[instr]}: 1 + 2^-j at k=0 and k={k_small}: exact up to j={s}")
    assert min(found.values()) >= 20, found


def test_fp8_instructions_truncate_small_products_within_a_run():
    # the same pair of products: next to each other in the first 8 codes of a
    # lane (one run of K), and further apart (other dwords of the lane, other
    # lane groups)
    found = {}
    for instr in F8_INSTRS:
        R, K, KL, _ = SHAPE[instr]
        near = {k: _survival(instr, k) for k in (1, 3, 7)}
        far = {k: _survival(instr, k) for k in sorted({8, 16, KL, K - 1})}
        found[instr] = (near, far)
        progress(f"[mfma] {NAME[instr]}: 1 + 2^-j exact up to j = {near} (k within the first "
                 f"8), {far} (k further apart)")
    for instr, (near, far) in found.items():
        assert max(near.values()) < 16, (NAME[instr], near)
        assert max(far.values()) >= 18, (NAME[instr], far)


def test_random_full_range_blocks_fp8_error_far_above_bf16():
    # random finite codes over the whole e4m3 range: error of each result
    # against the exact sum, relative to the largest product of that output
    r = inputs.rng(7)
    codes = e4m3.finite_codes()
    stats = {}
    for instr in sorted(SHAPE):
        R, K, _, _ = SHAPE[instr]
        worst = 0.0
        for trial in range(8):
            X = e4m3.decode(codes[r.integers(0, codes.size, (R, K))]).astype(F32)
            Y = e4m3.decode(codes[r.integers(0, codes.size, (R, K))]).astype(F32)
            D = _run(instr, X, Y)
            Xd, Yd = X.astype(np.float64), Y.astype(np.float64)
            exact = Xd @ Yd.T                       # exact: K <= 128 products on a 2^-18 grid
            pmax = np.max(np.abs(Xd[:, None, :] * Yd[None, :, :]), axis=2)
            worst = max(worst, float(np.max(np.abs(D - exact) / np.where(pmax > 0, pmax, 1))))
        stats[instr] = worst
        progress(f"[mfma] {NAME[instr]}: random full-range blocks, max |D - exact| / max "
                 f"product = 2^{np.log2(worst) if worst > 0 else -np.inf:.1f}")
    bf = max(stats[i] for i in BF16_INSTRS)
    assert bf <= 2.0 ** -20, bf
    for i in F8_INSTRS:
        assert stats[i] >= 16 * max(bf, 2.0 ** -30), (NAME[i], stats[i], bf)


def test_fp8_mfma_gemm_exact_where_sums_are_exact():
    # the evidence kernel itself is correct: with small-integer codes every
    # sum is exact in any instruction, so it equals the oracle bitwise
    from oracle import gemm as og
    vals = np.arange(-8, 9, dtype=F32)
    codes = e4m3.encode(vals)
    r = inputs.rng(21)
    for M, N, K in [(70, 264, 1024), (130, 520, 2064), (5, 24, 48)]:
        A = codes[r.integers(0, codes.size, (M, K))]
        B = codes[r.integers(0, codes.size, (N, K))]
        sa = np.exp2(r.integers(-4, 4, M)).astype(F32)
        sb = np.exp2(r.integers(-4, 4, N)).astype(F32)
        c = fp8sm.scaled_mm_fp8mfma(torch.from_numpy(A).to(cuda()), torch.from_numpy(B).to(cuda()),
                                    torch.from_numpy(sa).to(cuda()), torch.from_numpy(sb).to(cuda()),
                                    fp8sm.KIND_ROW, fp8sm.KIND_COL)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(c), og.scaled_mm(A, B, sa, sb).bits), (M, N, K)


def _time_gemm(fn, reps=10):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return float(np.median(ts))


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_fp8_mfma_gemm_on_the_full_qkv_workload_leaves_the_bound():
    # the whole QKV output computed both ways against the oracle: the bf16
    # path stays within the bound, the fp8-instruction path does not
    name = "qkv"
    M, N, K = inputs.ROWWISE_SHAPES[name]
    progress(f"[case] fp8-instruction GEMM vs bf16 path, full {name} {M}x{K}x{N}")
    w = inputs.workload(name)
    qa, sa = fp8sm.quant_group(w.x.to(cuda()), -1)
    qb, sb = fp8sm.quant_group(w.w.to(cuda()), -1)
    sa, sb = sa.reshape(-1), sb.reshape(-1)
    c8 = torch.empty((M, N), dtype=torch.bfloat16, device=cuda())
    c16 = torch.empty((M, N), dtype=torch.bfloat16, device=cuda())
    us8 = _time_gemm(lambda: fp8sm.scaled_mm_fp8mfma(qa, qb, sa, sb, fp8sm.KIND_ROW,
                                                     fp8sm.KIND_COL, c=c8))
    us16 = _time_gemm(lambda: fp8sm.scaled_mm(qa, qb, sa, sb, fp8sm.KIND_ROW, fp8sm.KIND_COL,
                                              c=c16))
    flop = 2.0 * M * N * K
    progress(f"[mfma] {name}: fp8-instruction GEMM {us8:.1f} us = {flop / us8 / 1e6:.0f} TFLOP/s; "
             f"bf16 path {us16:.1f} us = {flop / us16 / 1e6:.0f} TFLOP/s (median of 10)")
    ga, gb = qa.cpu().numpy(), qb.cpu().numpy()
    gsa, gsb = sa.cpu().numpy(), sb.cpu().numpy()
    b8, b16 = bf16_bits(c8), bf16_bits(c16)
    del c8, c16, qa, qb
    torch.cuda.empty_cache()
    oa = oq.quant_group(inputs.widen(w.x), K)
    assert np.array_equal(ga, oa.codes)
    del oa, w
    n, v16, mx16, at16 = full_tolerance_report(b16, ga, gb, gsa, gsb, K, f"{name} bf16 path")
    n, v8, mx8, at8 = full_tolerance_report(b8, ga, gb, gsa, gsb, K, f"{name} fp8 instructions")
    progress(f"[tol] {name} full output, bf16 path: violations={v16} max_err/tol={mx16:.4f}")
    progress(f"[tol] {name} full output, fp8 instructions: violations={v8} of {n} "
             f"({100.0 * v8 / n:.3f}%) max_err/tol={mx8:.2f} at {at8}")
    assert v16 == 0
    assert v8 > 0

"""The C-ABI library loads, exports every symbol include/fp8sm.h declares, and
rejects bad arguments on the host before touching a device (no compute calls:
these run without a GPU)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

LIB = os.path.join(ROOT, "column_scaled_gemm_amd", "libfp8sm.so")
HEADER = os.path.join(ROOT, "include", "fp8sm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfp8sm.so not built")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8sm_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported_and_bound():
    from column_scaled_gemm_amd import fp8sm
    lib = ctypes.CDLL(LIB)
    names = _declared()
    assert "fp8sm_scaled_mm" in names and "fp8sm_quant_group" in names
    for n in names:
        assert hasattr(lib, n), n
        assert n in fp8sm.SIGNATURES, f"binding lacks {n}"


def test_status_strings_and_scale_bytes():
    from column_scaled_gemm_amd import fp8sm
    assert fp8sm.status_str(0) == "ok"
    assert "alignment" in fp8sm.status_str(3)
    assert fp8sm.scale_bytes(fp8sm.SCALE_FP32, fp8sm.LAYOUT_ROW_MAJOR, 10, 512, 128) == 10 * 4 * 4
    assert fp8sm.scale_bytes(fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_ROW_MAJOR, 10, 512, 128) == 40
    assert fp8sm.scale_bytes(fp8sm.SCALE_UE8M0_BYTE, fp8sm.LAYOUT_MN_MAJOR, 10, 512, 128) == 12 * 4
    assert fp8sm.scale_bytes(fp8sm.SCALE_FP32, fp8sm.LAYOUT_ROW_MAJOR, 10, 512, 512) == 40
    assert fp8sm.scale_bytes(fp8sm.SCALE_FP32, fp8sm.LAYOUT_ROW_MAJOR, 10, 500, 128) == 0


def _mm(lib, **kw):
    a = dict(A=16, lda=512, B=16, ldb=512, C=16, ldc=256, M=64, N=256, K=512, ka=1, sa=16, kb=2,
             sb=16)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.fp8sm_scaled_mm(P(a["A"]), a["lda"], P(a["B"]), a["ldb"], P(a["C"]), a["ldc"],
                               a["M"], a["N"], a["K"], a["ka"], P(a["sa"]), a["kb"], P(a["sb"]),
                               P(0))


def test_scaled_mm_rejects_bad_arguments_before_any_launch():
    from column_scaled_gemm_amd import fp8sm
    lib = fp8sm.lib()
    E = {v: k for k, v in fp8sm.STATUS.items()}
    assert _mm(lib, K=100) == E["ERR_ALIGN"]                 # K % 16
    assert _mm(lib, lda=520) == E["ERR_ALIGN"]
    assert _mm(lib, N=250, ldc=256) == E["ERR_ALIGN"]         # N % 8
    assert _mm(lib, lda=256) == E["ERR_SHAPE"]                # lda < K
    assert _mm(lib, M=-1) == E["ERR_SHAPE"]
    assert _mm(lib, ka=2) == E["ERR_UNSUPPORTED"]             # COL is not an A kind
    assert _mm(lib, ka=3, kb=2) == E["ERR_UNSUPPORTED"]       # group A needs block B
    assert _mm(lib, ka=1, kb=5) == E["ERR_UNSUPPORTED"]
    assert _mm(lib, A=0) == E["ERR_NULL"]
    assert _mm(lib, C=0) == E["ERR_NULL"]
    assert _mm(lib, A=8) == E["ERR_ALIGN"]                    # 16-byte rule
    assert _mm(lib, K=1 << 17, lda=1 << 17, ldb=1 << 17) == E["ERR_RANGE"]
    # row strides beyond 2^24 bytes: 32-bit operand offsets over a 64-row panel
    assert _mm(lib, lda=(1 << 24) + 16) == E["ERR_RANGE"]
    assert _mm(lib, ldb=(1 << 24) + 16) == E["ERR_RANGE"]
    assert _mm(lib, M=0) == E["OK"]                           # empty: nothing launched
    assert _mm(lib, N=0, ldc=8) == E["OK"]


def _mm_ex(lib, bias=0, out=0, **kw):
    a = dict(A=16, lda=512, B=16, ldb=512, C=16, ldc=256, M=64, N=256, K=512, ka=1, sa=16, kb=2,
             sb=16)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.fp8sm_scaled_mm_ex(P(a["A"]), a["lda"], P(a["B"]), a["ldb"], P(a["C"]), a["ldc"],
                                  a["M"], a["N"], a["K"], a["ka"], P(a["sa"]), a["kb"],
                                  P(a["sb"]), P(bias), out, P(0))


def test_scaled_mm_ex_rejects_bad_epilogues_before_any_launch():
    from column_scaled_gemm_amd import fp8sm
    lib = fp8sm.lib()
    E = {v: k for k, v in fp8sm.STATUS.items()}
    assert _mm_ex(lib, out=2) == E["ERR_UNSUPPORTED"]                    # bf16 / fp16 only
    assert _mm_ex(lib, ka=3, kb=5, bias=16) == E["ERR_UNSUPPORTED"]      # blockwise: no bias
    assert _mm_ex(lib, ka=3, kb=5, out=1) == E["ERR_UNSUPPORTED"]        # blockwise: bf16 only
    assert _mm_ex(lib, bias=17) == E["ERR_ALIGN"]                        # 2-byte bias
    assert _mm_ex(lib, K=100, bias=16, out=1) == E["ERR_ALIGN"]          # the shared rules hold
    assert _mm_ex(lib, M=0, bias=16, out=1) == E["OK"]


def test_quant_group_rejects_bad_arguments():
    from column_scaled_gemm_amd import fp8sm
    lib = fp8sm.lib()
    E = {v: k for k, v in fp8sm.STATUS.items()}
    P = ctypes.c_void_p

    def q(**kw):
        a = dict(x=16, dt=0, M=4, K=256, ldx=256, group=128, flags=0, fmt=0, lay=0, q=16, ldq=256,
                 s=16)
        a.update(kw)
        return lib.fp8sm_quant_group(P(a["x"]), a["dt"], a["M"], a["K"], a["ldx"], a["group"],
                                     a["flags"], a["fmt"], a["lay"], P(a["q"]), a["ldq"],
                                     P(a["s"]), P(0))
    assert q(group=64) == E["ERR_SHAPE"]
    assert q(K=200, ldx=200, ldq=200) == E["ERR_SHAPE"]       # 200 % 128
    assert q(K=196, ldx=196, ldq=196, group=196) == E["ERR_ALIGN"]
    assert q(flags=1) == E["ERR_SHAPE"]                       # fused needs ld_x >= 2K
    assert q(dt=2) == E["ERR_UNSUPPORTED"]
    assert q(fmt=3) == E["ERR_UNSUPPORTED"]
    assert q(lay=2) == E["ERR_UNSUPPORTED"]
    assert q(flags=4) == E["ERR_UNSUPPORTED"]
    assert q(x=0) == E["ERR_NULL"]
    assert q(x=8) == E["ERR_ALIGN"]
    assert q(M=0) == E["OK"]


def test_batched_calls_reject_bad_batches_before_any_launch():
    from column_scaled_gemm_amd import fp8sm
    lib = fp8sm.lib()
    E = {v: k for k, v in fp8sm.STATUS.items()}
    P = ctypes.c_void_p

    def qb(**kw):
        a = dict(x=16, B=3, M=4, K=256, bsx=2048, ldx=256, rows=0, group=128, q=16, bsq=1024,
                 ldq=256, s=16)
        a.update(kw)
        return lib.fp8sm_quant_group_batched(P(a["x"]), 0, a["B"], a["M"], a["K"], a["bsx"],
                                             a["ldx"], P(a["rows"]), a["group"], 0, 0, 0,
                                             P(a["q"]), a["bsq"], a["ldq"], P(a["s"]), P(0))
    assert qb(B=-1) == E["ERR_SHAPE"]
    assert qb(B=65536) == E["ERR_RANGE"]
    assert qb(bsx=-8) == E["ERR_SHAPE"]
    assert qb(bsx=2052) == E["ERR_ALIGN"]                    # batch stride of x % 8
    assert qb(bsq=1020) == E["ERR_ALIGN"]
    assert qb(bsq=1016) == E["ERR_SHAPE"]                    # batches of q would overlap
    assert qb(rows=18) == E["ERR_ALIGN"]                     # int32 counts
    assert qb(B=0) == E["OK"] and qb(M=0) == E["OK"]
    assert qb(x=0) == E["ERR_NULL"]

    def sb(**kw):
        a = dict(x=16, B=2, M=4, K=64, bsx=256, ldx=64, s=16, q=16, bsq=256, ldq=64)
        a.update(kw)
        return lib.fp8sm_quant_static_batched(P(a["x"]), 0, a["B"], a["M"], a["K"], a["bsx"],
                                              a["ldx"], P(a["s"]), P(a["q"]), a["bsq"], a["ldq"],
                                              P(0))
    assert sb(bsq=248) == E["ERR_SHAPE"]
    assert sb(bsx=-8) == E["ERR_SHAPE"]
    assert sb(bsx=12) == E["ERR_ALIGN"]
    assert sb(B=70000) == E["ERR_RANGE"]
    assert sb(q=0) == E["ERR_NULL"]

    def mb(**kw):
        a = dict(B=4, rows=0, A=16, bsa=64 * 512, lda=512, Bp=16, bsb=0, ldb=512, C=16,
                 bsc=64 * 256, ldc=256, M=64, N=256, K=512, ka=1, sa=16, bssa=64, kb=2, sb=16,
                 bssb=0, bias=0, out=0)
        a.update(kw)
        return lib.fp8sm_scaled_mm_batched(a["B"], P(a["rows"]), P(a["A"]), a["bsa"], a["lda"],
                                           P(a["Bp"]), a["bsb"], a["ldb"], P(a["C"]), a["bsc"],
                                           a["ldc"], a["M"], a["N"], a["K"], a["ka"], P(a["sa"]),
                                           a["bssa"], a["kb"], P(a["sb"]), a["bssb"], P(a["bias"]),
                                           a["out"], P(0))
    assert mb(B=-2) == E["ERR_SHAPE"]
    assert mb(B=65536) == E["ERR_RANGE"]
    assert mb(bsa=8) == E["ERR_ALIGN"]                       # fp8 rows stay 16-byte aligned
    assert mb(bsb=24) == E["ERR_ALIGN"]
    assert mb(bsc=12) == E["ERR_ALIGN"]
    assert mb(bsc=64 * 256 - 8) == E["ERR_SHAPE"]            # C batches would overlap
    assert mb(bssa=-1) == E["ERR_SHAPE"]
    assert mb(rows=2) == E["ERR_ALIGN"]
    assert mb(ka=3, kb=5, out=1) == E["ERR_UNSUPPORTED"]     # blockwise: bf16 only
    assert mb(B=0) == E["OK"]
    assert mb(A=0) == E["ERR_NULL"]


def test_weight_preparation_rejects_bad_arguments():
    from column_scaled_gemm_amd import fp8sm
    lib = fp8sm.lib()
    E = {v: k for k, v in fp8sm.STATUS.items()}
    P = ctypes.c_void_p

    def rq(widths=(4, 4), N=8, K=32, ldw=32, ldq=32, w=16, q=32, s=16, m=16):
        arr = (ctypes.c_int64 * max(1, len(widths)))(*widths)
        return lib.fp8sm_requantize_max_scale(P(w), ldw, N, K, arr, len(widths), P(s), P(q), ldq,
                                              P(m), P(0))
    assert rq(widths=()) == E["ERR_RANGE"]
    assert rq(widths=(1,) * 17, N=17) == E["ERR_RANGE"]
    assert rq(widths=(4, 3)) == E["ERR_SHAPE"]                # sum != N
    assert rq(widths=(9, -1)) == E["ERR_SHAPE"]
    assert rq(K=24, ldw=32, ldq=32) == E["ERR_ALIGN"]          # K % 16
    assert rq(ldq=16) == E["ERR_SHAPE"]                       # ld < K
    assert rq(q=16, ldq=48) == E["ERR_SHAPE"]                 # in place needs ldq == ldw
    assert rq(s=0) == E["ERR_NULL"] and rq(w=0) == E["ERR_NULL"]
    assert rq(w=8) == E["ERR_ALIGN"]
    assert lib.fp8sm_requantize_max_scale(P(16), 32, 8, 32, None, 2, P(16), P(32), 32, P(16),
                                          P(0)) == E["ERR_NULL"]

    def cw(widths=(2, 3), s=16, o=16):
        arr = (ctypes.c_int64 * max(1, len(widths)))(*widths)
        return lib.fp8sm_scales_to_channelwise(P(s), arr, len(widths), P(o), P(0))
    assert cw(widths=()) == E["ERR_RANGE"]
    assert cw(widths=(2, -3)) == E["ERR_SHAPE"]
    assert cw(widths=(0, 0)) == E["OK"]
    assert cw(o=0) == E["ERR_NULL"]
    assert cw(o=2) == E["ERR_ALIGN"]


def test_scatter_quant_rejects_bad_arguments():
    from column_scaled_gemm_amd import fp8sm
    lib = fp8sm.lib()
    E = {v: k for k, v in fp8sm.STATUS.items()}
    P = ctypes.c_void_p

    def sc(x=16, T=4, K=256, ldx=256, dst=16, topk=2, R=8, fmt=2, lay=1, q=16, ldq=256, s=16):
        return lib.fp8sm_quant_group_scatter(P(x), 0, T, K, ldx, P(dst), topk, R, fmt, lay, P(q),
                                             ldq, P(s), P(0))
    assert sc(K=200, ldx=200, ldq=200) == E["ERR_SHAPE"]      # K % 128
    assert sc(topk=-1) == E["ERR_SHAPE"] and sc(topk=1025) == E["ERR_RANGE"]
    assert sc(ldq=128) == E["ERR_SHAPE"]
    assert sc(fmt=5) == E["ERR_UNSUPPORTED"] and sc(lay=3) == E["ERR_UNSUPPORTED"]
    assert sc(dst=0) == E["ERR_NULL"]
    assert sc(dst=2) == E["ERR_ALIGN"]
    assert sc(T=0) == E["OK"] and sc(topk=0) == E["OK"] and sc(R=0) == E["OK"]


def test_rate_probe_rejects_bad_arguments_before_any_launch():
    from column_scaled_gemm_amd import fp8sm
    lib = fp8sm.lib()
    E = {v: k for k, v in fp8sm.STATUS.items()}
    P = ctypes.c_void_p

    def rp(widen=0, blocks=4, wpb=4, iters=8, sink=16):
        return lib.fp8sm_rate_probe(widen, blocks, wpb, iters, P(sink), P(0))
    assert rp(widen=2) == E["ERR_UNSUPPORTED"] and rp(widen=-1) == E["ERR_UNSUPPORTED"]
    assert rp(wpb=2) == E["ERR_UNSUPPORTED"] and rp(wpb=32) == E["ERR_UNSUPPORTED"]
    assert rp(sink=0) == E["ERR_NULL"] and rp(sink=2) == E["ERR_ALIGN"]
    assert rp(blocks=0) == E["ERR_SHAPE"] and rp(iters=0) == E["ERR_SHAPE"]
    assert rp(blocks=65537) == E["ERR_RANGE"] and rp(iters=(1 << 24) + 1) == E["ERR_RANGE"]


def test_variant_names_and_forcing():
    from column_scaled_gemm_amd import fp8sm
    assert fp8sm.variant_count() >= 3
    names = [fp8sm.variant_name(i) for i in range(fp8sm.variant_count())]
    assert len(set(names)) == len(names)
    prev = fp8sm.force_variant(0)
    try:
        assert fp8sm.pick_variant(1, 4096, 4096) == 0
    finally:
        fp8sm.force_variant(prev)
    assert fp8sm.pick_variant(8320, 21504, 5376) == fp8sm.pick_variant(8320, 21504, 5376)


def test_variant_accepts_bounds_decode_variants_by_m():
    from column_scaled_gemm_amd import fp8sm
    names = {fp8sm.variant_name(v): v for v in range(fp8sm.variant_count())}
    for name, cap in (("decode32", 32), ("decode32w4", 32), ("decode16", 32), ("decode64", 64)):
        v = names[name]
        assert fp8sm.variant_accepts(v, cap, 4096, 65536)
        assert not fp8sm.variant_accepts(v, cap + 1, 4096, 4096)
    for name in ("tile128x256", "tile128x128", "tile256x128"):
        assert fp8sm.variant_accepts(names[name], 1 << 20, 16, 65536)
    assert not fp8sm.variant_accepts(-1, 1, 1, 16)
    assert not fp8sm.variant_accepts(fp8sm.variant_count(), 1, 1, 16)


def test_binding_rejects_views_with_a_strided_last_dimension():
    # the C ABI takes one row stride; a view whose elements are not contiguous
    # within a row must not reach it (checked before any call)
    import torch
    from column_scaled_gemm_amd import fp8sm
    x = torch.zeros(4, 512, dtype=torch.bfloat16)[:, ::2]
    codes = torch.zeros(8, 64, dtype=torch.uint8)
    for call in (lambda: fp8sm.quant_group(x, 128),
                 lambda: fp8sm.quant_static(x, torch.ones(1)),
                 lambda: fp8sm.scaled_mm(codes[:, ::2], codes[:, :32], torch.ones(1), torch.ones(1),
                                         fp8sm.KIND_TENSOR, fp8sm.KIND_TENSOR),
                 lambda: fp8sm.quant_group_batched(x[None], 128)):
        with pytest.raises(ValueError):
            call()


def test_binding_strides_of_empty_tensors_satisfy_the_layout_rules():
    # torch gives a zero-width matrix a row stride of 1; the binding passes the
    # smallest stride the ABI accepts for a tensor with no elements or a single
    # row (row length rounded up to 16), a zero batch stride for an empty
    # tensor, and the tensor's own strides otherwise
    import torch
    from column_scaled_gemm_amd import fp8sm
    assert torch.empty((64, 0)).stride(0) == 1
    assert fp8sm._ld(torch.empty((64, 0))) == 0
    assert fp8sm._ld(torch.empty((0, 512))) == 512
    assert fp8sm._ld(torch.empty((0, 500))) == 512
    assert fp8sm._ld(torch.empty((3, 64, 0))) == 0
    assert fp8sm._bs(torch.empty((3, 64, 0)), 3) == 0
    assert fp8sm._bs(torch.empty((3, 0, 512)), 3) == 0
    x = torch.empty((3, 10, 256))[:, 1:9, :128]
    assert fp8sm._ld(x) == 256 and fp8sm._bs(x, 3) == 2560 and fp8sm._bs(x, 1) == 0
    assert fp8sm._ld(torch.empty((5, 48))) == 48
    # one row: only row 0 is addressed, whatever torch reports as its stride
    col_t = torch.empty((512, 1)).T
    assert col_t.shape == (1, 512) and col_t.stride(0) == 1
    assert fp8sm._ld(col_t) == 512
    assert fp8sm._ld(torch.empty((4, 1, 100))) == 112


def test_binding_rejects_outputs_and_operands_too_small_before_any_call():
    # the C ABI cannot see buffer sizes: every caller-supplied tensor is checked
    # against what the call reads or writes (host tensors: a check that let a
    # call through would fail on the stream lookup, not with these errors)
    import torch
    from column_scaled_gemm_amd import fp8sm
    ROW, COL, U8, BF = fp8sm.KIND_ROW, fp8sm.KIND_COL, torch.uint8, torch.bfloat16
    x = torch.zeros(8, 256, dtype=BF)
    codes = torch.zeros(8, 256, dtype=U8)
    w = torch.zeros(16, 256, dtype=U8)

    def ones(n):
        return torch.ones(n)

    cases = [
        (ValueError, lambda: fp8sm.quant_group(x, 128, fuse_silu_mul=True, q=torch.zeros(8, 64, dtype=U8))),
        (ValueError, lambda: fp8sm.quant_group(x, 128, q=codes, scales=torch.zeros(8, 1))),
        (TypeError, lambda: fp8sm.quant_group(x, 128, fp8sm.SCALE_UE8M0_BYTE, q=codes,
                                              scales=torch.zeros(8, 2))),
        (TypeError, lambda: fp8sm.quant_group(x, 128, q=torch.zeros(8, 256, dtype=torch.int8))),
        (ValueError, lambda: fp8sm.quant_static(x, ones(1), q=codes[:4])),
        (ValueError, lambda: fp8sm.quant_weight_block128(x, scales=torch.zeros(1))),
        (ValueError, lambda: fp8sm.silu_mul_f32(x, y=torch.zeros(8, 64))),
        (ValueError, lambda: fp8sm.scaled_mm(codes, w, ones(8), ones(16), ROW, COL,
                                             c=torch.zeros(8, 8, dtype=BF))),
        (ValueError, lambda: fp8sm.scaled_mm(codes, w[:, :128], ones(8), ones(16), ROW, COL)),
        (ValueError, lambda: fp8sm.scaled_mm(codes, w, ones(4), ones(16), ROW, COL)),
        (ValueError, lambda: fp8sm.scaled_mm(codes, w, ones(8), ones(8), ROW, COL)),
        (TypeError, lambda: fp8sm.scaled_mm(codes, w, ones(8).double(), ones(16), ROW, COL)),
        (ValueError, lambda: fp8sm.scaled_mm(codes, w, ones(8), ones(16), ROW, COL, M=9)),
        (ValueError, lambda: fp8sm.scaled_mm(codes, w, torch.zeros(8, 1, dtype=U8), ones(2),
                                             fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_BLOCK128)),
        (ValueError, lambda: fp8sm.quant_group_batched(x[None], 128,
                                                       q=torch.zeros(1, 4, 256, dtype=U8))),
        (ValueError, lambda: fp8sm.quant_static_batched(x[None], ones(1),
                                                        q=torch.zeros(1, 8, 128, dtype=U8))),
        (ValueError, lambda: fp8sm.scaled_mm_batched(codes[None], w, ones(8), ones(16), ROW, COL,
                                                     c=torch.zeros(1, 8, 8, dtype=BF))),
        (ValueError, lambda: fp8sm.scaled_mm_batched(codes[None], w[:, :64], ones(8), ones(16),
                                                     ROW, COL)),
        (ValueError, lambda: fp8sm.scaled_mm_batched(codes[None], w, ones(8), ones(16), ROW, COL,
                                                     bias=torch.zeros(8, dtype=BF))),
        (ValueError, lambda: fp8sm.scaled_mm(codes, w, ones(8), ones(16), ROW, COL,
                                             bias=torch.zeros(8, dtype=BF))),
        (ValueError, lambda: fp8sm.requantize_max_scale(w, ones(1), [16],
                                                        q=torch.zeros(8, 256, dtype=U8))),
        (ValueError, lambda: fp8sm.requantize_max_scale(w, ones(1), [8, 8])),
        (ValueError, lambda: fp8sm.scales_to_channelwise(ones(2), [8, 8], out=torch.zeros(15))),
        (ValueError, lambda: fp8sm.quant_group_scatter(x, torch.zeros(8, 2, dtype=torch.int32), 16,
                                                       q=torch.zeros(8, 256, dtype=U8))),
    ]
    for i, (err, call) in enumerate(cases):
        with pytest.raises(err) as info:
            call()
        # the size / dtype check itself fired, not the later device check
        assert not isinstance(info.value, fp8sm.DeviceTensorError), i


def test_binding_refuses_host_tensors_before_any_call():
    # the kernels dereference every tensor address on the GPU: host tensors of
    # valid shapes are refused by the binding before the library is called
    import torch
    from column_scaled_gemm_amd import fp8sm
    ROW, COL, U8, BF = fp8sm.KIND_ROW, fp8sm.KIND_COL, torch.uint8, torch.bfloat16
    x = torch.zeros(8, 256, dtype=BF)
    codes = torch.zeros(8, 256, dtype=U8)
    w = torch.zeros(16, 256, dtype=U8)
    ones = torch.ones
    calls = [
        lambda: fp8sm.quant_group(x, 128),
        lambda: fp8sm.quant_group(x, -1, fuse_silu_mul=True),
        lambda: fp8sm.quant_static(x, ones(1)),
        lambda: fp8sm.quant_weight_block128(x),
        lambda: fp8sm.silu_mul_f32(x),
        lambda: fp8sm.scaled_mm(codes, w, ones(8), ones(16), ROW, COL),
        lambda: fp8sm.scaled_mm(codes, w, ones(8), ones(16), ROW, COL,
                                bias=torch.zeros(16, dtype=BF)),
        lambda: fp8sm.scaled_mm_fp8mfma(codes, w, ones(8), ones(16), ROW, COL),
        lambda: fp8sm.quant_group_batched(x[None], 128),
        lambda: fp8sm.quant_static_batched(x[None], ones(1)),
        lambda: fp8sm.scaled_mm_batched(codes[None], w, ones(8), ones(16), ROW, COL),
        lambda: fp8sm.requantize_max_scale(w, ones(1), [16]),
        lambda: fp8sm.scales_to_channelwise(ones(2), [8, 8]),
        lambda: fp8sm.quant_group_scatter(x, torch.zeros(8, 2, dtype=torch.int32), 16),
        lambda: fp8sm.mfma_probe(0, torch.zeros(64, 8, dtype=torch.int32),
                                 torch.zeros(64, 8, dtype=torch.int32)),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(fp8sm.DeviceTensorError):
            call()

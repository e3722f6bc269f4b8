"""Thin ctypes binding of libfp8sm.so (the C ABI declared in include/fp8sm.h).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch device tensors (torch provides device memory and the
current stream); outputs are either passed in or allocated here with
torch.empty.  The library is loaded on first use; if it is missing or fails to
load, every call raises -- there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8sm.so")

OK = 0
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_ALIGN", 4: "ERR_UNSUPPORTED",
          5: "ERR_LAUNCH", 6: "ERR_DEVICE", 7: "ERR_RANGE"}

BF16, FP16 = 0, 1
SCALE_FP32, SCALE_UE8M0_FP32, SCALE_UE8M0_BYTE = 0, 1, 2
LAYOUT_ROW_MAJOR, LAYOUT_MN_MAJOR = 0, 1
KIND_TENSOR, KIND_ROW, KIND_COL = 0, 1, 2
KIND_GROUP128_UE8M0, KIND_GROUP128_FP32, KIND_BLOCK128 = 3, 4, 5
FUSE_SILU_MUL = 1

# Every symbol include/fp8sm.h declares, with (restype, argtypes).
_i64, _i32, _u32, _p = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p
_int = ctypes.c_int
SIGNATURES = {
    "fp8sm_quant_group": (_int, [_p, _int, _i64, _i64, _i64, _i32, _u32, _int, _int, _p, _i64, _p, _p]),
    "fp8sm_quant_static": (_int, [_p, _int, _i64, _i64, _i64, _p, _p, _i64, _p]),
    "fp8sm_quant_weight_block128": (_int, [_p, _int, _i64, _i64, _i64, _p, _i64, _p, _p]),
    "fp8sm_scaled_mm": (_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _int, _p, _int, _p, _p]),
    "fp8sm_scaled_mm_ex": (_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _int, _p, _int, _p,
                                  _p, _int, _p]),
    "fp8sm_silu_mul_f32": (_int, [_p, _int, _i64, _i64, _i64, _p, _i64, _p]),
    "fp8sm_quant_group_scatter": (_int, [_p, _int, _i64, _i64, _i64, _p, _i32, _i64, _int, _int, _p,
                                         _i64, _p, _p]),
    "fp8sm_requantize_max_scale": (_int, [_p, _i64, _i64, _i64, _p, _i32, _p, _p, _i64, _p, _p]),
    "fp8sm_scales_to_channelwise": (_int, [_p, _p, _i32, _p, _p]),
    "fp8sm_quant_group_batched": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i64, _p, _i32, _u32,
                                         _int, _int, _p, _i64, _i64, _p, _p]),
    "fp8sm_quant_static_batched": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i64, _p, _p, _i64,
                                          _i64, _p]),
    "fp8sm_scaled_mm_batched": (_int, [_i64, _p, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                       _i64, _i64, _i64, _int, _p, _i64, _int, _p, _i64, _p, _int,
                                       _p]),
    "fp8sm_scale_bytes": (ctypes.c_size_t, [_int, _int, _i64, _i64, _i32]),
    "fp8sm_status_str": (ctypes.c_char_p, [_int]),
    "fp8sm_force_variant": (_int, [_int]),
    "fp8sm_variant_count": (_int, []),
    "fp8sm_variant_name": (ctypes.c_char_p, [_int]),
    "fp8sm_pick_variant": (_int, [_i64, _i64, _i64]),
    "fp8sm_variant_accepts": (_int, [_int, _i64, _i64, _i64]),
    "fp8sm_scaled_mm_fp8mfma": (_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _int, _p,
                                       _int, _p, _p]),
    "fp8sm_mfma_probe": (_int, [_i32, _p, _p, _p, _p]),
    "fp8sm_rate_probe": (_int, [_i32, _i32, _i32, _i32, _p, _p]),
}

_lib = None


class DeviceTensorError(ValueError):
    """A tensor argument is not on the current GPU (raised before any call)."""


class Fp8smError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _load().fp8sm_status_str(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "python -m column_scaled_gemm_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def lib():
    return _load()


def _check(status, where):
    if status != OK:
        raise Fp8smError(status, where)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    """Device address of a tensor argument (NULL for None).  The kernels
    dereference every such address on the GPU, so a host tensor, or one on
    another device than the current one, is refused here, before the library
    is called."""
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise DeviceTensorError("tensor arguments must be device (cuda) tensors; got one on "
                                f"{t.device}")
    if t.device.index != torch.cuda.current_device():
        raise DeviceTensorError(f"tensor on {t.device}, but the current device is "
                                f"cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return FP16
    raise TypeError("activations must be bfloat16 or float16")


# ---------------------------------------------------------------- raw calls

def scale_bytes(fmt, layout, M, K_out, group):
    return _load().fp8sm_scale_bytes(fmt, layout, M, K_out, group)


def status_str(status):
    return _load().fp8sm_status_str(status).decode()


def force_variant(vid):
    return _load().fp8sm_force_variant(vid)


def variant_count():
    return _load().fp8sm_variant_count()


def variant_name(vid):
    return _load().fp8sm_variant_name(vid).decode()


def pick_variant(M, N, K):
    return _load().fp8sm_pick_variant(M, N, K)


def variant_accepts(vid, M, N, K):
    """Whether kernel variant vid computes an M x N x K rowwise call."""
    return bool(_load().fp8sm_variant_accepts(vid, M, N, K))


# ---------------------------------------------------------------- tensor calls

def scale_shape(fmt, layout, M, K_out, group):
    G = K_out // group
    rows = ((M + 3) // 4) * 4 if layout == LAYOUT_MN_MAJOR else M
    return (G, rows) if layout == LAYOUT_MN_MAJOR else (M, G)


def quant_group(x, group, fmt=SCALE_FP32, layout=LAYOUT_ROW_MAJOR, fuse_silu_mul=False,
                q=None, scales=None, stream=None):
    """x [M, K_in] bf16/fp16 (K_in = 2*K_out when fused) -> (codes uint8 [M, K_out], scales)."""
    M, K_in = x.shape
    _unit_last(x, "x")
    K_out = K_in // 2 if fuse_silu_mul else K_in
    if group == -1:
        group = K_out
    if q is None:
        q = torch.empty((M, K_out), dtype=torch.uint8, device=x.device)
    else:
        _unit_last(q, "q")
        _holds(q, (M, K_out), "q", torch.uint8)
    if scales is None:
        scales = torch.empty(scale_shape(fmt, layout, M, K_out, group), dtype=_scale_dtype(fmt),
                             device=x.device)
    else:
        _holds_bytes(scales, scale_bytes(fmt, layout, M, K_out, group), "scales",
                     _scale_dtype(fmt))
    st = _load().fp8sm_quant_group(_ptr(x), _dtype_code(x), M, K_out, _ld(x), group,
                                   FUSE_SILU_MUL if fuse_silu_mul else 0, fmt, layout,
                                   _ptr(q), _ld(q), _ptr(scales), _stream(stream))
    _check(st, "fp8sm_quant_group")
    return q, scales


def quant_static(x, scale, q=None, stream=None):
    """x [M, K] bf16/fp16, scale: 1-element fp32 device tensor -> codes [M, K]."""
    M, K = x.shape
    _unit_last(x, "x")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    else:
        _unit_last(q, "q")
        _holds(q, (M, K), "q", torch.uint8)
    _holds_bytes(scale, 4, "scale", torch.float32)
    st = _load().fp8sm_quant_static(_ptr(x), _dtype_code(x), M, K, _ld(x), _ptr(scale),
                                    _ptr(q), _ld(q), _stream(stream))
    _check(st, "fp8sm_quant_static")
    return q


def quant_weight_block128(w, q=None, scales=None, stream=None):
    N, K = w.shape
    _unit_last(w, "w")
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    else:
        _unit_last(q, "q")
        _holds(q, (N, K), "q", torch.uint8)
    if scales is None:
        scales = torch.empty(((N + 127) // 128, (K + 127) // 128), dtype=torch.float32,
                             device=w.device)
    else:
        _holds_bytes(scales, 4 * ((N + 127) // 128) * ((K + 127) // 128), "scales",
                     torch.float32)
    st = _load().fp8sm_quant_weight_block128(_ptr(w), _dtype_code(w), N, K, _ld(w), _ptr(q),
                                             _ld(q), _ptr(scales), _stream(stream))
    _check(st, "fp8sm_quant_weight_block128")
    return q, scales


def silu_mul_f32(x, y=None, stream=None):
    """x [M, 2K] bf16/fp16 [gate | up] -> y [M, K] fp32 = silu(gate) * up."""
    M, K2 = x.shape
    _unit_last(x, "x")
    K = K2 // 2
    if y is None:
        y = torch.empty((M, K), dtype=torch.float32, device=x.device)
    else:
        _unit_last(y, "y")
        _holds(y, (M, K), "y", torch.float32)
    st = _load().fp8sm_silu_mul_f32(_ptr(x), _dtype_code(x), M, K, _ld(x), _ptr(y),
                                    _ld(y), _stream(stream))
    _check(st, "fp8sm_silu_mul_f32")
    return y


def scaled_mm(a, b, sa, sb, kind_a, kind_b, c=None, M=None, stream=None, bias=None,
              out_dtype=None):
    """a [M, K] uint8, b [N, K] uint8 (E4M3FN codes) -> c [M, N] bf16, or
    fp16 with out_dtype=torch.float16; bias: optional [N] of the output dtype
    (fp8sm_scaled_mm_ex)."""
    Mx, K = a.shape
    M = Mx if M is None else M
    N = b.shape[0]
    _unit_last(a, "a")
    _unit_last(b, "b")
    if out_dtype is None:
        out_dtype = c.dtype if c is not None else torch.bfloat16
    if a.dtype != torch.uint8 or b.dtype != torch.uint8:
        raise TypeError("a and b must be uint8 E4M3FN codes")
    if M > Mx or b.dim() != 2 or b.shape[1] < K:
        raise ValueError(f"a [{Mx}, {K}] / b {tuple(b.shape)} do not hold an M={M}, K={K} product")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=b.device)
    else:
        _unit_last(c, "c")
        _holds(c, (M, N), "c")
    _holds_scale(sa, kind_a, M, N, K, "sa")
    _holds_scale(sb, kind_b, M, N, K, "sb")
    if bias is not None:
        _holds_bytes(bias, 2 * N, "bias")
    if bias is None and out_dtype == torch.bfloat16:
        st = _load().fp8sm_scaled_mm(_ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(c),
                                     _ld(c), M, N, K, kind_a, _ptr(sa), kind_b, _ptr(sb),
                                     _stream(stream))
        _check(st, "fp8sm_scaled_mm")
        return c
    out = {torch.bfloat16: BF16, torch.float16: FP16}[out_dtype]
    if c.dtype != out_dtype or (bias is not None and bias.dtype != out_dtype):
        raise TypeError("fp8sm_scaled_mm_ex: c and bias must have the output dtype")
    st = _load().fp8sm_scaled_mm_ex(_ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(c), _ld(c),
                                    M, N, K, kind_a, _ptr(sa), kind_b, _ptr(sb),
                                    None if bias is None else _ptr(bias), out, _stream(stream))
    _check(st, "fp8sm_scaled_mm_ex")
    return c


def scaled_mm_fp8mfma(a, b, sa, sb, kind_a, kind_b, c=None, stream=None):
    """Test hook fp8sm_scaled_mm_fp8mfma: the rowwise GEMM on the fp8 matrix
    instructions (inexact; evidence for the bf16 path, never dispatched)."""
    M, K = a.shape
    N = b.shape[0]
    _unit_last(a, "a")
    _unit_last(b, "b")
    if a.dtype != torch.uint8 or b.dtype != torch.uint8:
        raise TypeError("a and b must be uint8 E4M3FN codes")
    if b.dim() != 2 or b.shape[1] < K:
        raise ValueError(f"b {tuple(b.shape)} does not hold an N x {K} operand")
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=b.device)
    else:
        _unit_last(c, "c")
        _holds(c, (M, N), "c", torch.bfloat16)
    _holds_scale(sa, kind_a, M, N, K, "sa")
    _holds_scale(sb, kind_b, M, N, K, "sb")
    st = _load().fp8sm_scaled_mm_fp8mfma(_ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(c), _ld(c),
                                         M, N, K, kind_a, _ptr(sa), kind_b, _ptr(sb),
                                         _stream(stream))
    _check(st, "fp8sm_scaled_mm_fp8mfma")
    return c


MFMA_BF16_16x16x32, MFMA_BF16_32x32x16 = 0, 1
MFMA_F8_16x16x128, MFMA_F8_32x32x64, MFMA_F8_16x16x32 = 2, 3, 4


def mfma_probe(instr, a_regs, b_regs, stream=None):
    """Test hook fp8sm_mfma_probe: a_regs, b_regs device uint32-compatible
    [64, 8] register images (int32 tensors) -> device float32 [64, 16] result
    registers of one matrix instruction with a zero accumulator."""
    for t, what in ((a_regs, "a_regs"), (b_regs, "b_regs")):
        if t.dtype != torch.int32 or tuple(t.shape) != (64, 8) or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous int32 [64, 8] tensor")
    d = torch.zeros((64, 16), dtype=torch.float32, device=a_regs.device)
    st = _load().fp8sm_mfma_probe(instr, _ptr(a_regs), _ptr(b_regs), _ptr(d), _stream(stream))
    _check(st, "fp8sm_mfma_probe")
    return d


def rate_probe(widen, blocks, waves_per_block, iters, stream=None):
    """Test hook fp8sm_rate_probe: launches the matrix-pipe throughput kernel
    on the current device and returns its sink tensor (the caller times the
    launch; 2*32*32*16*4*iters flops per wavefront)."""
    dev = torch.device("cuda", torch.cuda.current_device())
    sink = torch.empty(blocks * 64 * waves_per_block, dtype=torch.float32, device=dev)
    st = _load().fp8sm_rate_probe(widen, blocks, waves_per_block, iters, _ptr(sink),
                                  _stream(stream))
    _check(st, "fp8sm_rate_probe")
    return sink


# ---------------------------------------------------------------- batched calls

def _rows_arg(rows, B):
    """Device int32 [B] live-row counts, or None."""
    if rows is None:
        return None
    if rows.dtype != torch.int32 or rows.dim() != 1 or rows.numel() != B or not rows.is_cuda:
        raise ValueError("rows must be a device int32 tensor with one count per batch")
    return rows


def _unit_last(t, what):
    if t.stride(-1) != 1:
        raise ValueError(f"{what}: the last dimension must be contiguous")


def _ld(t):
    """Row stride in elements of a matrix (or of a batch's rows).  With no
    elements, or one row per batch, the stride addresses nothing beyond row 0,
    and torch may report any value for it (1 for a zero-width matrix or a
    transposed column): pass the smallest row stride the layout rules accept
    instead, the row length rounded up to 16."""
    if t.numel() == 0 or t.shape[-2] == 1:
        return -(-t.shape[-1] // 16) * 16
    return t.stride(-2)


def _bs(t, B):
    """Batch stride in elements of a 3-D operand: 0 for one batch or for a
    tensor with no elements (which addresses no memory)."""
    return t.stride(0) if B > 1 and t.numel() else 0


def _holds(t, shape, what, dtype=None):
    """The C ABI cannot see buffer sizes: a tensor the caller supplies must
    span at least `shape` (dimension by dimension) and have the dtype the
    call reads or writes, checked here before any call."""
    sh = t.shape
    ok = len(sh) == len(shape)
    if ok:
        for have, need in zip(sh, shape):
            if have < need:
                ok = False
                break
    if not ok:
        raise ValueError(f"{what}: needs shape {tuple(shape)}, got {tuple(sh)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: needs dtype {dtype}, got {t.dtype}")


def _holds_bytes(t, nbytes, what, dtype=None):
    """A flat buffer the caller supplies (scales) must be contiguous and hold
    `nbytes` bytes."""
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: needs dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what}: needs {nbytes} contiguous bytes")


def _scale_dtype(fmt):
    return torch.uint8 if fmt == SCALE_UE8M0_BYTE else torch.float32


def _holds_scale(t, kind, M, N, K, what):
    """A GEMM scale operand holds its kind's elements (bytes for
    GROUP128_UE8M0, fp32 otherwise; unknown kinds are left to the ABI)."""
    if kind == KIND_TENSOR:
        nbytes = 4
    elif kind == KIND_ROW:
        nbytes = 4 * M
    elif kind == KIND_COL:
        nbytes = 4 * N
    elif kind == KIND_GROUP128_FP32:
        nbytes = 4 * M * ((K + 127) // 128)
    elif kind == KIND_BLOCK128:
        nbytes = 4 * ((N + 127) // 128) * ((K + 127) // 128)
    elif kind == KIND_GROUP128_UE8M0:
        _holds_bytes(t, M * ((K + 127) // 128), what, torch.uint8)
        return
    else:
        return
    _holds_bytes(t, nbytes, what, torch.float32)


def quant_group_batched(x, group, fmt=SCALE_FP32, layout=LAYOUT_ROW_MAJOR, fuse_silu_mul=False,
                        rows=None, q=None, scales=None, stream=None):
    """x [B, M, K_in] bf16/fp16 with any batch / row strides (unit element
    stride) -> (codes uint8 [B, M, K_out], scales [B, ...2-D scale shape]).
    rows: optional device int32 [B] live-row counts (the masked form)."""
    B, M, K_in = x.shape
    _unit_last(x, "x")
    K_out = K_in // 2 if fuse_silu_mul else K_in
    if group == -1:
        group = K_out
    if q is None:
        q = torch.empty((B, M, K_out), dtype=torch.uint8, device=x.device)
    if scales is None:
        dt = torch.uint8 if fmt == SCALE_UE8M0_BYTE else torch.float32
        scales = torch.empty((B,) + scale_shape(fmt, layout, M, K_out, group), dtype=dt,
                             device=x.device)
    _unit_last(q, "q")
    _holds(q, (B, M, K_out), "q", torch.uint8)
    if scales.dtype != _scale_dtype(fmt):
        raise TypeError(f"scales: needs dtype {_scale_dtype(fmt)}, got {scales.dtype}")
    per = scale_bytes(fmt, layout, M, K_out, group)
    if not scales.is_contiguous() or scales.numel() * scales.element_size() < B * per:
        raise ValueError("scales must be contiguous with room for every batch")
    rows = _rows_arg(rows, B)
    st = _load().fp8sm_quant_group_batched(
        _ptr(x), _dtype_code(x), B, M, K_out, _bs(x, B), _ld(x), _ptr(rows),
        group, FUSE_SILU_MUL if fuse_silu_mul else 0, fmt, layout, _ptr(q),
        _bs(q, B), _ld(q), _ptr(scales), _stream(stream))
    _check(st, "fp8sm_quant_group_batched")
    return q, scales


def quant_static_batched(x, scale, q=None, stream=None):
    """x [B, M, K] bf16/fp16 (any batch / row strides) -> codes [B, M, K]."""
    B, M, K = x.shape
    _unit_last(x, "x")
    if q is None:
        q = torch.empty((B, M, K), dtype=torch.uint8, device=x.device)
    _unit_last(q, "q")
    _holds(q, (B, M, K), "q", torch.uint8)
    _holds_bytes(scale, 4, "scale", torch.float32)
    st = _load().fp8sm_quant_static_batched(
        _ptr(x), _dtype_code(x), B, M, K, _bs(x, B), _ld(x), _ptr(scale),
        _ptr(q), _bs(q, B), _ld(q), _stream(stream))
    _check(st, "fp8sm_quant_static_batched")
    return q


# rank of one batch's scale operand per kind, and its element count
_KIND_RANK = {KIND_TENSOR: 0, KIND_ROW: 1, KIND_COL: 1, KIND_GROUP128_UE8M0: 2,
              KIND_GROUP128_FP32: 2, KIND_BLOCK128: 2}


def _scale_batch_stride(t, kind, B, need, what):
    """0 for a shared scale operand, its leading stride for a per-batch one;
    checks that every batch's `need` elements exist."""
    if kind == KIND_TENSOR:
        if t.numel() == 1:
            return 0
        if t.dim() == 1 and t.numel() == B:
            return t.stride(0)
        raise ValueError(f"{what}: a TENSOR scale is one element or one per batch")
    base = _KIND_RANK[kind]
    if t.dim() == base + 1 and t.shape[0] == B and B > 1:
        if t[0].numel() < need or not t[0].is_contiguous():
            raise ValueError(f"{what}: per-batch scales too small or not contiguous")
        return t.stride(0)
    if t.numel() < need or not t.is_contiguous():
        raise ValueError(f"{what}: scales too small or not contiguous")
    return 0


def scaled_mm_batched(a, b, sa, sb, kind_a, kind_b, rows=None, c=None, bias=None,
                      out_dtype=None, stream=None):
    """a [B, M, K] uint8 (any batch / row strides); b [N, K] (one weight) or
    [B, N, K] (one per batch) -> c [B, M, N].  Scales are shared (their 2-D
    shape) or per batch (a leading B dimension).  rows: optional device int32
    [B] live-row counts; rows past a batch's count are left as c held them."""
    B, M, K = a.shape
    _unit_last(a, "a")
    _unit_last(b, "b")
    if b.dim() == 3:
        if b.shape[0] != B:
            raise ValueError("a per-batch weight needs one [N, K] slab per batch")
        N, bs_b = b.shape[1], _bs(b, B)
        ldb = _ld(b)
    else:
        N, bs_b, ldb = b.shape[0], 0, _ld(b)
    if out_dtype is None:
        out_dtype = c.dtype if c is not None else torch.bfloat16
    if c is None:
        c = torch.empty((B, M, N), dtype=out_dtype, device=a.device)
    _unit_last(c, "c")
    _holds(a, (B, M, K), "a", torch.uint8)
    _holds(b, (B, N, K) if b.dim() == 3 else (N, K), "b", torch.uint8)
    _holds(c, (B, M, N), "c")
    if c.dtype != out_dtype or (bias is not None and bias.dtype != out_dtype):
        raise TypeError("c and bias must have the output dtype")
    if bias is not None:
        _holds_bytes(bias, 2 * N, "bias")
    G = (K + 127) // 128
    need_a = {KIND_TENSOR: 1, KIND_ROW: M, KIND_GROUP128_UE8M0: M * G,
              KIND_GROUP128_FP32: M * G}[kind_a]
    need_b = {KIND_TENSOR: 1, KIND_COL: N, KIND_BLOCK128: ((N + 127) // 128) * G}[kind_b]
    bs_sa = _scale_batch_stride(sa, kind_a, B, need_a, "sa")
    bs_sb = _scale_batch_stride(sb, kind_b, B, need_b, "sb")
    out = {torch.bfloat16: BF16, torch.float16: FP16}[out_dtype]
    rows = _rows_arg(rows, B)
    st = _load().fp8sm_scaled_mm_batched(
        B, _ptr(rows), _ptr(a), _bs(a, B), _ld(a), _ptr(b), bs_b, ldb,
        _ptr(c), _bs(c, B), _ld(c), M, N, K, kind_a, _ptr(sa), bs_sa, kind_b,
        _ptr(sb), bs_sb, None if bias is None else _ptr(bias), out, _stream(stream))
    _check(st, "fp8sm_scaled_mm_batched")
    return c


# ---------------------------------------------------------------- weight preparation

def _widths_arg(widths):
    arr = (ctypes.c_int64 * len(widths))(*[int(v) for v in widths])
    return arr, len(widths)


def requantize_max_scale(w, scales, widths, q=None, max_scale=None, stream=None):
    """w uint8 [N, K] fused weight codes, scales fp32 device [P], widths: host
    list of P row counts -> (max_scale fp32 [1], codes requantized to it).
    Pass q=w to convert in place."""
    N, K = w.shape
    _unit_last(w, "w")
    if q is None:
        q = torch.empty_like(w)
    if max_scale is None:
        max_scale = torch.empty(1, dtype=torch.float32, device=w.device)
    _holds(w, (N, K), "w", torch.uint8)
    _holds(q, (N, K), "q", torch.uint8)
    _holds_bytes(scales, 4 * len(widths), "scales", torch.float32)
    _holds_bytes(max_scale, 4, "max_scale", torch.float32)
    arr, n = _widths_arg(widths)
    st = _load().fp8sm_requantize_max_scale(_ptr(w), _ld(w), N, K, arr, n, _ptr(scales),
                                            _ptr(q), _ld(q), _ptr(max_scale),
                                            _stream(stream))
    _check(st, "fp8sm_requantize_max_scale")
    return max_scale, q


def scales_to_channelwise(scales, widths, out=None, stream=None):
    """Device fp32 [P] per-partition scalars -> fp32 [sum(widths)] per channel."""
    arr, n = _widths_arg(widths)
    if out is None:
        out = torch.empty(int(sum(widths)), dtype=torch.float32, device=scales.device)
    _holds_bytes(scales, 4 * len(widths), "scales", torch.float32)
    _holds_bytes(out, 4 * int(sum(widths)), "out", torch.float32)
    st = _load().fp8sm_scales_to_channelwise(_ptr(scales), arr, n, _ptr(out), _stream(stream))
    _check(st, "fp8sm_scales_to_channelwise")
    return out


def quant_group_scatter(x, dst, R, fmt=SCALE_UE8M0_BYTE, layout=LAYOUT_MN_MAJOR, q=None,
                        scales=None, stream=None):
    """x [T, K] bf16/fp16 tokens, dst device int32 [T, topk] destination rows
    -> (codes uint8 [R, K], scales) with each token's 1x128 group quant
    written to its destination rows (other rows untouched)."""
    T, K = x.shape
    _unit_last(x, "x")
    if dst.dtype != torch.int32 or dst.dim() != 2 or dst.shape[0] != T or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous int32 [T, topk] tensor")
    if q is None:
        q = torch.empty((R, K), dtype=torch.uint8, device=x.device)
    _unit_last(q, "q")
    _holds(q, (R, K), "q", torch.uint8)
    if scales is None:
        scales = torch.empty(scale_shape(fmt, layout, R, K, 128), dtype=_scale_dtype(fmt),
                             device=x.device)
    _holds_bytes(scales, scale_bytes(fmt, layout, R, K, 128), "scales", _scale_dtype(fmt))
    st = _load().fp8sm_quant_group_scatter(_ptr(x), _dtype_code(x), T, K, _ld(x), _ptr(dst),
                                           dst.shape[1], R, fmt, layout, _ptr(q), _ld(q),
                                           _ptr(scales), _stream(stream))
    _check(st, "fp8sm_quant_group_scatter")
    return q, scales

"""Helpers for the GPU parity tests (compare the HIP path with the oracle)."""
import numpy as np
import torch

from oracle import bf16 as obf16
from oracle import fp16 as ofp16

F32 = np.float32


def cuda():
    return torch.device("cuda:0")


def to_gpu_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(cuda())


def to_gpu_f32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=F32).reshape(-1))).to(cuda())


def bf16_bits(t):
    """bf16 device tensor -> uint16 numpy bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_bits(t):
    return t.contiguous().cpu().numpy().view(np.uint32)


def tolerance_report(gpu_bits, res, K):
    """GEMM accuracy bound: |gpu - oracle| <= 2^-7 |oracle| + 1e-3 sa sb sqrt(K).

    The GPU bits are decoded in the oracle result's output dtype (bf16 or
    fp16); equal values, infinities included, count as no error.
    Returns (violations, max err/tol, worst index)."""
    dec = ofp16.bits_to_f64 if getattr(res, "dtype", "bf16") == "fp16" else obf16.bits_to_f64
    gpu = dec(gpu_bits)
    ora = res.out
    with np.errstate(invalid="ignore"):
        err = np.where(gpu == ora, 0.0, np.abs(gpu - ora))
    tol = 2.0 ** -7 * np.abs(ora) + 1e-3 * res.sab * np.sqrt(K)
    ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1), np.where(err > 0, np.inf, 0))
    idx = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
    return int(np.sum(err > tol)), float(ratio.max()) if ratio.size else 0.0, idx


def assert_within_tolerance(gpu_bits, res, K, what=""):
    v, mx, idx = tolerance_report(gpu_bits, res, K)
    print(f"[tol] {what}: outputs={gpu_bits.size} violations={v} max_err/tol={mx:.4f}")
    assert v == 0, f"{what}: {v} outputs outside the bound (max err/tol {mx:.3f} at {idx})"

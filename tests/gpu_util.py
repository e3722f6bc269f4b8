"""Helpers for the GPU parity tests (compare the HIP path with the oracle)."""
import os
import time
from concurrent.futures import ThreadPoolExecutor

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


def progress(msg):
    """A progress line on stdout and appended to progress.log in the run-output
    folder (long full-size checks print while they run, not only when they end)."""
    line = f"[{time.strftime('%H:%M:%S')}] {msg}"
    print(line, flush=True)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    try:
        os.makedirs(os.path.join(root, "gpurun_out"), exist_ok=True)
        with open(os.path.join(root, "gpurun_out", "progress.log"), "a") as f:
            f.write(line + "\n")
    except OSError:
        pass


def full_tolerance_report(gpu_bits, a_codes, b_codes, sa, sb, K, what, slab=1024, workers=4):
    """Every output of a rowwise GEMM against the oracle (og.scaled_mm on row
    slabs of A; rows are independent in the oracle's definition).  Returns
    (outputs, violations, max err/tol, worst [row, col])."""
    from threadpoolctl import threadpool_limits
    from oracle import gemm as og
    M = a_codes.shape[0]
    sa = np.asarray(sa, dtype=F32).reshape(-1)
    sb = np.asarray(sb, dtype=F32).reshape(-1)
    cores = len(os.sched_getaffinity(0))
    starts = list(range(0, M, slab))

    def one(r0):
        r1 = min(M, r0 + slab)
        res = og.scaled_mm(a_codes[r0:r1], b_codes, sa[r0:r1], sb)
        v, mx, idx = tolerance_report(gpu_bits[r0:r1], res, K)
        return r0, v, mx, idx

    total_v, worst, worst_at, done = 0, 0.0, None, 0
    t0 = time.time()
    with threadpool_limits(limits=max(1, cores // workers)):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for r0, v, mx, idx in ex.map(one, starts):
                total_v += v
                if mx > worst:
                    worst, worst_at = mx, (r0 + int(idx[0]), int(idx[1]))
                done += 1
                if done % max(1, len(starts) // 8) == 0 or done == len(starts):
                    progress(f"{what}: {done}/{len(starts)} row slabs, violations so far "
                             f"{total_v}, max err/tol {worst:.4f} ({time.time() - t0:.0f} s)")
    return gpu_bits.size, total_v, worst, worst_at

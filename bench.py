"""Benchmark of the FP8 quant + scaled-GEMM hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:
per-token E4M3FN quant of the bf16 activations (fp32 scales), then the rowwise
scaled GEMM against pre-quantized per-channel weights, writing bf16.  The
default workload is the attention-QKV projection the pages benchmark
("Route large SM90 row/column-scaled FP8 GEMMs to Torch", Kernel results):
M=8320, K=5376, N=21504.  Inputs are resident in HBM before timing starts.

Prints one JSON line (rank 0).  `value` is GEMM TFLOP/s over the whole step
(2*M*N*K / mean step time, quant included).  Each step's quant and GEMM
launches are bracketed by HIP events on the launch stream; their median, min
and max over the timed steps are reported.  `roofline` is the GEMM kernel's
own achieved rate (2*M*N*K / median launch time) against the dense FP8 matrix
peak the metric names (5.0 PFLOP/s); `frac_of_bf16_peak` gives the same rate
against the dense bf16 peak (2.5 PFLOP/s) of the instruction the kernel runs
on (fp8 codes widened exactly to bf16: the fp8 instructions truncate sums
below fp32 precision).  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload (a block of rows: their per-token quant plus their
GEMM rows).

Other modes: --suite (every hot-path kernel on its own workload), --sweep
(every rowwise kernel variant over a grid of M and (N, K): the measurements
the shape dispatch table is generated from), --ceilings (measured matrix-pipe
and HBM ceilings), --copy-calibration (a plain copy of known size for scaling
the traffic counters).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp8_scaled_mm TFLOP/s and % of FP8 MFMA peak on H3 dense shapes; quant GB/s"
PEAK_BF16_MFMA = 2500.0     # TFLOP/s, dense
PEAK_FP8_MFMA = 5000.0      # TFLOP/s, dense
PEAK_HBM = 8000.0           # GB/s

# HBM traffic of one QKV GEMM launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, scaled by a plain-copy calibration (FETCH_SIZE x2, WRITE_SIZE x1;
# profiles/gemm_rowwise_qkv_traffic.md).  Valid only for the gemm.hip source
# and kernel variant it was measured on; reported as null once either changes.
TRAFFIC = {"gemm_src_sha256_prefix": "cd3142395b89e366", "workload": "qkv",
           "kernel": "tile128x128", "bytes": 3120.1e6 + 367.7e6}


def measured_traffic(workload, variant):
    import hashlib
    src = os.path.join(ROOT, "column_scaled_gemm_amd", "csrc", "gemm.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if (h == TRAFFIC["gemm_src_sha256_prefix"] and workload == TRAFFIC["workload"]
            and variant == TRAFFIC["kernel"]):
        return TRAFFIC["bytes"]
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=15,
                   help="untimed steps; the GEMM settles over its first ~10 back-to-back launches")
    p.add_argument("--workload", default="qkv",
                   choices=["qkv", "mlp_gateup_23216", "mlp_gateup_15760", "mlp_down", "tiny"])
    p.add_argument("--variant", default=None,
                   help="force a GEMM kernel variant by name (default: the dispatch table)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--suite", action="store_true",
                   help="time every hot-path kernel on its own workload (one JSON line each)")
    p.add_argument("--sweep", action="store_true",
                   help="time every rowwise variant over the dispatch grid (one JSON line each)")
    p.add_argument("--sweep-out", default=None,
                   help="also write the sweep's lines to this file")
    p.add_argument("--ceilings", action="store_true",
                   help="measured matrix-pipe and HBM ceilings (one JSON line each)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (a known-size "
                        "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reads": n, "writes": n, "launches": 3}))


def ceilings(repeats=5):
    """Measured ceilings of the machine, one JSON line each: the matrix pipe
    on the GEMMs' instruction and accumulator count (fp8sm_rate_probe at 1, 2
    and 4 wavefronts per SIMD, without and with the widen feeding the
    operands) and HBM (a 1 GiB copy, read and write, caches evicted first
    by the other buffer).  Each figure is the median over `repeats` launches
    timed with HIP events.  Last, the QKV GEMM on three data sets of the same
    shape (the quantized workload, all-zero codes, all codes 1.0): the
    difference is what the values themselves cost."""
    import numpy as np
    import torch
    from column_scaled_gemm_amd import fp8sm
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    iters = 20000

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(repeats):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return float(np.median(ts))

    for widen in (0, 1):
        for wpb in (4, 8, 16):
            us = timed(lambda: fp8sm.rate_probe(widen, cus, wpb, iters))
            flop = 2.0 * 32 * 32 * 16 * 4 * iters * cus * wpb
            tf = flop / us / 1e6
            print(json.dumps({"ceiling": "matrix pipe, v_mfma_f32_32x32x16_bf16, 4 accumulators/wavefront"
                              + (", widen feeding the operands" if widen else ""),
                              "waves_per_simd": wpb // 4, "us": round(us, 1),
                              "TFLOPs": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_MFMA, 4)}),
                  flush=True)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    other = torch.ones(n // 8, dtype=torch.int64, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)

    def copy_cold():
        torch.sum(other, dim=0, out=sink)   # evicts src / dst (1 GiB read)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    def read_cold():
        dst.copy_(src)                     # evicts `other`
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        torch.sum(other, dim=0, out=sink)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    def write_cold():
        torch.sum(other, dim=0, out=sink)   # evicts dst (1 GiB read)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.fill_(7)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    for name, fn, nbytes in (("HBM copy (torch copy_, 1 GiB read + 1 GiB write)", copy_cold, 2 * n),
                             ("HBM read (torch sum, 1 GiB)", read_cold, n),
                             ("HBM write (torch fill_, 1 GiB)", write_cold, n)):
        fn()
        us = float(np.median([fn() for _ in range(repeats)]))
        gbs = nbytes / us / 1e3
        print(json.dumps({"ceiling": name, "us": round(us, 1), "GBps": round(gbs, 1),
                          "frac_of_hbm_peak": round(gbs / PEAK_HBM, 4)}), flush=True)
    del src, dst, other

    # Data-dependent cost of the rowwise GEMM: the QKV GEMM the dispatch picks,
    # on the quantized workload, on all-zero codes and on codes that all
    # encode 1.0 (0x38), interleaved over three rounds (median of each).  The
    # kernel's instructions, addresses and memory traffic are the same in all
    # three; only the values (and so the switching activity) differ.
    from column_scaled_gemm_amd import inputs
    M, N, K = inputs.ROWWISE_SHAPES["qkv"]
    w = inputs.workload("qkv")
    qb, sb = fp8sm.quant_group(w.w.to(dev), -1)
    qa, sa = fp8sm.quant_group(w.x.to(dev), -1)
    del w
    sa, sb = sa.reshape(-1), sb.reshape(-1)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    data = {"quantized workload": (qa, qb),
            "all-zero codes": (torch.zeros_like(qa), torch.zeros_like(qb)),
            "all codes 0x38 (1.0)": (torch.full_like(qa, 0x38), torch.full_like(qb, 0x38))}
    per = {k: [] for k in data}
    for _ in range(3):
        for k, (a, b) in data.items():
            per[k].append(timed(lambda: fp8sm.scaled_mm(a, b, sa, sb, fp8sm.KIND_ROW,
                                                        fp8sm.KIND_COL, c=c)))
    variant = fp8sm.variant_name(fp8sm.pick_variant(M, N, K))
    for k, xs in per.items():
        us = float(np.median(xs))
        print(json.dumps({"probe": "QKV rowwise GEMM %dx%dx%d, %s" % (M, K, N, k),
                          "variant": variant, "us": round(us, 1),
                          "TFLOPs": round(2.0 * M * N * K / us / 1e6, 1)}), flush=True)


def cpu_baseline(w, M, N, K, target_s):
    """Time the CPU oracle on the first R rows of the workload (quant of those
    rows + their GEMM rows against the full weight), R sized to ~target_s."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from column_scaled_gemm_amd import inputs
    from oracle import gemm as og, quant as oq

    ob = oq.quant_group(inputs.widen(w.w), K)            # offline weight quant, untimed

    def run(R):
        t0 = time.perf_counter()
        oa = oq.quant_group(inputs.widen(w.x[:R]), K)
        og.scaled_mm(oa.codes, ob.codes, oa.scale.reshape(-1), ob.scale.reshape(-1))
        return time.perf_counter() - t0

    R = 16
    t = run(R)                       # also warms up the BLAS threads
    for _ in range(4):               # rescale until the sample is near the target
        R = int(max(16, min(M, R * target_s / max(t, 1e-3))))
        t = run(R)
        if t >= 0.5 * target_s or R == M:
            break
    passes = 1
    if R == M and t < 0.5 * target_s:  # the whole workload is short: repeat it
        passes = int(math.ceil(target_s / max(t, 1e-3)))
        t = sum(run(R) for _ in range(passes))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    what = f"first {R} of {M} rows" if R < M else f"all {M} rows x {passes} passes"
    return {"value": round(2.0 * passes * R * N * K / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{what}: per-token quant + GEMM rows vs the full {N}x{K} weight "
                      f"({t:.1f} s)"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _stats(xs, nd=2):
    """median / min / max of a list of timings."""
    import numpy as np
    return {"median": round(float(np.median(xs)), nd), "min": round(float(np.min(xs)), nd),
            "max": round(float(np.max(xs)), nd), "n": len(xs)}


def _time_launches(fn, reps, nrot, stream, batches=3):
    """Mean kernel duration (us) of fn(i), launched `reps` times back to back.

    fn(i) launches on input set i % nrot; with nrot > 1 the sets together
    exceed the 256 MB last-level cache, so every launch reads from HBM.
    Two measurements of the same launch sequence:
      * graph: the `reps` launches captured once in a HIP graph and replayed
        (no host work between launches); HIP events around each replay;
      * queued: each batch enqueued behind a device read sized to outlast the
        host's enqueueing (measured during warm-up); a batch whose enqueue
        still outlasted that read is flagged host-bound.
    Returns (median graph mean, median queued mean, host_bound)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(nrot):
        fn(i)
    per_call = (time.perf_counter() - t0) / nrot
    torch.cuda.synchronize()
    # a read at ~4 TB/s lasting 3x the batch's enqueue time, 256 MiB .. 6 GiB
    nbytes = int(min(max(3 * reps * per_call * 4e12, 256 << 20), 6 << 30))
    spacer = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    means, host_bound = [], False
    for _ in range(batches):
        s0 = torch.cuda.Event(enable_timing=True)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        spacer.amax()
        a.record(stream)
        t0 = time.perf_counter()
        for i in range(reps):
            fn(i)
        host_us = (time.perf_counter() - t0) * 1e6
        b.record(stream)
        torch.cuda.synchronize()
        if host_us > s0.elapsed_time(a) * 1e3:
            host_bound = True
        means.append(a.elapsed_time(b) * 1e3 / reps)
    del spacer
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    gmeans = []
    for _ in range(batches):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        gmeans.append(a.elapsed_time(b) * 1e3 / reps)
    del g
    return sorted(gmeans)[len(gmeans) // 2], sorted(means)[len(means) // 2], host_bound


# The dispatch grid: M in powers of two (decode to large prefill) against the
# (N, K) of the H3 projections ("Route large SM90 row/column-scaled FP8 GEMMs
# to Torch", Kernel results: QKV, gate/up and down at TP1, with their TP2
# shards), and the decode widths (prhub digest of sglang PR #33148: the
# per-tensor decode shapes, K = 4096, N = 4096 / 14336).
SWEEP_NK = [(21504, 5376), (28672, 5376), (5376, 14336), (14336, 5376), (10752, 5376),
            (5376, 7168), (4096, 4096), (14336, 4096)]
SWEEP_M = [1 << i for i in range(16)]


def _time_graph(fn, reps, stream, repeats=5):
    """Per-launch time (us) of fn(i), i < reps, captured once in a HIP graph:
    one untimed replay, then `repeats` timed replays; (median, min, max)."""
    import numpy as np
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    g.replay()
    ts = []
    for _ in range(repeats):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / reps)
    del g
    return float(np.median(ts)), float(np.min(ts)), float(np.max(ts))


def sweep(out_path=None):
    """Every rowwise variant on every (M, N, K) of the dispatch grid: per-token
    quantized N(0,1) activations against per-channel quantized N(0, 0.02)
    weights (the H3 recipe without outliers), weights rotated through copies
    larger than the last-level cache, launches replayed from a graph."""
    import torch
    from column_scaled_gemm_amd import fp8sm
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    out = open(out_path, "w") if out_path else None
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    with torch.cuda.stream(stream):
        for N, K in SWEEP_NK:
            w = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            qb, sb = fp8sm.quant_group(w, -1, stream=stream)
            del w
            nrot = _rotations(N * K, True)
            qbs = [qb] + [qb.clone() for _ in range(nrot - 1)]
            x = torch.randn((SWEEP_M[-1], K), generator=gen, device=dev).to(torch.bfloat16)
            qa, sa = fp8sm.quant_group(x, -1, stream=stream)
            del x
            sa, sb = sa.reshape(-1), sb.reshape(-1)
            for M in SWEEP_M:
                c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                est_us = 2.0 * M * N * K / 1.2e15 * 1e6 + N * K / 4e12 * 1e6
                reps = int(min(200, max(3, nrot, -(-2000 // max(est_us, 1.0)))))
                for v in range(fp8sm.variant_count()):
                    if not fp8sm.variant_accepts(v, M, N, K):
                        continue
                    prev = fp8sm.force_variant(v)
                    try:
                        med, lo, hi = _time_graph(
                            lambda i: fp8sm.scaled_mm(qa[:M], qbs[i % nrot], sa[:M], sb,
                                                      fp8sm.KIND_ROW, fp8sm.KIND_COL, c=c,
                                                      stream=stream), reps, stream)
                    finally:
                        fp8sm.force_variant(prev)
                    line = json.dumps({"sweep": 1, "M": M, "N": N, "K": K,
                                       "variant": fp8sm.variant_name(v), "us": round(med, 2),
                                       "us_min": round(lo, 2), "us_max": round(hi, 2),
                                       "reps": reps, "weight_copies": nrot})
                    print(line, flush=True)
                    if out:
                        out.write(line + "\n")
                        out.flush()
                del c
            del qa, sa, qbs, qb, sb
            torch.cuda.empty_cache()
    if out:
        out.close()


def _rotations(bytes_per_set, cold):
    """Input sets a cold batch rotates through: 4 GiB of them.  The 256 MB
    memory-side cache keeps a share of a cyclic working set much larger than
    itself (measured: rotating 0.5 GB of decode weights still read at up to
    10 TB/s), so the set is 16x the cache and at most ~6% of a launch's bytes
    can be served from it."""
    return max(1, -(-(4 << 30) // max(bytes_per_set, 1))) if cold else 1


def suite(reps):
    """One JSON line per hot-path row.  Quant and decode rows are cold (each
    launch reads its inputs from HBM); the rowwise and blockwise GEMMs, which
    are compute-bound, are warm."""
    import torch
    # a stream of its own (default priority) so launch sequences can be captured
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        return _suite_rows(reps, stream)


def _suite_rows(reps, stream):
    import numpy as np
    import torch
    from column_scaled_gemm_amd import fp8sm, inputs
    dev = torch.device("cuda:0")
    out = []

    def emit(row, **kv):
        d = {"row": row}
        d.update(kv)
        print(json.dumps(d), flush=True)
        out.append(d)

    # a1 / a5: per-token quant + rowwise GEMM on the H3 shapes
    for name in ("qkv", "mlp_gateup_23216", "mlp_gateup_15760", "mlp_down"):
        M, N, K = inputs.ROWWISE_SHAPES[name]
        w = inputs.workload(name)
        qb, sb = fp8sm.quant_group(w.w.to(dev), -1)
        nrot = _rotations(3 * M * K, True)
        xs = [w.x.to(dev) for _ in range(nrot)]
        del w
        qas = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(nrot)]
        sas = [torch.empty((M, 1), dtype=torch.float32, device=dev) for _ in range(nrot)]
        us_q, qus_q, hb = _time_launches(
            lambda i: fp8sm.quant_group(xs[i % nrot], -1, q=qas[i % nrot], scales=sas[i % nrot],
                                        stream=stream), max(reps, nrot), nrot, stream)
        qbytes = 2 * M * K + M * K + 4 * M
        emit("a1 per-token quant", workload=f"{name} bf16[{M},{K}]", us=round(us_q, 2), us_queued=round(qus_q, 2),
             GBps=round(qbytes / us_q / 1e3, 1), hbm_frac=round(qbytes / us_q / 1e3 / PEAK_HBM, 3),
             cache="cold", host_bound=hb)
        qa, sa = qas[0], sas[0]
        del xs, qas[1:], sas[1:]
        c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us_g, qus_g, hb = _time_launches(
            lambda i: fp8sm.scaled_mm(qa, qb, sa.reshape(-1), sb.reshape(-1), fp8sm.KIND_ROW,
                                      fp8sm.KIND_COL, c=c, stream=stream),
            max(3, reps // 2), 1, stream, batches=2)
        tf = 2.0 * M * N * K / us_g / 1e6
        emit("a5 rowwise GEMM", workload=f"{name} {M}x{K}x{N}", us=round(us_g, 1), us_queued=round(qus_g, 1),
             TFLOPs=round(tf, 1), bf16_peak_frac=round(tf / PEAK_BF16_MFMA, 4),
             fp8_peak_frac=round(tf / PEAK_FP8_MFMA, 4), cache="warm",
             variant=fp8sm.variant_name(fp8sm.pick_variant(M, N, K)))
        if name == "qkv":
            # evidence only: the same GEMM on the fp8 matrix instructions
            # (outside the accuracy bound; never dispatched)
            us_8, qus_8, _ = _time_launches(
                lambda i: fp8sm.scaled_mm_fp8mfma(qa, qb, sa.reshape(-1), sb.reshape(-1),
                                                  fp8sm.KIND_ROW, fp8sm.KIND_COL, c=c,
                                                  stream=stream),
                max(3, reps // 2), 1, stream, batches=2)
            tf8 = 2.0 * M * N * K / us_8 / 1e6
            emit("a5 evidence: fp8-instruction rowwise GEMM (inexact)",
                 workload=f"{name} {M}x{K}x{N}", us=round(us_8, 1), us_queued=round(qus_8, 1),
                 TFLOPs=round(tf8, 1), fp8_peak_frac=round(tf8 / PEAK_FP8_MFMA, 4),
                 cache="warm")
        del qa, sa, qas, sas, qb, sb, c
        torch.cuda.empty_cache()

    # a3 / a6: static quant + per-tensor decode GEMM
    d = inputs.decode()
    Kd = inputs.DECODE_K
    xsc = torch.tensor([d.x_scale], dtype=torch.float32, device=dev)
    x = d.x.to(dev)
    for N in inputs.DECODE_NS:
        ws = torch.tensor([d.w_scale[N]], dtype=torch.float32, device=dev)
        qw0 = fp8sm.quant_static(d.w[N].to(dev), ws)
        nrot = _rotations(N * Kd, True)
        qws = [qw0] + [qw0.clone() for _ in range(nrot - 1)]
        for M in inputs.DECODE_MS:
            qx = torch.empty((M, Kd), dtype=torch.uint8, device=dev)
            cs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(nrot)]
            us_s, qus_s, hb_s = _time_launches(lambda i: fp8sm.quant_static(x[:M], xsc, q=qx, stream=stream),
                                        max(reps, 20), 1, stream)
            us_d, qus_d, hb = _time_launches(
                lambda i: fp8sm.scaled_mm(qx, qws[i % nrot], xsc, ws, fp8sm.KIND_TENSOR,
                                          fp8sm.KIND_TENSOR, c=cs[i % nrot], stream=stream),
                max(reps, nrot), nrot, stream)
            byts = N * Kd + M * Kd + 2 * M * N
            emit("a3 static quant", workload=f"bf16[{M},{Kd}]", us=round(us_s, 2), us_queued=round(qus_s, 2), cache="warm",
                 host_bound=hb_s)
            emit("a6 decode GEMM", workload=f"M={M} K={Kd} N={N} per-tensor",
                 us=round(us_d, 2), us_queued=round(qus_d, 2), GBps=round(byts / us_d / 1e3, 1),
                 hbm_frac=round(byts / us_d / 1e3 / PEAK_HBM, 3),
                 TFLOPs=round(2.0 * M * N * Kd / us_d / 1e6, 2), cache="cold", host_bound=hb,
                 variant=fp8sm.variant_name(fp8sm.pick_variant(M, N, Kd)))
        del qws, qw0, cs
        torch.cuda.empty_cache()

    # a4 / a7: fused SiLU-and-mul + 1x128 UE8M0 quant, blockwise GEMM
    f = inputs.fused()
    Mf, Kf, Nf = inputs.FUSED_M, inputs.FUSED_K, inputs.FUSED_N
    qb, sbb = fp8sm.quant_weight_block128(f.w.to(dev))
    for tag, xin in (("bf16", f.gu_bf16), ("fp16", f.gu_fp16)):
        nrot = _rotations(4 * Mf * Kf, True)
        xgs = [xin.to(dev) for _ in range(nrot)]
        qas = [torch.empty((Mf, Kf), dtype=torch.uint8, device=dev) for _ in range(nrot)]
        eas = [torch.empty((Mf, Kf // 128), dtype=torch.uint8, device=dev) for _ in range(nrot)]
        us_f, qus_f, hb = _time_launches(
            lambda i: fp8sm.quant_group(xgs[i % nrot], 128, fp8sm.SCALE_UE8M0_BYTE,
                                        fuse_silu_mul=True, q=qas[i % nrot], scales=eas[i % nrot],
                                        stream=stream), max(reps, nrot), nrot, stream)
        fbytes = 4 * Mf * Kf + Mf * Kf + Mf * Kf // 128
        emit("a4 fused SiLU-mul + 1x128 UE8M0 quant", workload=f"{tag}[{Mf},{2 * Kf}]",
             us=round(us_f, 2), us_queued=round(qus_f, 2), GBps=round(fbytes / us_f / 1e3, 1),
             hbm_frac=round(fbytes / us_f / 1e3 / PEAK_HBM, 3), cache="cold", host_bound=hb)
        qa, ea = qas[0], eas[0]
        del xgs, qas, eas
        c = torch.empty((Mf, Nf), dtype=torch.bfloat16, device=dev)
        us_b, qus_b, hb = _time_launches(
            lambda i: fp8sm.scaled_mm(qa, qb, ea, sbb, fp8sm.KIND_GROUP128_UE8M0,
                                      fp8sm.KIND_BLOCK128, c=c, stream=stream),
            max(reps, 5), 1, stream, batches=2)
        tf = 2.0 * Mf * Nf * Kf / us_b / 1e6
        emit("a7 blockwise GEMM", workload=f"{tag} {Mf}x{Kf}x{Nf}", us=round(us_b, 1), us_queued=round(qus_b, 1),
             TFLOPs=round(tf, 1), bf16_peak_frac=round(tf / PEAK_BF16_MFMA, 4), cache="warm")
        del qa, ea, c
        torch.cuda.empty_cache()

    # f2: masked EP-MoE decode -- fused SiLU-and-mul + 1x128 UE8M0 quant of the
    # live rows of each expert's slab, then the grouped blockwise down GEMM
    mo = inputs.masked_moe()
    E, Tm, H, I = inputs.MOE_E, inputs.MOE_T, inputs.MOE_HIDDEN, inputs.MOE_INTER
    rows = torch.from_numpy(mo.rows).to(dev)
    live, active = int(mo.rows.sum()), int((mo.rows > 0).sum())
    nrot = _rotations(2 * E * Tm * 2 * I, True)
    gus = [mo.gu.to(dev) for _ in range(nrot)]
    q = torch.empty((E, Tm, I), dtype=torch.uint8, device=dev)
    es = torch.empty((E, Tm, I // 128), dtype=torch.uint8, device=dev)
    us_m, qus_m, hb = _time_launches(
        lambda i: fp8sm.quant_group_batched(gus[i % nrot], 128, fp8sm.SCALE_UE8M0_BYTE,
                                            fuse_silu_mul=True, rows=rows, q=q, scales=es,
                                            stream=stream), max(reps, nrot), nrot, stream)
    mbytes = live * (4 * I + I + I // 128)
    emit("f2 masked fused SiLU-mul + 1x128 UE8M0 quant",
         workload=f"bf16[{E},{Tm},{2 * I}] {live} live rows", us=round(us_m, 2), us_queued=round(qus_m, 2),
         GBps=round(mbytes / us_m / 1e3, 1), hbm_frac=round(mbytes / us_m / 1e3 / PEAK_HBM, 3),
         cache="cold", host_bound=hb)
    del gus
    nrot = _rotations(E * H * I, True)
    wqs, wss = [], []
    for _ in range(nrot):
        wq = torch.empty((E, H, I), dtype=torch.uint8, device=dev)
        ws = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            fp8sm.quant_weight_block128(mo.w[e].to(dev), q=wq[e], scales=ws[e])
        wqs.append(wq)
        wss.append(ws)
    del mo
    c = torch.empty((E, Tm, H), dtype=torch.bfloat16, device=dev)
    us_e, qus_e, hb = _time_launches(
        lambda i: fp8sm.scaled_mm_batched(q, wqs[i % nrot], es, wss[i % nrot],
                                          fp8sm.KIND_GROUP128_UE8M0, fp8sm.KIND_BLOCK128,
                                          rows=rows, c=c, stream=stream),
        max(reps, nrot), nrot, stream)
    ebytes = (active * H * I + live * (I + I // 128) + active * (H // 128) * (I // 128) * 4
              + live * H * 2)
    emit("f2 masked grouped blockwise GEMM",
         workload=f"{E} experts x {Tm}-row slabs, {live} live rows, K={I} N={H}",
         us=round(us_e, 1), us_queued=round(qus_e, 1), GBps=round(ebytes / us_e / 1e3, 1),
         hbm_frac=round(ebytes / us_e / 1e3 / PEAK_HBM, 3),
         TFLOPs=round(2.0 * live * H * I / us_e / 1e6, 1), cache="cold", host_bound=hb)
    del wqs, wss, q, es, c
    torch.cuda.empty_cache()

    # f3: 1x128 UE8M0 quant scattered to the top-k destination rows of the
    # grouped-GEMM input (MN-major scales); stand-in: 1024 tokens of hidden
    # 7168, top-8, 8192 destination rows (the pages print no shapes)
    Ts, Ks, topk = 1024, inputs.FUSED_K, 8
    Rs = Ts * topk
    nrot = _rotations(2 * Ts * Ks + Rs * Ks, True)
    gen = inputs.rng(50)
    xs_ = [inputs.to_dtype(gen.standard_normal((Ts, Ks), dtype=np.float32)).to(dev)
           for _ in range(nrot)]
    dsts = [torch.from_numpy(gen.permutation(Rs).reshape(Ts, topk).astype(np.int32)).to(dev)
            for _ in range(nrot)]
    qs_ = [torch.empty((Rs, Ks), dtype=torch.uint8, device=dev) for _ in range(nrot)]
    ss_ = torch.empty((Ks // 128, Rs), dtype=torch.uint8, device=dev)
    us_sc, qus_sc, hb = _time_launches(
        lambda i: fp8sm.quant_group_scatter(xs_[i % nrot], dsts[i % nrot], Rs, q=qs_[i % nrot],
                                            scales=ss_, stream=stream),
        max(reps, nrot), nrot, stream)
    scb = 2 * Ts * Ks + Rs * Ks + Rs * (Ks // 128) + 4 * Rs
    emit("f3 scatter 1x128 UE8M0 quant", workload=f"bf16[{Ts},{Ks}] top-{topk} -> {Rs} rows",
         us=round(us_sc, 2), us_queued=round(qus_sc, 2), GBps=round(scb / us_sc / 1e3, 1),
         hbm_frac=round(scb / us_sc / 1e3 / PEAK_HBM, 3), cache="cold", host_bound=hb)
    del xs_, dsts, qs_, ss_
    torch.cuda.empty_cache()

    # f4: load-time requantization of the fused QKV weight to its largest
    # partition scale (partition widths 16384 / 2560 / 2560 rows: a stand-in,
    # the pages print none), then the per-channel broadcast
    Nq, Kq = inputs.ROWWISE_SHAPES["qkv"][1], inputs.ROWWISE_SHAPES["qkv"][2]
    widths = [16384, 2560, 2560]
    nrot = _rotations(2 * Nq * Kq, True)
    wcs = [torch.from_numpy(inputs.random_codes((Nq, Kq), seed=40 + i)).to(dev)
           for i in range(nrot)]
    ps = torch.tensor([0.011, 0.017, 0.013], dtype=torch.float32, device=dev)
    wq = torch.empty((Nq, Kq), dtype=torch.uint8, device=dev)
    ms = torch.empty(1, dtype=torch.float32, device=dev)
    us_r, qus_r, hb = _time_launches(
        lambda i: fp8sm.requantize_max_scale(wcs[i % nrot], ps, widths, q=wq, max_scale=ms,
                                             stream=stream), max(reps, nrot), nrot, stream)
    rbytes = 2 * Nq * Kq
    emit("f4 requantize fused weight to the max scale", workload=f"qkv weight [{Nq},{Kq}], 3 partitions",
         us=round(us_r, 1), us_queued=round(qus_r, 1), GBps=round(rbytes / us_r / 1e3, 1),
         hbm_frac=round(rbytes / us_r / 1e3 / PEAK_HBM, 3), cache="cold", host_bound=hb)
    del wcs, wq
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library "
              "has no multi-GPU path; the GEMM's column-parallel sharding needs no exchange "
              "and would scale per GPU.", file=sys.stderr)
        sys.exit(2)
    if args.suite:
        suite(max(args.steps, 5))
        return
    if args.sweep:
        sweep(args.sweep_out)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.ceilings:
        ceilings()
        return
    import numpy as np
    import torch
    from column_scaled_gemm_amd import fp8sm, inputs

    dev = torch.device("cuda:0")
    if args.variant:
        names = [fp8sm.variant_name(i) for i in range(fp8sm.variant_count())]
        fp8sm.force_variant(names.index(args.variant))
    M, N, K = inputs.ROWWISE_SHAPES[args.workload]
    w = inputs.workload(args.workload)
    x = w.x.to(dev)
    qb, sb = fp8sm.quant_group(w.w.to(dev), -1)            # weights: quantized once
    sb = sb.reshape(-1)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, 1), dtype=torch.float32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fp8sm.quant_group(x, -1, q=qa, scales=sa, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        fp8sm.scaled_mm(qa, qb, sa.reshape(-1), sb, fp8sm.KIND_ROW, fp8sm.KIND_COL, c=c,
                        stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    gemm_us = [b.elapsed_time(c_) * 1e3 for a, b, c_ in evs]
    quant_us = [a.elapsed_time(b) * 1e3 for a, b, c_ in evs]
    step_ms = [a.elapsed_time(c_) for a, b, c_ in evs]
    gemm_med_us = float(np.median(gemm_us))
    flop = 2.0 * M * N * K
    value = flop / (ms_step * 1e-3) / 1e12
    gemm_tflops = flop / (gemm_med_us * 1e-6) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic: fp8 codes widened exactly to bf16, multiplied on the
        # bf16 matrix cores with fp32 accumulation (the roofline's peak)
        "dtype": "bf16",
        "operand_dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: per-token quant bf16[{M},{K}] + rowwise "
                               f"fp8_scaled_mm {M}x{K}x{N} -> bf16",
                   "M": M, "N": N, "K": K, "kernel_variant": fp8sm.variant_name(
                       fp8sm.pick_variant(M, N, K))},
        # achieved: 2MNK / median GEMM launch time (HIP events on the launch
        # stream); peak: the dense FP8 matrix peak the metric names
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 3),
                     "peak": PEAK_FP8_MFMA, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP8_MFMA, 4),
                     "traffic": measured_traffic(args.workload, fp8sm.variant_name(
                         fp8sm.pick_variant(M, N, K)))},
        "frac_of_bf16_peak": round(gemm_tflops / PEAK_BF16_MFMA, 4),
        "gemm_us": _stats(gemm_us, 1),
        "quant_us": _stats(quant_us, 2),
        "step_ms": _stats(step_ms, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, M, N, K, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""bench.py's contract pieces that need no GPU: the one-GPU refusal, the CPU
oracle baseline field, and traffic reported only for the GEMM source it was
measured on."""
import hashlib
import os
import subprocess
import sys

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    for extra in ([], ["--suite"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"] + extra,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr
        assert r.stdout == ""


def test_cpu_baseline_fields_on_the_tiny_workload():
    from column_scaled_gemm_amd import inputs
    M, N, K = inputs.ROWWISE_SHAPES["tiny"]
    cb = bench.cpu_baseline(inputs.workload("tiny"), M, N, K, 0.2)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample", "cpu_model"}
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert f"{N}x{K}" in cb["sample"]


def test_traffic_only_for_the_measured_source_workload_and_kernel():
    src = os.path.join(ROOT, "column_scaled_gemm_amd", "csrc", "gemm.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    t = bench.TRAFFIC
    got = bench.measured_traffic(t["workload"], t["kernel"])
    assert got == (t["bytes"] if h == t["gemm_src_sha256_prefix"] else None)
    assert bench.measured_traffic("mlp_down", t["kernel"]) is None
    assert bench.measured_traffic(t["workload"], "tile256x256") is None


def test_timing_stats_are_median_min_max():
    st = bench._stats([3.0, 1.0, 2.0, 10.0, 4.0])
    assert st == {"median": 3.0, "min": 1.0, "max": 10.0, "n": 5}


def test_sweep_grid_covers_decode_and_the_h3_shapes():
    from column_scaled_gemm_amd import inputs
    nk = set(bench.SWEEP_NK)
    for name in ("qkv", "mlp_gateup_23216", "mlp_down"):
        M, N, K = inputs.ROWWISE_SHAPES[name]
        assert (N, K) in nk
    for N in inputs.DECODE_NS:
        assert (N, inputs.DECODE_K) in nk
    assert bench.SWEEP_M[0] == 1 and bench.SWEEP_M[-1] >= 23216

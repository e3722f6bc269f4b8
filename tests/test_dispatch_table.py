"""The shape-dispatch table is generated from a measured sweep and picks each
swept shape's measured winner.

The pages route GEMM shapes to the implementation measured fastest on a sweep
("Route large SM90 row/column-scaled FP8 GEMMs to Torch", Kernel results) and
found that a route without an M bound slowed decode (same page, review
thread).  csrc/dispatch_sweep.jsonl holds `bench.py --sweep` from an MI355X
(every rowwise variant timed on every swept (M, N, K)); csrc/dispatch_table.h
is generated from it by gen_dispatch_table.py.  No GPU is needed here: the
table lookup (fp8sm_pick_variant) runs on the host.
"""
import json
import os
import random

import pytest

from conftest import ROOT

LIB = os.path.join(ROOT, "column_scaled_gemm_amd", "libfp8sm.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfp8sm.so not built")


def _gen():
    from column_scaled_gemm_amd import gen_dispatch_table as gen
    return gen


def test_variant_ids_match_the_library():
    from column_scaled_gemm_amd import fp8sm
    gen = _gen()
    assert len(gen.VARIANT_IDS) == fp8sm.variant_count()
    for name, vid in gen.VARIANT_IDS.items():
        assert fp8sm.variant_name(vid) == name


def test_header_is_generated_from_the_committed_sweep():
    gen = _gen()
    rows = gen.table_rows(gen.winners(gen.load()))
    with open(gen.HEADER) as f:
        assert f.read() == gen.render(rows), "dispatch_table.h is stale: rerun gen_dispatch_table"


def test_sweep_covers_every_variant_at_every_point_it_accepts():
    from column_scaled_gemm_amd import fp8sm
    gen = _gen()
    lines = gen.load()
    seen = {(d["M"], d["N"], d["K"], d["variant"]) for d in lines}
    shapes = {(d["M"], d["N"], d["K"]) for d in lines}
    for M, N, K in shapes:
        for v in range(fp8sm.variant_count()):
            if fp8sm.variant_accepts(v, M, N, K):
                assert (M, N, K, fp8sm.variant_name(v)) in seen, (M, N, K, v)
    for d in lines:
        assert d["us_min"] <= d["us"] <= d["us_max"]


def test_table_picks_each_swept_shapes_measured_winner():
    from column_scaled_gemm_amd import fp8sm
    gen = _gen()
    lines = gen.load()
    best = {}
    for d in lines:
        key = (d["M"], d["N"], d["K"])
        if key not in best or d["us"] < best[key][1]:
            best[key] = (d["variant"], d["us"])
    for (M, N, K), (name, us) in best.items():
        assert fp8sm.variant_name(fp8sm.pick_variant(M, N, K)) == name, (M, N, K, name, us)


def test_library_lookup_equals_the_generators_off_the_grid():
    # shapes between and beyond the swept ones: the compiled lookup and the
    # generator's model of it agree (nearest (N, K), M bucket ceil(log2 M))
    from column_scaled_gemm_amd import fp8sm
    gen = _gen()
    rows = gen.table_rows(gen.winners(gen.load()))
    r = random.Random(5)
    shapes = [(64, 256, 512), (1, 4096, 14336), (37, 5376, 4096), (100000, 28672, 5376)]
    shapes += [(r.randint(1, 70000), 8 * r.randint(1, 8000), 16 * r.randint(1, 4096))
               for _ in range(300)]
    for M, N, K in shapes:
        assert fp8sm.pick_variant(M, N, K) == gen.pick(rows, M, N, K), (M, N, K)


def test_every_pick_accepts_its_shape():
    from column_scaled_gemm_amd import fp8sm
    r = random.Random(6)
    for _ in range(500):
        M = r.choice([1, 2, 3, 15, 16, 17, 31, 33, 63, 64, 65, 127, 4097, r.randint(1, 1 << 17)])
        N, K = 8 * r.randint(1, 8000), 16 * r.randint(1, 4096)
        assert fp8sm.variant_accepts(fp8sm.pick_variant(M, N, K), M, N, K), (M, N, K)


def test_decode_batches_measured_fastest_on_the_decode_kernels():
    # the pages' decode regression: the per-tensor decode shapes (M = 1..16,
    # K = 4096, N = 4096 / 14336) route to a register-streamed decode kernel,
    # and the sweep measured them fastest there
    from column_scaled_gemm_amd import fp8sm
    for M in (1, 2, 4, 8, 16):
        for N in (4096, 14336):
            assert fp8sm.variant_name(fp8sm.pick_variant(M, N, 4096)).startswith("decode"), (M, N)

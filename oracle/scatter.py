"""Group quant with a scattered output: one token to its top-k destination rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

sglang PR #33533 "[JIT] per_token_group_quant: fix the fp16 UE8M0 multiplier
overflow ..." (commit messages, the scatter fusion) keeps one kernel beyond
the shared group quant: its output mapping replicates each source token to
its top-k destination rows of the grouped-GEMM input and writes each group's
UE8M0 scale byte into the MN-major (group-major) scale buffer at those rows,
so no separate fill kernel or intermediate buffer is needed.  The page prints
no code.  Reading taken: token t is quantized exactly as the plain 1x128
group quant quantizes a row, once; for every destination d = dst[t][j] with
0 <= d < R its codes become row d of the output and its scales row d's scale
entries; rows no token names keep their contents, and destination entries
outside [0, R) name no row.  Destinations are distinct (a row written twice
is not defined).

Pins (tests/test_oracle_scatter.py): quantize-then-scatter equals
replicate-then-quantize through the pinned plain group quant; power-of-two
closed forms per token; untouched rows and skipped destinations.
"""
import numpy as np

from .quant import quant_group

F32 = np.float32


def quant_group_scatter(x32, dst, R, group=128, pow2=True):
    """x32 float32 [T, K]; dst int [T, topk]; R output rows.

    Returns (codes uint8 [R, K], scale values float32 [R, G], UE8M0 bytes
    uint8 [R, G] or None, written bool [R]); rows with written False are
    rows no destination names (zeros here; the caller's contents there)."""
    x32 = np.asarray(x32, dtype=F32)
    T, K = x32.shape
    dst = np.asarray(dst, dtype=np.int64).reshape(T, -1)
    G = K // group
    gq = quant_group(x32, group, pow2)
    codes = np.zeros((R, K), np.uint8)
    scale = np.zeros((R, G), F32)
    byte = np.zeros((R, G), np.uint8) if pow2 else None
    written = np.zeros(R, dtype=bool)
    for t in range(T):
        for d in dst[t]:
            if 0 <= d < R:
                codes[d] = gq.codes[t]
                scale[d] = gq.scale[t]
                if pow2:
                    byte[d] = gq.ue8m0_byte[t]
                written[d] = True
    return codes, scale, byte, written

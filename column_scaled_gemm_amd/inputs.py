"""Seeded synthetic inputs for the FP8 scaled-GEMM path.

This module only draws numbers, rounds them to the input dtype (bf16 / fp16,
round-to-nearest-even via torch's CPU cast) and lays them out.  It holds none
of the path's arithmetic, and it is the only code the HIP path and the CPU
oracle both see: the tests feed the same tensors to each side.

Every draw comes from numpy's PCG64 generator, seed 0 unless a test asks for
another, in a fixed order per workload: activations, then the outlier
channels, then weights.  The shapes are the pages' own ("Route large SM90
row/column-scaled FP8 GEMMs to Torch", Kernel results table: the H3 QKV and MLP
projections); synthetic normal data stands in for real activations and
weights, since no checkpoint or dataset is used.

Workloads
---------
tiny        A [64, 512] N(0,1), B [256, 512] N(0, 0.02); per-row quant of both.
decode      A [16, 4096] N(0,1) (M = 1 and 4 use its first rows); W [N, 4096]
            N(0, 0.02) for N = 4096 and 14336; one static fp32 scale per tensor,
            standing in for the checkpoint scale of the prhub digest of
            PR #33148: s = fp32(max|T|) / 448 in fp32.
qkv         A [8320, 5376] N(0,1) with floor(K/100) channels (chosen by a seeded
            permutation) multiplied by 20 before rounding -- the outliers;
            W [21504, 5376] N(0, 0.02).
mlp_*       the same recipe at 23216x5376x28672, 15760x5376x28672 (gate/up)
            and 8320x14336x5376 (down).
fused       gate|up [4096, 2 x 7168] N(0,1); a seeded Bernoulli(0.05) choice of
            (row, 128-column group) pairs multiplies that group of the up half
            by 1e-5 (product absmax below 1e-3; in fp16 these become
            subnormal on purpose); rows with r % 512 == 7 are all zero.
            Returned in bf16 and in fp16 from the same draws.  W [4096, 7168]
            N(0, 0.02) for the blockwise GEMM.
masked_moe  the masked EP-MoE decode step of sglang PR #33533 (Speed Tests:
            graph-captured decode, bf16, group 128, UE8M0, fused SiLU-and-mul,
            masked), whose shapes the pages do not print.  Stand-in: 32 local
            experts (256 routed experts over 8 ranks), each with a 128-row
            slab; live rows per expert ~ Poisson(32) clamped to the slab (a
            decode batch of 128 tokens per rank, top-8 routing); gate|up
            [32, 128, 2 x 2048] N(0,1) (all slab rows drawn, dead ones
            included); down-projection weights [32, 7168, 2048] N(0, 0.02),
            hidden 7168 as in the fused workload.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

SEED = 0

# name -> (M, N, K) of the rowwise GEMM workloads
ROWWISE_SHAPES = {
    "tiny": (64, 256, 512),
    "qkv": (8320, 21504, 5376),
    "mlp_gateup_23216": (23216, 28672, 5376),
    "mlp_gateup_15760": (15760, 28672, 5376),
    "mlp_down": (8320, 5376, 14336),
}
DECODE_K = 4096
DECODE_NS = (4096, 14336)
DECODE_MS = (1, 4, 16)
FUSED_M, FUSED_K, FUSED_N = 4096, 7168, 4096
FUSED_GROUP = 128
MOE_E, MOE_T, MOE_HIDDEN, MOE_INTER, MOE_MEAN_ROWS = 32, 128, 7168, 2048, 32


def rng(seed=SEED):
    return np.random.Generator(np.random.PCG64(seed))


def to_dtype(x32: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """float32 numpy -> CPU tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(dtype)


def widen(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp16 CPU tensor -> float32 numpy, exactly."""
    return t.to(torch.float32).numpy()


@dataclass
class RowwiseInputs:
    name: str
    x: torch.Tensor          # activations [M, K]
    w: torch.Tensor          # weights [N, K]
    outlier_channels: Optional[np.ndarray] = None


def rowwise(M, N, K, seed=SEED, outliers=True, x_std=1.0, w_std=0.02,
            dtype=torch.bfloat16, name="custom") -> RowwiseInputs:
    r = rng(seed)
    x = r.standard_normal((M, K), dtype=np.float32)
    if x_std != 1.0:
        x *= np.float32(x_std)
    ch = None
    if outliers and K >= 100:
        ch = np.sort(r.permutation(K)[: K // 100])
        x[:, ch] *= np.float32(20.0)
    w = r.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)
    return RowwiseInputs(name, to_dtype(x, dtype), to_dtype(w, dtype), ch)


def workload(name, seed=SEED) -> RowwiseInputs:
    """The named rowwise workload (see the module docstring)."""
    M, N, K = ROWWISE_SHAPES[name]
    return rowwise(M, N, K, seed=seed, outliers=(name != "tiny"), name=name)


def static_scale(t: torch.Tensor) -> float:
    """Synthetic checkpoint scale: fp32(max|t|) / 448 evaluated in fp32."""
    a = torch.tensor(float(t.float().abs().max()), dtype=torch.float32)
    return float(a / torch.tensor(448.0, dtype=torch.float32))


@dataclass
class DecodeInputs:
    x: torch.Tensor                    # [16, 4096]
    w: Dict[int, torch.Tensor]         # N -> [N, 4096]
    x_scale: float
    w_scale: Dict[int, float]


def decode(seed=SEED) -> DecodeInputs:
    r = rng(seed)
    x = to_dtype(r.standard_normal((max(DECODE_MS), DECODE_K), dtype=np.float32))
    ws = {}
    for n in DECODE_NS:
        ws[n] = to_dtype(r.standard_normal((n, DECODE_K), dtype=np.float32) * np.float32(0.02))
    return DecodeInputs(x, ws, static_scale(x), {n: static_scale(w) for n, w in ws.items()})


@dataclass
class FusedInputs:
    gu_bf16: torch.Tensor              # [M, 2K] gate | up
    gu_fp16: torch.Tensor
    w: torch.Tensor                    # [N, K] bf16
    tiny_groups: np.ndarray = field(default=None)   # bool [M, K/128]
    zero_rows: np.ndarray = field(default=None)


def fused(M=FUSED_M, K=FUSED_K, N=FUSED_N, seed=SEED) -> FusedInputs:
    r = rng(seed)
    gu = r.standard_normal((M, 2 * K), dtype=np.float32)
    G = K // FUSED_GROUP
    tiny = r.random((M, G)) < 0.05
    up = gu[:, K:].reshape(M, G, FUSED_GROUP)
    up[tiny] *= np.float32(1e-5)
    gu[:, K:] = up.reshape(M, K)
    zero_rows = np.arange(M) % 512 == 7
    gu[zero_rows] = 0.0
    w = r.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return FusedInputs(to_dtype(gu, torch.bfloat16), to_dtype(gu, torch.float16),
                       to_dtype(w, torch.bfloat16), tiny, zero_rows)


@dataclass
class MaskedMoEInputs:
    gu: torch.Tensor                   # [E, T, 2 * inter] bf16 gate | up
    rows: np.ndarray                   # int32 [E] live rows per expert
    w: torch.Tensor                    # [E, hidden, inter] bf16


def masked_moe(E=MOE_E, T=MOE_T, hidden=MOE_HIDDEN, inter=MOE_INTER, mean_rows=MOE_MEAN_ROWS,
               seed=SEED) -> MaskedMoEInputs:
    r = rng(seed)
    rows = np.minimum(r.poisson(mean_rows, E), T).astype(np.int32)
    gu = r.standard_normal((E, T, 2 * inter), dtype=np.float32)
    w = np.empty((E, hidden, inter), dtype=np.float32)
    for e in range(E):                 # one expert at a time bounds the fp32 peak
        w[e] = r.standard_normal((hidden, inter), dtype=np.float32) * np.float32(0.02)
    return MaskedMoEInputs(to_dtype(gu), rows, to_dtype(w))


def random_codes(shape, seed=SEED) -> np.ndarray:
    """Uniform random E4M3FN codes, never a NaN pattern (0x7F / 0xFF)."""
    r = rng(seed)
    c = r.integers(0, 254, size=shape, dtype=np.int32)
    c = c + (c >= 0x7F)            # skip 0x7F
    c = c + (c >= 0xFF)            # skip 0xFF
    return c.astype(np.uint8)

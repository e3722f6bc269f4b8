"""Batched and masked forms of the activation quant and the scaled GEMMs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Two page passages ask for a batch dimension on the same arithmetic:

* sglang PR #33533 "[JIT] per_token_group_quant: fix the fp16 UE8M0
  multiplier overflow ..." (commit messages; Speed Tests) has a *masked* mode
  of the group quant, fused with SiLU-and-mul on the EP-MoE decode path:
  tokens are grouped per local expert, each expert's slab has room for M rows
  and a per-expert count says how many of them are live.  The grouped GEMM
  that consumes those codes (a per-expert weight and block scales) is the
  blockwise consumer named in Modifications 3.
* sglang PR #44861 (deterministic static-FP8 linears, Modifications) tests
  the linear with strided 3-D inputs: [batch, rows, K] activations whose
  batch and row strides are not those of a dense 2-D matrix, against one
  shared weight.

Reading taken here (the pages print no formula): batch b owns an [M, ...]
slab of every operand; its live rows are m < m_b with
m_b = clamp(rows[b], 0, M), or M when no counts are given; every live row
is processed exactly as the 2-D operation processes it, with batch b's own
operands (the weight, its scales and the activation scales of batch b, or
the shared ones); rows m >= m_b produce nothing, so whatever the caller's
output held there stays.  Strides are a memory-layout matter, not
arithmetic: the oracle takes the gathered [B, M, ...] values.

The functions below compose the pinned 2-D definitions batch by batch; the
pins of this module (tests/test_oracle_batched.py) are closed forms whose
values differ from batch to batch, count clamping, and permutation
equivariance, so a batch read from the wrong slab, a count not clamped or a
shared operand indexed per batch fails one of them.
"""
import numpy as np

from . import gemm, quant

F32 = np.float32


def valid_rows(rows, nbatch, M):
    """m_b = clamp(rows[b], 0, M) per batch; M for every batch when rows is None."""
    if rows is None:
        return np.full(nbatch, M, dtype=np.int64)
    r = np.asarray(rows, dtype=np.int64).reshape(-1)
    if r.size != nbatch:
        raise ValueError("one row count per batch")
    return np.clip(r, 0, M)


def quant_group_batched(x32, group, pow2=False, fused=False, rows=None):
    """Group / per-token quant of each batch's live rows.

    x32: float32 [B, M, K] (or [B, M, 2K] = [gate | up] when fused).
    Returns one GroupQuant per batch holding only its m_b live rows.
    """
    x32 = np.asarray(x32, dtype=F32)
    B, M = x32.shape[:2]
    mb = valid_rows(rows, B, M)
    out = []
    for b in range(B):
        xb = x32[b, :mb[b]]
        out.append(quant.quant_group_silu_mul(xb, group, pow2) if fused
                   else quant.quant_group(xb, group, pow2))
    return out


def quant_static_batched(x32, s):
    """Static per-tensor quant of every row of every batch, one shared scale."""
    x32 = np.asarray(x32, dtype=F32)
    return np.stack([quant.quant_static(x32[b], s) for b in range(x32.shape[0])])


def scaled_mm_batched(a_codes, b_codes, sa, sb, rows=None, bias=None, out="bf16"):
    """Rowwise / per-tensor GEMM of each batch's live rows.

    a_codes [B, M, K]; b_codes [N, K] (one shared weight) or [B, N, K] (one
    weight per batch).  Scales are given per batch, shared ones repeated:
    sa [B] (a scalar per batch) or [B, M] (per row); sb [B] or [B, N].
    bias: None or [N] output-dtype values, shared.  Returns one MMResult per
    batch with its m_b rows.
    """
    a_codes = np.asarray(a_codes)
    B, M = a_codes.shape[:2]
    per_b = np.asarray(b_codes).ndim == 3
    mb = valid_rows(rows, B, M)
    sa = np.asarray(sa, dtype=F32)
    sb = np.asarray(sb, dtype=F32)
    if sa.shape[0] != B or sb.shape[0] != B:
        raise ValueError("scales are given per batch")
    res = []
    for b in range(B):
        sab = sa[b, :mb[b]] if sa.ndim == 2 else sa[b]
        bb = b_codes[b] if per_b else b_codes
        res.append(gemm.scaled_mm(a_codes[b, :mb[b]], bb, sab, sb[b], bias=bias, out=out))
    return res


def blockwise_mm_batched(a_codes, a_scale, b_codes, b_scale, rows=None, block=128):
    """1x128-group x 128x128-block GEMM of each batch's live rows.

    a_codes [B, M, K], a_scale [B, M, ceil(K/128)] (fp32 values of the group
    scales); b_codes [N, K] or [B, N, K] with b_scale [NB, KB] or [B, NB, KB].
    Returns one MMResult per batch with its m_b rows.
    """
    a_codes = np.asarray(a_codes)
    B, M = a_codes.shape[:2]
    per_b = np.asarray(b_codes).ndim == 3
    mb = valid_rows(rows, B, M)
    res = []
    for b in range(B):
        bb = b_codes[b] if per_b else b_codes
        bs = b_scale[b] if per_b else b_scale
        res.append(gemm.blockwise_mm(a_codes[b, :mb[b]], np.asarray(a_scale)[b, :mb[b]], bb, bs,
                                     block=block))
    return res

"""Load-time preparation of a fused per-tensor FP8 weight.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The prhub digest of sglang PR #33148 (key source excerpts, the linear's
process_weights_after_loading) calls two routines whose bodies the page does
not print:

* requantize_with_max_scale(weight, weight_scale, logical_widths) returns the
  largest of the per-partition weight scales and the weight requantized to it.
  A fused weight (e.g. Q, K and V stacked along the output channels) holds one
  row block per logical partition, each quantized with its own per-tensor
  scale.  Reading taken: partition i's codes are decoded exactly, scaled back
  with their own scale in fp32, and quantized again with the static per-tensor
  rule of the same digest against the maximum scale:

      s_max = max_i s_i
      w     = RN32(dec(q) * s_i)
      q'    = E4M3(clamp(RN32(w * RN32(1 / s_max)), -448, 448))

  so one scalar (s_max) then serves the whole fused weight.
* convert_to_channelwise(scales, logical_widths) broadcasts one scalar per
  partition to the output channels of that partition (the page's comment:
  the scalar weight scale made per-channel), giving the [N] column scales the
  rowwise GEMM takes.

The activation side of the same excerpt keeps input_scale.max(), the largest
per-partition activation scale; that is the same maximum.

Pins: tests/test_oracle_weights.py -- a partition already at the maximum
scale keeps its codes (closed form), power-of-two scale ratios give the codes
of dec(q) * 2^-j exactly, torch's own float8_e4m3fn casts and fp32 arithmetic
reproduce the codes on random scales, and the channelwise broadcast has its
closed form.
"""
import numpy as np

from . import e4m3
from .quant import quant_static

F32 = np.float32


def _offsets(widths, n):
    w = np.asarray(widths, dtype=np.int64).reshape(-1)
    if np.any(w < 0) or int(w.sum()) != n:
        raise ValueError("logical widths must be non-negative and sum to the rows")
    return np.concatenate([[0], np.cumsum(w)])


def requantize_with_max_scale(codes, scales, widths):
    """codes uint8 [N, K] (E4M3FN), scales fp32 [P] per partition, widths [P]
    summing to N.  Returns (s_max as fp32, requantized codes [N, K])."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=F32).reshape(-1)
    off = _offsets(widths, codes.shape[0])
    if scales.size != off.size - 1:
        raise ValueError("one scale per partition")
    s_max = F32(np.max(scales))
    out = np.empty_like(codes)
    for i in range(scales.size):
        blk = codes[off[i]:off[i + 1]]
        w = (e4m3.decode(blk).astype(F32) * scales[i]).astype(F32)
        out[off[i]:off[i + 1]] = quant_static(w, s_max).reshape(blk.shape)
    return s_max, out


def convert_to_channelwise(scales, widths):
    """One scalar per partition -> fp32 [N], channel n of partition i = s_i."""
    scales = np.asarray(scales, dtype=F32).reshape(-1)
    w = np.asarray(widths, dtype=np.int64).reshape(-1)
    if scales.size == 1 and w.size > 1:
        scales = np.repeat(scales, w.size)
    if scales.size != w.size or np.any(w < 0):
        raise ValueError("one scale per partition")
    return np.repeat(scales, w).astype(F32)

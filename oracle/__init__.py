"""CPU oracle for the FP8 (E4M3FN) activation-quant + scaled-GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the C-ABI library,
its HIP kernels or the Python binding) may import, call or link anything in
this package; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path: the two meet only in the seeded synthetic inputs both are fed.

What it computes, and where each definition comes from (pages are cited by
title and section):

* ``e4m3``   -- exact decode of OCP FP8 E4M3FN codes and round-to-nearest-even
               encode, written as a nearest-value search.  Format named in
               "Route large SM90 row/column-scaled FP8 GEMMs to Torch"
               (Summary); the tie example (168 -> 160, one fp32 ulp above ->
               176) is in sglang PR #33533 "[JIT] per_token_group_quant: fix
               the fp16 UE8M0 multiplier overflow ..." (Motivation).
* ``quant``  -- per-token / per-1x128-group activation quant with fp32 or
               UE8M0 (power-of-two) scales, fused SiLU-and-mul, static
               per-tensor quant, per-channel and 128x128-block weight quant
               (PR #33533: commit messages, Motivation, Modifications 1-2;
               prhub digest of sglang PR #33148, implementation section).
* ``gemm``   -- rowwise / per-tensor / blockwise scaled GEMM: exact fp64
               accumulation of decoded codes, scales applied, one rounding
               to bf16 ("Route large SM90 ..." Summary; PR #33148 digest,
               key source excerpts).
* ``bf16``   -- round-to-nearest-even from float64 to bfloat16.
* ``fp16``   -- round-to-nearest-even from float64 to IEEE half.
* ``weights`` -- load-time preparation of a fused per-tensor weight:
               requantization of every logical partition to the largest
               partition scale, and the per-partition scalar broadcast to
               per-channel scales (prhub digest of PR #33148, key source
               excerpts).
* ``scatter`` -- the 1x128 group quant with a scattered output: each token's
               codes and scales written to its top-k destination rows
               (PR #33533 commit messages, the scatter fusion).
* ``batched`` -- the batched / masked forms: each batch's live rows (a
               per-batch count, clamped to the slab) go through the 2-D
               definitions with that batch's operands (PR #33533 commit
               messages and Speed Tests: the masked fused quant of the EP-MoE
               path; sglang PR #44861 Modifications: strided 3-D inputs).

Every function states which pins in ``tests/test_oracle_*.py`` tie it to
something other than itself.
"""
from . import e4m3, bf16, quant, gemm  # noqa: F401

/*
 * fp8sm -- FP8 (E4M3FN) activation quant + scaled GEMM for MI355X (gfx950).
 *
 * C ABI of libfp8sm.so.  Every pointer argument named x, q, A, B, C, scale(s),
 * sa, sb is a DEVICE pointer owned by the caller; the library allocates no
 * device memory, never synchronizes, and enqueues its kernels on the caller's
 * stream.  Results are valid once that stream has run them.  All arguments are
 * validated on the host before anything is launched; a non-OK status means
 * nothing was enqueued.  The library never aborts or throws.
 *
 * Pages cited (by title and section):
 *  [P1] sglang PR #34318 "Route large SM90 row/column-scaled FP8 GEMMs to Torch"
 *  [P2] sglang PR #44861 (SM12x deterministic static-FP8 linears)
 *  [P3] prhub digest of sglang PR #33148 (SM90 per-tensor FP8 -> FlashInfer)
 *  [P4] sglang PR #33533 "[JIT] per_token_group_quant: fix the fp16 UE8M0
 *       multiplier overflow, 1.23x on the fused EP-MoE path, unify the scale
 *       allocation"
 *
 * Number format: OCP FP8 E4M3FN codes, one byte each (max 448, no infinities,
 * 0x7F / 0xFF are NaN) -- the input type required in [P1] Summary.  gfx950
 * converts to and from this format natively; the gfx94x FNUZ variant that
 * [P4] Modifications 3 warns about is not supported.
 */
#ifndef FP8SM_H
#define FP8SM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8SM_OK = 0,
  FP8SM_ERR_NULL = 1,        /* a required pointer is NULL                      */
  FP8SM_ERR_SHAPE = 2,       /* negative/zero size, ld < row length, bad group */
  FP8SM_ERR_ALIGN = 3,       /* a pointer, leading dimension or size breaks the
                                16-byte alignment rule of the call             */
  FP8SM_ERR_UNSUPPORTED = 4, /* enum value or combination not supported        */
  FP8SM_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch       */
  FP8SM_ERR_DEVICE = 6,      /* current device is not gfx950, or no device     */
  FP8SM_ERR_RANGE = 7        /* size beyond what the call supports             */
} fp8sm_status;

typedef enum { FP8SM_BF16 = 0, FP8SM_FP16 = 1 } fp8sm_dtype;

/* Scale rounding and storage ([P4] Modifications 3: rounding, storage and
 * layout are three separate choices, named explicitly by the caller).       */
typedef enum {
  FP8SM_SCALE_FP32 = 0,        /* s = RN32(amax / 448), stored as float      */
  FP8SM_SCALE_UE8M0_FP32 = 1,  /* 2^ceil(log2 s), stored as float            */
  FP8SM_SCALE_UE8M0_BYTE = 2   /* same power of two, stored as the biased
                                  exponent byte e + 127                      */
} fp8sm_scale_fmt;

typedef enum {
  FP8SM_LAYOUT_ROW_MAJOR = 0,  /* scales[m * G + g]                          */
  FP8SM_LAYOUT_MN_MAJOR = 1    /* scales[g * M_pad + m], M_pad = M rounded up
                                  to a multiple of 4 (group-major, the layout
                                  a grouped consumer reads column by column) */
} fp8sm_scale_layout;

/* Scale kinds of the GEMM operands. */
typedef enum {
  FP8SM_KIND_TENSOR = 0,          /* one fp32 scalar (device pointer)          */
  FP8SM_KIND_ROW = 1,             /* A: fp32 [M], one per row (per token)      */
  FP8SM_KIND_COL = 2,             /* B: fp32 [N], one per output channel       */
  FP8SM_KIND_GROUP128_UE8M0 = 3,  /* A: uint8 [M][ceil(K/128)] biased exponents
                                     (scale 2^(byte-127)) per 1x128 group     */
  FP8SM_KIND_GROUP128_FP32 = 4,   /* A: fp32 [M][ceil(K/128)] per 1x128 group  */
  FP8SM_KIND_BLOCK128 = 5         /* B: fp32 [ceil(N/128)][ceil(K/128)] per
                                     128x128 weight block                      */
} fp8sm_scale_kind;

#define FP8SM_FUSE_SILU_MUL 0x1u

/*
 * Per-token or per-1x128-group activation quant ([P4] commit messages and
 * Motivation; the fused form of Modifications 2; the UE8M0 overflow fix of
 * Modifications 1).  For each group of `group` consecutive outputs of a row:
 *   a' = max(max|y|, 1e-10);  s = RN32(a'/448)
 *   FP32 scales:   q = E4M3(clamp(RN32(y * RN32(448/a')), +-448))
 *   UE8M0 scales:  e = ceil(log2 s), q = E4M3(clamp(RN32(y * 2^-e), +-448))
 * with E4M3 round-to-nearest-even.  All scaling is done in fp32 whatever the
 * input dtype, so no multiplier can overflow (the fp16 failure of [P4]).
 *
 *   x      device, bf16 or fp16 (`in`), row-major, M rows, row stride ld_x
 *          elements.  Without FUSE_SILU_MUL a row holds K_out values y.  With
 *          FUSE_SILU_MUL a row holds 2*K_out values [gate | up] and
 *          y = RN32(silu(gate) * up), silu(g) = RN32(g / RN32(1 + e^-g)) with
 *          e^-g the correctly rounded fp32 exponential.
 *   M      rows, >= 0 (0: nothing is launched).
 *   K_out  output columns, > 0, multiple of 8.
 *   ld_x   >= K_out (2*K_out when fused), multiple of 8; x 16-byte aligned.
 *   group  128 (K_out a multiple of 128) or K_out (per token).
 *   flags  0 or FP8SM_FUSE_SILU_MUL.
 *   fmt, lay  scale format and layout (see above).
 *   q      device uint8 [M][ld_q] codes; ld_q >= K_out, multiple of 8;
 *          q 8-byte aligned.
 *   scales device, fp8sm_scale_bytes(fmt, lay, M, K_out, group) bytes.
 * Errors: NULL pointers -> ERR_NULL; sizes -> ERR_SHAPE; alignment ->
 * ERR_ALIGN; unknown enums -> ERR_UNSUPPORTED; non-gfx950 -> ERR_DEVICE.
 */
fp8sm_status fp8sm_quant_group(const void* x, fp8sm_dtype in, int64_t M, int64_t K_out,
                               int64_t ld_x, int32_t group, uint32_t flags,
                               fp8sm_scale_fmt fmt, fp8sm_scale_layout lay,
                               uint8_t* q, int64_t ld_q, void* scales, hipStream_t stream);

/*
 * 1x128 group quant with a scattered output ([P4] commit messages: the
 * scatter fusion of the EP-MoE path).  Token t (row t of x, T rows of K
 * values, K % 128 == 0) is quantized exactly as fp8sm_quant_group quantizes a
 * row with group 128, once; its codes and scales are then written to every
 * destination row d = dst[t][j] (j < topk) with 0 <= d < R of the R-row
 * output: q row d, and scale row d of a fp8sm_scale_bytes(fmt, lay, R, K, 128)
 * buffer (MN-major: [G][R_pad], the grouped GEMM's layout).  Entries of dst
 * outside [0, R) name no row and are skipped (checked on the device); rows no
 * entry names are not written.  Destinations must be distinct (a row named
 * twice is written by two threads: not defined).
 *   dst  device int32 [T][topk], 4-byte aligned; topk 0..1024.
 *   x, q, ld_x, ld_q, in, fmt, lay as fp8sm_quant_group (ld_x >= K).
 * Errors as fp8sm_quant_group; K % 128 != 0 -> ERR_SHAPE.
 */
fp8sm_status fp8sm_quant_group_scatter(const void* x, fp8sm_dtype in, int64_t T, int64_t K,
                                       int64_t ld_x, const int32_t* dst, int32_t topk, int64_t R,
                                       fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, uint8_t* q,
                                       int64_t ld_q, void* scales, hipStream_t stream);

/*
 * Static per-tensor quant with a checkpoint scale ([P3] motivation and key
 * source excerpts: one scalar activation scale per layer):
 *   q = E4M3(clamp(RN32(x * RN32(1/s)), +-448)).
 *   scale  device pointer to one positive fp32 s.
 * Shapes/alignment as fp8sm_quant_group without groups (K multiple of 8).
 */
fp8sm_status fp8sm_quant_static(const void* x, fp8sm_dtype in, int64_t M, int64_t K,
                                int64_t ld_x, const float* scale, uint8_t* q, int64_t ld_q,
                                hipStream_t stream);

/*
 * Weight quant per 128x128 block (the weight side of the blockwise GEMM):
 * for each block, a' = max(max|w|, 1e-10), s = RN32(a'/448),
 * q = E4M3(clamp(RN32(w * RN32(448/a')))).  w: device bf16/fp16 [N][ld_w];
 * q: uint8 [N][ld_q]; scales: fp32 [ceil(N/128)][ceil(K/128)].
 * K multiple of 8, ld_w / ld_q multiples of 8, w 16-byte aligned.
 */
fp8sm_status fp8sm_quant_weight_block128(const void* w, fp8sm_dtype in, int64_t N, int64_t K,
                                         int64_t ld_w, uint8_t* q, int64_t ld_q, float* scales,
                                         hipStream_t stream);

/*
 * Scaled FP8 GEMM, bf16 output, no bias ([P1] Summary: E4M3FN inputs, fp32
 * row/column scales, bf16 output; [P3] key source excerpts: the per-tensor
 * form with two scalar scales):
 *   rowwise / per-tensor:  C[m,n] = bf16( acc[m,n] * sa[m] * sb[n] )
 *   blockwise:             C[m,n] = bf16( sum_kb sa[m,kb] * sb[n/128,kb] * P_kb[m,n] )
 * acc / P_kb are the sums over k (over one 128-wide k block) of
 * dec(A[m,k]) * dec(B[n,k]).  Every product and sum is taken in at least
 * fp32 precision (fp8 operands are widened exactly before the matrix cores),
 * and the reduction order over k is fixed: row m of C depends only on row m of
 * A, B and the scales -- not on M, on the other rows, or on which kernel
 * variant the shape dispatch picked ([P2] Motivation and the reviewers'
 * row-variance check).
 *
 *   A   device uint8 [M][lda] E4M3FN, K contiguous.
 *   B   device uint8 [N][ldb] E4M3FN, K contiguous (the [K, N] column-major
 *       weight of [P3]'s excerpt).
 *   C   device bf16 [M][ldc].
 *   ka/sa, kb/sb  scale kinds and device pointers.  Supported pairs:
 *       {TENSOR, ROW} x {TENSOR, COL}, and {GROUP128_UE8M0, GROUP128_FP32} x
 *       {BLOCK128}.
 * Rules ([P3] implementation section and review: fp8 rows need 16-byte
 * alignment, K % 16, and bf16 output rows N % 8): K % 16 == 0, lda, ldb % 16
 * == 0, A, B 16-byte aligned; N % 8 == 0, ldc % 8 == 0, C 16-byte aligned;
 * M, N >= 0 (0: nothing launched); K >= 0 (K == 0 writes zeros);
 * K <= 65536; lda, ldb <= 2^24 bytes (ERR_RANGE beyond).  Violations return
 * an error status; there is no fallback path.
 * Performance: calls with M <= 64 stream B once and are bound by that stream;
 * a weight stored with ldb = K + 64 instead of K ran 11-13% faster at
 * N = 14336, K = 4096, M = 1..16 and 2-3% faster at N = 4096 (measured).
 * The result does not depend on ldb.
 */
fp8sm_status fp8sm_scaled_mm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                             void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             fp8sm_scale_kind ka, const void* sa, fp8sm_scale_kind kb,
                             const void* sb, hipStream_t stream);

/*
 * Rowwise / per-tensor scaled GEMM with an optional bias and a bf16 or fp16
 * output ([P2] Modifications: the deterministic FP8 linear is tested with
 * bias, BF16/FP16 outputs, strided inputs and K tails; [P3] key source
 * excerpts: the linear's apply() passes an optional bias):
 *   C[m,n] = rnd( RN32( RN32(acc[m,n] * sa[m]) * sb[n] ) + bias[n] )
 * bias: device [N] values of the output dtype (2-byte aligned), widened
 * exactly to fp32 and added in fp32; NULL for none.  out: FP8SM_BF16 or
 * FP8SM_FP16; rnd is round-to-nearest-even to that dtype (fp16 overflows to
 * +-inf).  C holds that dtype.  Arguments, rules, reduction order and row
 * invariance are those of fp8sm_scaled_mm, which equals this call with
 * bias == NULL and out == FP8SM_BF16.  Blockwise scale kinds are accepted
 * only with bias == NULL and out == FP8SM_BF16 (else FP8SM_ERR_UNSUPPORTED).
 */
fp8sm_status fp8sm_scaled_mm_ex(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                fp8sm_scale_kind ka, const void* sa, fp8sm_scale_kind kb,
                                const void* sb, const void* bias, fp8sm_dtype out,
                                hipStream_t stream);

/*
 * Batched forms.  A batch is nbatch (0..65535) problems of one shape; batch b
 * reads and writes every operand at that operand's base pointer + b * its
 * batch stride (strides >= 0, in elements of the operand; a stride of 0
 * shares the operand between batches).  Two uses from the pages:
 *  - strided 3-D activations [nbatch, M, K] against one weight ([P2]
 *    Modifications: the deterministic linear is tested with strided 3-D
 *    inputs): bs_x / bs_a is the batch stride, ld_x / lda the row stride;
 *  - the masked per-expert form of the EP-MoE decode path ([P4] commit
 *    messages and Speed Tests: the fused SiLU-and-mul group quant, masked):
 *    `rows` is a DEVICE int32 [nbatch] array of live rows per batch (expert);
 *    batch b processes rows m < clamp(rows[b], 0, M) and leaves the outputs
 *    of its other rows (codes, scales, C rows) untouched.  NULL: all M rows.
 *    The counts are read on the device, so the call needs no host sync and
 *    can be captured in a graph.
 * Every live row gives bitwise the result the 2-D call gives for that row
 * with batch b's operands.  Output batch strides must keep batches disjoint
 * (stride >= (M - 1) * ld + row length when nbatch > 1, else ERR_SHAPE).
 * Inputs may overlap.  Batch strides obey the alignment of the matching
 * leading dimension (ERR_ALIGN otherwise); a negative stride or nbatch is
 * ERR_SHAPE, nbatch > 65535 is ERR_RANGE; rows must be 4-byte aligned.
 * Other arguments and errors are those of the 2-D call.
 */

/* fp8sm_quant_group per batch.  x: [nbatch][M][ld_x] with batch stride bs_x
 * elements; q: batch stride bs_q bytes; scales: nbatch consecutive blocks of
 * fp8sm_scale_bytes(fmt, lay, M, K_out, group) bytes each (batch-outermost,
 * so the MN-major layout is [nbatch][G][M_pad], the per-expert column-major
 * form a grouped GEMM reads). */
fp8sm_status fp8sm_quant_group_batched(const void* x, fp8sm_dtype in, int64_t nbatch, int64_t M,
                                       int64_t K_out, int64_t bs_x, int64_t ld_x,
                                       const int32_t* rows, int32_t group, uint32_t flags,
                                       fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, uint8_t* q,
                                       int64_t bs_q, int64_t ld_q, void* scales,
                                       hipStream_t stream);

/* fp8sm_quant_static per batch, one shared scale (no row counts). */
fp8sm_status fp8sm_quant_static_batched(const void* x, fp8sm_dtype in, int64_t nbatch, int64_t M,
                                        int64_t K, int64_t bs_x, int64_t ld_x,
                                        const float* scale, uint8_t* q, int64_t bs_q,
                                        int64_t ld_q, hipStream_t stream);

/* fp8sm_scaled_mm_ex per batch.  bs_a, bs_b: bytes (bs_b = 0: one weight for
 * every batch, the 3-D linear; > 0: one weight per batch, the grouped
 * per-expert GEMM); bs_c: output elements; bs_sa, bs_sb: elements of the
 * scale kind's type (bytes for GROUP128_UE8M0, floats otherwise), 0 to share:
 * a TENSOR scale with stride 1 is one scalar per batch, ROW / COL vectors,
 * GROUP128 [M][G] and BLOCK128 [NB][KB] arrays repeat per batch.  bias, when
 * given, is shared.  Dispatch picks the kernel from (M, N, K) as for the 2-D
 * call. */
fp8sm_status fp8sm_scaled_mm_batched(int64_t nbatch, const int32_t* rows, const uint8_t* A,
                                     int64_t bs_a, int64_t lda, const uint8_t* B, int64_t bs_b,
                                     int64_t ldb, void* C, int64_t bs_c, int64_t ldc, int64_t M,
                                     int64_t N, int64_t K, fp8sm_scale_kind ka, const void* sa,
                                     int64_t bs_sa, fp8sm_scale_kind kb, const void* sb,
                                     int64_t bs_sb, const void* bias, fp8sm_dtype out,
                                     hipStream_t stream);

/*
 * Load-time preparation of a fused per-tensor weight ([P3] key source
 * excerpts: the weights-after-loading step requantizes the fused weight to
 * its largest partition scale, then broadcasts scalar scales per channel when
 * the rowwise GEMM consumes them).  The weight's N rows are split into nparts
 * (1..16) logical partitions of widths[i] consecutive rows (a HOST int64
 * array summing to N; e.g. the Q, K and V blocks of a fused projection), row
 * block i quantized with the device fp32 scale scales[i] > 0.
 *
 * fp8sm_requantize_max_scale: s_max = max_i scales[i] is written to the
 * device float *max_scale, and every code is requantized against it:
 *   q'[n][k] = E4M3(clamp(RN32(RN32(dec(w[n][k]) * s_i) * RN32(1 / s_max)), +-448))
 * for n in partition i (codes of a partition whose scale is s_max are
 * unchanged).  w, q: device uint8 [N][ldw] / [N][ldq], K % 16 == 0, ldw and
 * ldq multiples of 16, 16-byte aligned; q == w (with ldq == ldw) converts in
 * place, other overlaps are not allowed.  NaN codes are not specified.
 * Errors: widths NULL -> ERR_NULL; nparts out of 1..16 -> ERR_RANGE; a
 * negative width or a sum != N -> ERR_SHAPE; alignment -> ERR_ALIGN.
 */
fp8sm_status fp8sm_requantize_max_scale(const uint8_t* w, int64_t ldw, int64_t N, int64_t K,
                                        const int64_t* widths, int32_t nparts,
                                        const float* scales, uint8_t* q, int64_t ldq,
                                        float* max_scale, hipStream_t stream);

/*
 * Per-partition scalars broadcast per output channel: out[n] = scales[i] for
 * every row n of partition i (widths: HOST int64 [nparts], nparts 1..16).
 * scales: device fp32 [nparts]; out: device fp32 [sum of widths].  To give
 * every channel the requantized scale, pass max_scale with nparts = 1 and the
 * total width.
 */
fp8sm_status fp8sm_scales_to_channelwise(const float* scales, const int64_t* widths,
                                         int32_t nparts, float* out, hipStream_t stream);

/*
 * The fused product alone, in fp32: y[m][k] = RN32(silu(x[m][k]) * x[m][K_out+k])
 * with the same silu as fp8sm_quant_group's FUSE_SILU_MUL ([P4] Modifications
 * 2).  x: device bf16/fp16 [M][ld_x], ld_x >= 2*K_out; y: device fp32
 * [M][ld_y].  K_out, ld_x, ld_y multiples of 8; x 16-byte, y 16-byte aligned.
 */
fp8sm_status fp8sm_silu_mul_f32(const void* x, fp8sm_dtype in, int64_t M, int64_t K_out,
                                int64_t ld_x, float* y, int64_t ld_y, hipStream_t stream);

/* Bytes needed for the scales of fp8sm_quant_group (0 on invalid input). */
size_t fp8sm_scale_bytes(fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, int64_t M, int64_t K_out,
                         int32_t group);

/* Static description of a status code. */
const char* fp8sm_status_str(fp8sm_status status);

/*
 * Test hook: force fp8sm_scaled_mm's rowwise/per-tensor dispatch to kernel
 * variant `id` (see fp8sm_variant_name), or -1 for the measured table.
 * Returns the previous setting.  Used to check that rows are bitwise identical
 * whichever variant computes them.  Not thread-safe; process-wide.
 */
int fp8sm_force_variant(int id);

/* Number of rowwise/per-tensor GEMM variants, and a name for each. */
int fp8sm_variant_count(void);
const char* fp8sm_variant_name(int id);

/* Variant the dispatch table picks for a shape (no launch, no validation). */
int fp8sm_pick_variant(int64_t M, int64_t N, int64_t K);

/* Test hook: 1 if variant `id` computes rowwise/per-tensor calls of this
 * shape, else 0 (a forced variant that does not is ERR_UNSUPPORTED).  The
 * decode variants bound M (32 or 64); the tile variants take any shape
 * the call accepts. */
int fp8sm_variant_accepts(int id, int64_t M, int64_t N, int64_t K);

/*
 * Test hook (evidence, not part of the path): the rowwise / per-tensor GEMM
 * of fp8sm_scaled_mm computed on the fp8 matrix instructions
 * (v_mfma_f32_32x32x64_f8f6f4, e4m3 x e4m3) instead of the bf16 ones.  These
 * instructions sum each run of products with the smaller ones truncated well
 * below fp32 precision (fp8sm_mfma_probe measures it), so outputs that nearly
 * cancel miss the accuracy bound of the pages' GEMM ([P1] Summary: fp32
 * accumulation of E4M3FN products); the shape dispatch never uses it, and
 * its rows need not equal fp8sm_scaled_mm's.  Arguments, rules and errors are
 * those of fp8sm_scaled_mm; blockwise kinds -> ERR_UNSUPPORTED.
 */
fp8sm_status fp8sm_scaled_mm_fp8mfma(const uint8_t* A, int64_t lda, const uint8_t* B,
                                     int64_t ldb, void* C, int64_t ldc, int64_t M, int64_t N,
                                     int64_t K, fp8sm_scale_kind ka, const void* sa,
                                     fp8sm_scale_kind kb, const void* sb, hipStream_t stream);

/*
 * Test hook: one wavefront executes one matrix instruction with a zero
 * accumulator on register images given by the caller, and writes the result
 * registers back -- the probe of how each instruction sums its products (the
 * reason the GEMMs widen fp8 to bf16 before the matrix cores, [P1] Summary:
 * fp32 accumulation).
 *   instr  0: v_mfma_f32_16x16x32_bf16      (a, b: 4 dwords/lane; d: 4 floats)
 *          1: v_mfma_f32_32x32x16_bf16      (a, b: 4 dwords/lane; d: 16 floats)
 *          2: v_mfma_f32_16x16x128_f8f6f4   (e4m3 x e4m3; 8 dwords; d: 4 floats)
 *          3: v_mfma_f32_32x32x64_f8f6f4    (e4m3 x e4m3; 8 dwords; d: 16 floats)
 *          4: v_mfma_f32_16x16x32_fp8_fp8   (2 dwords; d: 4 floats)
 *   a_regs, b_regs  device uint32 [64][8]: lane-major register images of the
 *          instruction's first and second operands (unused dwords ignored).
 *   d_regs device float [64][16]: lane-major result registers (unused ones 0).
 * All three 16-byte aligned.  Errors: instr out of range -> ERR_UNSUPPORTED;
 * NULL -> ERR_NULL; alignment -> ERR_ALIGN.
 */
fp8sm_status fp8sm_mfma_probe(int32_t instr, const uint32_t* a_regs, const uint32_t* b_regs,
                              float* d_regs, hipStream_t stream);

/*
 * Test hook (evidence, not part of the path): the matrix pipe's throughput
 * ceiling for the GEMMs' inner loop.  A grid of `blocks` workgroups of
 * 64 * waves_per_block threads; every wavefront runs `iters` iterations of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands
 * (2 * 32 * 32 * 16 * 4 flops per iteration), with widen = 1 also sixteen
 * v_cvt_scalef32_pk_bf16_fp8 per iteration whose results are the next
 * iteration's operands (the GEMMs' widen-to-matrix ratio for a 64 x 64
 * wavefront tile; the operand values are then arbitrary bit patterns, NaN
 * included).  Reads no memory, so it measures issue rate near the rated
 * clock, not the power-limited clock of real operands streaming from memory
 * (the GEMMs on real data run measurably slower than on constant codes).
 * The caller times the launch (the dense bf16 peak, [P1] Kernel results'
 * compute-bound shapes, is the reference).
 *   sink   device float [blocks * 64 * waves_per_block], 4-byte aligned:
 *          one value per lane, written so no work is optimized away.
 * Errors: widen not 0/1 or waves_per_block not 4, 8 or 16 -> ERR_UNSUPPORTED;
 * NULL -> ERR_NULL; blocks or iters < 1 -> ERR_SHAPE; blocks > 65536 or
 * iters > 2^24 -> ERR_RANGE.
 */
fp8sm_status fp8sm_rate_probe(int32_t widen, int32_t blocks, int32_t waves_per_block,
                              int32_t iters, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8SM_H */

// Scaled E4M3FN GEMM kernels for gfx950, bf16 output.
//
// Operation ("Route large SM90 row/column-scaled FP8 GEMMs to Torch", Summary;
// prhub digest of sglang PR #33148, key source excerpts for the per-tensor
// form): C[m,n] = bf16(acc[m,n] * sa[m] * sb[n]), acc = sum_k A[m,k] * B[n,k],
// A [M][lda] and B [N][ldb] E4M3FN with K contiguous.
//
// Arithmetic of the rowwise / per-tensor path, identical in every variant so a
// row of C never depends on M, on its neighbours or on the variant the shape
// dispatch picked (the property sglang PR #44861's reviewers checked row by
// row):
//  * fp8 codes are widened exactly to bf16 in registers and multiplied on the
//    bf16 matrix cores (v_mfma_f32_32x32x16_bf16).  The fp8 matrix
//    instructions sum each run of 8 products with the smaller ones truncated
//    ~13 bits below the largest (measured through fp8sm_mfma_probe), far
//    outside fp32 accumulation; the bf16 instruction keeps fp32 precision.
//  * K is walked in 64-wide chunks, ascending; positions past K hold zero
//    codes.  Within a chunk, matrix step s (0..3) multiplies the 16 positions
//    k = 32h + 8s + j, h = 0, 1, j = 0..7 (lane half h of the instruction
//    holds k = 32h .. 32h + 31 of its row), one instruction per 32 x 32
//    output subtile: the step adds the 16 products to its accumulator operand
//    and rounds once to fp32.
//  * The chunks are grouped in blocks of kBlockChunks (512 K).  A block's
//    fp32 partial starts at +0 and is chained through the block's 32 steps;
//    it is then added (fp32, round to nearest) into the output's fp32 master,
//    which starts at +0; blocks ascending.  (One fp32 chain over all of K lets
//    the accumulator reach ~3e5 code-product units on the H3 workloads, whose
//    rounding left one gate/up output beyond the accuracy bound; per-block
//    partials keep the chain's magnitude, and so its rounding, several times
//    smaller.  Blocks are also what lets the decode kernel run several
//    chains at once without changing any result.)
//  * Epilogue: bf16_rne((master * sa[m]) * sb[n]).
//
// Blockwise (1x128 activation groups x 128x128 weight blocks): a fresh fp32
// partial per 128-wide K block, multiplied by sa[m,kb] * sb[n/128,kb] in fp64
// and accumulated in an fp64 master; bf16 of the master at the end.  With
// UE8M0 activation scales the power of two sa[m,kb] is applied exactly while
// widening A, so only the weight scale, one per tile and block, multiplies
// the partial; that kernel uses v_mfma_f32_32x32x16_bf16 (near-fp32 sums,
// measured like the 16x16 instruction) and its own K order, since blockwise
// rows are compared with the oracle, not with the rowwise variants.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace fp8sm {

constexpr int kChunk = 64;        // K bytes per pipeline stage / canonical chunk
constexpr int kBlockChunks = 8;   // chunks per fp32 partial of the rowwise path (512 K)

__device__ __forceinline__ bf16x8 widen_e4m3_x8(uint32_t d0, uint32_t d1) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ bf16x8 widen_e4m3_x8_scaled(uint32_t d0, uint32_t d1, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Same chunk with A as the first operand (blockwise kernel: lane l has column
// 16j + l%16 and rows 16i + 4(l/16) .. +3).
template <int TM, int TN>
__device__ __forceinline__ void mma_chunk64(const uint4 (&fa)[TM], const uint4 (&fb)[TN],
                                            f32x4 (&acc)[TM][TN]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    bf16x8 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = s == 0 ? widen_e4m3_x8(fa[i].x, fa[i].y) : widen_e4m3_x8(fa[i].z, fa[i].w);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = s == 0 ? widen_e4m3_x8(fb[j].x, fb[j].y) : widen_e4m3_x8(fb[j].z, fb[j].w);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// 32 x 32 chunk of the UE8M0 blockwise path.  A 64-wide K chunk is four
// v_mfma_f32_32x32x16_bf16 steps.  Lane half
// h = lane / 32 holds k = 32h .. 32h + 31 of its row (two 16-byte pieces),
// and step s multiplies k = 32h + 8s .. 32h + 8s + 7 of both halves.  B is the
// instruction's first operand, so in a 32 x 32 output subtile lane l holds
// output row l % 32 and the columns 8v + 4h .. 8v + 4h + 3 in
// acc[4v .. 4v + 3], v = 0..3, which the epilogue stores as 8-byte writes.
struct Frag32 {
  uint4 q[2];  // a lane's 32 bytes of one row of a chunk
};

template <bool SCALED, int S>
__device__ __forceinline__ bf16x8 widen_step(const Frag32& f, float scale) {
  const uint4 v = f.q[S >> 1];
  const uint32_t d0 = (S & 1) ? v.z : v.x, d1 = (S & 1) ? v.w : v.y;
  if constexpr (SCALED) return widen_e4m3_x8_scaled(d0, d1, scale);
  return widen_e4m3_x8(d0, d1);
}

// FRESH: the step starts a new partial (C = +0 instead of the accumulator).
template <int TM, int TN, bool SCALED, int S, bool FRESH = false>
__device__ __forceinline__ void mma32_step(const Frag32 (&fa)[TM], const float (&asc)[TM],
                                           const Frag32 (&fb)[TN], f32x16 (&acc)[TM][TN]) {
  bf16x8 a[TM], b[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a[i] = widen_step<SCALED, S>(fa[i], asc[i]);
#pragma unroll
  for (int j = 0; j < TN; ++j) b[j] = widen_step<false, S>(fb[j], 1.0f);
  const f32x16 zero = {};
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], FRESH ? zero : acc[i][j], 0, 0, 0);
}

// master += partial, elementwise in fp32 (the end of a canonical block).
template <int TM, int TN>
__device__ __forceinline__ void promote_block(const f32x16 (&acc)[TM][TN], f32x16 (&mast)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) mast[i][j][v] = mast[i][j][v] + acc[i][j][v];
}

// With SCALED, A row subtile i is widened times asc[i], a power of two: the
// widen is exact (every finite E4M3 value times 2^e, |e| <= 100, is a bf16
// value), so products and fp32 sums are the unscaled ones times 2^e.
// FRESH: the chunk opens a K block, whose partial starts from zero.
template <int TM, int TN, bool SCALED, bool FRESH = false>
__device__ __forceinline__ void mma32_chunk(const Frag32 (&fa)[TM], const float (&asc)[TM],
                                            const Frag32 (&fb)[TN], f32x16 (&acc)[TM][TN]) {
  mma32_step<TM, TN, SCALED, 0, FRESH>(fa, asc, fb, acc);
  mma32_step<TM, TN, SCALED, 1>(fa, asc, fb, acc);
  mma32_step<TM, TN, SCALED, 2>(fa, asc, fb, acc);
  mma32_step<TM, TN, SCALED, 3>(fa, asc, fb, acc);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float rowwise_epilogue(float acc, float sa, float sb) {
  const float v = acc * sa;
  return v * sb;
}

// Rowwise epilogue variants: EPI_F16 writes fp16 instead of bf16, EPI_BIAS
// adds bias[c] (a value of the output dtype, widened exactly) in fp32 before
// the final rounding: out = rnd(RN32(RN32(acc * sa) * sb) + bias).
enum { EPI_F16 = 1, EPI_BIAS = 2 };

// Both conversions are the hardware's round-to-nearest-even (overflow to
// +-inf); the bf16 one (v_cvt_pk_bf16_f32) equals f32_to_bf16_rne for every
// fp32 value that is not NaN (checked over all 2^32 patterns on gfx950).
template <int EPI>
__device__ __forceinline__ uint16_t epi_round(float v) {
  if constexpr ((EPI & EPI_F16) != 0)
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  else
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int EPI>
__device__ __forceinline__ float epi_value(float acc, float sa, float sb,
                                           const uint16_t* __restrict__ bias, int c) {
  float v = rowwise_epilogue(acc, sa, sb);
  if constexpr ((EPI & EPI_BIAS) != 0) {
    if constexpr ((EPI & EPI_F16) != 0)
      v = v + (float)__builtin_bit_cast(_Float16, bias[c]);
    else
      v = v + __uint_as_float((uint32_t)bias[c] << 16);
  }
  return v;
}

// Scale and store one lane's four consecutive outputs of row r (columns c..c+3,
// c a multiple of 4; N % 8 == 0 so all four are in range when c < N).
template <int EPI>
__device__ __forceinline__ void store_row4(uint16_t* __restrict__ C, int64_t ldc, int r, int c,
                                           const f32x4& acc, float sar,
                                           const float* __restrict__ sb, int sb_vec,
                                           const uint16_t* __restrict__ bias) {
  float y[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) y[v] = epi_value<EPI>(acc[v], sar, sb[sb_vec ? c + v : 0], bias, c + v);
  uint32_t lo, hi;
  if constexpr ((EPI & EPI_F16) != 0) {
    lo = (uint32_t)epi_round<EPI>(y[0]) | ((uint32_t)epi_round<EPI>(y[1]) << 16);
    hi = (uint32_t)epi_round<EPI>(y[2]) | ((uint32_t)epi_round<EPI>(y[3]) << 16);
  } else {  // two values per conversion instruction
    lo = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)y[0], (__bf16)y[1]});
    hi = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)y[2], (__bf16)y[3]});
  }
  *reinterpret_cast<uint2*>(C + (int64_t)r * ldc + c) = make_uint2(lo, hi);
}

// The same for two consecutive outputs (columns c, c + 1, c even): one 4-byte
// store.
template <int EPI>
__device__ __forceinline__ void store_row2(uint16_t* __restrict__ C, int64_t ldc, int r, int c,
                                           float a0, float a1, float sar,
                                           const float* __restrict__ sb, int sb_vec,
                                           const uint16_t* __restrict__ bias) {
  const float y0 = epi_value<EPI>(a0, sar, sb[sb_vec ? c : 0], bias, c);
  const float y1 = epi_value<EPI>(a1, sar, sb[sb_vec ? c + 1 : 0], bias, c + 1);
  uint32_t v;
  if constexpr ((EPI & EPI_F16) != 0)
    v = (uint32_t)epi_round<EPI>(y0) | ((uint32_t)epi_round<EPI>(y1) << 16);
  else
    v = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)y0, (__bf16)y1});
  *reinterpret_cast<uint32_t*>(C + (int64_t)r * ldc + c) = v;
}

// Hardware places consecutive workgroups on the 8 XCDs in turn; give each XCD
// a contiguous range of logical tiles (so tiles sharing A / B panels share an
// L2), then walk the logical tiles in groups of kGroupM tile rows.
__device__ __forceinline__ void tile_coords(int bid, int nbid, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  constexpr int kXcd = 8, kGroupM = 8;
  const int xcd = bid % kXcd, idx = bid / kXcd;
  const int lid = xcd * (nbid / kXcd) + min(xcd, nbid % kXcd) + idx;
  const int per_group = kGroupM * tiles_n;
  const int group = lid / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = lid - group * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// Fourth word of a raw buffer resource on gfx9-family chips (gfx950): 32-bit
// data format, no swizzle, no per-lane index.
constexpr int kBufferWord3 = 0x00020000;

// 16 zero bytes: the DMA source for chunk positions past K.
__device__ __attribute__((aligned(16))) uint8_t g_zero16[16];

// 16-byte global -> LDS copy (global_load_lds_dwordx4).  Issued as inline asm
// so the compiler does not wait for every such copy before each LDS read; the
// kernel waits for exactly the stages it needs with wait_vmcnt.  lds_addr is
// the wave-uniform LDS byte address of lane 0's destination; lane i writes
// lds_addr + 16 i.
// m0 is clobbered on purpose: these kernels use it for nothing else.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_addr), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS chunk swizzle for 64-byte rows: the 16-byte chunk c of row r is stored
// at position c ^ swz16(r mod 16).  A 16-lane group reading the same chunk of
// 16 consecutive rows (and any 8-lane phase of it) then hits distinct banks.
__device__ __forceinline__ int swz16(int x) { return ((x >> 1) ^ (x >> 3)) & 3; }

// LDS byte offset of piece q (0, 1) of this lane's 32 bytes within a 64-byte
// chunk row of a 32-row subtile (subtiles start at multiples of 16 rows).
// Each 8-lane phase of a 16-byte read then covers 8 consecutive rows and hits
// 8 distinct bank groups.
__device__ __forceinline__ int frag32_off(int lane, int q) {
  return (lane & 31) * kChunk + ((((lane >> 5) * 2 + q) ^ swz16(lane & 15)) << 4);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor starting at base (wave-uniform, so it lives in SGPRs);
// byte offsets below 2^31 are in range.
__device__ __forceinline__ i32x4 sgpr_rsrc(const void* base) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));  // stride field 0
  r[2] = 0x7FFFFFFF;
  r[3] = kBufferWord3;
  return r;
}

// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds): reads
// base + voff + soff, lane i writes lds_addr + 16 i.  Inline asm for the same
// reason as dma16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_buf(uint32_t voff, i32x4 rsrc, int soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy plan of one wavefront for a ring stage of the BM + BN row tile (A rows
// then B rows): copy i of wavefront w (of NW) fills 16-row segment NW i + w;
// lane l copies row 16 seg + l/4, 16-byte piece (l%4) ^ swz16(l/4) of the
// 64-byte chunk, so the slot holds swizzled rows.  Rows past M / N repeat the last
// row.  Whole chunks are copied by buffer loads from a per-segment SGPR
// descriptor with the chunk offset in a scalar register (no vector
// instruction per copy; row strides <= 2^24 keep 15 rows + K below 2^31);
// a partial last chunk (K % 64 != 0) takes guarded global copies that read
// zeros past K.
template <int DPS, int BM, int NW = 4>
struct DmaPlan {
  i32x4 rs[DPS];     // per-segment descriptor (wave-uniform: SGPRs)
  uint32_t vo[DPS];  // the lane's byte offset from its segment's base
  int koff;          // the lane's 16-byte piece within a chunk row (every segment)

  __device__ __forceinline__ void init(const uint8_t* A, int64_t lda, const uint8_t* B,
                                       int64_t ldb, int m0, int n0, int M, int N, int w,
                                       int lane) {
    const int r = lane >> 2;
    koff = ((lane & 3) ^ swz16(r)) * 16;
#pragma unroll
    for (int i = 0; i < DPS; ++i) {
      const int seg = i * NW + w;
      const bool isa = seg * 16 < BM;
      const uint8_t* base = isa ? A : B;
      const int64_t ld = isa ? lda : ldb;
      const int first = isa ? m0 + seg * 16 : n0 + seg * 16 - BM;
      const int last = (isa ? M : N) - 1;
      const int r0 = min(first, last), rr = min(first + r, last);
      rs[i] = sgpr_rsrc(base + (int64_t)r0 * ld);
      vo[i] = (uint32_t)((int64_t)(rr - r0) * ld) + (uint32_t)koff;
    }
  }

  // copies of the chunk at byte offset kb into the slot at LDS address slot
  __device__ __forceinline__ void issue(uint32_t slot, int kb, int K, int w) const {
    if (kb + kChunk <= K) {
#pragma unroll
      for (int i = 0; i < DPS; ++i) dma16_buf(vo[i], rs[i], kb, slot + (uint32_t)((i * NW + w) * 1024));
    } else {
#pragma unroll
      for (int i = 0; i < DPS; ++i) {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(
            ((uint64_t)(uint32_t)rs[i][1] << 32) | (uint32_t)rs[i][0]);
        const void* p = kb + koff < K ? (const void*)(base + vo[i] + kb) : (const void*)g_zero16;
        dma16(p, slot + (uint32_t)((i * NW + w) * 1024));
      }
    }
  }
};

// Wait until at most `after` ring stages (DPS copies each) issued behind the
// one about to be read are still in flight (0 <= after <= MAXA).
template <int DPS, int MAXA>
__device__ __forceinline__ void wait_stages(int after) {
  if constexpr (MAXA >= 4) {
    if (after >= 4) {
      wait_vmcnt<4 * DPS>();
      return;
    }
  }
  if constexpr (MAXA >= 3) {
    if (after == 3) {
      wait_vmcnt<3 * DPS>();
      return;
    }
  }
  if constexpr (MAXA >= 2) {
    if (after == 2) {
      wait_vmcnt<2 * DPS>();
      return;
    }
  }
  if (after == 1)
    wait_vmcnt<DPS>();
  else
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Rowwise tile kernel: BM x BN workgroup tile, WM x WN wavefronts of 64 x 64
// outputs (2 x 2 subtiles of 32 x 32), 64-wide K chunks in an NSLOT-slot LDS
// ring filled by global->LDS DMA, one barrier per chunk.  Software
// pipelined: the barrier that makes chunk k + 1 visible comes before chunk
// k's matrix work, chunk k + 1's fragments are read right after it (into a
// second register set) while chunk k is multiplied from registers; chunk k's
// slot is then free (every wavefront holds its fragments) and takes the copy
// of chunk k + NSLOT.  Each output keeps a block partial and a master (two
// fp32 registers), which is what bounds a wavefront's tile at 64 x 64 with
// two wavefronts per SIMD.  OCC is the number of workgroups meant to share a
// CU (their waits hide each other's).
template <int BM, int BN, int WM, int WN, int NSLOT, int OCC, int EPI>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_rowwise_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, const float* __restrict__ sa,
    int sa_vec, const float* __restrict__ sb, int sb_vec, const uint16_t* __restrict__ bias,
    int tiles_m, int tiles_n, GemmBatch gb) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int SLOT = ROWS * kChunk;          // bytes per ring slot
  constexpr int SEGS = SLOT / 1024;            // 1 KB segments per slot (16 rows each)
  constexpr int DPS = SEGS / NW;               // DMA instructions per thread per stage
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "wavefront tiles of 32 x 32 subtiles");
  static_assert(NSLOT >= 2 && NSLOT <= 6, "ring depth");
  static_assert(SEGS % NW == 0, "segments must split over the wavefronts");
  static_assert(kBlockChunks % 2 == 0, "fragment sets alternate by chunk parity");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSLOT * SLOT];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  {
    const int64_t bi = blockIdx.y;
    A += bi * gb.a;
    B += bi * gb.b;
    C += bi * gb.c;
    sa += bi * gb.sa;
    sb += bi * gb.sb;
    M = (int)batch_rows(gb.rows, M);
    if (m0 >= M) return;  // the whole workgroup, before any barrier
  }
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WN, wn = w % WN;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);

  DmaPlan<DPS, BM, NW> dma;
  dma.init(A, lda, B, ldb, m0, n0, M, N, w, lane);
  const int nkc = (K + kChunk - 1) / kChunk;
  auto issue = [&](int kc) {
    dma.issue(lds0 + (uint32_t)((kc % NSLOT) * SLOT), kc * kChunk, K, w);
  };

  // fragment read offsets (bytes within a slot): two 16-byte pieces per row
  const int a_off0 = wm * (BM / WM) * kChunk + frag32_off(lane, 0);
  const int a_off1 = wm * (BM / WM) * kChunk + frag32_off(lane, 1);
  const int b_off0 = (BM + wn * (BN / WN)) * kChunk + frag32_off(lane, 0);
  const int b_off1 = (BM + wn * (BN / WN)) * kChunk + frag32_off(lane, 1);
  auto read_frags = [&](int kc, Frag32 (&fa)[TM], Frag32 (&fb)[TN]) {
    const uint8_t* slot = lds + (kc % NSLOT) * SLOT;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      fa[i].q[0] = *reinterpret_cast<const uint4*>(slot + a_off0 + i * 32 * kChunk);
      fa[i].q[1] = *reinterpret_cast<const uint4*>(slot + a_off1 + i * 32 * kChunk);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      fb[j].q[0] = *reinterpret_cast<const uint4*>(slot + b_off0 + j * 32 * kChunk);
      fb[j].q[1] = *reinterpret_cast<const uint4*>(slot + b_off1 + j * 32 * kChunk);
    }
  };

  f32x16 acc[TM][TN], mast[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[i][j][v] = 0.f;
        mast[i][j][v] = 0.f;
      }
  const float one[TM] = {};  // unused scale operand of the unscaled widen

  Frag32 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  for (int c = 0; c < NSLOT - 1 && c < nkc; ++c) issue(c);
  wait_stages<DPS, NSLOT - 2>(min(NSLOT - 2, nkc - 1));
  __syncthreads();  // chunk 0 visible
  if (NSLOT - 1 < nkc) issue(NSLOT - 1);
  read_frags(0, fa0, fb0);
  // chunk kc, whose fragments are in (fa, fb): make chunk kc + 1 visible,
  // start reading it into (na, nb), queue the copy of chunk kc + NSLOT into
  // chunk kc's slot, multiply chunk kc (FRESH: it opens a block)
  auto step = [&](int kc, auto fresh, const Frag32 (&fa)[TM], const Frag32 (&fb)[TN],
                  Frag32 (&na)[TM], Frag32 (&nb)[TN]) {
    constexpr bool F = decltype(fresh)::value;
    if (kc + 1 < nkc) {
      wait_stages<DPS, NSLOT - 2>(min(NSLOT - 2, nkc - 2 - kc));
      __syncthreads();
      if (kc + NSLOT < nkc) issue(kc + NSLOT);
      read_frags(kc + 1, na, nb);
    }
    mma32_chunk<TM, TN, false, F>(fa, one, fb, acc);
  };
  // blocks of kBlockChunks chunks; chunk kc uses fragment set kc % 2
  for (int kb = 0; kb < nkc; kb += kBlockChunks) {
    const int kend = min(kb + kBlockChunks, nkc);
    step(kb, std::true_type{}, fa0, fb0, fa1, fb1);
    int kc = kb + 1;
    for (; kc + 1 < kend; kc += 2) {
      step(kc, std::false_type{}, fa1, fb1, fa0, fb0);
      step(kc + 1, std::false_type{}, fa0, fb0, fa1, fb1);
    }
    if (kc < kend) step(kc, std::false_type{}, fa1, fb1, fa0, fb0);
    promote_block<TM, TN>(acc, mast);
  }

  // lane l holds output row l % 32 of each row subtile and the columns
  // 8v + 4(l / 32) .. +3 of each column subtile in mast[.][.][4v .. 4v + 3]
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = m0 + wm * (BM / WM) + 32 * i + (lane & 31);
    if (r >= M) continue;
    const float sar = sa[sa_vec ? r : 0];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = n0 + wn * (BN / WN) + 32 * j + 8 * v + 4 * (lane >> 5);
        if (c >= N) continue;
        const f32x4 a4 = {mast[i][j][4 * v], mast[i][j][4 * v + 1], mast[i][j][4 * v + 2],
                          mast[i][j][4 * v + 3]};
        store_row4<EPI>(C, ldc, r, c, a4, sar, sb, sb_vec, bias);
      }
  }
}

// ---------------------------------------------------------------------------
// The rowwise GEMM on the fp8 matrix instructions (v_mfma_f32_32x32x64_f8f6f4,
// e4m3 x e4m3): no widening, twice the matrix rate of the bf16 path.  It is
// kept only as measured evidence for the choice of the bf16 path: these
// instructions sum each run of products with the smaller ones truncated far
// below fp32 precision, so the result misses the accuracy bound on outputs
// that nearly cancel.  The shape dispatch never selects it; it is reached
// only through its own test entry point.  Same DMA ring and tile walk as
// gemm_rowwise_kernel; wavefronts of BM/2 x BN/2 in 32 x 32 subtiles; lane
// half h holds k = 32h .. 32h + 31 of each 64-wide chunk for both operands
// (the same register positions carry the same k in A and B, so the products
// pair up whatever order the instruction sums them in).
template <int BM, int BN, int NSLOT, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_rowwise_fp8mfma_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, const float* __restrict__ sa,
    int sa_vec, const float* __restrict__ sb, int sb_vec, int tiles_m, int tiles_n) {
  constexpr int TM = BM / 64, TN = BN / 64;  // 32-row subtiles per wavefront
  constexpr int ROWS = BM + BN;
  constexpr int SLOT = ROWS * kChunk;
  constexpr int SEGS = SLOT / 1024;
  constexpr int DPS = SEGS / 4;
  static_assert(NSLOT >= 2 && NSLOT <= 4, "ring depth");
  static_assert(SEGS % 4 == 0, "segments must split over the four wavefronts");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSLOT * SLOT];
  typedef int i32x8 __attribute__((ext_vector_type(8)));

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);

  DmaPlan<DPS, BM> dma;
  dma.init(A, lda, B, ldb, m0, n0, M, N, w, lane);
  const int nkc = (K + kChunk - 1) / kChunk;
  auto issue = [&](int kc) {
    dma.issue(lds0 + (uint32_t)((kc % NSLOT) * SLOT), kc * kChunk, K, w);
  };
  const int a_off0 = wm * (BM / 2) * kChunk + frag32_off(lane, 0);
  const int a_off1 = wm * (BM / 2) * kChunk + frag32_off(lane, 1);
  const int b_off0 = (BM + wn * (BN / 2)) * kChunk + frag32_off(lane, 0);
  const int b_off1 = (BM + wn * (BN / 2)) * kChunk + frag32_off(lane, 1);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  for (int c = 0; c < NSLOT - 1 && c < nkc; ++c) issue(c);
  for (int kc = 0; kc < nkc; ++kc) {
    const int after = min(NSLOT - 2, nkc - 1 - kc);
    if (after >= 2)
      wait_vmcnt<2 * DPS>();
    else if (after == 1)
      wait_vmcnt<DPS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (kc + NSLOT - 1 < nkc) issue(kc + NSLOT - 1);
    const uint8_t* slot = lds + (kc % NSLOT) * SLOT;
    i32x8 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint4 p = *reinterpret_cast<const uint4*>(slot + a_off0 + i * 32 * kChunk);
      const uint4 q = *reinterpret_cast<const uint4*>(slot + a_off1 + i * 32 * kChunk);
      fa[i] = i32x8{(int)p.x, (int)p.y, (int)p.z, (int)p.w, (int)q.x, (int)q.y, (int)q.z, (int)q.w};
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint4 p = *reinterpret_cast<const uint4*>(slot + b_off0 + j * 32 * kChunk);
      const uint4 q = *reinterpret_cast<const uint4*>(slot + b_off1 + j * 32 * kChunk);
      fb[j] = i32x8{(int)p.x, (int)p.y, (int)p.z, (int)p.w, (int)q.x, (int)q.y, (int)q.z, (int)q.w};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0,
                                                                    0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = m0 + wm * (BM / 2) + 32 * i + (lane & 31);
    if (r >= M) continue;
    const float sar = sa[sa_vec ? r : 0];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = n0 + wn * (BN / 2) + 32 * j + 8 * v + 4 * (lane >> 5);
        if (c >= N) continue;
        const f32x4 a4 = {acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2],
                          acc[i][j][4 * v + 3]};
        store_row4<0>(C, ldc, r, c, a4, sar, sb, sb_vec, nullptr);
      }
  }
}

// fp64 -> bf16 with one rounding (nearest even).  Normal results: rounded to
// 8 significant bits in fp64, then converted exactly.  Below 2^-126 (the bf16
// subnormal range, spacing 2^-133): rounded to a multiple of 2^-133 in fp64,
// which fp32 and then bf16 hold exactly.  Zeros and NaN go through fp32.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  if (!(fabs(x) >= 0x1p-126)) {
    const double r = __builtin_rint(x * 0x1p133) * 0x1p-133;  // nearest even multiple
    return f32_to_bf16_rne((float)r);                         // both conversions exact
  }
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u += ((uint64_t)1 << 44) - 1 + ((u >> 45) & 1);  // round to 8 significant bits
  u &= ~(((uint64_t)1 << 45) - 1);
  return f32_to_bf16_rne((float)__longlong_as_double((long long)u));  // exact now
}

// ---------------------------------------------------------------------------
// Blockwise kernel for 1x128 UE8M0 activation groups and 128x128 fp32 weight
// blocks.  Same ring, chunk order and B-first layout as the rowwise kernel,
// with a 128 x 128 tile (wavefronts of 64 x 64).  The activation scale
// 2^(byte - 127) is applied exactly: its exponent clamped to +-kWidenExp in
// the widen, so each 128-wide K block's fresh fp32 partial already carries
// it, and the rest (bytes below 27 or above 227) with the block's weight
// scale (one value per tile: the tile spans one 128-column weight block) in
// the fp64 factor that adds the partial to an fp64 master.  The tile's scale
// bytes are staged in LDS, SEGB K blocks at a time.
//
// kWidenExp: every finite E4M3 value times 2^e, |e| <= 100, is a bf16 normal,
// every product of two such operands (the weight unscaled) is an fp32 normal,
// and a 128-wide block sum stays below 2^125.
constexpr int kWidenExp = 100;

template <int NSLOT, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_block_ue8m0_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, const uint8_t* __restrict__ ea,
    const float* __restrict__ sbb, int tiles_m, int tiles_n, GemmBatch gb) {
  constexpr int BM = 128, BN = 128, TM = 2, TN = 2;  // 32-row subtiles per wavefront
  constexpr int ROWS = BM + BN;
  constexpr int SLOT = ROWS * kChunk;
  constexpr int SEGS = SLOT / 1024;
  constexpr int DPS = SEGS / 4;
  constexpr int SEGB = 64;  // K blocks of activation scale bytes staged at a time
  // their row stride in LDS: 17 words, so the 32 rows a wavefront reads at
  // once fall in distinct banks (a 16-word stride folded them onto a few)
  constexpr int SEGP = SEGB + 4;
  static_assert(NSLOT >= 2 && NSLOT <= 4, "ring depth");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSLOT * SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t esc[BM * SEGP / 4];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  {
    const int64_t bi = blockIdx.y;
    A += bi * gb.a;
    B += bi * gb.b;
    C += bi * gb.c;
    ea += bi * gb.sa;
    sbb += bi * gb.sb;
    M = (int)batch_rows(gb.rows, M);
    if (m0 >= M) return;  // the whole workgroup, before any barrier
  }
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);

  DmaPlan<DPS, BM> dma;
  dma.init(A, lda, B, ldb, m0, n0, M, N, w, lane);
  const int nkc = (K + kChunk - 1) / kChunk;
  const int nkb = (K + 127) / 128;
  auto issue = [&](int kc) {
    dma.issue(lds0 + (uint32_t)((kc % NSLOT) * SLOT), kc * kChunk, K, w);
  };
  // scale bytes of K blocks kb0 .. kb0 + SEGB - 1 for the tile's rows: thread t
  // copies half a row (32 blocks); rows past M repeat row M - 1
  auto stage_scales = [&](int kb0) {
    const int row = t >> 1, half = t & 1;
    const uint8_t* er = ea + (int64_t)min(m0 + row, M - 1) * nkb;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int kb = kb0 + half * 32 + 4 * q + b;
        v |= (uint32_t)(kb < nkb ? er[kb] : 127) << (8 * b);
      }
      esc[(row * SEGP + half * 32 + 4 * q) / 4] = v;
    }
  };
  const uint8_t* escb = reinterpret_cast<const uint8_t*>(esc);
  const float* sbrow = sbb + (int64_t)tn * nkb;

  const bool live = m0 + wm * (BM / 2) < M;  // wavefront has a live row (uniform)
  const int a_off0 = wm * (BM / 2) * kChunk + frag32_off(lane, 0);
  const int a_off1 = wm * (BM / 2) * kChunk + frag32_off(lane, 1);
  const int b_off0 = (BM + wn * (BN / 2)) * kChunk + frag32_off(lane, 0);
  const int b_off1 = (BM + wn * (BN / 2)) * kChunk + frag32_off(lane, 1);

  f32x16 acc[TM][TN];
  double mast[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[i][j][v] = 0.f;
        mast[i][j][v] = 0.0;
      }
  float asc[TM];
  double sbk[TM] = {};  // per row subtile: weight scale x out-of-window power of two

  for (int c = 0; c < NSLOT - 1 && c < nkc; ++c) issue(c);
  stage_scales(0);  // visible after the first loop barrier
  // one chunk: wait for its copies, barrier, queue the copies NSLOT - 1
  // chunks ahead, read the fragments, multiply (FRESH: the chunk opens a K
  // block and its partial starts from zero, so no register clearing is needed
  // after a promotion)
  auto chunk = [&](int kc, auto fresh) {
    const int after = min(NSLOT - 2, nkc - 1 - kc);
    if (after >= 2)
      wait_vmcnt<2 * DPS>();
    else if (after == 1)
      wait_vmcnt<DPS>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // chunk kc visible to all; slot of chunk kc-1 free
    if constexpr (decltype(fresh)::value) {
      const int kb = kc >> 1;
      if (kb > 0 && kb % SEGB == 0) {  // every wavefront is past the previous segment
        stage_scales(kb);
        __syncthreads();
      }
      // 2^(byte - 127) for any byte: the part of the exponent inside
      // [-100, 100] goes into the widen (exact there), the rest into the
      // fp64 factor of the promotion.
      const double sb64 = (double)sbrow[kb];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int e = (int)escb[(wm * 64 + 32 * i + (lane & 31)) * SEGP + kb % SEGB] - 127;
        const int ein = min(max(e, -kWidenExp), kWidenExp);
        asc[i] = __uint_as_float((uint32_t)(ein + 127) << 23);
        sbk[i] = __builtin_ldexp(sb64, e - ein);
      }
    }
    if (kc + NSLOT - 1 < nkc) issue(kc + NSLOT - 1);
    const uint8_t* slot = lds + (kc % NSLOT) * SLOT;
    Frag32 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      fa[i].q[0] = *reinterpret_cast<const uint4*>(slot + a_off0 + i * 32 * kChunk);
      fa[i].q[1] = *reinterpret_cast<const uint4*>(slot + a_off1 + i * 32 * kChunk);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      fb[j].q[0] = *reinterpret_cast<const uint4*>(slot + b_off0 + j * 32 * kChunk);
      fb[j].q[1] = *reinterpret_cast<const uint4*>(slot + b_off1 + j * 32 * kChunk);
    }
    // a wavefront whose rows all lie past the live rows (a masked expert's
    // few rows) neither multiplies nor promotes: none of its rows is stored
    if (live) mma32_chunk<TM, TN, true, decltype(fresh)::value>(fa, asc, fb, acc);
  };
  // one K block (two chunks; the last block of a K tail may have one) per
  // iteration, then its partial is promoted into the fp64 master
  for (int kc = 0; kc < nkc; kc += 2) {
    chunk(kc, std::true_type{});
    if (kc + 1 < nkc) chunk(kc + 1, std::false_type{});
    if (live)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) mast[i][j][v] = fma((double)acc[i][j][v], sbk[i], mast[i][j][v]);
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = m0 + wm * (BM / 2) + 32 * i + (lane & 31);
    if (r >= M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = n0 + wn * (BN / 2) + 32 * j + 8 * v + 4 * (lane >> 5);
        if (c >= N) continue;
        const double* m4 = &mast[i][j][4 * v];
        const uint32_t lo = (uint32_t)f64_to_bf16_rne(m4[0]) | ((uint32_t)f64_to_bf16_rne(m4[1]) << 16);
        const uint32_t hi = (uint32_t)f64_to_bf16_rne(m4[2]) | ((uint32_t)f64_to_bf16_rne(m4[3]) << 16);
        *reinterpret_cast<uint2*>(C + (int64_t)r * ldc + c) = make_uint2(lo, hi);
      }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 32 * TMD): a workgroup of NWD wavefronts owns PW output
// columns (32, or 16 for twice the workgroups: the 32-row B operand then
// repeats rows 0..15 in lanes 16..31 from the same LDS bytes, and output
// columns 16..31 of the instruction are not stored).  Wavefront w computes
// the canonical blocks w, w + NWD, ... of K, each a fresh partial chained
// through its chunks; after each round of NWD blocks the partials meet in
// LDS and every wavefront adds its slice (16 / NWD of each lane's 16
// accumulator elements) of every partial to its master, in ascending block
// order, and finally stores that slice: the same fp32 operations in the same
// order as the tile kernels, so every row is bitwise identical to theirs,
// while the wavefronts' chains, reductions and stores run side by side.
//
// The weight block (PW rows x 512 bytes) is what streams from HBM.  It is
// copied by global->LDS DMA into the wavefront's own LDS region, pair of
// chunks by pair of chunks (each copy instruction takes 8 rows x 128 bytes:
// whole cache lines), and read back in the matrix layout through a bank
// swizzle; no other wavefront reads the region, so waiting for the
// wavefront's own copies is enough (no barrier).  With one round of blocks
// the matrix steps of each chunk pair start as soon as its copies have
// landed; with several, the copies of a wavefront's next block are issued as
// soon as the current block's fragments are in registers, so they overlap
// its chain.  The few A rows (L2-resident, shared by every workgroup) are
// read straight into registers.
//
// A chunk slot past the wavefront's whole chunks (its block is the last one
// and partial, or it has no block this round) is multiplied with its A
// operand zeroed, which adds exactly +0 to a partial that started at +0; its
// copies re-read the row's first bytes, so no copy leaves the row.  With
// PART (K % 64 != 0) the chunk past the whole chunks is loaded from clamped
// addresses (pieces past K re-read the row's last 16 bytes) and multiplied
// with its A values past K -- and all of them outside the block that owns
// that chunk -- zeroed.
// f(std::integral_constant<int, i>) for i = 0 .. N - 1 (compile-time indices,
// e.g. for wait counts that must be immediates).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

template <int TMD, int NWD, int PW, bool PART, bool REFILL, int EPI>
__global__ __launch_bounds__(64 * NWD) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, const float* __restrict__ sa,
    int sa_vec, const float* __restrict__ sb, int sb_vec, const uint16_t* __restrict__ bias,
    GemmBatch gb) {
  constexpr int D = kBlockChunks;
  constexpr int RB = D * kChunk;   // bytes of a block row (512)
  constexpr int REG = PW * RB;     // a wavefront's LDS region: PW rows of a block
  constexpr int NCP = REG / 1024;  // copy instructions per block (two rows each)
  static_assert(RB == 512, "two block rows per 64-lane copy of 16 bytes each");
  static_assert(PW == 16 || PW == 32, "panel width");
  __shared__ __attribute__((aligned(1024))) uint8_t bls[NWD * REG];
  __shared__ float part[NWD][TMD][16][64];  // element-major: conflict-free slices
  constexpr int EPW = 16 / NWD;              // accumulator elements each wavefront reduces
  static_assert(EPW * NWD == 16 && 4 % EPW == 0, "slices of the 16 accumulator elements");
  {
    const int64_t bi = blockIdx.y;
    A += bi * gb.a;
    B += bi * gb.b;
    C += bi * gb.c;
    sa += bi * gb.sa;
    sb += bi * gb.sb;
    M = (int)batch_rows(gb.rows, M);
    if (M == 0) return;  // the whole workgroup, before any barrier
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int n0 = blockIdx.x * PW;
  const int nf = K / kChunk;  // whole chunks
  const int nkc = (K + kChunk - 1) / kChunk;
  const int nblk = (nkc + D - 1) / D;
  const int last = N - 1 - n0;  // B rows past N repeat the last row

  // One round: the region is pair-major: chunk pair p of the block holds PW
  // rows x 128 bytes (chunks 2p, 2p + 1 of each row: one whole cache line),
  // the 16-byte pieces of row r XOR-swizzled by (r / 2) % 8 so a 16-lane read
  // of 16 rows hits 16 distinct bank groups.  Copy g of pair p fills rows
  // 8g .. 8g + 7: lane l copies row 8g + l / 8, logical piece
  // (l % 8) ^ ((row / 2) % 8) into position l % 8.  Row offsets stay below
  // 2^31 (32 rows of at most 2^24 bytes, plus K).
  constexpr int NP = D / 2;          // chunk pairs per block
  constexpr int NGP = PW / 8;        // copies per pair
  constexpr int PB = PW * 2 * kChunk;  // region bytes per pair
  const uint8_t* bbase = B + (int64_t)n0 * ldb;
  const i32x4 rsb = sgpr_rsrc(bbase);
  const uint32_t region =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)bls) + (uint32_t)(w * REG);
  // Several rounds (REFILL) stream better with the row-major layout: copy j
  // takes rows 2j, 2j + 1 whole (lane l: row 2j + l / 32, logical piece
  // (l % 32) ^ (row % 16) into position l % 32).
  const int crow = lane >> 3;
  auto issue_block = [&](int blk) {
    const int kwhole = nf * kChunk;
    if constexpr (REFILL) {
#pragma unroll
      for (int j = 0; j < NCP; ++j) {
        const int row = min(2 * j + h, last);
        const int kp = blk * RB + 16 * (r32 ^ (row & 15));
        const uint32_t off = (uint32_t)(row * ldb) + (uint32_t)(kp + 16 <= kwhole ? kp : 0);
        dma16_buf(off, rsb, 0, region + (uint32_t)(j * 1024));
      }
    } else {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int g = 0; g < NGP; ++g) {
          const int rl = 8 * g + crow;
          const int row = min(rl, last);
          const int kp = blk * RB + p * 2 * kChunk + 16 * ((lane & 7) ^ ((rl >> 1) & 7));
          const uint32_t off = (uint32_t)(row * ldb) + (uint32_t)(kp + 16 <= kwhole ? kp : 0);
          dma16_buf(off, rsb, 0, region + (uint32_t)(p * PB + g * 1024));
        }
    }
  };
  // fragment read of chunk d: logical pieces 4d + 2h + q of row prow (row-major
  // layout) or 4 (d % 2) + 2h + q of row prow in pair d / 2 (pair-major)
  const int prow = r32 % PW;  // PW = 16: lanes 16..31 repeat rows 0..15
  const uint8_t* myrow = bls + w * REG + prow * (REFILL ? RB : 2 * kChunk);
  const int rsw = REFILL ? (prow & 15) : ((prow >> 1) & 7);
  auto read_chunk = [&](int d) -> Frag32 {
    Frag32 f;
    if constexpr (REFILL) {
      f.q[0] = *reinterpret_cast<const uint4*>(myrow + 16 * ((4 * d + 2 * h) ^ rsw));
      f.q[1] = *reinterpret_cast<const uint4*>(myrow + 16 * ((4 * d + 2 * h + 1) ^ rsw));
    } else {
      const uint8_t* pr = myrow + (d >> 1) * PB;
      f.q[0] = *reinterpret_cast<const uint4*>(pr + 16 * ((4 * (d & 1) + 2 * h) ^ rsw));
      f.q[1] = *reinterpret_cast<const uint4*>(pr + 16 * ((4 * (d & 1) + 2 * h + 1) ^ rsw));
    }
    return f;
  };

  uint32_t arow[TMD];
#pragma unroll
  for (int i = 0; i < TMD; ++i) arow[i] = (uint32_t)(min(32 * i + r32, M - 1) * lda);
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0x7FFFFFFF, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsbv =
      __builtin_amdgcn_make_buffer_rsrc((void*)bbase, (short)0, 0x7FFFFFFF, kBufferWord3);
  auto ld16 = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, int soff) -> uint4 {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // A chunks of block blk (clamped into the whole chunks; masked where used)
  auto load_a = [&](int blk, Frag32 (&ra)[D][TMD]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kc = min(blk * D + d, nf - 1);
#pragma unroll
      for (int i = 0; i < TMD; ++i) {
        ra[d][i].q[0] = ld16(rsa, arow[i] + 32 * h, kc * kChunk);
        ra[d][i].q[1] = ld16(rsa, arow[i] + 32 * h + 16, kc * kChunk);
      }
    }
  };
  const float one[TMD] = {};
  const uint4 z4 = make_uint4(0, 0, 0, 0);
  // the chunk past the whole chunks, at clamped offsets
  const int kpart = nf * kChunk + 32 * h;
  const int poff0 = min(kpart, K - 16), poff1 = min(kpart + 16, K - 16);
  const uint32_t brow = (uint32_t)(min(prow, last) * ldb);

  // wavefront w keeps the master of accumulator elements w*EPW .. w*EPW+EPW-1
  float mast[TMD][EPW];
  f32x16 acc[TMD][1];
#pragma unroll
  for (int i = 0; i < TMD; ++i)
#pragma unroll
    for (int e = 0; e < EPW; ++e) mast[i][e] = 0.f;
  Frag32 ra[D][TMD];
  // One round (REFILL false): A loads first, then the copies pair by pair, so
  // a wait for pair p's copies (at most (NP - 1 - p) NGP copies outstanding)
  // also covers every A load and each pair's matrix steps start as soon as
  // its copies have landed.  Several rounds (REFILL): the weight copies go
  // out first (they are the long pole), the next round's copies are issued
  // as soon as this round's fragments are in registers, and its A loads
  // after the chain.
  if (nf > 0) {
    if constexpr (REFILL) {
      issue_block(min(w, nblk - 1));
      load_a(min(w, nblk - 1), ra);
    } else {
      load_a(min(w, nblk - 1), ra);
      issue_block(min(w, nblk - 1));
    }
  }
  for (int r = 0; r < nblk; r += NWD) {
    const int blk = r + w;
#pragma unroll
    for (int i = 0; i < TMD; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][0][v] = 0.f;
    if (nf > 0) {
      const int nwhole = max(0, min(D, nf - blk * D));  // 0 when blk >= nblk
      auto chunk_mma = [&](int d, const Frag32& fbd) {
        const bool own = d < nwhole;
        Frag32 fa[TMD];
#pragma unroll
        for (int i = 0; i < TMD; ++i) {
          fa[i].q[0] = own ? ra[d][i].q[0] : z4;
          fa[i].q[1] = own ? ra[d][i].q[1] : z4;
        }
        const Frag32 fb[1] = {fbd};
        mma32_chunk<TMD, 1, false>(fa, one, fb, acc);
      };
      if constexpr (!REFILL) {
        static_for<NP>([&](auto pc) {
          constexpr int p = decltype(pc)::value;
          wait_vmcnt<(NP - 1 - p) * NGP>();
          const Frag32 f0 = read_chunk(2 * p), f1 = read_chunk(2 * p + 1);
          chunk_mma(2 * p, f0);
          chunk_mma(2 * p + 1, f1);
        });
      } else {
        wait_vmcnt<0>();  // this round's copies and A loads
        Frag32 rb[D];
#pragma unroll
        for (int d = 0; d < D; ++d) rb[d] = read_chunk(d);
        const bool next = r + NWD < nblk;  // uniform
        if (next) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the region has been read
          issue_block(blk + NWD < nblk ? blk + NWD : nblk - 1);
        }
#pragma unroll
        for (int d = 0; d < D; ++d) chunk_mma(d, rb[d]);
        if (next) load_a(min(blk + NWD, nblk - 1), ra);
      }
    }
    if constexpr (PART) {
      const bool own = blk == nf / D;
      Frag32 pb[1], pa[TMD];
      pb[0].q[0] = ld16(rsbv, brow + (uint32_t)poff0, 0);
      pb[0].q[1] = ld16(rsbv, brow + (uint32_t)poff1, 0);
#pragma unroll
      for (int i = 0; i < TMD; ++i) {
        const uint4 v0 = ld16(rsa, arow[i] + (uint32_t)poff0, 0);
        const uint4 v1 = ld16(rsa, arow[i] + (uint32_t)poff1, 0);
        pa[i].q[0] = own && kpart < K ? v0 : z4;
        pa[i].q[1] = own && kpart + 16 < K ? v1 : z4;
      }
      mma32_chunk<TMD, 1, false>(pa, one, pb, acc);
    }
#pragma unroll
    for (int i = 0; i < TMD; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) part[w][i][e][lane] = acc[i][0][e];
    __syncthreads();
    // every wavefront adds its slice of each block's partial, blocks ascending
    for (int b = 0; b < NWD && r + b < nblk; ++b)
#pragma unroll
      for (int i = 0; i < TMD; ++i)
#pragma unroll
        for (int e = 0; e < EPW; ++e) mast[i][e] = mast[i][e] + part[b][i][w * EPW + e][lane];
    if (r + NWD < nblk) __syncthreads();  // (uniform) the next round rewrites part
  }
  // accumulator element e of lane l is output row 32i + l % 32, column
  // 8 (e / 4) + 4 (l / 32) + e % 4; wavefront w stores its elements
  const int v = (w * EPW) / 4, t0 = (w * EPW) % 4;
  if (v >= PW / 8) return;  // PW = 16: the instruction's upper 16 columns
#pragma unroll
  for (int i = 0; i < TMD; ++i) {
    const int rr = 32 * i + r32;
    const int c = n0 + 8 * v + 4 * h + t0;
    if (rr >= M || c >= N) continue;
    const float sar = sa[sa_vec ? rr : 0];
    if constexpr (EPW == 4) {
      const f32x4 a4 = {mast[i][0], mast[i][1], mast[i][2], mast[i][3]};
      store_row4<EPI>(C, ldc, rr, c, a4, sar, sb, sb_vec, bias);
    } else {
      store_row2<EPI>(C, ldc, rr, c, mast[i][0], mast[i][1], sar, sb, sb_vec, bias);
    }
  }
}

// ---------------------------------------------------------------------------
// Blockwise kernel: 128 x 128 workgroup tile, 4 wavefronts of 64 x 64, 128-wide
// K tiles double-buffered through LDS (register-staged 16-byte loads, XOR
// swizzled 128-byte rows).  Each K tile is one scale block.
__device__ __forceinline__ int swz8(int row) { return ((row >> 1) ^ (row << 2)) & 7; }

template <bool UE8M0>
__global__ __launch_bounds__(256, 1) void gemm_blockwise_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, const void* __restrict__ sa_p,
    const float* __restrict__ sb_p, int tiles_m, int tiles_n, GemmBatch gb) {
  constexpr int BM = 128, BN = 128, TM = 4, TN = 4;
  constexpr int ROWS = BM + BN, CPT = ROWS * 8 / 256, STAGE = ROWS * 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  {
    const int64_t bi = blockIdx.y;
    A += bi * gb.a;
    B += bi * gb.b;
    C += bi * gb.c;
    sa_p = static_cast<const uint8_t*>(sa_p) + bi * gb.sa * (UE8M0 ? 1 : 4);
    sb_p += bi * gb.sb;
    M = (int)batch_rows(gb.rows, M);
    if (m0 >= M) return;  // the whole workgroup, before any barrier
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int g = lane >> 4, r16 = lane & 15;
  const uint8_t* gsrc[CPT];
  int ldst[CPT], kc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int id = t + 256 * i, row = id >> 3, c = id & 7;
    gsrc[i] = row < BM ? A + (int64_t)min(m0 + row, M - 1) * lda + c * 16
                       : B + (int64_t)min(n0 + row - BM, N - 1) * ldb + c * 16;
    ldst[i] = row * 128 + ((c ^ swz8(row)) << 4);
    kc[i] = c * 16;
  }
  const int nk = (K + 127) / 128;
  uint4 pre[CPT];
  f32x4 part[TM][TN];
  double mast[TM][TN][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) mast[i][j][v] = 0.0;
    }
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    pre[i] = kc[i] < K ? *reinterpret_cast<const uint4*>(gsrc[i]) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(lds + ldst[i]) = pre[i];
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      const int64_t koff = (int64_t)(kt + 1) * 128;
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        pre[i] = koff + kc[i] < K ? *reinterpret_cast<const uint4*>(gsrc[i] + koff)
                                  : make_uint4(0, 0, 0, 0);
    }
    const uint8_t* base = lds + (kt & 1) * STAGE;
    // each 128-wide tile is two 64-wide halves; lane group g takes 16 bytes of
    // each half per row (k = 64h + 16g + 8s + j within the tile)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * 64 + 16 * i + r16;
        fa[i] = *reinterpret_cast<const uint4*>(base + row * 128 + (((4 * h + g) ^ swz8(row)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = BM + wn * 64 + 16 * j + r16;
        fb[j] = *reinterpret_cast<const uint4*>(base + row * 128 + (((4 * h + g) ^ swz8(row)) << 4));
      }
      mma_chunk64<TM, TN>(fa, fb, part);
    }
    const float sbv = sb_p[(int64_t)tn * nk + kt];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = min(m0 + wm * 64 + 16 * i + 4 * g + v, M - 1);
        double s64;
        if constexpr (UE8M0) {
          const int byte = static_cast<const uint8_t*>(sa_p)[(int64_t)r * nk + kt];
          s64 = ldexp((double)sbv, byte - 127);
        } else {
          s64 = (double)static_cast<const float*>(sa_p)[(int64_t)r * nk + kt] * (double)sbv;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) mast[i][j][v] = fma((double)part[i][j][v], s64, mast[i][j][v]);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kt + 1 < nk) {
      uint8_t* nb = lds + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(nb + ldst[i]) = pre[i];
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int c = n0 + wn * 64 + 16 * j + r16;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = m0 + wm * 64 + 16 * i + 4 * g + v;
        if (r < M && c < N) C[(int64_t)r * ldc + c] = f32_to_bf16_rne((float)mast[i][j][v]);
      }
  }
}

// K == 0: every accumulator is zero, so C = rnd(0 + bias) = bias (a value of
// the output dtype) or +0.
__global__ void fill_k0_kernel(uint16_t* C, int64_t ldc, int64_t M, int64_t N,
                               const uint16_t* __restrict__ bias, GemmBatch gb) {
  C += (int64_t)blockIdx.y * gb.c;
  M = batch_rows(gb.rows, M);
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / N, c = i - r * N;
    C[r * ldc + c] = bias ? bias[c] : (uint16_t)0;
  }
}

// ---------------------------------------------------------------------------
// host launchers

const char* variant_name(int v) {
  switch (v) {
    case VAR_TILE_128x128: return "tile128x128";
    case VAR_TILE_128x256: return "tile128x256";
    case VAR_TILE_256x128: return "tile256x128";
    case VAR_DECODE_32: return "decode32";
    case VAR_DECODE_64: return "decode64";
    case VAR_DECODE_32_W4: return "decode32w4";
    case VAR_DECODE_16: return "decode16";
    default: return "unknown";
  }
}

bool variant_accepts(int v, int64_t M) {
  switch (v) {
    case VAR_TILE_128x128:
    case VAR_TILE_128x256:
    case VAR_TILE_256x128: return true;
    case VAR_DECODE_32:
    case VAR_DECODE_32_W4:
    case VAR_DECODE_16: return M <= 32;
    case VAR_DECODE_64: return M <= 64;
    default: return false;
  }
}

static dim3 grid2(int64_t blocks, const GemmArgs& g) {
  return dim3((unsigned)blocks, (unsigned)g.batch.count);
}

// Runs f(std::integral_constant<int, EPI>) for the arguments' epilogue.
template <typename Fn>
static hipError_t with_epi(const GemmArgs& g, Fn&& f) {
  switch ((g.out_f16 ? EPI_F16 : 0) | (g.bias ? EPI_BIAS : 0)) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case EPI_F16: f(std::integral_constant<int, EPI_F16>{}); break;
    case EPI_BIAS: f(std::integral_constant<int, EPI_BIAS>{}); break;
    default: f(std::integral_constant<int, EPI_F16 | EPI_BIAS>{}); break;
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NSLOT, int OCC>
static hipError_t launch_rowwise_tile(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  return with_epi(g, [&](auto e) {
    constexpr int EPI = decltype(e)::value;
    hipLaunchKernelGGL((gemm_rowwise_kernel<BM, BN, WM, WN, NSLOT, OCC, EPI>),
                       grid2(tiles_m * tiles_n, g), dim3(64 * WM * WN), 0, s, g.A, g.lda, g.B,
                       g.ldb, g.C, g.ldc, (int)g.M, (int)g.N,
                       (int)g.K, static_cast<const float*>(g.sa), (int)(g.sa_kind == 1),
                       static_cast<const float*>(g.sb), (int)(g.sb_kind == 2),
                       static_cast<const uint16_t*>(g.bias), tiles_m, tiles_n, g.batch);
  });
}

template <int TMD, int NWD, int PW = 32>
static hipError_t launch_decode(const GemmArgs& g, hipStream_t s) {
  const int grid = (int)((g.N + PW - 1) / PW);
  auto go = [&](auto part, auto refill) {
    return with_epi(g, [&](auto e) {
      constexpr int EPI = decltype(e)::value;
      constexpr bool PART = decltype(part)::value, REFILL = decltype(refill)::value;
      hipLaunchKernelGGL((gemm_decode_kernel<TMD, NWD, PW, PART, REFILL, EPI>), grid2(grid, g),
                         dim3(64 * NWD), 0, s, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, (int)g.M,
                         (int)g.N, (int)g.K, static_cast<const float*>(g.sa),
                         (int)(g.sa_kind == 1), static_cast<const float*>(g.sb),
                         (int)(g.sb_kind == 2), static_cast<const uint16_t*>(g.bias), g.batch);
    });
  };
  // REFILL: K has more blocks than the workgroup has wavefronts, so the
  // kernel runs several rounds with each next block's copies issued ahead;
  // otherwise one round whose chunk pairs are multiplied as they land
  const int64_t nblk = (g.K + kChunk * kBlockChunks - 1) / (kChunk * kBlockChunks);
  if (nblk > NWD)
    return g.K % kChunk ? go(std::true_type{}, std::true_type{})
                        : go(std::false_type{}, std::true_type{});
  return g.K % kChunk ? go(std::true_type{}, std::false_type{})
                      : go(std::false_type{}, std::false_type{});
}

hipError_t launch_gemm_rowwise(int variant, const GemmArgs& g, hipStream_t s) {
  switch (variant) {
    case VAR_TILE_128x128: return launch_rowwise_tile<128, 128, 2, 2, 4, 2>(g, s);
    case VAR_TILE_128x256: return launch_rowwise_tile<128, 256, 2, 4, 4, 1>(g, s);
    case VAR_TILE_256x128: return launch_rowwise_tile<256, 128, 4, 2, 4, 1>(g, s);
    case VAR_DECODE_32: return launch_decode<1, 8>(g, s);
    case VAR_DECODE_64: return launch_decode<2, 4>(g, s);
    case VAR_DECODE_32_W4: return launch_decode<1, 4>(g, s);
    case VAR_DECODE_16: return launch_decode<1, 8, 16>(g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_rowwise_fp8mfma(const GemmArgs& g, hipStream_t s) {
  constexpr int BM = 128, BN = 256;
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_rowwise_fp8mfma_kernel<BM, BN, 3, 2>), dim3(tiles_m * tiles_n),
                     dim3(256), 0, s, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, (int)g.M, (int)g.N,
                     (int)g.K, static_cast<const float*>(g.sa), (int)(g.sa_kind == 1),
                     static_cast<const float*>(g.sb), (int)(g.sb_kind == 2), tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm_blockwise(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (int)((g.M + 127) / 128), tiles_n = (int)((g.N + 127) / 128);
  if (g.sa_kind == 3)
    hipLaunchKernelGGL((gemm_block_ue8m0_kernel<4, 2>), grid2(tiles_m * tiles_n, g), dim3(256),
                       0, s, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, (int)g.M, (int)g.N, (int)g.K,
                       static_cast<const uint8_t*>(g.sa), static_cast<const float*>(g.sb), tiles_m,
                       tiles_n, g.batch);
  else
    hipLaunchKernelGGL((gemm_blockwise_kernel<false>), grid2(tiles_m * tiles_n, g), dim3(256), 0,
                       s, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, (int)g.M, (int)g.N, (int)g.K, g.sa,
                       static_cast<const float*>(g.sb), tiles_m, tiles_n, g.batch);
  return hipGetLastError();
}

hipError_t launch_fill_k0(uint16_t* C, int64_t ldc, int64_t M, int64_t N, const void* bias,
                          hipStream_t s, const GemmBatch& bt) {
  int64_t blocks = (M * N + 255) / 256;
  const int64_t cap = std::max<int64_t>(1, 65536 / std::max<int64_t>(1, bt.count));
  if (blocks > cap) blocks = cap;
  if (blocks == 0 || bt.count == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_k0_kernel, dim3((unsigned)blocks, (unsigned)bt.count), dim3(256), 0, s,
                     C, ldc, M, N, static_cast<const uint16_t*>(bias), bt);
  return hipGetLastError();
}

}  // namespace fp8sm

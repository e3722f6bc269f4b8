// Scaled E4M3FN GEMM kernels for gfx950, bf16 output.
//
// Operation ("Route large SM90 row/column-scaled FP8 GEMMs to Torch", Summary;
// prhub digest of sglang PR #33148, key source excerpts for the per-tensor
// form): C[m,n] = bf16(acc[m,n] * sa[m] * sb[n]), acc = sum_k A[m,k] * B[n,k],
// A [M][lda] and B [N][ldb] E4M3FN with K contiguous.
//
// Arithmetic, identical in every variant (so a row of C never depends on M,
// on its neighbours, or on the variant the shape dispatch picked -- the
// property sglang PR #44861's reviewers checked row by row):
//  * fp8 codes are widened exactly to bf16 in registers and multiplied on the
//    bf16 matrix cores (v_mfma_f32_16x16x32_bf16).  The fp8 matrix
//    instructions were measured to sum each run of 8 products with the
//    smaller ones truncated ~13 bits below the largest, far outside fp32
//    accumulation; the bf16 instruction keeps near-fp32 precision.
//  * Within a 128-wide K tile, MFMA step s (0..3) of lane group g (0..3)
//    multiplies k = 32g + 8s + j, j = 0..7.
//  * Products of kPromoteTiles consecutive K tiles are chained into a fresh
//    fp32 partial (the first MFMA of a block starts from zero); partials are
//    added into an fp32 master in ascending block order.
//  * Epilogue: bf16_rne((master * sa[m]) * sb[n]).
// The decode kernel splits the K blocks across wavefronts but merges the
// partials in the same ascending order, so it is bitwise identical.
//
// Blockwise (1x128 activation groups x 128x128 weight blocks): a fresh fp32
// partial per 128-wide K tile, multiplied by sa[m,kb] * sb[n/128,kb] in fp64
// and accumulated in an fp64 master; bf16 of the master at the end.
#include "device_common.h"
#include "launch.h"

namespace fp8sm {

#ifndef FP8SM_PROMOTE_TILES
#define FP8SM_PROMOTE_TILES 4
#endif
constexpr int kPromoteTiles = FP8SM_PROMOTE_TILES;  // 128-wide K tiles per fp32 partial

enum { MODE_ROWWISE = 0, MODE_BLOCK_UE8M0 = 1, MODE_BLOCK_FP32 = 2 };

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row, chosen so
// that the 16 rows read by one 16-lane group (and the 8 rows of any 8-lane
// phase) land in distinct bank groups.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row << 2)) & 7; }

__device__ __forceinline__ bf16x8 widen_e4m3_x8(uint32_t d0, uint32_t d1) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One 128-wide K tile for TM x TN 16x16 output tiles.  af/bf hold each lane's
// 32 bytes (k = 32g .. 32g+31 of the tile) for every row/column subtile.
template <int TM, int TN>
__device__ __forceinline__ void mma_tile128(const uint32_t (&af)[TM][8], const uint32_t (&bf)[TN][8],
                                            f32x4 (&acc)[TM][TN]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = widen_e4m3_x8(af[i][2 * s], af[i][2 * s + 1]);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = widen_e4m3_x8(bf[j][2 * s], bf[j][2 * s + 1]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
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

// ---------------------------------------------------------------------------
// LDS-staged tile kernel: BM x BN workgroup tile, 4 wavefronts in a WM x WN
// grid, 128-wide K tiles double-buffered through LDS (16-byte global loads
// into registers, swizzled 16-byte LDS stores, one barrier per K tile).
template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, const void* __restrict__ sa_p,
    int sa_vec, const float* __restrict__ sb_p, int sb_vec, int tiles_m, int tiles_n) {
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int ROWS = BM + BN;
  static_assert((ROWS * 8) % 256 == 0, "tile rows must split evenly over 256 threads");
  constexpr int CPT = ROWS * 8 / 256;
  constexpr int STAGE = ROWS * 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w / WN, wn = w % WN;
  const int g = lane >> 4, r16 = lane & 15;

  const uint8_t* gsrc[CPT];
  int ldst[CPT], kc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int id = t + 256 * i, row = id >> 3, c = id & 7;
    if (row < BM)
      gsrc[i] = A + (int64_t)min(m0 + row, M - 1) * lda + c * 16;
    else
      gsrc[i] = B + (int64_t)min(n0 + row - BM, N - 1) * ldb + c * 16;
    ldst[i] = row * 128 + ((c ^ swz(row)) << 4);
    kc[i] = c * 16;
  }
  const int nk = (K + 127) / 128;
  const int KB = nk;
  uint4 pre[CPT];

  f32x4 part[TM][TN], mast[TM][TN];
  double mastd[TM][TN][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      mast[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) mastd[i][j][v] = 0.0;
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
    uint32_t af[TM][8], bfr[TN][8];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * (BM / WM) + 16 * i + r16;
      const uint8_t* p = base + row * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(p + (((2 * g) ^ swz(row)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(p + (((2 * g + 1) ^ swz(row)) << 4));
      af[i][0] = lo.x; af[i][1] = lo.y; af[i][2] = lo.z; af[i][3] = lo.w;
      af[i][4] = hi.x; af[i][5] = hi.y; af[i][6] = hi.z; af[i][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = BM + wn * (BN / WN) + 16 * j + r16;
      const uint8_t* p = base + row * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(p + (((2 * g) ^ swz(row)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(p + (((2 * g + 1) ^ swz(row)) << 4));
      bfr[j][0] = lo.x; bfr[j][1] = lo.y; bfr[j][2] = lo.z; bfr[j][3] = lo.w;
      bfr[j][4] = hi.x; bfr[j][5] = hi.y; bfr[j][6] = hi.z; bfr[j][7] = hi.w;
    }
    mma_tile128<TM, TN>(af, bfr, part);

    if constexpr (MODE == MODE_ROWWISE) {
      if ((kt + 1) % kPromoteTiles == 0 || kt + 1 == nk) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            mast[i][j] += part[i][j];
            part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
    } else {
      // blockwise: this K tile is exactly one 128-wide scale block
      const float sbv = sb_p[(int64_t)(n0 / 128) * KB + kt];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = min(m0 + wm * (BM / WM) + 16 * i + 4 * g + v, M - 1);
          double s64;
          if constexpr (MODE == MODE_BLOCK_UE8M0) {
            const int byte = static_cast<const uint8_t*>(sa_p)[(int64_t)r * KB + kt];
            s64 = ldexp((double)sbv, byte - 127);
          } else {
            s64 = (double)static_cast<const float*>(sa_p)[(int64_t)r * KB + kt] * (double)sbv;
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) mastd[i][j][v] = fma((double)part[i][j][v], s64, mastd[i][j][v]);
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (kt + 1 < nk) {
      uint8_t* nb = lds + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(nb + ldst[i]) = pre[i];
    }
    __syncthreads();
  }

  // epilogue
  const float* sa_f = static_cast<const float*>(sa_p);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int c = n0 + wn * (BN / WN) + 16 * j + r16;
    const float sbc = MODE == MODE_ROWWISE ? sb_p[sb_vec ? min(c, N - 1) : 0] : 1.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = m0 + wm * (BM / WM) + 16 * i + 4 * g + v;
        if (r < M && c < N) {
          float val;
          if constexpr (MODE == MODE_ROWWISE)
            val = rowwise_epilogue(mast[i][j][v], sa_f[sa_vec ? r : 0], sbc);
          else
            val = (float)mastd[i][j][v];
          C[(int64_t)r * ldc + c] = f32_to_bf16_rne(val);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16 * TM): a workgroup owns 16 output columns; its four
// wavefronts take the 512-wide K blocks in turn (block b by wavefront b % 4),
// each streaming its operands straight from global memory into registers, and
// wavefront 0 adds the partials into the master in ascending block order.
template <int TM>
__global__ __launch_bounds__(256) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, const float* __restrict__ sa,
    int sa_vec, const float* __restrict__ sb, int sb_vec) {
  __shared__ f32x4 red[4][TM][64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int nk = (K + 127) / 128;
  const int nblk = (nk + kPromoteTiles - 1) / kPromoteTiles;
  const uint8_t* brow = B + (int64_t)min(n0 + r16, N - 1) * ldb + 32 * g;
  const uint8_t* arow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) arow[i] = A + (int64_t)min(16 * i + r16, M - 1) * lda + 32 * g;

  f32x4 mast[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) mast[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int b0 = 0; b0 < nblk; b0 += 4) {
    const int blk = b0 + w;
    f32x4 part[TM][1];
#pragma unroll
    for (int i = 0; i < TM; ++i) part[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (blk < nblk) {
      uint4 bv[kPromoteTiles][2], av[kPromoteTiles][TM][2];
#pragma unroll
      for (int tt = 0; tt < kPromoteTiles; ++tt) {
        const int64_t k0 = (int64_t)(blk * kPromoteTiles + tt) * 128 + 32 * g;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = k0 + 16 * h < K;
          bv[tt][h] = ok ? *reinterpret_cast<const uint4*>(brow + (k0 - 32 * g) + 16 * h)
                         : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            av[tt][i][h] = ok ? *reinterpret_cast<const uint4*>(arow[i] + (k0 - 32 * g) + 16 * h)
                              : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int tt = 0; tt < kPromoteTiles; ++tt) {
        if (blk * kPromoteTiles + tt < nk) {
          uint32_t af[TM][8], bfr[1][8];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            af[i][0] = av[tt][i][0].x; af[i][1] = av[tt][i][0].y;
            af[i][2] = av[tt][i][0].z; af[i][3] = av[tt][i][0].w;
            af[i][4] = av[tt][i][1].x; af[i][5] = av[tt][i][1].y;
            af[i][6] = av[tt][i][1].z; af[i][7] = av[tt][i][1].w;
          }
          bfr[0][0] = bv[tt][0].x; bfr[0][1] = bv[tt][0].y; bfr[0][2] = bv[tt][0].z;
          bfr[0][3] = bv[tt][0].w; bfr[0][4] = bv[tt][1].x; bfr[0][5] = bv[tt][1].y;
          bfr[0][6] = bv[tt][1].z; bfr[0][7] = bv[tt][1].w;
          mma_tile128<TM, 1>(af, bfr, part);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) red[w][i][lane] = part[i][0];
    __syncthreads();
    if (w == 0) {
      for (int ww = 0; ww < 4; ++ww)
        if (b0 + ww < nblk)
#pragma unroll
          for (int i = 0; i < TM; ++i) mast[i] += red[ww][i][lane];
    }
    __syncthreads();
  }
  if (w != 0) return;
  const int c = n0 + r16;
  if (c >= N) return;
  const float sbc = sb[sb_vec ? c : 0];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * i + 4 * g + v;
      if (r < M) C[(int64_t)r * ldc + c] = f32_to_bf16_rne(rowwise_epilogue(mast[i][v], sa[sa_vec ? r : 0], sbc));
    }
}

__global__ void fill_zero_bf16_kernel(uint16_t* C, int64_t ldc, int64_t M, int64_t N) {
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / N, c = i - r * N;
    C[r * ldc + c] = 0;
  }
}

// ---------------------------------------------------------------------------
// host launchers

const char* variant_name(int v) {
  switch (v) {
    case VAR_TILE_256x128: return "tile256x128";
    case VAR_TILE_128x128: return "tile128x128";
    case VAR_DECODE_16: return "decode16";
    case VAR_DECODE_32: return "decode32";
    case VAR_DECODE_64: return "decode64";
    default: return "unknown";
  }
}

bool variant_accepts(int v, int64_t M) {
  switch (v) {
    case VAR_TILE_256x128:
    case VAR_TILE_128x128: return true;
    case VAR_DECODE_16: return M <= 16;
    case VAR_DECODE_32: return M <= 32;
    case VAR_DECODE_64: return M <= 64;
    default: return false;
  }
}

template <int BM, int BN, int WM, int WN, int MODE>
static hipError_t launch_tile(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  const int grid = tiles_m * tiles_n;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, WN, MODE>), dim3(grid), dim3(256), 0, s, g.A,
                     g.lda, g.B, g.ldb, g.C, g.ldc, (int)g.M, (int)g.N, (int)g.K, g.sa,
                     (int)(g.sa_kind == 1), static_cast<const float*>(g.sb),
                     (int)(g.sb_kind == 2), tiles_m, tiles_n);
  return hipGetLastError();
}

template <int TM>
static hipError_t launch_decode(const GemmArgs& g, hipStream_t s) {
  const int grid = (int)((g.N + 15) / 16);
  hipLaunchKernelGGL((gemm_decode_kernel<TM>), dim3(grid), dim3(256), 0, s, g.A, g.lda, g.B,
                     g.ldb, g.C, g.ldc, (int)g.M, (int)g.N, (int)g.K,
                     static_cast<const float*>(g.sa), (int)(g.sa_kind == 1),
                     static_cast<const float*>(g.sb), (int)(g.sb_kind == 2));
  return hipGetLastError();
}

hipError_t launch_gemm_rowwise(int variant, const GemmArgs& g, hipStream_t s) {
  switch (variant) {
    case VAR_TILE_256x128: return launch_tile<256, 128, 2, 2, MODE_ROWWISE>(g, s);
    case VAR_TILE_128x128: return launch_tile<128, 128, 2, 2, MODE_ROWWISE>(g, s);
    case VAR_DECODE_16: return launch_decode<1>(g, s);
    case VAR_DECODE_32: return launch_decode<2>(g, s);
    case VAR_DECODE_64: return launch_decode<4>(g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_blockwise(const GemmArgs& g, hipStream_t s) {
  if (g.sa_kind == 3) return launch_tile<128, 128, 2, 2, MODE_BLOCK_UE8M0>(g, s);
  return launch_tile<128, 128, 2, 2, MODE_BLOCK_FP32>(g, s);
}

hipError_t launch_fill_zero_bf16(uint16_t* C, int64_t ldc, int64_t M, int64_t N, hipStream_t s) {
  int64_t blocks = (M * N + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, C, ldc, M, N);
  return hipGetLastError();
}

}  // namespace fp8sm

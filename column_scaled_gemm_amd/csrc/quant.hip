// Activation / weight quantization kernels to OCP E4M3FN (gfx950).
//
// Group rule (sglang PR #33533 "[JIT] per_token_group_quant: fix the fp16
// UE8M0 multiplier overflow ...", commit messages and Motivation): for each
// group, a' = max(max|y|, 1e-10), s = RN32(a'/448); fp32 scales quantize with
// the correctly rounded multiplier RN32(448/a'), UE8M0 scales with 2^-e,
// e = ceil(log2 s).  Every multiply is fp32, whatever the input dtype, so the
// fp16 multiplier overflow of that PR's Modifications 1 cannot occur.
// Fused SiLU-and-mul follows Modifications 2 (silu per element, plain divide).
//
// Memory layout: x row-major [M][ld_x] bf16/fp16 (a fused row is [gate|up]),
// codes row-major [M][ld_q], scales row-major [M][G] or group-major
// [G][M_pad].  Every kernel reads each input element once from HBM with
// 16-byte loads that are contiguous across a wavefront, and writes codes with
// 8-byte stores that are contiguous across the wavefront.
#include "device_common.h"
#include "launch.h"
#include "silu_table.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace fp8sm {

enum { FMT_FP32 = 0, FMT_UE8M0_FP32 = 1, FMT_UE8M0_BYTE = 2 };

// Largest grid of the per-token kernels (workgroups); more rows than the grid
// covers are walked by its wavefronts.
constexpr int64_t kMaxRowBlocks = 1 << 20;

template <int FMT>
__device__ __forceinline__ float group_multiplier(float amax, float* scale_val, int* ebyte) {
  const float a = fmaxf(amax, kAmaxFloor);
  if constexpr (FMT == FMT_FP32) {
    *scale_val = a / kQMax;
    *ebyte = 0;
    return kQMax / a;
  } else {
    // e = ceil(log2 RN32(a / 448)) without the divide.  a is a normal fp32
    // value (a >= 1e-10), a = (1 + m 2^-23) 2^(E-127).  RN32(a/448) <= 2^k
    // exactly when a <= 448 * 2^k = 1.75 * 2^(k+8): if a is at most that,
    // so is a/448 and its rounding; if a is larger it is at least one ulp
    // (2^(k-15)) larger, so a/448 exceeds 2^k by more than 2^(k-24), half an
    // ulp of 2^k, and rounds above it.  Hence e = E - 135 when m <= 0x600000
    // (1 + m 2^-23 <= 1.75) and E - 134 otherwise: adding 0x1FFFFF carries
    // into the exponent field exactly when m > 0x600000.
    const uint32_t t = (__float_as_uint(a) + 0x1FFFFFu) & 0xFF800000u;  // E' << 23
    const int e = (int)(t >> 23) - 135;
    *scale_val = pow2f(e);
    *ebyte = e + 127;
    return pow2f(-e);
  }
}

// Codes need the clamp to [-448, 448] only with fp32 scales: a UE8M0
// multiplier 2^-e has 448 * 2^e >= the group's absmax (above), and scaling by
// a power of two is exact, so every scaled value already lies in range.
template <int FMT>
constexpr bool kClampCodes = FMT == FMT_FP32;

template <int FMT>
__device__ __forceinline__ void store_scale(void* scales, int64_t idx, float v, int ebyte) {
  if constexpr (FMT == FMT_UE8M0_BYTE) {
    static_cast<uint8_t*>(scales)[idx] = (uint8_t)ebyte;
  } else {
    static_cast<float*>(scales)[idx] = v;
  }
}

// Moves a workgroup's x, q and scale pointers to its batch (blockIdx.y) and
// returns the batch's live rows.
template <int FMT>
__device__ __forceinline__ int64_t enter_batch(const QuantBatch& bt,
                                               const uint16_t* __restrict__& x,
                                               uint8_t* __restrict__& q,
                                               void* __restrict__& scales, int64_t M) {
  const int64_t b = blockIdx.y;
  x += b * bt.sx;
  q += b * bt.sq;
  scales = static_cast<uint8_t*>(scales) + b * bt.ss * (FMT == FMT_UE8M0_BYTE ? 1 : 4);
  return batch_rows(bt.rows, M);
}

// y = silu(gate) * up in fp32 (fused) or the widened input; `tab` is the
// workgroup's silu table (fused only).
template <bool F16, bool FUSED>
__device__ __forceinline__ void load_values(const uint4 gv, const uint4 uv, float* y,
                                            const void* tab) {
  widen8<F16>(gv, y);
  if constexpr (FUSED) {
    float u[8];
    widen8<F16>(uv, u);
    if constexpr (F16) {
      // fp16 gates: index the table from the raw 16-bit halves
      const uint32_t w[4] = {gv.x, gv.y, gv.z, gv.w};
      float sl[8];
      SiluTable<true>::lookup8(tab, w, y, sl);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = sl[i] * u[i];
    } else {
      // bf16 gates: index the table from the raw 16-bit halves
      const uint32_t w[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = SiluTable<false>::lookup_bits(tab, y[2 * i], w[i] & 0x7FFFu, (w[i] >> 15) & 1u) * u[2 * i];
        y[2 * i + 1] = SiluTable<false>::lookup_bits(tab, y[2 * i + 1], (w[i] >> 16) & 0x7FFFu, w[i] >> 31) * u[2 * i + 1];
      }
    }
  }
}

// Codes of one 1x128 group held by a 16-lane quarter (8 values per lane), and
// its scale (value and UE8M0 byte).  Every lane of the quarter takes part.
template <int FMT>
__device__ __forceinline__ uint2 group128_codes(float* y, float* sval, int* eb) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = group_max<16>(amax);
  const float mult = group_multiplier<FMT>(amax, sval, eb);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = y[i] * mult;
  return to_e4m3_x8<kClampCodes<FMT>>(y);
}

// Quantize one 1x128 group and store its codes and scale (row < 0: nothing).
template <int FMT>
__device__ __forceinline__ void quant_group128(float* y, int l16, int64_t row, int64_t grp,
                                               uint8_t* __restrict__ q, int64_t ld_q,
                                               void* __restrict__ scales, int64_t G,
                                               int mn_major, int64_t mpad) {
  float sval;
  int eb;
  const uint2 codes = group128_codes<FMT>(y, &sval, &eb);
  if (row >= 0) {
    store_stream8(q + row * ld_q + grp * 128 + l16 * 8, codes);
    if (l16 == 0) {
      const int64_t idx = mn_major ? grp * mpad + row : row * G + grp;
      store_scale<FMT>(scales, idx, sval, eb);
    }
  }
}

// The same group conversion with 32-bit byte offsets: qo is the group's first
// code offset in q plus l16 * 8, so = its scale index.
template <int FMT>
__device__ __forceinline__ void quant_group128_o32(float* y, int l16, bool valid,
                                                   uint8_t* __restrict__ q, uint32_t qo,
                                                   void* __restrict__ scales, uint32_t so) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = group_max<16>(amax);
  float sval;
  int eb;
  const float mult = group_multiplier<FMT>(amax, &sval, &eb);
  if (valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * mult;
    store_stream8(q + qo, to_e4m3_x8<kClampCodes<FMT>>(y));
    if (l16 == 0) store_scale<FMT>(scales, so, sval, eb);
  }
}

// ---------------------------------------------------------------------------
// 1x128 groups.  A 16-lane quarter of a wavefront owns one group (16 lanes x 8
// values); a wavefront owns kQuads x 4 consecutive groups of the flattened
// (row, group) index, issuing all its loads before any arithmetic.
constexpr int kQuads = 4;

template <bool F16, int FMT>
__global__ __launch_bounds__(256) void quant_g128_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t G, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, void* __restrict__ scales, int mn_major,
    int64_t mpad, QuantBatch bt) {
  M = enter_batch<FMT>(bt, x, q, scales, M);
  const int lane = threadIdx.x & 63;
  const int quarter = lane >> 4;
  const int l16 = lane & 15;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = M * G;
  uint4 gv[kQuads];
  int64_t row[kQuads], grp[kQuads];
#pragma unroll
  for (int u = 0; u < kQuads; ++u) {
    const int64_t gid = (wave * kQuads + u) * 4 + quarter;
    row[u] = -1;
    grp[u] = 0;
    gv[u] = make_uint4(0, 0, 0, 0);
    if (gid < total) {
      row[u] = gid / G;
      grp[u] = gid - row[u] * G;
      gv[u] = load_stream16(x + row[u] * ld_x + grp[u] * 128 + l16 * 8);
    }
  }
#pragma unroll
  for (int u = 0; u < kQuads; ++u) {
    float y[8];
    widen8<F16>(gv[u], y);
    quant_group128<FMT>(y, l16, row[u], grp[u], q, ld_q, scales, G, mn_major, mpad);
  }
}

// 1x128 groups with a scattered output (sglang PR #33533, commit messages: the
// scatter fusion): token t's groups are quantized once, as above, and each
// group's codes and scale go to every destination row d = dst[t][j] with
// 0 <= d < R (the bound is checked here: other entries name no row).  The 16
// lanes of a quarter read the same destination list (one cache line).  A
// wavefront takes kScatterQuads x 4 groups: 2 measured 5% faster than 4 and
// 9% faster than 1 on [1024, 7168] top-8.
constexpr int kScatterQuads = 2;
template <bool F16, int FMT>
__global__ __launch_bounds__(256) void quant_g128_scatter_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t G, int64_t ld_x,
    const int32_t* __restrict__ dst, int topk, int64_t R, uint8_t* __restrict__ q, int64_t ld_q,
    void* __restrict__ scales, int mn_major, int64_t rpad) {
  const int lane = threadIdx.x & 63;
  const int quarter = lane >> 4;
  const int l16 = lane & 15;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = T * G;
  uint4 gv[kScatterQuads];
  int64_t tok[kScatterQuads], grp[kScatterQuads];
#pragma unroll
  for (int u = 0; u < kScatterQuads; ++u) {
    const int64_t gid = (wave * kScatterQuads + u) * 4 + quarter;
    tok[u] = -1;
    grp[u] = 0;
    gv[u] = make_uint4(0, 0, 0, 0);
    if (gid < total) {
      tok[u] = gid / G;
      grp[u] = gid - tok[u] * G;
      gv[u] = load_stream16(x + tok[u] * ld_x + grp[u] * 128 + l16 * 8);
    }
  }
#pragma unroll
  for (int u = 0; u < kScatterQuads; ++u) {
    float y[8], sval;
    int eb;
    widen8<F16>(gv[u], y);
    const uint2 codes = group128_codes<FMT>(y, &sval, &eb);
    if (tok[u] < 0) continue;
    const int32_t* dl = dst + tok[u] * topk;
    for (int j = 0; j < topk; ++j) {
      const int64_t d = dl[j];
      if (d < 0 || d >= R) continue;
      store_stream8(q + d * ld_q + grp[u] * 128 + l16 * 8, codes);
      if (l16 == 0) store_scale<FMT>(scales, mn_major ? grp[u] * rpad + d : d * G + grp[u], sval, eb);
    }
  }
}

// Fused SiLU-and-mul + 1x128 groups: one 1024-thread workgroup per CU copies
// the silu table into LDS, then its 16 wavefronts walk the flattened
// (row, group) space 4 groups (one per 16-lane quarter) per step, loading the
// next step while converting the current one.  Steps are interleaved across
// the grid: wavefront w at step t covers groups (t nw + w) 4 .. + 3 (nw
// wavefronts in the grid), so consecutive wavefronts take consecutive 4-group
// runs and a short batch (a masked expert's few rows) spreads over every
// workgroup instead of a few.  One run per step (not several) keeps the
// walk's fill and drain short: 4 runs per step measured 11% slower (32.7 vs
// 28.9 us on [4096, 2 x 7168]), and neither a second workgroup per CU nor
// loads two or three steps ahead changed it.  A fused row is [gate | up],
// each K wide.  M and G are at most 2^30 (checked at the boundary), so rows
// and groups fit in int.  Each lane keeps a (row, group) cursor and advances
// it without division; loads past the last row read the last row and are
// never stored, so the loads are branch-free and the compiler's wait counts
// leave the next step's loads in flight.
constexpr int kFusedRuns = 1;  // 4-group runs per wavefront and step

struct G128Step {
  uint4 g[kFusedRuns], u[kFusedRuns];
  int row[kFusedRuns], grp[kFusedRuns];  // row = -1: past the end
};

template <bool F16, int FMT, bool O32>
__global__ __launch_bounds__(1024) void quant_g128_fused_kernel(
    const uint16_t* __restrict__ x, int M, int G, int64_t K, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, void* __restrict__ scales, int mn_major,
    int64_t mpad, QuantBatch bt) {
  __shared__ __attribute__((aligned(16))) uint8_t tab[SiluTable<F16>::kBytes];
  M = (int)enter_batch<FMT>(bt, x, q, scales, M);
  // a workgroup whose first group (that of its first wavefront's run 0 at
  // step 0) is past the batch's groups has no work at any step: it leaves
  // before copying the table (uniform, before the barrier)
  if ((int64_t)blockIdx.x * 64 >= (int64_t)M * G) return;
  const int lane = threadIdx.x & 63;
  const int quarter = lane >> 4;
  const int l16 = lane & 15;
  const int64_t total = (int64_t)M * G;
  // g0: first group of this wavefront's run 0 at the current step; every
  // step moves each cursor by 4 kFusedRuns nw groups = (drow, dgrp)
  const int64_t nw = (int64_t)gridDim.x * 16;
  const int64_t w = (int64_t)blockIdx.x * 16 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t g0 = w * 4;
  int drow, dgrp;
  int cr[kFusedRuns], cc[kFusedRuns];
  if constexpr (O32) {
    // M * G < 2^23 here (the host checked every byte offset against 2^32),
    // and the first groups are below 4 nw: 32-bit divisions are exact and
    // far cheaper than 64-bit ones
    const uint32_t ug = (uint32_t)G, step = (uint32_t)nw * (4u * kFusedRuns);
    drow = (int)(step / ug);
    dgrp = (int)(step - (uint32_t)drow * ug);
#pragma unroll
    for (int u = 0; u < kFusedRuns; ++u) {
      const uint32_t gid = ((uint32_t)u * (uint32_t)nw + (uint32_t)w) * 4u + (uint32_t)quarter;
      cr[u] = (int)(gid / ug);
      cc[u] = (int)(gid - (uint32_t)cr[u] * ug);
    }
  } else {
    drow = (int)(nw * (4 * kFusedRuns) / G);
    dgrp = (int)(nw * (4 * kFusedRuns) - (int64_t)drow * G);
#pragma unroll
    for (int u = 0; u < kFusedRuns; ++u) {
      const int64_t gid = (u * nw + w) * 4 + quarter;
      cr[u] = (int)(gid / G);
      cc[u] = (int)(gid - (int64_t)cr[u] * G);
    }
  }
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  auto fetch = [&](G128Step& st) {
#pragma unroll
    for (int u = 0; u < kFusedRuns; ++u) {
      const int r = min(cr[u], M - 1);
      if constexpr (O32) {
        const uint32_t off = (uint32_t)r * (uint32_t)(2 * ld_x) + (uint32_t)cc[u] * 256u + l16 * 16u;
        st.g[u] = load_stream16(xb + off);
        st.u[u] = load_stream16(xb + (off + (uint32_t)(2 * K)));
      } else {
        const uint16_t* src = x + (int64_t)r * ld_x + (int64_t)cc[u] * 128 + l16 * 8;
        st.g[u] = load_stream16(src);
        st.u[u] = load_stream16(src + K);
      }
      st.row[u] = cr[u] < M ? cr[u] : -1;
      st.grp[u] = cc[u];
      // advance the cursor to the wavefront's next step
      int c = cc[u] + dgrp, rr = cr[u] + drow;
      const bool wrap = c >= G;
      cc[u] = wrap ? c - G : c;
      cr[u] = wrap ? rr + 1 : rr;
    }
  };
  auto convert = [&](const G128Step& st) {
#pragma unroll
    for (int u = 0; u < kFusedRuns; ++u) {
      float y[8];
      load_values<F16, true>(st.g[u], st.u[u], y, tab);
      if constexpr (O32) {
        const uint32_t rr = (uint32_t)max(st.row[u], 0), gg = (uint32_t)st.grp[u];
        const uint32_t qo = rr * (uint32_t)ld_q + gg * 128u + l16 * 8u;
        const uint32_t so = mn_major ? gg * (uint32_t)mpad + rr : rr * (uint32_t)G + gg;
        quant_group128_o32<FMT>(y, l16, st.row[u] >= 0, q, qo, scales, so);
      } else {
        quant_group128<FMT>(y, l16, st.row[u], st.grp[u], q, ld_q, scales, G, mn_major, mpad);
      }
    }
  };
  G128Step a, b;
  fetch(a);  // the first loads overlap the table copy
  SiluTable<F16>::load(tab, threadIdx.x, 1024);
  __syncthreads();
  const int64_t step = (4 * kFusedRuns) * nw;
  while (g0 < total) {
    g0 += step;
    fetch(b);
    convert(a);
    if (g0 >= total) break;
    g0 += step;
    fetch(a);
    convert(b);
  }
}

// ---------------------------------------------------------------------------
// Per token, row kept in registers: wavefronts walk the rows (row, row +
// waves in the grid, ...; the host gives every row its own wavefront up to
// kMaxRowBlocks workgroups, which measured faster from HBM than a grid of
// resident wavefronts walking several rows), holding a row as NC 16-byte chunks per
// lane (chunk c = lane + 64 i; the host picks the smallest listed NC with
// 64 * NC * 8 >= K, so the last chunks of a lane may lie past the row end:
// those read the row's last chunk and are masked out of the maximum and the
// stores; chunks below NFULL, the next smaller listed NC, always lie inside
// the row).  When a wavefront has another row, its loads are issued before
// the current row is reduced, quantized and stored.  Codes go out as
// streaming (nontemporal) stores.
template <bool F16, int NC, int NFULL, int FMT>
__global__ __launch_bounds__(256) void quant_token_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, void* __restrict__ scales, QuantBatch bt) {
  M = enter_batch<FMT>(bt, x, q, scales, M);
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nch = (int)(K >> 3);  // K <= 2^30
  int cidx[NC];
  bool ok[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    ok[i] = i < NFULL || c < nch;
    cidx[i] = i < NFULL ? c : min(c, nch - 1);
  }
  auto fetch = [&](uint4 (&v)[NC], int64_t r) {
    const uint16_t* xr = x + r * ld_x;
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = load_stream16(xr + (int64_t)cidx[i] * 8);
  };
  auto convert = [&](const uint4 (&v)[NC], int64_t r) {
    // |x| max on the 16-bit patterns: with the sign cleared, bf16 and fp16
    // values order like unsigned integers (inputs are finite)
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, ok[i] ? (w[k] & 0x7FFF7FFFu) : 0u));
    }
    const uint32_t mb = m2[0] > m2[1] ? m2[0] : m2[1];
    float amax;
    if constexpr (F16)
      amax = (float)__builtin_bit_cast(_Float16, (uint16_t)mb);
    else
      amax = __uint_as_float(mb << 16);
    amax = group_max<64>(amax);
    float sval;
    int eb;
    const float mult = group_multiplier<FMT>(amax, &sval, &eb);
    uint8_t* qr = q + r * ld_q;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      float y[8];
      widen8<F16>(v[i], y);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = y[j] * mult;
      const uint2 codes = to_e4m3_x8<kClampCodes<FMT>>(y);
      if (ok[i]) store_stream8(qr + (int64_t)cidx[i] * 8, codes);
    }
    if (lane == 0) store_scale<FMT>(scales, r, sval, eb);
  };
  uint4 va[NC], vb[NC];
  if (row < M) fetch(va, row);
  while (row < M) {
    const int64_t r1 = row + nw;
    if (r1 < M) fetch(vb, r1);
    convert(va, row);
    row = r1;
    if (row >= M) break;
    const int64_t r2 = row + nw;
    if (r2 < M) fetch(va, r2);
    convert(vb, row);
    row = r2;
  }
}

// Per token, long rows (K > 4096): the four wavefronts of a workgroup share a
// row, each holding NCW 16-byte chunks per lane (chunk c = 64 w + lane +
// 256 i); a workgroup per row (up to kMaxRowBlocks), a next row's quarter
// loaded while the current one is converted, streaming code stores.  The row
// maximum is exchanged through LDS (two slots, alternating by row, so one
// barrier per row suffices); chunks past the row end are clamped and masked.
template <bool F16, int NCW, int FMT>
__global__ __launch_bounds__(256) void quant_token_wg_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, void* __restrict__ scales, QuantBatch bt) {
  __shared__ float part[2][4];
  M = enter_batch<FMT>(bt, x, q, scales, M);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nch = (int)(K >> 3);  // K <= 2^30
  int cidx[NCW];
  bool ok[NCW];
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int c = 64 * w + lane + 256 * i;
    ok[i] = c < nch;
    cidx[i] = min(c, nch - 1);
  }
  auto fetch = [&](uint4 (&v)[NCW], int64_t r) {
    const uint16_t* xr = x + r * ld_x;
#pragma unroll
    for (int i = 0; i < NCW; ++i) v[i] = load_stream16(xr + (int64_t)cidx[i] * 8);
  };
  auto convert = [&](const uint4 (&v)[NCW], int64_t r, int par) {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, ok[i] ? (wd[k] & 0x7FFF7FFFu) : 0u));
    }
    const uint32_t mb = m2[0] > m2[1] ? m2[0] : m2[1];
    float amax;
    if constexpr (F16)
      amax = (float)__builtin_bit_cast(_Float16, (uint16_t)mb);
    else
      amax = __uint_as_float(mb << 16);
    amax = group_max<64>(amax);
    if (lane == 0) part[par][w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[par][0], part[par][1]), fmaxf(part[par][2], part[par][3]));
    float sval;
    int eb;
    const float mult = group_multiplier<FMT>(amax, &sval, &eb);
    uint8_t* qr = q + r * ld_q;
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      float y[8];
      widen8<F16>(v[i], y);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = y[j] * mult;
      const uint2 codes = to_e4m3_x8<kClampCodes<FMT>>(y);
      if (ok[i]) store_stream8(qr + (int64_t)cidx[i] * 8, codes);
    }
    if (threadIdx.x == 0) store_scale<FMT>(scales, r, sval, eb);
  };
  uint4 va[NCW], vb[NCW];
  int64_t row = blockIdx.x;
  const int64_t stride = gridDim.x;
  if (row < M) fetch(va, row);
  while (row < M) {
    const int64_t r1 = row + stride;
    if (r1 < M) fetch(vb, r1);
    convert(va, row, 0);
    row = r1;
    if (row >= M) break;
    const int64_t r2 = row + stride;
    if (r2 < M) fetch(va, r2);
    convert(vb, row, 1);
    row = r2;
  }
}

// Per token, any K: two passes over the row (the second pass re-reads it from
// L2) so no register budget limits K.  The row pass is shared by the plain
// kernel below (one wavefront per row) and the fused one (persistent
// 1024-thread workgroups that hold the silu table).
template <bool F16, bool FUSED, int FMT>
__device__ __forceinline__ void quant_row_2pass(const uint16_t* __restrict__ xr, int64_t K,
                                                uint8_t* __restrict__ qr, void* __restrict__ scales,
                                                int64_t row, int lane, const void* tab) {
  const int64_t nch = K >> 3;
  float amax = 0.0f;
  for (int64_t c = lane; c < nch; c += 64) {
    const uint4 g = *reinterpret_cast<const uint4*>(xr + c * 8);
    uint4 u = make_uint4(0, 0, 0, 0);
    if constexpr (FUSED) u = *reinterpret_cast<const uint4*>(xr + K + c * 8);
    float y[8];
    load_values<F16, FUSED>(g, u, y, tab);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(y[j]));
  }
  amax = group_max<64>(amax);
  float sval;
  int eb;
  const float mult = group_multiplier<FMT>(amax, &sval, &eb);
  for (int64_t c = lane; c < nch; c += 64) {
    const uint4 g = *reinterpret_cast<const uint4*>(xr + c * 8);
    uint4 u = make_uint4(0, 0, 0, 0);
    if constexpr (FUSED) u = *reinterpret_cast<const uint4*>(xr + K + c * 8);
    float y[8];
    load_values<F16, FUSED>(g, u, y, tab);
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = y[j] * mult;
    *reinterpret_cast<uint2*>(qr + c * 8) = to_e4m3_x8<kClampCodes<FMT>>(y);
  }
  if (lane == 0) store_scale<FMT>(scales, row, sval, eb);
}

template <bool F16, int FMT>
__global__ __launch_bounds__(256) void quant_token_2pass_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, void* __restrict__ scales, QuantBatch bt) {
  M = enter_batch<FMT>(bt, x, q, scales, M);
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // whole wavefront; the kernel has no barrier
  quant_row_2pass<F16, false, FMT>(x + row * ld_x, K, q + row * ld_q, scales, row,
                                   threadIdx.x & 63, nullptr);
}

template <bool F16, int FMT>
__global__ __launch_bounds__(1024) void quant_token_fused_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, void* __restrict__ scales, QuantBatch bt) {
  __shared__ __attribute__((aligned(16))) uint8_t tab[SiluTable<F16>::kBytes];
  M = enter_batch<FMT>(bt, x, q, scales, M);
  if ((int64_t)blockIdx.x * 16 >= M) return;  // no row for any wavefront (uniform)
  SiluTable<F16>::load(tab, threadIdx.x, 1024);
  __syncthreads();
  for (int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 6); row < M;
       row += (int64_t)gridDim.x * 16)
    quant_row_2pass<F16, true, FMT>(x + row * ld_x, K, q + row * ld_q, scales, row,
                                    threadIdx.x & 63, tab);
}

// ---------------------------------------------------------------------------
// Static per-tensor quant: q = E4M3(clamp(RN32(x * RN32(1/s)))).  Each thread
// converts one 16-byte chunk (8 values) of the flattened (row, chunk) space.
template <bool F16>
__global__ __launch_bounds__(256) void quant_static_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld_x,
    const float* __restrict__ scale, uint8_t* __restrict__ q, int64_t ld_q, QuantBatch bt) {
  x += (int64_t)blockIdx.y * bt.sx;
  q += (int64_t)blockIdx.y * bt.sq;
  M = batch_rows(bt.rows, M);
  const int64_t nch = K >> 3;
  const int64_t total = M * nch;
  const float inv = 1.0f / scale[0];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nch, c = i - r * nch;
    const uint4 v = *reinterpret_cast<const uint4*>(x + r * ld_x + c * 8);
    float y[8];
    widen8<F16>(v, y);
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = y[j] * inv;
    *reinterpret_cast<uint2*>(q + r * ld_q + c * 8) = to_e4m3_x8(y);
  }
}

// ---------------------------------------------------------------------------
// The fused product alone in fp32, through the same table and lookup as the
// fused quant kernels.
template <bool F16>
__global__ __launch_bounds__(1024) void silu_mul_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                        int64_t K, int64_t ld_x,
                                                        float* __restrict__ y, int64_t ld_y) {
  __shared__ __attribute__((aligned(16))) uint8_t tab[SiluTable<F16>::kBytes];
  SiluTable<F16>::load(tab, threadIdx.x, 1024);
  __syncthreads();
  const int64_t nch = K >> 3;
  const int64_t total = M * nch;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nch, c = i - r * nch;
    const uint16_t* src = x + r * ld_x + c * 8;
    float v[8];
    load_values<F16, true>(*reinterpret_cast<const uint4*>(src),
                           *reinterpret_cast<const uint4*>(src + K), v, tab);
    float4* dst = reinterpret_cast<float4*>(y + r * ld_y + c * 8);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: one workgroup (4 wavefronts) per block; each thread
// holds 8 chunks of 8 values; the block maximum is reduced across the
// workgroup through LDS.
template <bool F16>
__global__ __launch_bounds__(256) void quant_wblock_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales, int64_t KB) {
  __shared__ float red[4];
  const int64_t nb = blockIdx.y, kb = blockIdx.x;
  const int t = threadIdx.x;
  uint4 v[8];
  bool ok[8];
  int64_t rr[8], cc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = t + 256 * i;         // 0..2047: 128 rows x 16 chunks
    rr[i] = nb * 128 + (idx >> 4);
    cc[i] = kb * 128 + (idx & 15) * 8;
    ok[i] = rr[i] < N && cc[i] < K;
    v[i] = ok[i] ? *reinterpret_cast<const uint4*>(w + rr[i] * ld_w + cc[i]) : make_uint4(0, 0, 0, 0);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y[8];
    widen8<F16>(v[i], y);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(y[j]));
  }
  amax = group_max<64>(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float sval;
  int eb;
  const float mult = group_multiplier<FMT_FP32>(amax, &sval, &eb);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (ok[i]) {
      float y[8];
      widen8<F16>(v[i], y);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = y[j] * mult;
      *reinterpret_cast<uint2*>(q + rr[i] * ld_q + cc[i]) = to_e4m3_x8(y);
    }
  }
  if (t == 0) scales[nb * KB + kb] = sval;
}

// ---------------------------------------------------------------------------
// Load-time requantization of a fused per-tensor weight (the weight loading of
// the prhub digest of sglang PR #33148, key source excerpts): the rows of
// logical partition i (offsets in `parts`) hold codes quantized with scale
// s_i; every code is decoded exactly, scaled back in fp32 and quantized again
// against s_max = max_i s_i with the static rule:
//   q' = E4M3(clamp(RN32(RN32(dec(q) * s_i) * RN32(1 / s_max))))
// Each thread converts one 16-byte chunk (16 codes) of the flattened
// (row, chunk) space; reading and writing the same chunk makes q == w safe.
__global__ __launch_bounds__(256) void requant_max_kernel(
    const uint8_t* w, int64_t ldw, int64_t N, int64_t K, WeightParts parts,
    const float* __restrict__ scales, uint8_t* q, int64_t ldq, float* __restrict__ max_out) {
  float smax = scales[0];
  for (int i = 1; i < parts.n; ++i) smax = fmaxf(smax, scales[i]);
  const float inv = 1.0f / smax;
  if (blockIdx.x == 0 && threadIdx.x == 0) max_out[0] = smax;
  const int64_t nch = K >> 4;
  const int64_t total = N * nch;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / nch, c = idx - r * nch;
    int part = 0;
    while (part + 1 < parts.n && r >= parts.off[part + 1]) ++part;
    const float si = scales[part];
    const uint4 v = *reinterpret_cast<const uint4*>(w + r * ldw + c * 16);
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float y[8];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int word = (int)wd[2 * h + k];
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);  // bytes 0, 1 (exact)
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);   // bytes 2, 3
        y[4 * k] = (lo[0] * si) * inv;
        y[4 * k + 1] = (lo[1] * si) * inv;
        y[4 * k + 2] = (hi[0] * si) * inv;
        y[4 * k + 3] = (hi[1] * si) * inv;
      }
      const uint2 e = to_e4m3_x8(y);
      o[2 * h] = e.x;
      o[2 * h + 1] = e.y;
    }
    *reinterpret_cast<uint4*>(q + r * ldq + c * 16) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Per-partition scalar scales broadcast to the output channels.
__global__ __launch_bounds__(256) void channelwise_kernel(const float* __restrict__ scales,
                                                          WeightParts parts, int64_t N,
                                                          float* __restrict__ out) {
  for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < N;
       n += (int64_t)gridDim.x * blockDim.x) {
    int part = 0;
    while (part + 1 < parts.n && n >= parts.off[part + 1]) ++part;
    out[n] = scales[part];
  }
}

// ---------------------------------------------------------------------------
// host-side launchers

// Runs f(std::integral_constant<int, FMT>) for the runtime scale format.
template <typename Fn>
static hipError_t with_fmt(int fmt, Fn&& f) {
  switch (fmt) {
    case FMT_FP32: f(std::integral_constant<int, FMT_FP32>{}); break;
    case FMT_UE8M0_FP32: f(std::integral_constant<int, FMT_UE8M0_FP32>{}); break;
    default: f(std::integral_constant<int, FMT_UE8M0_BYTE>{}); break;
  }
  return hipGetLastError();
}

// Compute units of the current device (persistent fused kernels launch one
// 1024-thread workgroup per CU).
static int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups per batch for a persistent kernel: enough for the work, at most
// `cap` over all batches together (at least one per batch).
static unsigned persistent_blocks(int64_t work_per_block_units, int64_t units, int64_t batches = 1,
                                  int64_t cap = 0) {
  if (cap <= 0) cap = cu_count();
  const int64_t need = (units + work_per_block_units - 1) / work_per_block_units;
  const int64_t share = (cap + batches - 1) / batches;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(need, share));
}

static dim3 grid2(int64_t blocks, const QuantBatch& bt) {
  return dim3((unsigned)blocks, (unsigned)bt.count);
}

template <bool F16>
static hipError_t launch_g128(int fmt, const QuantArgs& a, hipStream_t s) {
  const int64_t G = a.K / 128;
  const int64_t waves = (a.M * G + 15) / 16;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  return with_fmt(fmt, [&](auto f) {
    constexpr int FMT = decltype(f)::value;
    hipLaunchKernelGGL((quant_g128_kernel<F16, FMT>), grid2((waves + 3) / 4, a.batch), dim3(256),
                       0, s, x, a.M, G, a.ld_x, a.q, a.ld_q, a.scales, a.mn_major, a.mpad,
                       a.batch);
  });
}

template <bool F16>
static hipError_t launch_g128_scatter(int fmt, const ScatterArgs& a, hipStream_t s) {
  const int64_t G = a.K / 128;
  const int64_t waves = (a.T * G + 4 * kScatterQuads - 1) / (4 * kScatterQuads);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  return with_fmt(fmt, [&](auto f) {
    constexpr int FMT = decltype(f)::value;
    hipLaunchKernelGGL((quant_g128_scatter_kernel<F16, FMT>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, s, x, a.T, G, a.ld_x, a.dst, a.topk, a.R, a.q, a.ld_q,
                       a.scales, a.mn_major, a.rpad);
  });
}

hipError_t launch_quant_scatter(const ScatterArgs& a, hipStream_t s) {
  if (a.T == 0 || a.topk == 0) return hipSuccess;
  return a.f16 ? launch_g128_scatter<true>(a.fmt, a, s) : launch_g128_scatter<false>(a.fmt, a, s);
}

template <bool F16>
static hipError_t launch_g128_fused(int fmt, const QuantArgs& a, hipStream_t s) {
  const int64_t G = a.K / 128;
  // a workgroup per 4 steps of its 16 wavefronts (64 groups a step), at most one per CU
  const unsigned blocks = persistent_blocks(16 * 16, a.M * G, a.batch.count);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  // every byte offset the kernel forms below 2^32: 32-bit address arithmetic
  const uint64_t lim = (uint64_t)1 << 32;
  const bool o32 = (uint64_t)a.M * (uint64_t)a.ld_x * 2 + 2 * (uint64_t)a.K < lim &&
                   (uint64_t)a.M * (uint64_t)a.ld_q < lim &&
                   (uint64_t)(a.mn_major ? G * a.mpad : a.M * G) < lim;
  return with_fmt(fmt, [&](auto f) {
    constexpr int FMT = decltype(f)::value;
    if (o32)
      hipLaunchKernelGGL((quant_g128_fused_kernel<F16, FMT, true>), grid2(blocks, a.batch),
                         dim3(1024), 0, s, x, (int)a.M, (int)G, a.K, a.ld_x, a.q, a.ld_q,
                         a.scales, a.mn_major, a.mpad, a.batch);
    else
      hipLaunchKernelGGL((quant_g128_fused_kernel<F16, FMT, false>), grid2(blocks, a.batch),
                         dim3(1024), 0, s, x, (int)a.M, (int)G, a.K, a.ld_x, a.q, a.ld_q,
                         a.scales, a.mn_major, a.mpad, a.batch);
  });
}

// NC chunks per lane; the caller guarantees the row has more than 64 * NFULL
// chunks (so chunks below NFULL are whole).
template <bool F16, int NC, int NFULL>
static hipError_t launch_token_nc(int fmt, const QuantArgs& a, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  return with_fmt(fmt, [&](auto f) {
    constexpr int FMT = decltype(f)::value;
    const int64_t blocks = std::min<int64_t>((a.M + 3) / 4, kMaxRowBlocks);
    hipLaunchKernelGGL((quant_token_kernel<F16, NC, NFULL, FMT>), grid2(blocks, a.batch),
                       dim3(256), 0, s, x, a.M, a.K, a.ld_x, a.q, a.ld_q, a.scales, a.batch);
  });
}

template <bool F16>
static hipError_t launch_token_2pass(int fmt, const QuantArgs& a, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  return with_fmt(fmt, [&](auto f) {
    constexpr int FMT = decltype(f)::value;
    hipLaunchKernelGGL((quant_token_2pass_kernel<F16, FMT>), grid2((a.M + 3) / 4, a.batch),
                       dim3(256), 0, s, x, a.M, a.K, a.ld_x, a.q, a.ld_q, a.scales, a.batch);
  });
}

template <bool F16>
static hipError_t launch_token_fused(int fmt, const QuantArgs& a, hipStream_t s) {
  const unsigned blocks = persistent_blocks(16, a.M, a.batch.count);  // one row per wavefront
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  return with_fmt(fmt, [&](auto f) {
    constexpr int FMT = decltype(f)::value;
    hipLaunchKernelGGL((quant_token_fused_kernel<F16, FMT>), grid2(blocks, a.batch), dim3(1024),
                       0, s, x, a.M, a.K, a.ld_x, a.q, a.ld_q, a.scales, a.batch);
  });
}

template <bool F16, int NCW>
static hipError_t launch_token_wg(int fmt, const QuantArgs& a, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  return with_fmt(fmt, [&](auto f) {
    constexpr int FMT = decltype(f)::value;
    const int64_t blocks = std::min<int64_t>(a.M, kMaxRowBlocks);
    hipLaunchKernelGGL((quant_token_wg_kernel<F16, NCW, FMT>), grid2(blocks, a.batch), dim3(256),
                       0, s, x, a.M, a.K, a.ld_x, a.q, a.ld_q, a.scales, a.batch);
  });
}

template <bool F16>
static hipError_t launch_token(int fmt, const QuantArgs& a, hipStream_t s) {
  const int64_t per_lane = (a.K / 8 + 63) / 64;
  if (per_lane <= 1) return launch_token_nc<F16, 1, 0>(fmt, a, s);
  if (per_lane <= 2) return launch_token_nc<F16, 2, 1>(fmt, a, s);
  if (per_lane <= 4) return launch_token_nc<F16, 4, 2>(fmt, a, s);
  if (per_lane <= 6) return launch_token_nc<F16, 6, 4>(fmt, a, s);
  if (per_lane <= 8) return launch_token_nc<F16, 8, 6>(fmt, a, s);
  const int64_t per_wave = (a.K / 8 + 255) / 256;  // chunks per lane with 4 waves per row
  if (per_wave <= 3) return launch_token_wg<F16, 3>(fmt, a, s);
  if (per_wave <= 4) return launch_token_wg<F16, 4>(fmt, a, s);
  if (per_wave <= 6) return launch_token_wg<F16, 6>(fmt, a, s);
  if (per_wave <= 8) return launch_token_wg<F16, 8>(fmt, a, s);
  if (per_wave <= 12) return launch_token_wg<F16, 12>(fmt, a, s);
  return launch_token_2pass<F16>(fmt, a, s);
}

hipError_t launch_quant_group(const QuantArgs& a, hipStream_t s) {
  if (a.M == 0 || a.batch.count == 0) return hipSuccess;
  const bool per_token = a.group == a.K;
  if (per_token) {
    if (a.fused) return a.f16 ? launch_token_fused<true>(a.fmt, a, s)
                              : launch_token_fused<false>(a.fmt, a, s);
    return a.f16 ? launch_token<true>(a.fmt, a, s) : launch_token<false>(a.fmt, a, s);
  }
  if (a.fused) return a.f16 ? launch_g128_fused<true>(a.fmt, a, s)
                            : launch_g128_fused<false>(a.fmt, a, s);
  return a.f16 ? launch_g128<true>(a.fmt, a, s) : launch_g128<false>(a.fmt, a, s);
}

hipError_t launch_quant_static(const void* x, bool f16, int64_t M, int64_t K, int64_t ld_x,
                               const float* scale, uint8_t* q, int64_t ld_q, hipStream_t s,
                               const QuantBatch& bt) {
  if (M == 0 || bt.count == 0) return hipSuccess;
  const int64_t chunks = M * (K / 8);
  int64_t blocks = (chunks + 255) / 256;
  const int64_t cap = std::max<int64_t>(1, 65536 / bt.count);
  if (blocks > cap) blocks = cap;
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  if (f16)
    hipLaunchKernelGGL((quant_static_kernel<true>), grid2(blocks, bt), dim3(256), 0, s, xx, M, K,
                       ld_x, scale, q, ld_q, bt);
  else
    hipLaunchKernelGGL((quant_static_kernel<false>), grid2(blocks, bt), dim3(256), 0, s, xx, M,
                       K, ld_x, scale, q, ld_q, bt);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void* x, bool f16, int64_t M, int64_t K, int64_t ld_x, float* y,
                           int64_t ld_y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const unsigned blocks = persistent_blocks(1024, M * (K / 8));
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  if (f16)
    hipLaunchKernelGGL((silu_mul_kernel<true>), dim3(blocks), dim3(1024), 0, s, xx, M, K, ld_x, y,
                       ld_y);
  else
    hipLaunchKernelGGL((silu_mul_kernel<false>), dim3(blocks), dim3(1024), 0, s, xx, M, K, ld_x,
                       y, ld_y);
  return hipGetLastError();
}

hipError_t launch_requant_max(const uint8_t* w, int64_t ldw, int64_t N, int64_t K,
                              const WeightParts& parts, const float* scales, uint8_t* q,
                              int64_t ldq, float* max_out, hipStream_t s) {
  const int64_t chunks = N * (K / 16);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((chunks + 255) / 256, 65536));
  hipLaunchKernelGGL(requant_max_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, ldw, N, K,
                     parts, scales, q, ldq, max_out);
  return hipGetLastError();
}

hipError_t launch_channelwise(const float* scales, const WeightParts& parts, int64_t N, float* out,
                              hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((N + 255) / 256, 65536);
  hipLaunchKernelGGL(channelwise_kernel, dim3((unsigned)blocks), dim3(256), 0, s, scales, parts, N,
                     out);
  return hipGetLastError();
}

hipError_t launch_quant_wblock(const void* w, bool f16, int64_t N, int64_t K, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, float* scales, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int64_t NB = (N + 127) / 128, KB = (K + 127) / 128;
  const dim3 grid((unsigned)KB, (unsigned)NB), block(256);
  const uint16_t* ww = static_cast<const uint16_t*>(w);
  if (f16)
    hipLaunchKernelGGL((quant_wblock_kernel<true>), grid, block, 0, s, ww, N, K, ld_w, q, ld_q,
                       scales, KB);
  else
    hipLaunchKernelGGL((quant_wblock_kernel<false>), grid, block, 0, s, ww, N, K, ld_w, q, ld_q,
                       scales, KB);
  return hipGetLastError();
}

}  // namespace fp8sm

// SiLU of a bf16 / fp16 gate through an LDS table (gfx950).
//
// silu(g) = RN32(g / RN32(1 + RN32(e^-g))) depends only on the gate, and a
// gate held in bf16 or fp16 takes one of 65536 values, so each element costs
// a table lookup instead of an fp64 exponential and an IEEE divide.  The
// tables are constant data of the code object, computed on the host at build
// time by gen_silu_tables.cpp with the formulas below; a workgroup copies its
// table from global memory (L2-resident after the first workgroups) into LDS
// with 16-byte loads.  Tables are indexed by the sign and the
// fp32 exponent field E of g, clamped to a window; outside 2^-26 <= |g| < 2^7
// (E = 101..133) the value has a closed form:
//  * |g| < 2^-26: RN32(e^-g) = 1, so silu = g / 2 (exact).
//  * g >= 2^7: RN32(e^-g) = 0, so silu = g.
//  * g <= -2^7: RN32(e^-g) = +inf, so silu = -0.
//
// bf16 (8 significant bits): one entry (a, b) per sign, E = 100..134 and
// 7-bit mantissa, with silu = fma(g, a, b).  Inside the window a = 0 and b is
// silu_f32(g); row E = 100 stands for every |g| < 2^-26 with (1/2, -0); row
// E = 134 for every |g| >= 2^7 with (1, -0) for g > 0 and (0, -0) for g < 0.
// A -0 addend keeps the sign of a zero product.  2 x 35 x 128 x 8 = 71680 B.
// fp16 (11 significant bits, too many for a direct table): e^-g is the
// product of two fp64 factors, e^-gh * e^-gl, where gh keeps the top five
// stored mantissa bits of g and gl the next five.  Each factor table has
// 2 signs x 34 rows (E = 101..134) x 32 entries; row 134 holds e^-gh = 0
// (g > 0) or +inf (g < 0) and e^-gl = 1, so the upper end of the window needs
// no branch, and the only fp16 gates below it are +-0.  The
// product rounded to fp32 is RN32(e^-g).  g / d is formed in fp64 -- the
// hardware reciprocal, one Newton step, one remainder correction -- and
// rounded once to fp32: no fp16 gate has g / d closer than 2^-48 (relative)
// to an fp32 rounding boundary, far above the error of that quotient.  2 x 2 x 34 x 32 x 8 = 34816 B.
// Both forms are checked against the oracle for every finite gate value of
// their dtype by the parity tests.  Non-finite gates are not specified.
#pragma once
#include "device_common.h"

namespace fp8sm {

#include "silu_tables.inc"  // kSiluBf16Table, kSiluF16Table (generated)

// Every thread of the workgroup calls this; the caller places a barrier
// before the first lookup.
template <int BYTES>
__device__ __forceinline__ void copy_table(void* lds, const void* src, int tid, int nthr) {
  static_assert(BYTES % 16 == 0, "16-byte chunks");
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(lds);
  for (int j = tid; j < BYTES / 16; j += nthr) d[j] = s[j];
}

template <bool F16>
struct SiluTable;

template <>
struct SiluTable<false> {
  static constexpr uint32_t kE0 = 100, kRows = 35;  // E = 100 .. 134
  static constexpr int kBytes = 2 * kRows * 128 * 8;

  static_assert(sizeof(kSiluBf16Table) == kBytes, "generated bf16 table size");

  __device__ static void load(void* lds, int tid, int nthr) {
    copy_table<kBytes>(lds, kSiluBf16Table, tid, nthr);
  }

  __device__ static float lookup(const void* lds, float g) {
    const uint32_t b = __float_as_uint(g);
    return lookup_bits(lds, g, (b >> 16) & 0x7FFFu, b >> 31);
  }

  // The same from the gate's bf16 pattern: mag = its low 15 bits, s = its
  // sign bit.  Clamping mag (positive bf16 patterns order like integers) to
  // [E=100 m=0, E=134 m=127] selects the row and mantissa in one step; the
  // table is [sign][row][mantissa], so the entry is s * 4480 + mag - 12800.
  __device__ static float lookup_bits(const void* lds, float g, uint32_t mag, uint32_t s) {
    const uint32_t lo = kE0 << 7, hi = ((kE0 + kRows - 1) << 7) | 127u;
    const uint32_t mc = min(max(mag, lo), hi);
    const uint32_t idx = s * (kRows * 128) + mc - lo;
    const float2 ab = static_cast<const float2*>(lds)[idx];
    return __builtin_fmaf(g, ab.x, ab.y);
  }
};

template <>
struct SiluTable<true> {
  static constexpr uint32_t kE0 = 101, kRows = 34;  // E = 101 .. 134
  static constexpr int kHalf = 2 * kRows * 32;      // entries per factor table
  static constexpr int kBytes = 2 * kHalf * 8;

  static_assert(sizeof(kSiluF16Table) == kBytes, "generated fp16 table size");

  __device__ static void load(void* lds, int tid, int nthr) {
    copy_table<kBytes>(lds, kSiluF16Table, tid, nthr);
  }

  __device__ static float lookup(const void* lds, float g) {
    const uint32_t b = __float_as_uint(g);
    const uint32_t e = min(max((b >> 23) & 255u, kE0), kE0 + kRows - 1) - kE0;
    const uint32_t row = ((b >> 31) * kRows + e) << 5;
    const double* h = static_cast<const double*>(lds);
    const double em = h[row | ((b >> 18) & 31u)] * h[kHalf + (row | ((b >> 13) & 31u))];
    const double d = (double)(1.0f + (float)em);
    const double g64 = (double)g;
    double r = __builtin_amdgcn_rcp(d);                 // approximate reciprocal
    r = __builtin_fma(__builtin_fma(-d, r, 1.0), r, r);  // one Newton step
    const double q0 = g64 * r;
    const float q = (float)__builtin_fma(__builtin_fma(-q0, d, g64), r, q0);  // remainder correction
    // The exact result is a signed zero only for g = +-0 or d = +inf (where the
    // steps above give +0 or NaN); nowhere else is it zero.
    return fabsf(q) > 0.0f ? q : g * 0.0f;
  }
};

}  // namespace fp8sm

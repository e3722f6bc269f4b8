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
// fp16: a direct table of the fp32 silu for every fp16 gate with
// 2^-10 <= |g| < 2^7 (exponent field 5..21, 2 x 17408 entries, 139264 B), indexed
// by the gate's 16-bit pattern.  Outside it: |g| >= 2^7 has the closed forms
// above; |g| < 2^-10 (zero and the smallest gates) evaluates RN32(e^-g) from
// the series of e^-g in fp64 and divides in fp32.
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
  // fp16 patterns with exponent field 5..21 (2^-10 <= |g| < 2^7), per sign
  static constexpr uint32_t kLo = 5u << 10, kSpan = 17u << 10, kHi = 22u << 10;
  static constexpr int kBytes = 2 * kSpan * 4;

  static_assert(sizeof(kSiluF16Table) == kBytes, "generated fp16 table size");

  __device__ static void load(void* lds, int tid, int nthr) {
    copy_table<kBytes>(lds, kSiluF16Table, tid, nthr);
  }

  // Gates outside the table's window.
  __device__ static float outside(float g, uint32_t mag) {
    if (mag >= kHi) return g > 0.0f ? g : -0.0f;  // RN32(e^-g) is 0 or +inf
    // |g| < 2^-10: e^-g by its series in fp64 -- the terms past t^4 are
    // below 2^-57 of the sum -- then rounded to fp32 once
    const double t = -(double)g;
    const double e = 1.0 + t * (1.0 + t * (0.5 + t * (1.0 / 6.0 + t * (1.0 / 24.0))));
    const float d = 1.0f + (float)e;
    return g / d;
  }

  // silu of eight fp16 gates (the 16-bit halves of w[0..3], widened in g):
  // branch-free table reads (clamped index) for all, then one test, so the
  // common case (every gate inside the window) takes a single branch; the
  // rare gates outside it take the exact path above.
  __device__ static void lookup8(const void* lds, const uint32_t (&w)[4], const float* g,
                                 float* r) {
    uint32_t mag[8];
    bool out = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
      mag[i] = bits & 0x7FFFu;
      const uint32_t off = mag[i] - kLo;
      out = out || off >= kSpan;
      r[i] = static_cast<const float*>(lds)[(bits >> 15) * kSpan + min(off, kSpan - 1)];
    }
    if (out) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (mag[i] - kLo >= kSpan) r[i] = outside(g[i], mag[i]);
    }
  }

};

}  // namespace fp8sm

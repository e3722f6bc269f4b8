// Shape dispatch for the rowwise / per-tensor GEMM.
//
// The pages route each shape to the implementation that measured fastest
// ("Route large SM90 row/column-scaled FP8 GEMMs to Torch", Summary and the
// 64-shape sweep under Kernel results), and a later review found a route that
// ignored M and slowed decode down (same page, review thread).  This table is
// keyed on M first for that reason.  Every variant computes bitwise-identical
// rows, so the table only changes speed.
#pragma once
#include <stdint.h>

#include "launch.h"

namespace fp8sm {

inline int pick_from_table(int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (M <= 16) return VAR_DECODE_16;
  if (M <= 32) return VAR_DECODE_32;
  if (M <= 64) return VAR_DECODE_64;
  if (M <= 1024 || N <= 1024) return VAR_TILE_128x128;
  return VAR_TILE_128x256;
}

}  // namespace fp8sm

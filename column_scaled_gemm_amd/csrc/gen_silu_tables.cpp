// Writes the constant SiLU tables that silu_table.h copies into LDS, as a HIP
// include file on stdout.  Host code, run by the build before the kernels are
// compiled; plain IEEE double / float arithmetic (built without contraction or
// fast-math), the formulas of silu_table.h's header comment:
//  * bf16: per sign, fp32 exponent field E = 100..134 and 7-bit mantissa, a
//    pair (a, b) with silu(g) = fma(g, a, b); inside the window a = 0 and
//    b = RN32(g / RN32(1 + RN32(e^-g))); E = 100 stands for |g| < 2^-26
//    (a = 1/2), E = 134 for |g| >= 2^7 (a = 1 for g > 0, 0 for g < 0); b = -0
//    outside the window.
//  * fp16: e^-gh and e^+-gl in fp64 per sign, E = 101..134 and 5 mantissa
//    bits; row 134 holds 0 or +inf and 1.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

static float as_float(uint32_t b) {
  float f;
  std::memcpy(&f, &b, sizeof f);
  return f;
}

static void put(double v) {
  if (std::isinf(v))
    std::printf("%s__builtin_huge_val(),", v < 0 ? "-" : "");
  else
    std::printf("%a,", v);
}

int main() {
  const uint32_t e0b = 100, rowsb = 35;
  std::printf("// Generated at build time by gen_silu_tables.cpp; not a source file.\n");
  std::printf("alignas(16) __device__ const float kSiluBf16Table[%u] = {\n", 2 * rowsb * 128 * 2);
  for (uint32_t j = 0; j < 2 * rowsb * 128; ++j) {
    const uint32_t s = j / (rowsb * 128), r = (j / 128) % rowsb, m = j % 128;
    float a = 0.0f, b = -0.0f;
    if (r == 0) {
      a = 0.5f;
    } else if (r == rowsb - 1) {
      a = s ? 0.0f : 1.0f;
    } else {
      const float g = as_float(s << 31 | (r + e0b) << 23 | m << 16);
      const float e = (float)std::exp(-(double)g);
      const float d = 1.0f + e;
      b = g / d;
    }
    put(a);
    put(b);
    if (j % 4 == 3) std::printf("\n");
  }
  std::printf("};\n");

  const uint32_t e0h = 101, rowsh = 34, half = 2 * rowsh * 32;
  std::printf("alignas(16) __device__ const double kSiluF16Table[%u] = {\n", 2 * half);
  double h[2 * 34 * 32], l[2 * 34 * 32];
  for (uint32_t j = 0; j < half; ++j) {
    const uint32_t s = j / (rowsh * 32), r = (j / 32) % rowsh, m = j % 32;
    if (r == rowsh - 1) {
      h[j] = s ? HUGE_VAL : 0.0;
      l[j] = 1.0;
    } else {
      h[j] = std::exp(-(double)as_float(s << 31 | (r + e0h) << 23 | m << 18));
      const double gl = std::ldexp((double)m, (int)(r + e0h) - 137);  // m * 2^(E-127-10)
      l[j] = std::exp(s ? gl : -gl);
    }
  }
  for (uint32_t j = 0; j < half; ++j) {
    put(h[j]);
    if (j % 4 == 3) std::printf("\n");
  }
  for (uint32_t j = 0; j < half; ++j) {
    put(l[j]);
    if (j % 4 == 3) std::printf("\n");
  }
  std::printf("};\n");
  return 0;
}

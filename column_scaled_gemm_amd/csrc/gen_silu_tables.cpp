// Writes the constant SiLU tables that silu_table.h copies into LDS, as a HIP
// include file on stdout.  Host code, run by the build before the kernels are
// compiled; plain IEEE double / float arithmetic (built without contraction or
// fast-math), the formulas of silu_table.h's header comment:
//  * bf16: per sign, fp32 exponent field E = 100..134 and 7-bit mantissa, a
//    pair (a, b) with silu(g) = fma(g, a, b); inside the window a = 0 and
//    b = RN32(g / RN32(1 + RN32(e^-g))); E = 100 stands for |g| < 2^-26
//    (a = 1/2), E = 134 for |g| >= 2^7 (a = 1 for g > 0, 0 for g < 0); b = -0
//    outside the window.
//  * fp16: RN32(g / RN32(1 + RN32(e^-g))) for every fp16 pattern with
//    exponent field 5..21 (2^-10 <= |g| < 2^7), per sign.
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

  // fp16: every pattern with exponent field 5..21, per sign, the same formula
  const uint32_t lo = 5u << 10, span = 17u << 10;
  std::printf("alignas(16) __device__ const float kSiluF16Table[%u] = {\n", 2 * span);
  for (uint32_t j = 0; j < 2 * span; ++j) {
    const uint32_t s = j / span, mag = lo + j % span;
    const uint32_t ex = mag >> 10, man = mag & 1023u;  // normal: 1.man x 2^(ex - 15)
    float g = std::ldexp((float)(1024u + man), (int)ex - 25);
    if (s) g = -g;
    const float e = (float)std::exp(-(double)g);
    const float d = 1.0f + e;
    put(g / d);
    if (j % 8 == 7) std::printf("\n");
  }
  std::printf("};\n");
  return 0;
}

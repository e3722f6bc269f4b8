// Matrix-instruction precision probe (test hook behind fp8sm_mfma_probe).
//
// One wavefront executes one matrix instruction with a zero accumulator on
// register images the caller supplies, and writes the raw result registers
// back.  The operand layouts are the caller's business: the probe places
// nothing, so a test can state the lane / register / byte position of every
// input value and ask how the instruction sums products that share a run of
// K.  This is the measurement behind the GEMMs' choice of the bf16 matrix
// instructions over the fp8 ones: the accuracy bound of the pages' GEMM
// (the per-output tolerance of the scaled FP8 GEMM, "Route large SM90
// row/column-scaled FP8 GEMMs to Torch", Summary, with fp32 accumulation)
// needs sums at fp32 precision.
#include "device_common.h"
#include "launch.h"

namespace fp8sm {

typedef float f32x16p __attribute__((ext_vector_type(16)));
typedef int i32x8p __attribute__((ext_vector_type(8)));

// a, b: 8 dwords per lane ([lane][8]); d: 16 floats per lane ([lane][16]).
__global__ __launch_bounds__(64) void mfma_probe_kernel(int instr, const uint32_t* __restrict__ a,
                                                        const uint32_t* __restrict__ b,
                                                        float* __restrict__ d) {
  const int l = threadIdx.x;
  uint32_t ra[8], rb[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    ra[r] = a[l * 8 + r];
    rb[r] = b[l * 8 + r];
  }
  float out[16] = {};
  if (instr == 0 || instr == 1) {  // bf16 operands: 4 dwords = 8 values per lane
    const bf16x8 x = __builtin_bit_cast(bf16x8, u32x4{ra[0], ra[1], ra[2], ra[3]});
    const bf16x8 y = __builtin_bit_cast(bf16x8, u32x4{rb[0], rb[1], rb[2], rb[3]});
    if (instr == 0) {
      const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, f32x4{}, 0, 0, 0);
      for (int v = 0; v < 4; ++v) out[v] = c[v];
    } else {
      const f32x16p c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, f32x16p{}, 0, 0, 0);
      for (int v = 0; v < 16; ++v) out[v] = c[v];
    }
  } else if (instr == 2 || instr == 3) {  // e4m3 x e4m3: 8 dwords = 32 codes per lane
    i32x8p x, y;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x[r] = (int)ra[r];
      y[r] = (int)rb[r];
    }
    if (instr == 2) {
      const f32x4 c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, f32x4{}, 0, 0, 0, 0, 0, 0);
      for (int v = 0; v < 4; ++v) out[v] = c[v];
    } else {
      const f32x16p c =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, f32x16p{}, 0, 0, 0, 0, 0, 0);
      for (int v = 0; v < 16; ++v) out[v] = c[v];
    }
  } else {  // instr 4: e4m3 x e4m3, 2 dwords = 8 codes per lane
    const long x = (long)(((uint64_t)ra[1] << 32) | ra[0]);
    const long y = (long)(((uint64_t)rb[1] << 32) | rb[0]);
    const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(x, y, f32x4{}, 0, 0, 0);
    for (int v = 0; v < 4; ++v) out[v] = c[v];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) d[l * 16 + v] = out[v];
}

hipError_t launch_mfma_probe(int instr, const uint32_t* a, const uint32_t* b, float* d,
                             hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, s, instr, a, b, d);
  return hipGetLastError();
}

}  // namespace fp8sm

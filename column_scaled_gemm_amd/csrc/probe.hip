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

// Matrix-pipe throughput ceiling (test hook behind fp8sm_rate_probe): every
// wavefront runs `iters` iterations of four independent
// v_mfma_f32_32x32x16_bf16 on register operands, the accumulator count and
// instruction of the GEMMs' inner loop.  WIDEN: each iteration also widens
// 16 fp8 dwords with v_cvt_scalef32_pk_bf16_fp8 (the GEMMs' ratio of widen
// to matrix instructions for a 64 x 64 wavefront tile) and the widened values
// are the next iteration's operands, so the widen sits on the matrix
// instructions' critical path as it does in the GEMMs.  Nothing is read from
// memory; each lane writes one float so no work is optimized away.
template <bool WIDEN>
__global__ __launch_bounds__(1024) void rate_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t base = 0x3f803f80u + (uint32_t)lane;
  u32x4 ra = {base, base ^ 1u, base ^ 2u, base ^ 3u}, rb = {base ^ 4u, base ^ 5u, base ^ 6u, base ^ 7u};
  uint32_t u[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) u[j] = 0x38383838u + (uint32_t)(lane * 16 + j);
  f32x16p acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  for (int i = 0; i < iters; ++i) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, ra), y = __builtin_bit_cast(bf16x8, rb);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[j], 0, 0, 0);
    if constexpr (WIDEN) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        u[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[j], 1.0f, false));
      ra = u32x4{u[0] ^ u[4], u[1] ^ u[5], u[2] ^ u[6], u[3] ^ u[7]};
      rb = u32x4{u[8] ^ u[12], u[9] ^ u[13], u[10] ^ u[14], u[11] ^ u[15]};
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) sum += acc[j][v];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum + (float)(ra[0] & 1u);
}

hipError_t launch_rate_probe(int widen, int blocks, int waves_per_block, int iters, float* sink,
                             hipStream_t s) {
  const dim3 grid((unsigned)blocks), block((unsigned)(64 * waves_per_block));
  if (widen)
    hipLaunchKernelGGL(rate_probe_kernel<true>, grid, block, 0, s, iters, sink);
  else
    hipLaunchKernelGGL(rate_probe_kernel<false>, grid, block, 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int instr, const uint32_t* a, const uint32_t* b, float* d,
                             hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, s, instr, a, b, d);
  return hipGetLastError();
}

}  // namespace fp8sm

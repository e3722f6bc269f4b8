// Internal launcher interface between the C-ABI layer (api.cpp) and the
// kernels (quant.hip, gemm.hip).  No device code here; the two batch structs
// are also passed to kernels by value.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fp8sm {

// A batch of problems of one shape, one per blockIdx.y: batch b reads and
// writes every operand at its base + b * that operand's stride; when `rows`
// is set (device int32 [count]) batch b has clamp(rows[b], 0, M) live rows and
// its other rows are left untouched.  A plain 2-D call is count 1, strides 0,
// rows null.
struct QuantBatch {
  int64_t count;
  int64_t sx;  // x, elements
  int64_t sq;  // q, bytes
  int64_t ss;  // scales, scale elements (bytes for UE8M0 bytes, floats otherwise)
  const int32_t* rows;
};

struct GemmBatch {
  int64_t count;
  int64_t a, b;    // A, B: bytes (b = 0: one weight for every batch)
  int64_t c;       // C: output elements
  int64_t sa, sb;  // scales: elements of their kind (0: shared)
  const int32_t* rows;
};

struct QuantArgs {
  const void* x;
  bool f16;
  int64_t M, K, ld_x;
  int64_t group;  // 128 or K
  bool fused;
  int fmt;        // 0 fp32, 1 ue8m0 as fp32, 2 ue8m0 byte
  int mn_major;
  int64_t mpad;
  uint8_t* q;
  int64_t ld_q;
  void* scales;
  QuantBatch batch{1, 0, 0, 0, nullptr};
};

hipError_t launch_quant_group(const QuantArgs& a, hipStream_t s);

struct ScatterArgs {
  const void* x;
  bool f16;
  int64_t T, K, ld_x;
  const int32_t* dst;  // device [T][topk]
  int topk;
  int64_t R;           // rows of q
  int fmt;
  int mn_major;
  int64_t rpad;
  uint8_t* q;
  int64_t ld_q;
  void* scales;
};
hipError_t launch_quant_scatter(const ScatterArgs& a, hipStream_t s);
hipError_t launch_quant_static(const void* x, bool f16, int64_t M, int64_t K, int64_t ld_x,
                               const float* scale, uint8_t* q, int64_t ld_q, hipStream_t s,
                               const QuantBatch& bt = QuantBatch{1, 0, 0, 0, nullptr});
hipError_t launch_silu_mul(const void* x, bool f16, int64_t M, int64_t K, int64_t ld_x, float* y,
                           int64_t ld_y, hipStream_t s);
hipError_t launch_quant_wblock(const void* w, bool f16, int64_t N, int64_t K, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, float* scales, hipStream_t s);

// Logical partitions of a fused weight's rows: partition i is rows
// off[i] .. off[i + 1] - 1 (off[0] = 0, off[n] = N).
constexpr int kMaxWeightParts = 16;
struct WeightParts {
  int64_t off[kMaxWeightParts + 1];
  int n;
};
hipError_t launch_requant_max(const uint8_t* w, int64_t ldw, int64_t N, int64_t K,
                              const WeightParts& parts, const float* scales, uint8_t* q,
                              int64_t ldq, float* max_out, hipStream_t s);
hipError_t launch_channelwise(const float* scales, const WeightParts& parts, int64_t N, float* out,
                              hipStream_t s);

struct GemmArgs {
  const uint8_t* A;
  int64_t lda;
  const uint8_t* B;
  int64_t ldb;
  uint16_t* C;
  int64_t ldc;
  int64_t M, N, K;
  const void* sa;
  int sa_kind;  // fp8sm_scale_kind
  const void* sb;
  int sb_kind;
  const void* bias;  // rowwise / per-tensor only: output-dtype [N] or nullptr
  int out_f16;       // rowwise / per-tensor only: fp16 output instead of bf16
  GemmBatch batch{1, 0, 0, 0, 0, 0, nullptr};
};

// Rowwise / per-tensor variants.  All of them produce bitwise-identical rows.
// The tile variants use wavefronts of 64 x 64 outputs and a DMA-fed LDS ring.
enum Variant {
  VAR_TILE_128x128 = 0,  // 128x128 tiles, 4 wavefronts, two workgroups per CU
  VAR_TILE_128x256 = 1,  // 128x256 tiles, 8 wavefronts, one workgroup per CU
  VAR_TILE_256x128 = 2,  // 256x128 tiles, 8 wavefronts, one workgroup per CU
  VAR_DECODE_32 = 3,     // M <= 32: eight wavefronts per 32 columns, one 512-K block each
  VAR_DECODE_64 = 4,     // M <= 64: four wavefronts per 32 columns
  VAR_DECODE_32_W4 = 5,  // M <= 32: four wavefronts per 32 columns, two workgroups per CU
  VAR_DECODE_16 = 6,     // M <= 32: eight wavefronts per 16 columns (twice the workgroups)
  VAR_COUNT = 7
};
const char* variant_name(int v);
bool variant_accepts(int v, int64_t M);
hipError_t launch_gemm_rowwise(int variant, const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_blockwise(const GemmArgs& g, hipStream_t s);
// The rowwise GEMM on the fp8 matrix instructions (evidence only: inexact).
hipError_t launch_gemm_rowwise_fp8mfma(const GemmArgs& g, hipStream_t s);
// One matrix instruction on host-supplied register images (probe.hip).
hipError_t launch_mfma_probe(int instr, const uint32_t* a, const uint32_t* b, float* d,
                             hipStream_t s);
hipError_t launch_rate_probe(int widen, int blocks, int waves_per_block, int iters, float* sink,
                             hipStream_t s);
hipError_t launch_fill_k0(uint16_t* C, int64_t ldc, int64_t M, int64_t N, const void* bias,
                          hipStream_t s, const GemmBatch& bt = GemmBatch{1, 0, 0, 0, 0, 0, nullptr});

}  // namespace fp8sm

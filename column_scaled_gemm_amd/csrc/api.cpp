// C ABI of libfp8sm.so: argument validation, scale sizing, shape dispatch and
// launch.  Every check runs on the host before anything is enqueued, and the
// kernel that runs is exactly the one validated -- no silent fallback (the
// load-time / run-time gate mismatch described in the prhub digest of sglang
// PR #33148, implementation section, is the failure this avoids).
#include <hip/hip_runtime_api.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "../../include/fp8sm.h"
#include "launch.h"
#include "dispatch_table.h"

using namespace fp8sm;

namespace {

std::atomic<int> g_forced_variant{-1};

// gfx950 check, cached per device id.
fp8sm_status check_device() {
  static std::mutex mu;
  static signed char ok_cache[64];
  static bool init = false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8SM_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return FP8SM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!init) {
    memset(ok_cache, -1, sizeof ok_cache);
    init = true;
  }
  if (ok_cache[dev] < 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FP8SM_ERR_DEVICE;
    ok_cache[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  }
  return ok_cache[dev] ? FP8SM_OK : FP8SM_ERR_DEVICE;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline fp8sm_status launched(hipError_t e) { return e == hipSuccess ? FP8SM_OK : FP8SM_ERR_LAUNCH; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxK = 65536;
// GEMM operand row strides (bytes): the kernels address up to 64 rows of A or
// B with 32-bit offsets from one base, so 64 * stride + K must stay below 2^31.
constexpr int64_t kMaxGemmLd = (int64_t)1 << 24;
constexpr int64_t kMaxBatch = 65535;  // one grid row (blockIdx.y) per batch

// Batch arguments common to every batched call: the count, non-negative
// strides, and an int32-aligned row-count array (or NULL).
fp8sm_status check_batch(int64_t nbatch, const int32_t* rows, std::initializer_list<int64_t> strides) {
  if (nbatch < 0) return FP8SM_ERR_SHAPE;
  if (nbatch > kMaxBatch) return FP8SM_ERR_RANGE;
  for (int64_t st : strides)
    if (st < 0) return FP8SM_ERR_SHAPE;
  if (rows && !aligned(rows, 4)) return FP8SM_ERR_ALIGN;
  return FP8SM_OK;
}

// Batches write disjoint outputs: a batch stride of an output at least spans
// one batch's rows (rows - 1 strides of ld plus one row of `len`).
inline bool disjoint(int64_t nbatch, int64_t stride, int64_t rows, int64_t ld, int64_t len) {
  return nbatch <= 1 || rows == 0 || stride >= (rows - 1) * ld + len;
}

}  // namespace

extern "C" {

const char* fp8sm_status_str(fp8sm_status s) {
  switch (s) {
    case FP8SM_OK: return "ok";
    case FP8SM_ERR_NULL: return "null pointer argument";
    case FP8SM_ERR_SHAPE: return "invalid shape, leading dimension or group size";
    case FP8SM_ERR_ALIGN: return "pointer, leading dimension or size breaks the 16-byte alignment rule";
    case FP8SM_ERR_UNSUPPORTED: return "unsupported enum value or combination";
    case FP8SM_ERR_LAUNCH: return "kernel launch failed";
    case FP8SM_ERR_DEVICE: return "current device is not gfx950 (MI355X) or unavailable";
    case FP8SM_ERR_RANGE: return "size beyond the supported range";
    default: return "unknown status";
  }
}

size_t fp8sm_scale_bytes(fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, int64_t M, int64_t K_out,
                         int32_t group) {
  if (M < 0 || K_out <= 0 || group <= 0 || K_out % group) return 0;
  if (fmt != FP8SM_SCALE_FP32 && fmt != FP8SM_SCALE_UE8M0_FP32 && fmt != FP8SM_SCALE_UE8M0_BYTE)
    return 0;
  if (lay != FP8SM_LAYOUT_ROW_MAJOR && lay != FP8SM_LAYOUT_MN_MAJOR) return 0;
  const int64_t G = K_out / group;
  const int64_t esz = fmt == FP8SM_SCALE_UE8M0_BYTE ? 1 : 4;
  const int64_t rows = lay == FP8SM_LAYOUT_MN_MAJOR ? ((M + 3) / 4) * 4 : M;
  return (size_t)(rows * G * esz);
}

static fp8sm_status quant_group_impl(const void* x, fp8sm_dtype in, int64_t nbatch, int64_t M,
                                     int64_t K_out, int64_t bs_x, int64_t ld_x,
                                     const int32_t* rows, int32_t group, uint32_t flags,
                                     fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, uint8_t* q,
                                     int64_t bs_q, int64_t ld_q, void* scales,
                                     hipStream_t stream) {
  fp8sm_status bst = check_batch(nbatch, rows, {bs_x, bs_q});
  if (bst != FP8SM_OK) return bst;
  if (in != FP8SM_BF16 && in != FP8SM_FP16) return FP8SM_ERR_UNSUPPORTED;
  if (fmt != FP8SM_SCALE_FP32 && fmt != FP8SM_SCALE_UE8M0_FP32 && fmt != FP8SM_SCALE_UE8M0_BYTE)
    return FP8SM_ERR_UNSUPPORTED;
  if (lay != FP8SM_LAYOUT_ROW_MAJOR && lay != FP8SM_LAYOUT_MN_MAJOR) return FP8SM_ERR_UNSUPPORTED;
  if (flags & ~FP8SM_FUSE_SILU_MUL) return FP8SM_ERR_UNSUPPORTED;
  const bool fused = (flags & FP8SM_FUSE_SILU_MUL) != 0;
  if (M < 0 || K_out <= 0) return FP8SM_ERR_SHAPE;
  if (M > kMaxDim || K_out > kMaxDim) return FP8SM_ERR_RANGE;
  if (group != 128 && group != K_out) return FP8SM_ERR_SHAPE;
  if (K_out % group) return FP8SM_ERR_SHAPE;
  const int64_t row_in = fused ? 2 * K_out : K_out;
  if (ld_x < row_in || ld_q < K_out) return FP8SM_ERR_SHAPE;
  if (K_out % 8 || ld_x % 8 || ld_q % 8 || bs_x % 8 || bs_q % 8) return FP8SM_ERR_ALIGN;
  if (!disjoint(nbatch, bs_q, M, ld_q, K_out)) return FP8SM_ERR_SHAPE;
  if (M == 0 || nbatch == 0) return FP8SM_OK;
  if (!x || !q || !scales) return FP8SM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scales, fmt == FP8SM_SCALE_UE8M0_BYTE ? 1 : 4))
    return FP8SM_ERR_ALIGN;
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  QuantArgs a;
  a.x = x;
  a.f16 = in == FP8SM_FP16;
  a.M = M;
  a.K = K_out;
  a.ld_x = ld_x;
  a.group = group;
  a.fused = fused;
  a.fmt = (int)fmt;
  a.mn_major = lay == FP8SM_LAYOUT_MN_MAJOR;
  a.mpad = ((M + 3) / 4) * 4;
  a.q = q;
  a.ld_q = ld_q;
  a.scales = scales;
  const int64_t esz = fmt == FP8SM_SCALE_UE8M0_BYTE ? 1 : 4;
  a.batch = QuantBatch{nbatch, bs_x, bs_q,
                       (int64_t)fp8sm_scale_bytes(fmt, lay, M, K_out, group) / esz, rows};
  return launched(launch_quant_group(a, stream));
}

fp8sm_status fp8sm_quant_group(const void* x, fp8sm_dtype in, int64_t M, int64_t K_out,
                               int64_t ld_x, int32_t group, uint32_t flags,
                               fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, uint8_t* q,
                               int64_t ld_q, void* scales, hipStream_t stream) {
  return quant_group_impl(x, in, 1, M, K_out, 0, ld_x, nullptr, group, flags, fmt, lay, q, 0,
                          ld_q, scales, stream);
}

fp8sm_status fp8sm_quant_group_batched(const void* x, fp8sm_dtype in, int64_t nbatch, int64_t M,
                                       int64_t K_out, int64_t bs_x, int64_t ld_x,
                                       const int32_t* rows, int32_t group, uint32_t flags,
                                       fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, uint8_t* q,
                                       int64_t bs_q, int64_t ld_q, void* scales,
                                       hipStream_t stream) {
  return quant_group_impl(x, in, nbatch, M, K_out, bs_x, ld_x, rows, group, flags, fmt, lay, q,
                          bs_q, ld_q, scales, stream);
}

fp8sm_status fp8sm_quant_group_scatter(const void* x, fp8sm_dtype in, int64_t T, int64_t K,
                                       int64_t ld_x, const int32_t* dst, int32_t topk, int64_t R,
                                       fp8sm_scale_fmt fmt, fp8sm_scale_layout lay, uint8_t* q,
                                       int64_t ld_q, void* scales, hipStream_t stream) {
  if (in != FP8SM_BF16 && in != FP8SM_FP16) return FP8SM_ERR_UNSUPPORTED;
  if (fmt != FP8SM_SCALE_FP32 && fmt != FP8SM_SCALE_UE8M0_FP32 && fmt != FP8SM_SCALE_UE8M0_BYTE)
    return FP8SM_ERR_UNSUPPORTED;
  if (lay != FP8SM_LAYOUT_ROW_MAJOR && lay != FP8SM_LAYOUT_MN_MAJOR) return FP8SM_ERR_UNSUPPORTED;
  if (T < 0 || R < 0 || K <= 0 || topk < 0) return FP8SM_ERR_SHAPE;
  if (T > kMaxDim || R > kMaxDim || K > kMaxDim || topk > 1024) return FP8SM_ERR_RANGE;
  if (K % 128) return FP8SM_ERR_SHAPE;
  if (ld_x < K || ld_q < K) return FP8SM_ERR_SHAPE;
  if (ld_x % 8 || ld_q % 8) return FP8SM_ERR_ALIGN;
  if (T == 0 || topk == 0 || R == 0) return FP8SM_OK;
  if (!x || !dst || !q || !scales) return FP8SM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(dst, 4) ||
      !aligned(scales, fmt == FP8SM_SCALE_UE8M0_BYTE ? 1 : 4))
    return FP8SM_ERR_ALIGN;
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  ScatterArgs a;
  a.x = x;
  a.f16 = in == FP8SM_FP16;
  a.T = T;
  a.K = K;
  a.ld_x = ld_x;
  a.dst = dst;
  a.topk = topk;
  a.R = R;
  a.fmt = (int)fmt;
  a.mn_major = lay == FP8SM_LAYOUT_MN_MAJOR;
  a.rpad = ((R + 3) / 4) * 4;
  a.q = q;
  a.ld_q = ld_q;
  a.scales = scales;
  return launched(launch_quant_scatter(a, stream));
}

static fp8sm_status quant_static_impl(const void* x, fp8sm_dtype in, int64_t nbatch, int64_t M,
                                      int64_t K, int64_t bs_x, int64_t ld_x, const float* scale,
                                      uint8_t* q, int64_t bs_q, int64_t ld_q,
                                      hipStream_t stream) {
  fp8sm_status bst = check_batch(nbatch, nullptr, {bs_x, bs_q});
  if (bst != FP8SM_OK) return bst;
  if (in != FP8SM_BF16 && in != FP8SM_FP16) return FP8SM_ERR_UNSUPPORTED;
  if (M < 0 || K <= 0) return FP8SM_ERR_SHAPE;
  if (M > kMaxDim || K > kMaxDim) return FP8SM_ERR_RANGE;
  if (ld_x < K || ld_q < K) return FP8SM_ERR_SHAPE;
  if (K % 8 || ld_x % 8 || ld_q % 8 || bs_x % 8 || bs_q % 8) return FP8SM_ERR_ALIGN;
  if (!disjoint(nbatch, bs_q, M, ld_q, K)) return FP8SM_ERR_SHAPE;
  if (M == 0 || nbatch == 0) return FP8SM_OK;
  if (!x || !q || !scale) return FP8SM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 4)) return FP8SM_ERR_ALIGN;
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  return launched(launch_quant_static(x, in == FP8SM_FP16, M, K, ld_x, scale, q, ld_q, stream,
                                      QuantBatch{nbatch, bs_x, bs_q, 0, nullptr}));
}

fp8sm_status fp8sm_quant_static(const void* x, fp8sm_dtype in, int64_t M, int64_t K,
                                int64_t ld_x, const float* scale, uint8_t* q, int64_t ld_q,
                                hipStream_t stream) {
  return quant_static_impl(x, in, 1, M, K, 0, ld_x, scale, q, 0, ld_q, stream);
}

fp8sm_status fp8sm_quant_static_batched(const void* x, fp8sm_dtype in, int64_t nbatch, int64_t M,
                                        int64_t K, int64_t bs_x, int64_t ld_x,
                                        const float* scale, uint8_t* q, int64_t bs_q,
                                        int64_t ld_q, hipStream_t stream) {
  return quant_static_impl(x, in, nbatch, M, K, bs_x, ld_x, scale, q, bs_q, ld_q, stream);
}

fp8sm_status fp8sm_quant_weight_block128(const void* w, fp8sm_dtype in, int64_t N, int64_t K,
                                         int64_t ld_w, uint8_t* q, int64_t ld_q, float* scales,
                                         hipStream_t stream) {
  if (in != FP8SM_BF16 && in != FP8SM_FP16) return FP8SM_ERR_UNSUPPORTED;
  if (N < 0 || K <= 0) return FP8SM_ERR_SHAPE;
  if (N > kMaxDim || K > kMaxDim || (N + 127) / 128 > 65535) return FP8SM_ERR_RANGE;
  if (ld_w < K || ld_q < K) return FP8SM_ERR_SHAPE;
  if (K % 8 || ld_w % 8 || ld_q % 8) return FP8SM_ERR_ALIGN;
  if (N == 0) return FP8SM_OK;
  if (!w || !q || !scales) return FP8SM_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 8) || !aligned(scales, 4)) return FP8SM_ERR_ALIGN;
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  return launched(launch_quant_wblock(w, in == FP8SM_FP16, N, K, ld_w, q, ld_q, scales, stream));
}

// Partition offsets from host widths: 1..16 non-negative widths summing to N.
static fp8sm_status weight_parts(const int64_t* widths, int32_t nparts, int64_t N,
                                 WeightParts* parts) {
  if (!widths) return FP8SM_ERR_NULL;
  if (nparts < 1 || nparts > kMaxWeightParts) return FP8SM_ERR_RANGE;
  parts->n = nparts;
  parts->off[0] = 0;
  for (int i = 0; i < nparts; ++i) {
    if (widths[i] < 0) return FP8SM_ERR_SHAPE;
    parts->off[i + 1] = parts->off[i] + widths[i];
    if (parts->off[i + 1] > kMaxDim) return FP8SM_ERR_RANGE;
  }
  if (N >= 0 && parts->off[nparts] != N) return FP8SM_ERR_SHAPE;
  return FP8SM_OK;
}

fp8sm_status fp8sm_requantize_max_scale(const uint8_t* w, int64_t ldw, int64_t N, int64_t K,
                                        const int64_t* widths, int32_t nparts,
                                        const float* scales, uint8_t* q, int64_t ldq,
                                        float* max_scale, hipStream_t stream) {
  if (N < 0 || K < 0) return FP8SM_ERR_SHAPE;
  if (N > kMaxDim || K > kMaxDim) return FP8SM_ERR_RANGE;
  WeightParts parts;
  fp8sm_status st = weight_parts(widths, nparts, N, &parts);
  if (st != FP8SM_OK) return st;
  if (ldw < K || ldq < K) return FP8SM_ERR_SHAPE;
  if (K % 16 || ldw % 16 || ldq % 16) return FP8SM_ERR_ALIGN;
  if (q == w && ldq != ldw) return FP8SM_ERR_SHAPE;  // in place only row for row
  if (!scales || !max_scale) return FP8SM_ERR_NULL;
  if (!aligned(scales, 4) || !aligned(max_scale, 4)) return FP8SM_ERR_ALIGN;
  if ((N > 0 && K > 0) && (!w || !q)) return FP8SM_ERR_NULL;
  if ((w && !aligned(w, 16)) || (q && !aligned(q, 16))) return FP8SM_ERR_ALIGN;
  st = check_device();
  if (st != FP8SM_OK) return st;
  return launched(launch_requant_max(w, ldw, N, K, parts, scales, q, ldq, max_scale, stream));
}

fp8sm_status fp8sm_scales_to_channelwise(const float* scales, const int64_t* widths,
                                         int32_t nparts, float* out, hipStream_t stream) {
  WeightParts parts;
  fp8sm_status st = weight_parts(widths, nparts, -1, &parts);
  if (st != FP8SM_OK) return st;
  const int64_t N = parts.off[nparts];
  if (N == 0) return FP8SM_OK;
  if (!scales || !out) return FP8SM_ERR_NULL;
  if (!aligned(scales, 4) || !aligned(out, 4)) return FP8SM_ERR_ALIGN;
  st = check_device();
  if (st != FP8SM_OK) return st;
  return launched(launch_channelwise(scales, parts, N, out, stream));
}

fp8sm_status fp8sm_silu_mul_f32(const void* x, fp8sm_dtype in, int64_t M, int64_t K_out,
                                int64_t ld_x, float* y, int64_t ld_y, hipStream_t stream) {
  if (in != FP8SM_BF16 && in != FP8SM_FP16) return FP8SM_ERR_UNSUPPORTED;
  if (M < 0 || K_out <= 0) return FP8SM_ERR_SHAPE;
  if (M > kMaxDim || K_out > kMaxDim) return FP8SM_ERR_RANGE;
  if (ld_x < 2 * K_out || ld_y < K_out) return FP8SM_ERR_SHAPE;
  if (K_out % 8 || ld_x % 8 || ld_y % 8) return FP8SM_ERR_ALIGN;
  if (M == 0) return FP8SM_OK;
  if (!x || !y) return FP8SM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return FP8SM_ERR_ALIGN;
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  return launched(launch_silu_mul(x, in == FP8SM_FP16, M, K_out, ld_x, y, ld_y, stream));
}

int fp8sm_variant_count(void) { return VAR_COUNT; }

const char* fp8sm_variant_name(int id) { return variant_name(id); }

int fp8sm_force_variant(int id) {
  if (id < -1 || id >= VAR_COUNT) id = -1;
  return g_forced_variant.exchange(id);
}

int fp8sm_variant_accepts(int id, int64_t M, int64_t N, int64_t K) {
  (void)N;
  (void)K;  // no variant bounds N or K beyond the call's own limits
  return id >= 0 && id < VAR_COUNT && variant_accepts(id, M) ? 1 : 0;
}

int fp8sm_pick_variant(int64_t M, int64_t N, int64_t K) {
  const int forced = g_forced_variant.load();
  if (forced >= 0) return forced;
  return pick_from_table(M, N, K);
}

static fp8sm_status scaled_mm_impl(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                   void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                   fp8sm_scale_kind ka, const void* sa, fp8sm_scale_kind kb,
                                   const void* sb, const void* bias, fp8sm_dtype out,
                                   hipStream_t stream,
                                   const GemmBatch& bt = GemmBatch{1, 0, 0, 0, 0, 0, nullptr},
                                   bool fp8mfma = false) {
  fp8sm_status bst = check_batch(bt.count, bt.rows, {bt.a, bt.b, bt.c, bt.sa, bt.sb});
  if (bst != FP8SM_OK) return bst;
  const bool rowwise = (ka == FP8SM_KIND_TENSOR || ka == FP8SM_KIND_ROW) &&
                       (kb == FP8SM_KIND_TENSOR || kb == FP8SM_KIND_COL);
  const bool blockwise = (ka == FP8SM_KIND_GROUP128_UE8M0 || ka == FP8SM_KIND_GROUP128_FP32) &&
                         kb == FP8SM_KIND_BLOCK128;
  if (!rowwise && !blockwise) return FP8SM_ERR_UNSUPPORTED;
  if (out != FP8SM_BF16 && out != FP8SM_FP16) return FP8SM_ERR_UNSUPPORTED;
  if (blockwise && (bias || out != FP8SM_BF16)) return FP8SM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0) return FP8SM_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxK) return FP8SM_ERR_RANGE;
  if (lda < K || ldb < K || ldc < N) return FP8SM_ERR_SHAPE;
  if (lda > kMaxGemmLd || ldb > kMaxGemmLd) return FP8SM_ERR_RANGE;
  if (K % 16 || lda % 16 || ldb % 16 || bt.a % 16 || bt.b % 16) return FP8SM_ERR_ALIGN;
  if (N % 8 || ldc % 8 || bt.c % 8) return FP8SM_ERR_ALIGN;
  if (!disjoint(bt.count, bt.c, M, ldc, N)) return FP8SM_ERR_SHAPE;
  if (M == 0 || N == 0 || bt.count == 0) return FP8SM_OK;
  if (!C) return FP8SM_ERR_NULL;
  if (!aligned(C, 16)) return FP8SM_ERR_ALIGN;
  if (bias && !aligned(bias, 2)) return FP8SM_ERR_ALIGN;
  if (K > 0) {
    if (!A || !B || !sa || !sb) return FP8SM_ERR_NULL;
    if (!aligned(A, 16) || !aligned(B, 16)) return FP8SM_ERR_ALIGN;
    if (!aligned(sb, 4) || (ka != FP8SM_KIND_GROUP128_UE8M0 && !aligned(sa, 4)))
      return FP8SM_ERR_ALIGN;
  }
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  uint16_t* Cb = static_cast<uint16_t*>(C);
  if (K == 0) return launched(launch_fill_k0(Cb, ldc, M, N, bias, stream, bt));
  GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.C = Cb;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.sa = sa;
  g.sa_kind = (int)ka;
  g.sb = sb;
  g.sb_kind = (int)kb;
  g.bias = bias;
  g.out_f16 = out == FP8SM_FP16;
  g.batch = bt;
  if (fp8mfma) return launched(launch_gemm_rowwise_fp8mfma(g, stream));
  if (blockwise) return launched(launch_gemm_blockwise(g, stream));
  int v = fp8sm_pick_variant(M, N, K);
  if (!variant_accepts(v, M)) return FP8SM_ERR_UNSUPPORTED;
  return launched(launch_gemm_rowwise(v, g, stream));
}

fp8sm_status fp8sm_scaled_mm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                             void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             fp8sm_scale_kind ka, const void* sa, fp8sm_scale_kind kb,
                             const void* sb, hipStream_t stream) {
  return scaled_mm_impl(A, lda, B, ldb, C, ldc, M, N, K, ka, sa, kb, sb, nullptr, FP8SM_BF16,
                        stream);
}

fp8sm_status fp8sm_scaled_mm_ex(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                fp8sm_scale_kind ka, const void* sa, fp8sm_scale_kind kb,
                                const void* sb, const void* bias, fp8sm_dtype out,
                                hipStream_t stream) {
  return scaled_mm_impl(A, lda, B, ldb, C, ldc, M, N, K, ka, sa, kb, sb, bias, out, stream);
}

fp8sm_status fp8sm_scaled_mm_fp8mfma(const uint8_t* A, int64_t lda, const uint8_t* B,
                                     int64_t ldb, void* C, int64_t ldc, int64_t M, int64_t N,
                                     int64_t K, fp8sm_scale_kind ka, const void* sa,
                                     fp8sm_scale_kind kb, const void* sb, hipStream_t stream) {
  const bool rowwise = (ka == FP8SM_KIND_TENSOR || ka == FP8SM_KIND_ROW) &&
                       (kb == FP8SM_KIND_TENSOR || kb == FP8SM_KIND_COL);
  if (!rowwise) return FP8SM_ERR_UNSUPPORTED;
  return scaled_mm_impl(A, lda, B, ldb, C, ldc, M, N, K, ka, sa, kb, sb, nullptr, FP8SM_BF16,
                        stream, GemmBatch{1, 0, 0, 0, 0, 0, nullptr}, true);
}

fp8sm_status fp8sm_mfma_probe(int32_t instr, const uint32_t* a_regs, const uint32_t* b_regs,
                              float* d_regs, hipStream_t stream) {
  if (instr < 0 || instr > 4) return FP8SM_ERR_UNSUPPORTED;
  if (!a_regs || !b_regs || !d_regs) return FP8SM_ERR_NULL;
  if (!aligned(a_regs, 16) || !aligned(b_regs, 16) || !aligned(d_regs, 16)) return FP8SM_ERR_ALIGN;
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  return launched(launch_mfma_probe(instr, a_regs, b_regs, d_regs, stream));
}

fp8sm_status fp8sm_rate_probe(int32_t widen, int32_t blocks, int32_t waves_per_block,
                              int32_t iters, float* sink, hipStream_t stream) {
  if (widen < 0 || widen > 1) return FP8SM_ERR_UNSUPPORTED;
  if (waves_per_block != 4 && waves_per_block != 8 && waves_per_block != 16)
    return FP8SM_ERR_UNSUPPORTED;
  if (!sink) return FP8SM_ERR_NULL;
  if (!aligned(sink, 4)) return FP8SM_ERR_ALIGN;
  if (blocks < 1 || iters < 1) return FP8SM_ERR_SHAPE;
  if (blocks > 65536 || iters > (1 << 24)) return FP8SM_ERR_RANGE;
  fp8sm_status st = check_device();
  if (st != FP8SM_OK) return st;
  return launched(launch_rate_probe(widen, blocks, waves_per_block, iters, sink, stream));
}

fp8sm_status fp8sm_scaled_mm_batched(int64_t nbatch, const int32_t* rows, const uint8_t* A,
                                     int64_t bs_a, int64_t lda, const uint8_t* B, int64_t bs_b,
                                     int64_t ldb, void* C, int64_t bs_c, int64_t ldc, int64_t M,
                                     int64_t N, int64_t K, fp8sm_scale_kind ka, const void* sa,
                                     int64_t bs_sa, fp8sm_scale_kind kb, const void* sb,
                                     int64_t bs_sb, const void* bias, fp8sm_dtype out,
                                     hipStream_t stream) {
  return scaled_mm_impl(A, lda, B, ldb, C, ldc, M, N, K, ka, sa, kb, sb, bias, out, stream,
                        GemmBatch{nbatch, bs_a, bs_b, bs_c, bs_sa, bs_sb, rows});
}

}  // extern "C"

// extern "C" entry points of librvq.so (declared in include/rvq.h): argument validation, workspace
// layout, and calls into the kernel launchers.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rvq.h"
#include "device.hpp"
#include "launch.hpp"

using namespace rvq;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? RVQ_OK : RVQ_ERR_HIP; }

// Largest element count the kernels index with 32-bit row/column arithmetic.
constexpr int64_t kMaxDim = 1 << 24;

inline bool valid_matrix_shape(int64_t rows, int64_t cols) {
  return rows >= 1 && cols >= 8 && cols % 8 == 0 && rows <= kMaxDim && cols <= kMaxDim;
}

inline bool table_dtype(int32_t d) { return d == RVQ_F32 || d == RVQ_F16; }

int check_bank(const rvq_expert_bank_t* bank) {
  if (!bank || !bank->codes || !bank->codebooks) return RVQ_ERR_NULL;
  if (bank->num_experts < 1 || bank->num_experts > kMaxExperts) return RVQ_ERR_SHAPE;
  if (!valid_matrix_shape(bank->inter, bank->hidden) || bank->inter % 8 != 0) return RVQ_ERR_SHAPE;
  if (!aligned(bank->codes, 16) || !aligned(bank->codebooks, 16)) return RVQ_ERR_ALIGN;
  if (bank->record_stride % 256 != 0) return RVQ_ERR_ALIGN;
  if (bank->record_stride < (int64_t)rvq_bank_record_bytes(bank->hidden, bank->inter)) return RVQ_ERR_SHAPE;
  return RVQ_OK;
}

}  // namespace

extern "C" {

const char* rvq_status_string(int status) {
  switch (status) {
    case RVQ_OK: return "RVQ_OK";
    case RVQ_ERR_NULL: return "RVQ_ERR_NULL: a required pointer is NULL";
    case RVQ_ERR_SHAPE: return "RVQ_ERR_SHAPE: a size is out of range or inconsistent";
    case RVQ_ERR_DTYPE: return "RVQ_ERR_DTYPE: unsupported dtype";
    case RVQ_ERR_ALIGN: return "RVQ_ERR_ALIGN: pointer or stride misaligned";
    case RVQ_ERR_WORKSPACE: return "RVQ_ERR_WORKSPACE: workspace too small";
    case RVQ_ERR_EXPERT_ID: return "RVQ_ERR_EXPERT_ID: an expert id outside [0, num_experts) was seen";
    case RVQ_ERR_HIP: return "RVQ_ERR_HIP: a HIP runtime call failed";
    case RVQ_ERR_DEVICE_STALL: return "RVQ_ERR_DEVICE_STALL: a kernel's bounded internal wait gave up";
    case RVQ_ERR_RECORD: return "RVQ_ERR_RECORD: an expert record failed its header or payload check";
    default: return "RVQ: unknown status";
  }
}

size_t rvq_packed_bytes(int32_t rows, int32_t cols) {
  if (!valid_matrix_shape(rows, cols)) return 0;
  return (size_t)packed_bytes(rows, cols);
}

int rvq_pack_codes(const uint8_t* src, int32_t rows, int32_t cols, uint8_t* dst, hipStream_t stream) {
  if (!src || !dst) return RVQ_ERR_NULL;
  if (!valid_matrix_shape(rows, cols)) return RVQ_ERR_SHAPE;
  if (!aligned(dst, 16)) return RVQ_ERR_ALIGN;
  return hip_status(launch_pack(src, rows, cols, dst, stream));
}

int rvq_lut_build(const float* x, int32_t cols, const float* codebooks, int32_t lut_dtype, void* lut,
                  int32_t* log2_scale, hipStream_t stream) {
  if (!x || !codebooks || !lut || !log2_scale) return RVQ_ERR_NULL;
  if (cols < 8 || cols % 8 != 0 || cols > kMaxDim) return RVQ_ERR_SHAPE;
  if (!table_dtype(lut_dtype)) return RVQ_ERR_DTYPE;
  if (!aligned(codebooks, 16) || !aligned(lut, 16) || !aligned(x, 4)) return RVQ_ERR_ALIGN;
  return hip_status(launch_lut_build(x, cols, codebooks, lut_dtype == RVQ_F16, lut, log2_scale, stream));
}

size_t rvq_expert_gemv_workspace_bytes(int32_t rows, int32_t cols, int32_t lut_dtype) {
  if (!valid_matrix_shape(rows, cols) || !table_dtype(lut_dtype)) return 0;
  return gemv_workspace_bytes(rows, cols, lut_dtype == RVQ_F16);
}

int rvq_expert_gemv(const rvq_matrix_t* W, const float* x, int32_t lut_dtype, float* y, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (!W || !W->codes || !W->codebooks || !x || !y || !workspace) return RVQ_ERR_NULL;
  if (!valid_matrix_shape(W->rows, W->cols)) return RVQ_ERR_SHAPE;
  if (!table_dtype(lut_dtype)) return RVQ_ERR_DTYPE;
  if (!aligned(W->codes, 16) || !aligned(W->codebooks, 16) || !aligned(workspace, 256) || !aligned(x, 4) ||
      !aligned(y, 4))
    return RVQ_ERR_ALIGN;
  if (workspace_bytes < gemv_workspace_bytes(W->rows, W->cols, lut_dtype == RVQ_F16)) return RVQ_ERR_WORKSPACE;
  return hip_status(
      launch_gemv(W->codes, W->codebooks, W->rows, W->cols, x, lut_dtype == RVQ_F16, y, workspace, stream));
}

int rvq_router_topk(const void* w_router_bf16, const void* x, int32_t x_dtype, int32_t T, int32_t E, int32_t H,
                    int32_t k, int32_t* ids, float* gates, double* logits, hipStream_t stream) {
  if (!w_router_bf16 || !x || !ids || !gates || !logits) return RVQ_ERR_NULL;
  if (T < 1 || E < 1 || E > kMaxExperts || H < 1 || H > kMaxDim || k < 1 || k > E || k > kMaxTopK)
    return RVQ_ERR_SHAPE;
  if ((int64_t)T * E > ((int64_t)1 << 31) || (int64_t)T * H > ((int64_t)1 << 40)) return RVQ_ERR_SHAPE;
  if (x_dtype != RVQ_F32 && x_dtype != RVQ_BF16) return RVQ_ERR_DTYPE;
  if (!aligned(w_router_bf16, 2) || !aligned(x, x_dtype == RVQ_F32 ? 4 : 2) || !aligned(logits, 8) ||
      !aligned(ids, 4) || !aligned(gates, 4))
    return RVQ_ERR_ALIGN;
  return hip_status(launch_router_topk(static_cast<const uint16_t*>(w_router_bf16), x, x_dtype == RVQ_BF16, T, E, H,
                                       k, ids, gates, logits, stream));
}

size_t rvq_bank_record_bytes(int32_t hidden, int32_t inter) {
  if (!valid_matrix_shape(inter, hidden) || !valid_matrix_shape(hidden, inter)) return 0;
  return (size_t)(2 * packed_bytes(inter, hidden) + packed_bytes(hidden, inter));
}

// Largest chunk the bucketing workgroup handles (its per-expert token bitmaps live in 64 KiB of LDS).
inline bool chunk_shape_ok(const rvq_expert_bank_t* bank, int32_t T, int32_t k) {
  if (T < 2 || T > 4096 || k < 1 || k > kMaxTopK || k > bank->num_experts) return false;
  if (bank->hidden % 64 != 0 || bank->inter % 64 != 0) return false;
  const int64_t words = (int64_t)bank->num_experts * ((T + 31) / 32) + bank->num_experts + 1;
  return words <= 16384;
}

size_t rvq_moe_layer_workspace_bytes(const rvq_expert_bank_t* bank, int32_t T, int32_t k, int32_t compute_dtype) {
  if (!bank || k < 1 || k > kMaxTopK) return 0;
  if (!valid_matrix_shape(bank->inter, bank->hidden) || bank->inter % 8 != 0) return 0;
  if (T == 1) {
    if (!table_dtype(compute_dtype)) return 0;
    return moe_workspace_layout(bank->hidden, bank->inter, k, compute_dtype == RVQ_F16).total;
  }
  if (compute_dtype != RVQ_F16 && compute_dtype != RVQ_BF16) return 0;
  if (bank->num_experts < 1 || bank->num_experts > kMaxExperts || !chunk_shape_ok(bank, T, k)) return 0;
  return chunk_workspace_bytes(bank->num_experts, bank->hidden, bank->inter, T, k);
}

namespace {
int moe_layer_forward_impl(const rvq_expert_bank_t* bank, const void* x, int32_t x_dtype, int32_t T,
                           const int32_t* ids, const float* gates, int32_t k, const float* residual, float* y,
                           int32_t compute_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream,
                           hipEvent_t* events) {
  int st = check_bank(bank);
  if (st != RVQ_OK) return st;
  if (!x || !ids || !gates || !y || !workspace) return RVQ_ERR_NULL;
  if (T > 1) {
    if (events) return RVQ_ERR_SHAPE;
    if (!chunk_shape_ok(bank, T, k)) return RVQ_ERR_SHAPE;
    if (x_dtype != RVQ_BF16 || (compute_dtype != RVQ_F16 && compute_dtype != RVQ_BF16)) return RVQ_ERR_DTYPE;
    if (!aligned(workspace, 256) || !aligned(x, 16) || !aligned(y, 4) || !aligned(ids, 4) || !aligned(gates, 4) ||
        (residual && !aligned(residual, 4)))
      return RVQ_ERR_ALIGN;
    if (workspace_bytes < chunk_workspace_bytes(bank->num_experts, bank->hidden, bank->inter, T, k))
      return RVQ_ERR_WORKSPACE;
    return hip_status(launch_moe_chunk(bank->codes, bank->codebooks, bank->record_stride, bank->num_experts,
                                       bank->hidden, bank->inter, static_cast<const uint16_t*>(x), T, ids, gates, k,
                                       residual, y, compute_dtype == RVQ_F16, workspace, stream));
  }
  if (T != 1 || k < 1 || k > kMaxTopK) return RVQ_ERR_SHAPE;
  if (x_dtype != RVQ_F32 || !table_dtype(compute_dtype)) return RVQ_ERR_DTYPE;
  if (!aligned(workspace, 256) || !aligned(x, 4) || !aligned(y, 4) || !aligned(ids, 4) || !aligned(gates, 4) ||
      (residual && !aligned(residual, 4)))
    return RVQ_ERR_ALIGN;
  const bool f16 = compute_dtype == RVQ_F16;
  if (workspace_bytes < moe_workspace_layout(bank->hidden, bank->inter, k, f16).total) return RVQ_ERR_WORKSPACE;
  return hip_status(launch_moe_decode(bank->codes, bank->codebooks, bank->record_stride, bank->num_experts,
                                      bank->hidden, bank->inter, static_cast<const float*>(x), ids, gates, k,
                                      residual, y, f16, workspace, stream, events));
}
}  // namespace

int rvq_moe_layer_forward(const rvq_expert_bank_t* bank, const void* x, int32_t x_dtype, int32_t T,
                          const int32_t* ids, const float* gates, int32_t k, const float* residual, float* y,
                          int32_t compute_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return moe_layer_forward_impl(bank, x, x_dtype, T, ids, gates, k, residual, y, compute_dtype, workspace,
                                workspace_bytes, stream, nullptr);
}

int rvq_moe_layer_forward_timed(const rvq_expert_bank_t* bank, const void* x, int32_t x_dtype, int32_t T,
                                const int32_t* ids, const float* gates, int32_t k, const float* residual, float* y,
                                int32_t compute_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* events) {
  if (!events) return RVQ_ERR_NULL;
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return RVQ_ERR_NULL;
  return moe_layer_forward_impl(bank, x, x_dtype, T, ids, gates, k, residual, y, compute_dtype, workspace,
                                workspace_bytes, stream, events);
}

size_t rvq_moe_batch_decode_workspace_bytes(const rvq_expert_bank_t* bank, int32_t T, int32_t k,
                                            int32_t table_dtype_) {
  if (!bank || T < 1 || T > kMaxBatchDecode || k < 1 || k > kMaxTopK) return 0;
  if (!valid_matrix_shape(bank->inter, bank->hidden) || bank->inter % 8 != 0) return 0;
  if (!table_dtype(table_dtype_)) return 0;
  return moe_workspace_layout(bank->hidden, bank->inter, T * k, table_dtype_ == RVQ_F16).total;
}

int rvq_moe_batch_decode(const rvq_expert_bank_t* bank, const float* x, int32_t T, const int32_t* ids,
                         const float* gates, int32_t k, const float* residual, float* y, int32_t table_dtype_,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_bank(bank);
  if (st != RVQ_OK) return st;
  if (!x || !ids || !gates || !y || !workspace) return RVQ_ERR_NULL;
  if (T < 1 || T > kMaxBatchDecode || k < 1 || k > kMaxTopK) return RVQ_ERR_SHAPE;
  if (!table_dtype(table_dtype_)) return RVQ_ERR_DTYPE;
  if (!aligned(workspace, 256) || !aligned(x, 4) || !aligned(y, 4) || !aligned(ids, 4) || !aligned(gates, 4) ||
      (residual && !aligned(residual, 4)))
    return RVQ_ERR_ALIGN;
  const bool f16 = table_dtype_ == RVQ_F16;
  if (workspace_bytes < moe_workspace_layout(bank->hidden, bank->inter, T * k, f16).total) return RVQ_ERR_WORKSPACE;
  return hip_status(launch_moe_batch_decode(bank->codes, bank->codebooks, bank->record_stride, bank->num_experts,
                                            bank->hidden, bank->inter, x, T, ids, gates, k, residual, y, f16,
                                            workspace, stream));
}

int rvq_encode(const float* W, int32_t rows, int32_t cols, const float* codebooks, uint8_t* codes,
               hipStream_t stream) {
  if (!W || !codebooks || !codes) return RVQ_ERR_NULL;
  if (rows < 1 || cols < 8 || cols % 8 != 0) return RVQ_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(codebooks, 16)) return RVQ_ERR_ALIGN;
  return hip_status(launch_rvq_encode(W, rows, cols, codebooks, codes, stream));
}

static bool fit_shape_ok(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 8 || cols % 8 != 0) return false;
  return (int64_t)rows * (cols / 8) <= INT32_MAX;   // sub-vector indices are int32
}

size_t rvq_fit_workspace_bytes(int32_t rows, int32_t cols) {
  if (!fit_shape_ok(rows, cols)) return 0;
  return fit_workspace_bytes((int64_t)rows * (cols / 8));
}

int rvq_fit(const float* W, int32_t rows, int32_t cols, int32_t iters, const int32_t* init_idx, float* codebooks,
            uint8_t* codes, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!W || !init_idx || !codebooks || !codes || !workspace) return RVQ_ERR_NULL;
  if (!fit_shape_ok(rows, cols) || iters < 0 || iters > kMaxFitIters) return RVQ_ERR_SHAPE;
  const int64_t N = (int64_t)rows * (cols / 8);
  for (int i = 0; i < 3 * 256; ++i)
    if (init_idx[i] < 0 || init_idx[i] >= N) return RVQ_ERR_SHAPE;
  if (!aligned(W, 4) || !aligned(codebooks, 16) || !aligned(workspace, 256)) return RVQ_ERR_ALIGN;
  if (workspace_bytes < fit_workspace_bytes(N)) return RVQ_ERR_WORKSPACE;
  return hip_status(launch_rvq_fit(W, rows, cols, iters, init_idx, codebooks, codes, workspace, stream));
}

size_t rvq_bank_crc32_workspace_bytes(const rvq_expert_bank_t* bank) {
  if (check_bank(bank) != RVQ_OK) return 0;
  return crc_workspace_bytes(bank->num_experts, bank->hidden, bank->inter);
}

int rvq_bank_crc32(const rvq_expert_bank_t* bank, uint32_t* crc, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  const int st = check_bank(bank);
  if (st != RVQ_OK) return st;
  if (!crc || !workspace) return RVQ_ERR_NULL;
  if (!aligned(crc, 4) || !aligned(workspace, 256)) return RVQ_ERR_ALIGN;
  if (workspace_bytes < crc_workspace_bytes(bank->num_experts, bank->hidden, bank->inter)) return RVQ_ERR_WORKSPACE;
  return hip_status(launch_bank_crc32(bank->codes, bank->record_stride, bank->num_experts, bank->hidden, bank->inter,
                                      crc, workspace, stream));
}

int rvq_moe_decode_routed(const rvq_expert_bank_t* bank, const void* w_router_bf16, const float* x, int32_t k,
                          const float* residual, float* y, int32_t* ids, float* gates, double* logits,
                          int32_t compute_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_bank(bank);
  if (st != RVQ_OK) return st;
  if (!w_router_bf16 || !x || !y || !ids || !gates || !logits || !workspace) return RVQ_ERR_NULL;
  if (k < 1 || k > kMaxTopK || k > bank->num_experts || bank->num_experts > kMaxExperts) return RVQ_ERR_SHAPE;
  if (!table_dtype(compute_dtype)) return RVQ_ERR_DTYPE;
  if (!aligned(workspace, 256) || !aligned(w_router_bf16, 2) || !aligned(x, 4) || !aligned(y, 4) ||
      !aligned(ids, 4) || !aligned(gates, 4) || !aligned(logits, 8) || (residual && !aligned(residual, 4)))
    return RVQ_ERR_ALIGN;
  const bool f16 = compute_dtype == RVQ_F16;
  if (workspace_bytes < moe_workspace_layout(bank->hidden, bank->inter, k, f16).total) return RVQ_ERR_WORKSPACE;
  const hipError_t err = launch_router_logits(static_cast<const uint16_t*>(w_router_bf16), x, false, 1,
                                              bank->num_experts, bank->hidden, logits, stream);
  if (err != hipSuccess) return RVQ_ERR_HIP;
  const Route route{logits, ids, gates};
  return hip_status(launch_moe_decode(bank->codes, bank->codebooks, bank->record_stride, bank->num_experts,
                                      bank->hidden, bank->inter, x, nullptr, nullptr, k, residual, y, f16, workspace,
                                      stream, nullptr, &route));
}

int rvq_moe_decode_routed_scratch(const rvq_expert_bank_t* bank, const void* w_router_bf16, const float* x, int32_t k,
                                  const float* residual, float* y, int32_t* ids, float* gates, double* logits,
                                  int32_t compute_dtype, int32_t* status, hipStream_t stream) {
  int st = check_bank(bank);
  if (st != RVQ_OK) return st;
  if (!w_router_bf16 || !x || !y || !ids || !gates || !logits || !status) return RVQ_ERR_NULL;
  if (k < 1 || k > kMaxTopK || k > bank->num_experts || bank->num_experts > kMaxExperts) return RVQ_ERR_SHAPE;
  if (!table_dtype(compute_dtype)) return RVQ_ERR_DTYPE;
  if (!aligned(status, 256) || !aligned(w_router_bf16, 2) || !aligned(x, 4) || !aligned(y, 4) || !aligned(ids, 4) ||
      !aligned(gates, 4) || !aligned(logits, 8) || (residual && !aligned(residual, 4)))
    return RVQ_ERR_ALIGN;
  const bool f16 = compute_dtype == RVQ_F16;
  if (moe_workspace_layout(bank->hidden, bank->inter, k, f16).total > kScratchBytes) return RVQ_ERR_WORKSPACE;
  return hip_status(launch_moe_decode_routed_scratch(bank->codes, bank->codebooks, bank->record_stride,
                                                     bank->num_experts, bank->hidden, bank->inter,
                                                     static_cast<const uint16_t*>(w_router_bf16), x, k, residual, y,
                                                     ids, gates, logits, f16, status, stream));
}

int rvq_moe_block_decode(const rvq_expert_bank_t* bank, const void* w_router_bf16, const float* h, int32_t k,
                         float eps, float* h_out, int32_t* ids, float* gates, double* logits, int32_t compute_dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_bank(bank);
  if (st != RVQ_OK) return st;
  if (!w_router_bf16 || !h || !h_out || !ids || !gates || !logits || !workspace) return RVQ_ERR_NULL;
  if (k < 1 || k > kMaxTopK || k > bank->num_experts || bank->num_experts > kMaxExperts || !(eps >= 0.f))
    return RVQ_ERR_SHAPE;
  if (!table_dtype(compute_dtype)) return RVQ_ERR_DTYPE;
  if (!aligned(workspace, 256) || !aligned(w_router_bf16, 2) || !aligned(h, 4) || !aligned(h_out, 4) ||
      !aligned(ids, 4) || !aligned(gates, 4) || !aligned(logits, 8))
    return RVQ_ERR_ALIGN;
  const bool f16 = compute_dtype == RVQ_F16;
  const MoeWorkspace w = moe_workspace_layout(bank->hidden, bank->inter, k, f16);
  if (workspace_bytes < w.total) return RVQ_ERR_WORKSPACE;
  float* n = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + w.norm_off);
  const hipError_t err = launch_router_norm_logits(static_cast<const uint16_t*>(w_router_bf16), h, bank->num_experts,
                                                   bank->hidden, eps, logits, n, stream);
  if (err != hipSuccess) return RVQ_ERR_HIP;
  const Route route{logits, ids, gates};
  return hip_status(launch_moe_decode(bank->codes, bank->codebooks, bank->record_stride, bank->num_experts,
                                      bank->hidden, bank->inter, n, nullptr, nullptr, k, h, h_out, f16, workspace,
                                      stream, nullptr, &route));
}

int rvq_workspace_set_wait_limit(void* workspace, size_t workspace_bytes, int32_t polls, hipStream_t stream) {
  if (!workspace) return RVQ_ERR_NULL;
  if (!aligned(workspace, 256)) return RVQ_ERR_ALIGN;
  if (workspace_bytes < 256) return RVQ_ERR_WORKSPACE;
  if (polls == INT32_MAX) return RVQ_ERR_SHAPE;
  const int32_t word = polls < 0 ? 0 : polls + 1;
  return hip_status(launch_set_word(static_cast<int32_t*>(workspace) + kWaitLimitWord, word, stream));
}

int rvq_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return RVQ_ERR_NULL;
  if (!aligned(workspace, 256)) return RVQ_ERR_ALIGN;
  if (workspace_bytes == 0) return RVQ_OK;
  return hip_status(launch_zero(workspace, workspace_bytes, stream));
}

int rvq_stream_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream) {
  if (!src || !dst) return RVQ_ERR_NULL;
  if (nbytes % 16 != 0) return RVQ_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return RVQ_ERR_ALIGN;
  if (nbytes == 0) return RVQ_OK;
  return hip_status(launch_stream_copy(src, dst, nbytes, stream));
}

int rvq_stream_read(const void* src, size_t nbytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return RVQ_ERR_NULL;
  if (nbytes % 16 != 0) return RVQ_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return RVQ_ERR_ALIGN;
  if (nbytes == 0) return RVQ_OK;
  return hip_status(launch_stream_read(src, nbytes, sink, stream));
}

int rvq_rmsnorm(const float* x, int32_t T, int32_t H, float eps, float* out, hipStream_t stream) {
  if (!x || !out) return RVQ_ERR_NULL;
  if (T < 1 || H < 1 || H > kMaxDim || !(eps >= 0.f)) return RVQ_ERR_SHAPE;
  if (!aligned(x, 4) || !aligned(out, 4)) return RVQ_ERR_ALIGN;
  return hip_status(launch_rmsnorm(x, T, H, eps, out, stream));
}

int rvq_check_device_status(void* workspace, hipStream_t stream) {
  if (!workspace) return RVQ_ERR_NULL;
  if (!aligned(workspace, 256)) return RVQ_ERR_ALIGN;
  if (hipStreamSynchronize(stream) != hipSuccess) return RVQ_ERR_HIP;
  int32_t st = 0;
  if (hipMemcpy(&st, workspace, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return RVQ_ERR_HIP;
  const int32_t zero = 0;
  if (hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return RVQ_ERR_HIP;
  return st;
}

}  // extern "C"

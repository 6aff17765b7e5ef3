// Internal host-side launch interface between abi.cpp (validation) and kernels.hip (kernels).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rvq {

constexpr int kMaxExperts = 4096;
constexpr int kMaxTopK = 64;

struct MoeWorkspace {
  int nt_in, nt_out;              // K-tiles of gate/up (over H) and of down (over I)
  size_t status_off;              // int32 sticky device status
  size_t part_gu_off;             // fp32 [k][2][nt_in][I]
  size_t part_d_off;              // fp32 [k][nt_out][H]
  size_t norm_off;                // fp32 [H]: RMSNorm(h) for the pre-norm block
  size_t total;
};

MoeWorkspace moe_workspace_layout(int H, int I, int k, bool f16);
int gemv_tiles(int cols, bool f16);
size_t gemv_workspace_bytes(int rows, int cols, bool f16);

hipError_t launch_pack(const uint8_t* src, int rows, int cols, uint8_t* dst, hipStream_t stream);
hipError_t launch_zero(void* p, size_t nbytes, hipStream_t stream);
hipError_t launch_stream_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t nbytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_lut_build(const float* x, int cols, const float* cb, bool f16, void* lut, int32_t* log2_scale,
                            hipStream_t stream);
hipError_t launch_gemv(const uint8_t* codes, const float* cb, int rows, int cols, const float* x, bool f16, float* y,
                       void* ws, hipStream_t stream);
hipError_t launch_router_topk(const uint16_t* w, const void* x, bool x_bf16, int T, int E, int H, int k, int32_t* ids,
                              float* gates, double* logits, hipStream_t stream);
hipError_t launch_rmsnorm(const float* x, int T, int H, float eps, float* out, hipStream_t stream);
// Word of the decode workspace header (int32 index) holding the polls per bounded wait of the
// wave-specialised kernels: 0 = the default, else polls + 1.  Word 0 is the sticky status.
constexpr int kWaitLimitWord = 1;
hipError_t launch_set_word(int32_t* p, int32_t v, hipStream_t stream);
// T tokens of decode through the table path (x, residual, y: [T][H]; ids, gates: [T][k]); the
// workspace holds moe_workspace_layout(H, I, T * k, f16).
hipError_t launch_moe_batch_decode(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                                   const float* x, int T, const int32_t* ids, const float* gates, int k,
                                   const float* residual, float* y, bool f16, void* ws, hipStream_t stream);
constexpr int kMaxBatchDecode = 256;
constexpr int kMaxFitIters = 10000;   // Lloyd iterations per stage accepted by rvq_fit
// Residual RVQ encoding of W fp32 [rows][cols] against codebooks [3][256][8] into canonical codes
// [rows][cols/8][3] (encode.hip).
// Residual k-means fit of a matrix's stage codebooks (starts: host int32 [3][256], each < rows*cols/8).
size_t fit_workspace_bytes(int64_t N);
hipError_t launch_rvq_fit(const float* W, int64_t rows, int64_t cols, int iters, const int32_t* starts, float* cb,
                          uint8_t* codes, void* ws, hipStream_t stream);
hipError_t launch_rvq_encode(const float* W, int64_t rows, int64_t cols, const float* cb, uint8_t* codes,
                             hipStream_t stream);
// CRC-32 of each expert record's code payload (verify.hip); the workspace holds one word per
// 64 KiB block of every record.
int64_t crc_payload_bytes(int H, int I);
size_t crc_workspace_bytes(int E, int H, int I);
hipError_t launch_bank_crc32(const uint8_t* codes, int64_t stride, int E, int H, int I, uint32_t* crc, void* ws,
                             hipStream_t stream);
// CRC-32 of one record's codes compared on the device with `expect`; a mismatch stores RVQ_ERR_RECORD
// and `tag` into status[0..1].  ws: crc_workspace_bytes(1, H, I) bytes.
hipError_t launch_record_crc_check(const uint8_t* codes, int H, int I, uint32_t expect, int32_t tag, int32_t* status,
                                   void* ws, hipStream_t stream);
hipError_t launch_router_norm_logits(const uint16_t* w, const float* h, int E, int H, float eps, double* logits,
                                     float* n, hipStream_t stream);
hipError_t launch_router_logits(const uint16_t* w, const void* x, bool x_bf16, int T, int E, int H, double* logits,
                                hipStream_t stream);
// Routing inputs of a decode step: the router logits (fp64 [E]) and where the top-k ids/gates go.
struct Route {
  const double* logits;
  int32_t* ids;
  float* gates;
};
// route == nullptr: ids/gates are inputs.  Otherwise ids/gates are ignored and the top-k of
// route->logits is taken first (inside the gate/up kernel when it can), written to route->ids/gates.
// status_hdr: the status and wait-limit words, when they are not the workspace's header (the
// static-scratch variant keeps them in caller memory).
hipError_t launch_moe_decode(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                             const float* x, const int32_t* ids, const float* gates, int k, const float* residual,
                             float* y, bool f16, void* ws, hipStream_t stream, hipEvent_t* ev,
                             const Route* route = nullptr, int32_t* status_hdr = nullptr);

// Routed decode through the library's static per-device scratch array (scratch.hip): no workspace
// argument, nothing allocated.  kScratchBytes bounds the layout moe_workspace_layout(H, I, k, f16).
constexpr size_t kScratchBytes = (size_t)24 << 20;
hipError_t launch_moe_decode_routed_scratch(const uint8_t* codes, const float* cb, int64_t stride, int E, int H,
                                            int I, const uint16_t* w_router, const float* x, int k,
                                            const float* residual, float* y, int32_t* ids, float* gates,
                                            double* logits, bool f16, int32_t* status, hipStream_t stream);

size_t chunk_workspace_bytes(int E, int H, int I, int T, int k);
hipError_t launch_moe_chunk(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                            const uint16_t* x, int T, const int32_t* ids, const float* gates, int k,
                            const float* residual, float* y, bool f16, void* ws, hipStream_t stream);

}  // namespace rvq

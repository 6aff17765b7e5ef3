// The routed decode step for callers that cannot allocate device memory (code under HIP graph capture
// that may not call hipMalloc, tight serving loops, harnesses that forbid allocation): the same kernels
// as rvq_moe_decode_routed, with the gate/up and down partial sums in a static per-device array
// instead of a caller's workspace.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on holds its own copy, of
// kScratchBytes, from the module's load until the process ends.  In host code the array's name is
// only a host-side stand-in, so its device address is taken once per device (with that device
// current) by hipGetSymbolAddress and kept; every launch uses that address, never the name.  All
// calls on one GPU share its array and it keeps the last call's contents: the partial sums are
// completely written before they are read within a call, so nothing in it needs clearing, and two
// calls that overlap on one GPU (on different streams) race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace rvq {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
static void* g_scratch_ptr[kMaxScratchDevices];
static std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, taken on the first call there.
static hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_moe_decode_routed_scratch(const uint8_t* codes, const float* cb, int64_t stride, int E, int H,
                                            int I, const uint16_t* w_router, const float* x, int k,
                                            const float* residual, float* y, int32_t* ids, float* gates,
                                            double* logits, bool f16, int32_t* status, hipStream_t stream) {
  void* ws = nullptr;
  hipError_t err = scratch_address(&ws);
  if (err != hipSuccess) return err;
  err = launch_router_logits(w_router, x, false, 1, E, H, logits, stream);
  if (err != hipSuccess) return err;
  const Route route{logits, ids, gates};
  return launch_moe_decode(codes, cb, stride, E, H, I, x, nullptr, nullptr, k, residual, y, f16, ws, stream, nullptr,
                           &route, status);
}

}  // namespace rvq

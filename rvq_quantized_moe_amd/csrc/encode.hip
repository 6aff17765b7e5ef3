// RVQ encoding: the codes of a weight matrix against given stage codebooks, computed on the GPU.
//
// A weight sub-vector (8 consecutive columns of one row) is stored as three stage entries whose sum
// reconstructs it ("Running a 2.78-Trillion-Parameter Model on a Laptop", Technical Insight: 3
// stages x 256 entries x 8 dims, 3.00 bits per weight); the pages convert checkpoints to this form
// offline (news.hada.io topic 32035, conversion section) without spelling out the search.  The
// plainest encoder consistent with the residual form is taken here: stage by stage, the entry
// nearest (squared Euclidean distance) to what the earlier stages left, which is then subtracted.
//
// One thread per sub-vector, the 3 x 256 x 8 codebook in LDS (every lane of a wave reads the same
// entry, a broadcast).  The decisions are taken in fp32 in a fixed order with no fused
// multiply-add (contraction is switched off in the kernel), ties to the lower index, so the codes
// are reproducible bit for bit by any implementation of the same arithmetic.  Plain ALU work:
// 3 x 256 x 8 x (sub, mul, add) per sub-vector.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "launch.hpp"

namespace rvq {

__global__ __launch_bounds__(256) void k_rvq_encode(const float* __restrict__ W, int64_t rows, int64_t cols,
                                                    const float* __restrict__ cb, uint8_t* __restrict__ codes) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) float C[3 * 256 * 8];
  for (int i = threadIdx.x; i < 3 * 256 * 8 / 4; i += 256)
    reinterpret_cast<f32x4*>(C)[i] = reinterpret_cast<const f32x4*>(cb)[i];
  __syncthreads();
  const int64_t G = cols / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * G) return;
  const int64_t r = idx / G, g = idx % G;
  const f32x4* src = reinterpret_cast<const f32x4*>(W + r * cols + 8 * g);
  const f32x4 lo = src[0], hi = src[1];
  float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t packed = 0;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const float* Cs = C + s * 256 * 8;
    int best = 0;
    float best_d = 0.f;
    for (int c = 0; c < 256; ++c) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(Cs + c * 8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Cs + c * 8 + 4);
      const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = v[j] - e[j];
        const float t2 = t * t;
        d = d + t2;
      }
      if (c == 0 || d < best_d) {
        best_d = d;
        best = c;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] - Cs[best * 8 + j];
    packed |= (uint32_t)best << (8 * s);
  }
  uint8_t* out = codes + idx * 3;
  out[0] = (uint8_t)packed;
  out[1] = (uint8_t)(packed >> 8);
  out[2] = (uint8_t)(packed >> 16);
}

hipError_t launch_rvq_encode(const float* W, int64_t rows, int64_t cols, const float* cb, uint8_t* codes,
                             hipStream_t stream) {
  const int64_t n = rows * (cols / 8);
  hipLaunchKernelGGL(k_rvq_encode, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, W, rows, cols, cb, codes);
  return hipGetLastError();
}

}  // namespace rvq

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
//
// Codebook fitting (rvq_fit).  The pages' codebooks come from their converter (K3's experts were
// trained for the format), which the pages name without its method; the plainest fit of the residual
// form is taken: residual k-means, stage by stage.  256 centroids start at given sub-vectors of what
// the earlier stages left; each Lloyd iteration assigns every sub-vector to its nearest centroid (the
// encoder's decision) and moves each centroid with members to their mean (one without members keeps
// its value); a last assignment gives the stage's codes, and the chosen centroids are subtracted.
// The mean's rounding depends on the order of its sum, so the order is fixed: fp64 sums over the
// members inside each run of kFitRun consecutive sub-vectors in ascending index, then over the runs
// in ascending order, divided by the count and rounded to fp32 once.  Kernels per iteration:
//  * k_fit_assign: one thread per sub-vector, the stage's 256 x 8 centroids in LDS (as the encoder);
//  * k_fit_partial: one workgroup per run, one thread per centroid walking the run's codes in order
//    and adding its members' residuals (staged through LDS, 1024 sub-vectors at a time) in fp64;
//  * k_fit_reduce: one thread per centroid dimension adding the run sums in run order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "launch.hpp"

namespace rvq {

// Index of the entry of C (256 x 8 fp32, in LDS) nearest to v: squared distance accumulated over the 8
// dims in order, in fp32 with no fused operations; ties to the lower index.
__device__ inline int nearest_entry(const float (&v)[8], const float* C) {
#pragma clang fp contract(off)
  int best = 0;
  float best_d = 0.f;
  for (int c = 0; c < 256; ++c) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(C + c * 8);
    const f32x4 b = *reinterpret_cast<const f32x4*>(C + c * 8 + 4);
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
  return best;
}

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
    const int best = nearest_entry(v, Cs);
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

// ------------------------------------------------------------------ codebook fitting
constexpr int kFitRun = 2048;     // sub-vectors per run of the mean's first summation level
constexpr int kFitChunk = 1024;   // sub-vectors staged in LDS at a time

struct FitStarts {
  int32_t idx[256];
};

// C[c] = R[idx[c]]: one stage's starting centroids.
__global__ __launch_bounds__(256) void k_fit_init(const float* __restrict__ R, FitStarts st, float* __restrict__ C) {
  const int c = threadIdx.x;
  const f32x4* src = reinterpret_cast<const f32x4*>(R + (int64_t)st.idx[c] * 8);
  f32x4* dst = reinterpret_cast<f32x4*>(C + c * 8);
  dst[0] = src[0];
  dst[1] = src[1];
}

// Nearest centroid of every residual sub-vector: into cur (Lloyd iterations), or, on the stage's last
// pass (codes != null), into the stage's code byte, with the centroid subtracted from the residual.
__global__ __launch_bounds__(256) void k_fit_assign(float* __restrict__ R, int64_t N, const float* __restrict__ cb,
                                                    uint8_t* __restrict__ cur, uint8_t* __restrict__ codes,
                                                    int stage) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) float C[256 * 8];
  for (int i = threadIdx.x; i < 256 * 8 / 4; i += 256)
    reinterpret_cast<f32x4*>(C)[i] = reinterpret_cast<const f32x4*>(cb)[i];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  f32x4* p = reinterpret_cast<f32x4*>(R + i * 8);
  const f32x4 lo = p[0], hi = p[1];
  const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  const int best = nearest_entry(v, C);
  if (!codes) {
    cur[i] = (uint8_t)best;
    return;
  }
  codes[i * 3 + stage] = (uint8_t)best;
  const float* e = C + best * 8;
  p[0] = f32x4{v[0] - e[0], v[1] - e[1], v[2] - e[2], v[3] - e[3]};
  p[1] = f32x4{v[4] - e[4], v[5] - e[5], v[6] - e[6], v[7] - e[7]};
}

// Run b's per-centroid sums: thread c adds, in ascending index, the residuals of the run's sub-vectors
// assigned to c.  Each 1024-sub-vector chunk of the run is staged in LDS and its indices are sorted by
// code, stably, so that thread c then walks exactly its own members in index order:
//  * count per code (LDS integer atomics: exact in any order) and an exclusive scan: off[c];
//  * four sub-chunks of 256 in index order; in each, wave w (64 consecutive sub-vectors) finds for
//    every lane the lanes below it with the same code (8 ballots, one per code bit) and writes its
//    per-code counts, and a sub-vector's slot is off[c] + (earlier sub-chunks' count of c) +
//    (earlier waves' count of c) + (same-code lanes below it);
//  * thread c adds its members' residuals (8 fp64 sums) from off[c] on.
// part[(c * 8 + d) * nruns + b] (fp64), cnt[c * nruns + b].
__global__ __launch_bounds__(256) void k_fit_partial(const float* __restrict__ R, int64_t N,
                                                     const uint8_t* __restrict__ cur, int nruns,
                                                     double* __restrict__ part, int32_t* __restrict__ cnt) {
  __shared__ __attribute__((aligned(16))) float Rb[kFitChunk * 8];
  __shared__ uint16_t order[kFitChunk];   // chunk-local indices, grouped by code, ascending within a code
  __shared__ int count[256], off[256], base[256];
  __shared__ int whist[4][256];
  const int c = threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int n = 0;
  const int64_t run0 = (int64_t)blockIdx.x * kFitRun;
  for (int h = 0; h < kFitRun; h += kFitChunk) {
    const int64_t left = N - (run0 + h);
    if (left <= 0) break;   // uniform across the workgroup
    const int nvalid = left < kFitChunk ? (int)left : kFitChunk;
    __syncthreads();   // the previous chunk has been read
    count[c] = 0;
    base[c] = 0;
    // stage: 4 sub-vectors per thread, loads first (indices clamped to the last one; entries past
    // nvalid are staged but take no slot)
    constexpr int kPer = kFitChunk / 256;
    int code[kPer];
    {
      f32x4 lo[kPer], hi[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        int64_t i = run0 + h + u * 256 + threadIdx.x;
        i = i < N ? i : N - 1;
        code[u] = cur[i];
        const f32x4* src = reinterpret_cast<const f32x4*>(R + i * 8);
        lo[u] = src[0];
        hi[u] = src[1];
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int q = u * 256 + threadIdx.x;
        reinterpret_cast<f32x4*>(Rb)[2 * q] = lo[u];
        reinterpret_cast<f32x4*>(Rb)[2 * q + 1] = hi[u];
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (u * 256 + threadIdx.x < nvalid) atomicAdd(&count[code[u]], 1);
    __syncthreads();
    if (wave == 0) {   // exclusive scan of the 256 counts: lane l holds codes 4l .. 4l+3
      const int c0 = count[4 * lane], c1 = count[4 * lane + 1], c2 = count[4 * lane + 2], c3 = count[4 * lane + 3];
      int incl = c0 + c1 + c2 + c3;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      const int ex = incl - (c0 + c1 + c2 + c3);
      off[4 * lane] = ex;
      off[4 * lane + 1] = ex + c0;
      off[4 * lane + 2] = ex + c0 + c1;
      off[4 * lane + 3] = ex + c0 + c1 + c2;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int q = u * 256 + threadIdx.x;
      const bool valid = q < nvalid;
      const int v = valid ? code[u] : 256;   // past the end: a code no lane shares with a valid one
      uint64_t peers = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) {
        const uint64_t m = __ballot((v >> bit) & 1);
        peers &= ((v >> bit) & 1) ? m : ~m;
      }
      const int below = __popcll(peers & ((1ull << lane) - 1ull));
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) whist[w2][c] = 0;
      __syncthreads();
      if (valid && below == 0) whist[wave][v] = __popcll(peers);
      __syncthreads();
      if (valid) {
        int slot = off[v] + base[v] + below;
        for (int w2 = 0; w2 < wave; ++w2) slot += whist[w2][v];
        order[slot] = (uint16_t)q;
      }
      __syncthreads();
      base[c] += whist[0][c] + whist[1][c] + whist[2][c] + whist[3][c];
      __syncthreads();
    }
    // thread c: its members in index order
    const int m0 = off[c], m1 = off[c] + count[c];
    n += m1 - m0;
    for (int i = m0; i < m1; ++i) {
      const int j = order[i];
      const f32x4 lo = reinterpret_cast<const f32x4*>(Rb)[2 * j];
      const f32x4 hi = reinterpret_cast<const f32x4*>(Rb)[2 * j + 1];
      s[0] += (double)lo.x;
      s[1] += (double)lo.y;
      s[2] += (double)lo.z;
      s[3] += (double)lo.w;
      s[4] += (double)hi.x;
      s[5] += (double)hi.y;
      s[6] += (double)hi.z;
      s[7] += (double)hi.w;
    }
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) part[(int64_t)(c * 8 + d) * nruns + blockIdx.x] = s[d];
  cnt[(int64_t)c * nruns + blockIdx.x] = n;
}

// Thread (c, d): the run sums in run order, then the mean (a centroid without members keeps its value).
// 2048 threads in workgroups of one wave, so that the serial sums spread over 32 CUs, each with many
// loads in flight.
__global__ __launch_bounds__(64) void k_fit_reduce(const double* __restrict__ part, const int32_t* __restrict__ cnt,
                                                   int nruns, float* __restrict__ C) {
  const int t = blockIdx.x * 64 + threadIdx.x;   // 2048 threads
  const int c = t >> 3;
  const double* p = part + (int64_t)t * nruns;
  const int32_t* q = cnt + (int64_t)c * nruns;
  constexpr int kAhead = 32;
  double s = 0.0;
  int64_t n = 0;
  int b = 0;
  for (; b + kAhead <= nruns; b += kAhead) {   // loads issued ahead, sums kept in order
    double v[kAhead];
    int32_t m[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      v[u] = p[b + u];
      m[u] = q[b + u];
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      s += v[u];
      n += m[u];
    }
  }
  for (; b < nruns; ++b) {
    s += p[b];
    n += q[b];
  }
  if (n > 0) C[t] = (float)(s / (double)n);
}

int64_t fit_runs(int64_t N) { return cdiv(N, kFitRun); }

size_t fit_workspace_bytes(int64_t N) {
  const int64_t nr = fit_runs(N);
  const auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  return (size_t)(up(N * 32) + up(N) + up(nr * 2048 * 8) + up(nr * 256 * 4));
}

hipError_t launch_rvq_fit(const float* W, int64_t rows, int64_t cols, int iters, const int32_t* starts, float* cb,
                          uint8_t* codes, void* ws, hipStream_t stream) {
  const int64_t N = rows * (cols / 8);
  const int nr = (int)fit_runs(N);
  const auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* R = reinterpret_cast<float*>(w);
  uint8_t* cur = w + up(N * 32);
  double* part = reinterpret_cast<double*>(cur + up(N));
  int32_t* cnt = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(part) + up((int64_t)nr * 2048 * 8));
  hipError_t err = hipMemcpyAsync(R, W, (size_t)N * 32, hipMemcpyDeviceToDevice, stream);
  if (err != hipSuccess) return err;
  const unsigned g = (unsigned)cdiv(N, 256);
  for (int s = 0; s < 3; ++s) {
    float* C = cb + s * 256 * 8;
    FitStarts st;
    for (int c = 0; c < 256; ++c) st.idx[c] = starts[s * 256 + c];
    hipLaunchKernelGGL(k_fit_init, dim3(1), dim3(256), 0, stream, R, st, C);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(k_fit_assign, dim3(g), dim3(256), 0, stream, R, N, C, cur, nullptr, s);
      hipLaunchKernelGGL(k_fit_partial, dim3((unsigned)nr), dim3(256), 0, stream, R, N, cur, nr, part, cnt);
      hipLaunchKernelGGL(k_fit_reduce, dim3(32), dim3(64), 0, stream, part, cnt, nr, C);
    }
    hipLaunchKernelGGL(k_fit_assign, dim3(g), dim3(256), 0, stream, R, N, C, cur, codes, s);
  }
  return hipGetLastError();
}

}  // namespace rvq

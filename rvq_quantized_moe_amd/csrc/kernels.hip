// HIP kernels (gfx950) of the RVQ-LUT MoE expert path and their host-side launchers.
// Argument checking happens in abi.cpp before any launcher is called; launchers assume valid input.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device.hpp"
#include "launch.hpp"

namespace rvq {

// =============================================================================================
// Packing: canonical [rows][cols/8][3] -> slab layout (see rvq.h).  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void k_pack(const uint8_t* __restrict__ src, int rows, int cols,
                                              uint8_t* __restrict__ dst, int64_t nchunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nchunks) return;
  const int lane = (int)(i % 64);
  const int j = (int)((i / 64) % 3);
  const int64_t slab = i / 192;
  const int64_t nrb = cdiv(rows, kSlabRows);
  const int64_t t = slab / nrb, rb = slab % nrb;
  const int64_t row = rb * kSlabRows + lane;
  const int64_t rowbytes = 3 * (int64_t)(cols / 8);
  const int64_t b0 = t * 48 + j * 16;
  uint32_t w[4] = {0, 0, 0, 0};
  if (row < rows) {
    const uint8_t* s = src + row * rowbytes;
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int64_t bb = b0 + ii;
      const uint32_t v = bb < rowbytes ? s[bb] : 0u;
      w[ii >> 2] |= v << (8 * (ii & 3));
    }
  }
  u32x4 out = {w[0], w[1], w[2], w[3]};
  *reinterpret_cast<u32x4*>(dst + i * 16) = out;
}

hipError_t launch_pack(const uint8_t* src, int rows, int cols, uint8_t* dst, hipStream_t stream) {
  const int64_t nchunks = packed_bytes(rows, cols) / 16;
  const int64_t grid = cdiv(nchunks, 256);
  hipLaunchKernelGGL(k_pack, dim3((unsigned)grid), dim3(256), 0, stream, src, rows, cols, dst, nchunks);
  return hipGetLastError();
}

// =============================================================================================
// Zero fill (used instead of hipMemsetAsync so that callers may graph-capture it).
__global__ __launch_bounds__(256) void k_zero(uint8_t* __restrict__ p, int64_t nbytes) {
  const int64_t n16 = nbytes / 16;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<u32x4*>(p)[i] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && (int64_t)threadIdx.x < nbytes - n16 * 16) p[n16 * 16 + threadIdx.x] = 0;
}

hipError_t launch_zero(void* p, size_t nbytes, hipStream_t stream) {
  int64_t grid = cdiv((int64_t)(nbytes / 16) + 1, 256);
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)grid), dim3(256), 0, stream, static_cast<uint8_t*>(p), (int64_t)nbytes);
  return hipGetLastError();
}

// =============================================================================================
// Standalone partial-dot tables lut[g][s][c] for all groups of x (global memory output).
// Block b builds groups [b*G, b*G+G) with G = Tile<F16>::kGroups.  fp16: one exponent for the
// whole table, from max_c ||C_s[c]|| * max_g ||x_g|| (each block recomputes the x maximum).
template <bool F16>
__global__ __launch_bounds__(256) void k_lut_build(const float* __restrict__ x, int cols,
                                                   const float* __restrict__ cb,
                                                   typename Tile<F16>::entry_t* __restrict__ lut,
                                                   int32_t* __restrict__ log2_scale) {
  constexpr int G = Tile<F16>::kGroups;
  __shared__ float vs[G * 8];
  __shared__ float red[4];
  const int groups = cols / 8;
  const int g0 = blockIdx.x * G;
  const int i = threadIdx.x;
  if (i < G * 8) vs[i] = (g0 * 8 + i < cols) ? x[g0 * 8 + i] : 0.f;
  float cv[3][8];
  load_codebook_entry<F16>(cb, cv);
  float scale = 1.f;
  int e = 0;
  if constexpr (F16) {
    float xm = 0.f;
    for (int g = i; g < groups; g += 256) {
      float n = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) n = fmaf(x[g * 8 + j], x[g * 8 + j], n);
      xm = fmaxf(xm, n);
    }
    const float xmax2 = block_max(xm, red);
    const float cmax2 = block_max(codebook_norm2(cv), red);
    e = f16_table_exponent(sqrtf(cmax2) * sqrtf(xmax2));
    scale = ldexpf(1.f, -e);
  }
  __syncthreads();
  // Build into registers-then-global: entries of groups past the end are not written.
  const int c = threadIdx.x;
  for (int g = 0; g < G && g0 + g < groups; ++g) {
    float xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = vs[g * 8 + j];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      float t = cv[s][0] * xv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) t = fmaf(cv[s][j], xv[j], t);
      const int64_t idx = ((int64_t)(g0 + g) * 3 + s) * kEntries + c;
      if constexpr (F16) lut[idx] = (f16)(t * scale);
      else lut[idx] = t;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && log2_scale) *log2_scale = e;
}

hipError_t launch_lut_build(const float* x, int cols, const float* cb, bool half_tables, void* lut, int32_t* log2_scale,
                            hipStream_t stream) {
  const int groups = cols / 8;
  if (half_tables) {
    hipLaunchKernelGGL(k_lut_build<true>, dim3((unsigned)cdiv(groups, Tile<true>::kGroups)), dim3(256), 0, stream, x,
                       cols, cb, static_cast<f16*>(lut), log2_scale);
  } else {
    hipLaunchKernelGGL(k_lut_build<false>, dim3((unsigned)cdiv(groups, Tile<false>::kGroups)), dim3(256), 0, stream,
                       x, cols, cb, static_cast<float*>(lut), log2_scale);
  }
  return hipGetLastError();
}

// =============================================================================================
// Shared prologue of every table-path workgroup: stage the tile's activation values `vs` (already
// in LDS), choose the fp16 exponent, build the tables.  Returns the output scale 2^e.
template <bool F16>
__device__ __forceinline__ float tile_tables(typename Tile<F16>::entry_t* lut, const float* __restrict__ cb,
                                             const float* vs, float my_v, float* red) {
  float cv[3][8];
  load_codebook_entry<F16>(cb, cv);
  float scale = 1.f, out_scale = 1.f;
  if constexpr (F16) {
    // my_v = this thread's element of the tile vector (threads 0..255 cover the 32 groups)
    const float xmax2 = block_max(group_norm2(my_v), red);
    const float cmax2 = block_max(codebook_norm2(cv), red);
    const int e = f16_table_exponent(sqrtf(cmax2) * sqrtf(xmax2));
    scale = ldexpf(1.f, -e);
    out_scale = ldexpf(1.f, e);
  }
  build_tile<F16>(lut, cv, vs, scale);
  __syncthreads();
  return out_scale;
}

// =============================================================================================
// Single-matrix GEMV.  Grid: (tiles, parts).  part[t][row] = tile t's contribution.
template <bool F16>
__global__ __launch_bounds__(256) void k_gemv_tiles(const uint8_t* __restrict__ codes, const float* __restrict__ cb,
                                                    int rows, int cols, const float* __restrict__ x,
                                                    float* __restrict__ part, int nparts) {
  constexpr int G = Tile<F16>::kGroups;
  __shared__ __attribute__((aligned(16))) typename Tile<F16>::entry_t lut[kLutBytes / sizeof(typename Tile<F16>::entry_t)];
  __shared__ float vs[256];
  __shared__ float red[4];
  const int tile = blockIdx.x, p = blockIdx.y;
  const int groups = cols / 8;
  const int nt16 = (int)cdiv(groups, kSlabGroups);
  const int nrb = (int)cdiv(rows, kSlabRows);
  const int i = threadIdx.x;
  const int k0 = tile * G * 8;
  const float v = (i < G * 8 && k0 + i < cols) ? x[k0 + i] : 0.f;
  if (i < G * 8) vs[i] = v;
  __syncthreads();
  const float out_scale = tile_tables<F16>(lut, cb, vs, v, red);
  const int per = (int)cdiv(nrb, nparts);
  const int rb0 = p * per;
  const int rb1 = rb0 + per < nrb ? rb0 + per : nrb;
  stream_tile<F16>(lut, codes, nrb, nt16, tile, rb0, rb1, rows, out_scale, part + (int64_t)tile * rows);
}

__global__ __launch_bounds__(256) void k_sum_tiles(const float* __restrict__ part, int ntiles, int rows,
                                                   float* __restrict__ y) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.f;
  for (int t = 0; t < ntiles; ++t) acc += part[(int64_t)t * rows + r];
  y[r] = acc;
}

int gemv_tiles(int cols, bool f16) {
  return (int)cdiv(cols / 8, f16 ? Tile<true>::kGroups : Tile<false>::kGroups);
}

size_t gemv_workspace_bytes(int rows, int cols, bool f16) {
  return (size_t)gemv_tiles(cols, f16) * (size_t)rows * sizeof(float);
}

hipError_t launch_gemv(const uint8_t* codes, const float* cb, int rows, int cols, const float* x, bool f16,
                       float* y, void* ws, hipStream_t stream) {
  const int nt = gemv_tiles(cols, f16);
  const int nrb = (int)cdiv(rows, kSlabRows);
  // enough workgroups to cover the chip: split rows when there are few tiles
  int nparts = 1;
  while (nt * nparts < 512 && (nparts * 2) * 4 <= nrb) nparts *= 2;
  float* part = static_cast<float*>(ws);
  if (f16)
    hipLaunchKernelGGL(k_gemv_tiles<true>, dim3(nt, nparts), dim3(256), 0, stream, codes, cb, rows, cols, x, part,
                       nparts);
  else
    hipLaunchKernelGGL(k_gemv_tiles<false>, dim3(nt, nparts), dim3(256), 0, stream, codes, cb, rows, cols, x, part,
                       nparts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_sum_tiles, dim3((unsigned)cdiv(rows, 256)), dim3(256), 0, stream, part, nt, rows, y);
  return hipGetLastError();
}

// =============================================================================================
// Router logits in fp64 (bf16 x fp32 and bf16 x bf16 products are exact in fp64).
// One wave per (expert, token); 16-byte weight loads when rows are 16-byte aligned.
__device__ inline double bf16_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }
__device__ inline double x_to_f64(float v) { return (double)v; }
__device__ inline double x_to_f64(uint16_t v) { return bf16_to_f64(v); }

template <typename XT>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ w, const XT* __restrict__ x, int T,
                                                       int E, int H, double* __restrict__ logits, int vec) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = blockIdx.y;
  if (e >= E) return;
  const uint16_t* wr = w + (int64_t)e * H;
  const XT* xr = x + (int64_t)t * H;
  double acc = 0.0;
  int h0 = 0;
  if (vec) {
    const int n8 = H / 8;
    for (int q = lane; q < n8; q += 64) {
      const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + q * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fma(bf16_to_f64((uint16_t)(wv[j] & 0xffffu)), x_to_f64(xr[q * 8 + 2 * j]), acc);
        acc = fma(bf16_to_f64((uint16_t)(wv[j] >> 16)), x_to_f64(xr[q * 8 + 2 * j + 1]), acc);
      }
    }
    h0 = n8 * 8;
  }
  for (int h = h0 + lane; h < H; h += 64) acc = fma(bf16_to_f64(wr[h]), x_to_f64(xr[h]), acc);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) logits[(int64_t)t * E + e] = acc;
}

// Top-k by (logit desc, id asc): the rank of e is the number of experts that precede it in that
// order; ranks < k are kept, at position rank.  gates = softmax over the kept logits (fp64).
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ gates) {
  __shared__ double L[kMaxExperts];
  __shared__ int sel[kMaxTopK];
  const int t = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) L[e] = logits[(int64_t)t * E + e];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const double le = L[e];
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const double lj = L[j];
      rank += (lj > le) || (lj == le && j < e);
    }
    if (rank < k) sel[rank] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double m = L[sel[0]];
    double z = 0.0;
    for (int i = 0; i < k; ++i) z += exp(L[sel[i]] - m);
    for (int i = 0; i < k; ++i) {
      ids[(int64_t)t * k + i] = sel[i];
      gates[(int64_t)t * k + i] = (float)(exp(L[sel[i]] - m) / z);
    }
  }
}

hipError_t launch_router_topk(const uint16_t* w, const void* x, bool x_bf16, int T, int E, int H, int k, int32_t* ids,
                              float* gates, double* logits, hipStream_t stream) {
  const int vec = (H % 8 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0);
  dim3 grid((unsigned)cdiv(E, 4), (unsigned)T);
  if (x_bf16)
    hipLaunchKernelGGL(k_router_logits<uint16_t>, grid, dim3(256), 0, stream, w, static_cast<const uint16_t*>(x), T,
                       E, H, logits, vec);
  else
    hipLaunchKernelGGL(k_router_logits<float>, grid, dim3(256), 0, stream, w, static_cast<const float*>(x), T, E, H,
                       logits, vec);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_topk, dim3((unsigned)T), dim3(256), 0, stream, logits, E, k, ids, gates);
  return hipGetLastError();
}

// =============================================================================================
// RMSNorm (unit weight), sum of squares accumulated in fp64, fixed reduction order.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, int H, float eps, float* out) {
  __shared__ double red[4];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * H;
  double ss = 0.0;
  for (int h = threadIdx.x; h < H; h += 256) ss = fma((double)xr[h], (double)xr[h], ss);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double tot = (red[0] + red[1]) + (red[2] + red[3]);
  const double inv = 1.0 / sqrt(tot / (double)H + (double)eps);
  float* o = out + t * H;
  for (int h = threadIdx.x; h < H; h += 256) o[h] = (float)((double)xr[h] * inv);
}

hipError_t launch_rmsnorm(const float* x, int T, int H, float eps, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)T), dim3(256), 0, stream, x, H, eps, out);
  return hipGetLastError();
}

// =============================================================================================
// MoE layer, one decode token.
//   gate/up:  grid k * 2 * nt_in   -> part_gu[slot][m][tile][row]   (rows of gate/up = I)
//   down:     grid k * nt_out * P  -> part_d[slot][tile][row]        (rows of down = H)
//             (each workgroup first rebuilds its 8*G entries of h = silu(g) * u from part_gu)
//   combine:  y[r] = residual[r] + sum_slot gate[slot] * sum_tile part_d[slot][tile][r]
struct BankArgs {
  const uint8_t* codes;
  const float* cb;
  int64_t stride;
  int E, H, I;
};

template <bool F16>
__global__ __launch_bounds__(256) void k_moe_gateup(BankArgs bank, const float* __restrict__ x,
                                                    const int32_t* __restrict__ ids, float* __restrict__ part_gu,
                                                    int32_t* __restrict__ status) {
  constexpr int G = Tile<F16>::kGroups;
  __shared__ __attribute__((aligned(16))) typename Tile<F16>::entry_t lut[kLutBytes / sizeof(typename Tile<F16>::entry_t)];
  __shared__ float vs[256];
  __shared__ float red[4];
  const int H = bank.H, I = bank.I;
  const int groups = H / 8;
  const int nt = (int)cdiv(groups, G);
  const int tile = blockIdx.x % nt;
  const int m = (blockIdx.x / nt) & 1;
  const int slot = blockIdx.x / (2 * nt);
  const int e = ids[slot];
  if (e < 0 || e >= bank.E) {
    if (tile == 0 && m == 0 && threadIdx.x == 0) atomicExch(status, 6 /* RVQ_ERR_EXPERT_ID */);
    return;
  }
  const uint8_t* codes = bank.codes + (int64_t)e * bank.stride + (int64_t)m * packed_bytes(I, H);
  const float* cb = bank.cb + ((int64_t)e * 3 + m) * kCodebookFloats;
  const int i = threadIdx.x;
  const int k0 = tile * G * 8;
  const float v = (i < G * 8 && k0 + i < H) ? x[k0 + i] : 0.f;
  if (i < G * 8) vs[i] = v;
  __syncthreads();
  const float out_scale = tile_tables<F16>(lut, cb, vs, v, red);
  const int nrb = (int)cdiv(I, kSlabRows);
  const int nt16 = (int)cdiv(groups, kSlabGroups);
  stream_tile<F16>(lut, codes, nrb, nt16, tile, 0, nrb, I, out_scale,
                   part_gu + (((int64_t)slot * 2 + m) * nt + tile) * I);
}

template <bool F16>
__global__ __launch_bounds__(256) void k_moe_down(BankArgs bank, const int32_t* __restrict__ ids,
                                                  const float* __restrict__ part_gu, float* __restrict__ part_d,
                                                  int nparts) {
  constexpr int G = Tile<F16>::kGroups;
  __shared__ __attribute__((aligned(16))) typename Tile<F16>::entry_t lut[kLutBytes / sizeof(typename Tile<F16>::entry_t)];
  __shared__ float vs[256];
  __shared__ float red[4];
  const int H = bank.H, I = bank.I;
  const int groups = I / 8;
  const int nt = (int)cdiv(groups, G);
  const int nt_in = (int)cdiv(H / 8, G);
  const int p = blockIdx.x % nparts;
  const int tile = (blockIdx.x / nparts) % nt;
  const int slot = blockIdx.x / (nparts * nt);
  const int e = ids[slot];
  if (e < 0 || e >= bank.E) return;  // gate/up kernel records the status
  const int i = threadIdx.x;
  const int k0 = tile * G * 8;
  float v = 0.f;
  if (i < G * 8 && k0 + i < I) {
    const float* pg = part_gu + ((int64_t)slot * 2 + 0) * nt_in * I + k0 + i;
    const float* pu = part_gu + ((int64_t)slot * 2 + 1) * nt_in * I + k0 + i;
    float gs = 0.f, us = 0.f;
    for (int t = 0; t < nt_in; ++t) {
      gs += pg[(int64_t)t * I];
      us += pu[(int64_t)t * I];
    }
    v = gs / (1.f + expf(-gs)) * us;
  }
  if (i < G * 8) vs[i] = v;
  __syncthreads();
  const uint8_t* codes = bank.codes + (int64_t)e * bank.stride + 2 * packed_bytes(I, H);
  const float* cb = bank.cb + ((int64_t)e * 3 + 2) * kCodebookFloats;
  const float out_scale = tile_tables<F16>(lut, cb, vs, v, red);
  const int nrb = (int)cdiv(H, kSlabRows);
  const int nt16 = (int)cdiv(groups, kSlabGroups);
  const int per = (int)cdiv(nrb, nparts);
  const int rb0 = p * per;
  const int rb1 = rb0 + per < nrb ? rb0 + per : nrb;
  stream_tile<F16>(lut, codes, nrb, nt16, tile, rb0, rb1, H, out_scale,
                   part_d + ((int64_t)slot * nt + tile) * H);
}

__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ part_d, int nt, int H,
                                                     const int32_t* __restrict__ ids, const float* __restrict__ gates,
                                                     int k, int E, const float* residual, float* y) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= H) return;
  float acc = residual ? residual[r] : 0.f;
  for (int slot = 0; slot < k; ++slot) {
    const int e = ids[slot];
    if (e < 0 || e >= E) continue;
    float s = 0.f;
    const float* pd = part_d + (int64_t)slot * nt * H + r;
    for (int t = 0; t < nt; ++t) s += pd[(int64_t)t * H];
    acc = fmaf(gates[slot], s, acc);
  }
  y[r] = acc;
}

static int down_parts(int H) {
  const int nrb = (int)cdiv(H, kSlabRows);
  return nrb >= 64 ? 2 : 1;
}

MoeWorkspace moe_workspace_layout(int H, int I, int k, bool f16) {
  const int G = f16 ? Tile<true>::kGroups : Tile<false>::kGroups;
  MoeWorkspace w;
  w.nt_in = (int)cdiv(H / 8, G);
  w.nt_out = (int)cdiv(I / 8, G);
  w.status_off = 0;
  w.part_gu_off = 256;
  const size_t gu = (size_t)k * 2 * w.nt_in * I * sizeof(float);
  w.part_d_off = w.part_gu_off + ((gu + 255) / 256) * 256;
  const size_t d = (size_t)k * w.nt_out * H * sizeof(float);
  w.total = w.part_d_off + ((d + 255) / 256) * 256;
  return w;
}

hipError_t launch_moe_decode(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                             const float* x, const int32_t* ids, const float* gates, int k, const float* residual,
                             float* y, bool f16, void* ws, hipStream_t stream) {
  const MoeWorkspace w = moe_workspace_layout(H, I, k, f16);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* status = reinterpret_cast<int32_t*>(base + w.status_off);
  float* part_gu = reinterpret_cast<float*>(base + w.part_gu_off);
  float* part_d = reinterpret_cast<float*>(base + w.part_d_off);
  BankArgs bank{codes, cb, stride, E, H, I};
  const int nparts = down_parts(H);
  if (f16) {
    hipLaunchKernelGGL(k_moe_gateup<true>, dim3(k * 2 * w.nt_in), dim3(256), 0, stream, bank, x, ids, part_gu, status);
    hipLaunchKernelGGL(k_moe_down<true>, dim3(k * w.nt_out * nparts), dim3(256), 0, stream, bank, ids, part_gu, part_d,
                       nparts);
  } else {
    hipLaunchKernelGGL(k_moe_gateup<false>, dim3(k * 2 * w.nt_in), dim3(256), 0, stream, bank, x, ids, part_gu,
                       status);
    hipLaunchKernelGGL(k_moe_down<false>, dim3(k * w.nt_out * nparts), dim3(256), 0, stream, bank, ids, part_gu,
                       part_d, nparts);
  }
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)cdiv(H, 256)), dim3(256), 0, stream, part_d, w.nt_out, H, ids,
                     gates, k, E, residual, y);
  return hipGetLastError();
}

}  // namespace rvq

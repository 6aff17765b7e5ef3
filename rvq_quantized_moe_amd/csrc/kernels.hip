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
// Streaming copy with the code stream's load instruction (16-byte global loads): the
// reference for the achievable read rate and for scaling memory-traffic counters.
__global__ __launch_bounds__(256) void k_stream_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  // the same non-temporal 16-byte load as the code stream, so its memory counters calibrate those
  // of the table kernels
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    dst[i] = __builtin_nontemporal_load(src + i);
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(nbytes / 16);
  int64_t grid = cdiv(n16, 256);
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)grid), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

// Read-only stream with the same loads: each thread folds its 16-byte pieces into one word, stored
// only if it equals a value no input produces in practice, so the loads cannot be dropped and the
// kernel writes (almost) nothing.  One workgroup per CU reads one contiguous part, 16 loads in flight
// per thread (64 KiB per CU): the fastest of the read patterns measured (grid-stride loops with 4-16
// loads in flight, per-workgroup parts with 256-4096 workgroups), 7.2 TB/s where a grid-stride loop
// gives 6.5.
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  constexpr int U = 16;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b = (int64_t)blockIdx.x * per, e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  int64_t i = b + threadIdx.x;
  for (; i + (U - 1) * 256 < e; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < e; i += 256) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

static int compute_units();

hipError_t launch_stream_read(const void* src, size_t nbytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = (int64_t)(nbytes / 16);
  const int ncu = compute_units();
  int64_t grid = ncu > 0 ? ncu : 256;
  if (grid > n16 / 256) grid = n16 / 256;   // at least a wave's worth per workgroup
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, stream, static_cast<const u32x4*>(src), n16,
                     sink);
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
__device__ __forceinline__ float tile_tables(typename Tile<F16>::entry_t* lut, const float (&cv)[3][8],
                                             const float* vs, float my_v, float* red) {
  float scale = 1.f, out_scale = 1.f;
  if constexpr (F16) {
    // my_v = this thread's element of the tile vector (threads 0..8G-1; zero elsewhere)
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

// Occupancy of the table kernels: with fp32 tables three 8-wave workgroups per CU (LDS allows
// three), i.e. at most 512/6 VGPRs per lane; fp16 tables keep twice the code bytes in registers per
// row block and run two workgroups per CU.
#define RVQ_OCC_F32 __attribute__((amdgpu_waves_per_eu(6, 8)))
#define RVQ_OCC_F16 __attribute__((amdgpu_waves_per_eu(4, 8)))

// =============================================================================================
// Dispatch of the row-blocks-per-wave specialisation (see RowStream).
#define RVQ_BPW_DISPATCH(bpw, ...)                 \
  switch (bpw) {                                   \
    case 1: { constexpr int B = 1; __VA_ARGS__; } break;   \
    case 2: { constexpr int B = 2; __VA_ARGS__; } break;   \
    case 4: { constexpr int B = 4; __VA_ARGS__; } break;   \
    case 7: { constexpr int B = 7; __VA_ARGS__; } break;   \
    case 8: { constexpr int B = 8; __VA_ARGS__; } break;   \
    case 14: { constexpr int B = 14; __VA_ARGS__; } break; \
    default: { constexpr int B = 0; __VA_ARGS__; } break;  \
  }

// Straight-line specialisation usable when `nparts` workgroups split nrb row blocks evenly over
// their waves; 0 (the general loop) otherwise.
static int pick_bpw(int nrb, int nparts, int waves) {
  if (nrb % nparts != 0) return 0;
  const int per = nrb / nparts;
  if (per % waves != 0) return 0;
  return fixed_bpw(per / waves) ? per / waves : 0;
}

__host__ __device__ inline int64_t pad_rows(int64_t rows) { return cdiv(rows, kSlabRows) * kSlabRows; }

// =============================================================================================
// Single-matrix GEMV.  Grid: (tiles, parts).  part[t][row] = tile t's contribution (rows padded).
template <bool F16, int BPW>
__device__ __forceinline__ void k_gemv_tiles_body(const uint8_t* __restrict__ codes, const float* __restrict__ cb,
                                                         int rows, int cols, const float* __restrict__ x,
                                                         float* __restrict__ part, int nparts) {
  constexpr int G = Tile<F16>::kGroups;
  __shared__ __attribute__((aligned(16))) typename Tile<F16>::entry_t lut[kLutBytes / sizeof(typename Tile<F16>::entry_t)];
  __shared__ float vs[256];
  __shared__ float red[kWaves];
  const int tile = blockIdx.x, p = blockIdx.y;
  const int groups = cols / 8;
  const int nt16 = (int)cdiv(groups, kSlabGroups);
  const int nrb = (int)cdiv(rows, kSlabRows);
  const int i = threadIdx.x;
  const int k0 = tile * G * 8;
  const int per = (int)cdiv(nrb, nparts);
  const int rb0 = p * per;
  const int rb1 = rb0 + per < nrb ? rb0 + per : nrb;
  // loads the tables need are issued before the code prefetch: waits on memory counters are in order
  const float v = (i < G * 8 && k0 + i < cols) ? x[k0 + i] : 0.f;
  float cv[3][8];
  load_codebook_entry<F16>(cb, cv);
  RowStream<F16, BPW> rs;
  rs.begin(codes, nrb, nt16, tile, rb0, rb1);
  if (i < G * 8) vs[i] = v;
  __syncthreads();
  const float out_scale = tile_tables<F16>(lut, cv, vs, v, red);
  rs.run(lut, out_scale, part + (int64_t)tile * pad_rows(rows));
}

template <int BPW>
__global__ __launch_bounds__(kThreads) RVQ_OCC_F32 void k_gemv_tiles_f32(const uint8_t* __restrict__ codes, const float* __restrict__ cb, int rows, int cols, const float* __restrict__ x, float* __restrict__ part, int nparts) {
  k_gemv_tiles_body<false, BPW>(codes, cb, rows, cols, x, part, nparts);
}
template <int BPW>
__global__ __launch_bounds__(kThreads) RVQ_OCC_F16 void k_gemv_tiles_f16(const uint8_t* __restrict__ codes, const float* __restrict__ cb, int rows, int cols, const float* __restrict__ x, float* __restrict__ part, int nparts) {
  k_gemv_tiles_body<true, BPW>(codes, cb, rows, cols, x, part, nparts);
}

__global__ __launch_bounds__(256) void k_sum_tiles(const float* __restrict__ part, int ntiles, int rows,
                                                   int64_t stride, float* __restrict__ y) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.f;
  for (int t = 0; t < ntiles; ++t) acc += part[(int64_t)t * stride + r];
  y[r] = acc;
}

int gemv_tiles(int cols, bool f16) {
  return (int)cdiv(cols / 8, f16 ? Tile<true>::kGroups : Tile<false>::kGroups);
}

size_t gemv_workspace_bytes(int rows, int cols, bool f16) {
  return (size_t)gemv_tiles(cols, f16) * (size_t)pad_rows(rows) * sizeof(float);
}

hipError_t launch_gemv(const uint8_t* codes, const float* cb, int rows, int cols, const float* x, bool f16,
                       float* y, void* ws, hipStream_t stream) {
  const int nt = gemv_tiles(cols, f16);
  const int nrb = (int)cdiv(rows, kSlabRows);
  // enough workgroups to cover the chip: split rows when there are few tiles
  int nparts = 1;
  while (nt * nparts < 512 && (nparts * 2) * kWaves <= nrb) nparts *= 2;
  float* part = static_cast<float*>(ws);
  const int bpw = pick_bpw(nrb, nparts, kWaves);
  if (f16) {
    RVQ_BPW_DISPATCH(bpw, hipLaunchKernelGGL((k_gemv_tiles_f16<B>), dim3(nt, nparts), dim3(kThreads), 0, stream,
                                             codes, cb, rows, cols, x, part, nparts))
  } else {
    RVQ_BPW_DISPATCH(bpw, hipLaunchKernelGGL((k_gemv_tiles_f32<B>), dim3(nt, nparts), dim3(kThreads), 0, stream,
                                             codes, cb, rows, cols, x, part, nparts))
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_sum_tiles, dim3((unsigned)cdiv(rows, 256)), dim3(256), 0, stream, part, nt, rows,
                     (int64_t)pad_rows(rows), y);
  return hipGetLastError();
}

// =============================================================================================
// Router logits in fp64 (bf16 x fp32 and bf16 x bf16 products are exact in fp64).
// One wave per (expert, token); 16-byte weight loads when rows are 16-byte aligned.
__device__ inline double bf16_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }
__device__ inline double x_to_f64(float v) { return (double)v; }
__device__ inline double x_to_f64(uint16_t v) { return bf16_to_f64(v); }

// Sum over the 64 lanes of a wave (every lane active), equal at every lane, bit for bit, to
//   for (off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64)
// without lane permutes through the LDS unit.  The xor-32 and xor-16 partners come from the permlane
// swaps (each half of the double swapped with itself); after those two steps a lane's value depends
// only on its place in its row of 16 lanes, so rotating the row by 8, 4, 2 and 1 lanes (DPP) reads
// a lane holding exactly the value of the xor-8, -4, -2 and -1 partner.  a + b equals b + a, so
// every lane adds the same two values as in the shuffle form, step by step.
__device__ __forceinline__ double wave_sum_f64(double v) {
  const unsigned lane = __lane_id();
  {
    const unsigned lo = (unsigned)__double2loint(v), hi = (unsigned)__double2hiint(v);
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const bool up = lane & 32u;   // its partner's value: first result on lanes 32..63, second below
    v += __hiloint2double((int)(up ? b[0] : b[1]), (int)(up ? a[0] : a[1]));
  }
  {
    const unsigned lo = (unsigned)__double2loint(v), hi = (unsigned)__double2hiint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const bool odd = lane & 16u;   // first result on the odd rows, second on the even ones
    v += __hiloint2double((int)(odd ? b[0] : b[1]), (int)(odd ? a[0] : a[1]));
  }
#define RVQ_ROW_ROR_ADD(n)                                                                              \
  {                                                                                                     \
    const int lo = __double2loint(v), hi = __double2hiint(v);                                           \
    v += __hiloint2double(__builtin_amdgcn_update_dpp(0, hi, 0x120 + (n), 0xF, 0xF, false),            \
                          __builtin_amdgcn_update_dpp(0, lo, 0x120 + (n), 0xF, 0xF, false));           \
  }
  RVQ_ROW_ROR_ADD(8)
  RVQ_ROW_ROR_ADD(4)
  RVQ_ROW_ROR_ADD(2)
  RVQ_ROW_ROR_ADD(1)
#undef RVQ_ROW_ROR_ADD
  return v;
}

// Eight x values as loaded (16 or 32 bytes), widened to fp64 only when used, so that a thread can
// have all of its loads in flight before the first product.
template <typename XT>
struct RawX8;
template <>
struct RawX8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ double get(int j) const { return (double)(j < 4 ? a[j] : b[j - 4]); }
};
template <>
struct RawX8<uint16_t> {
  u32x4 a;
  __device__ __forceinline__ void load(const uint16_t* p) { a = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ double get(int j) const {
    return bf16_to_f64((uint16_t)((j & 1) ? (a[j >> 1] >> 16) : (a[j >> 1] & 0xffffu)));
  }
};

constexpr int kRouterUnroll = 4;   // 8-element pieces per thread with loads in flight together

// This thread's part of sum_h w[h] * xf(x[h]) for one router row: pieces q = tid, tid + 256, ...
// in increasing q, even elements into a0 and odd into a1 (fp64 fma), then a scalar tail into a0.
// Loads use clamped (always valid) indices and are all issued before the products, which are
// predicated on the real index; the order of the products is that of the plain loop.
template <typename XT, typename XF>
__device__ __forceinline__ double router_dot(const uint16_t* __restrict__ wr, const XT* __restrict__ xr, int H, int vec,
                                             XF xf) {
  double a0 = 0.0, a1 = 0.0;
  int h0 = 0;
  if (vec) {
    const int n8 = H / 8;
    for (int q0 = threadIdx.x; q0 < n8; q0 += 256 * kRouterUnroll) {
      u32x4 wv[kRouterUnroll];
      RawX8<XT> xv[kRouterUnroll];
#pragma unroll
      for (int u = 0; u < kRouterUnroll; ++u) {
        const int q = min(q0 + 256 * u, n8 - 1);
        wv[u] = *reinterpret_cast<const u32x4*>(wr + q * 8);
        xv[u].load(xr + q * 8);
      }
#pragma unroll
      for (int u = 0; u < kRouterUnroll; ++u) {
        if (q0 + 256 * u < n8) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a0 = fma(bf16_to_f64((uint16_t)(wv[u][j] & 0xffffu)), xf(xv[u].get(2 * j)), a0);
            a1 = fma(bf16_to_f64((uint16_t)(wv[u][j] >> 16)), xf(xv[u].get(2 * j + 1)), a1);
          }
        }
      }
    }
    h0 = n8 * 8;
  }
  for (int h = h0 + threadIdx.x; h < H; h += 256) a0 = fma(bf16_to_f64(wr[h]), xf(x_to_f64(xr[h])), a0);
  return a0 + a1;
}

// This thread's part of sum_h x[h]^2 in fp64: h = tid, tid + 256, ... in increasing order (fma),
// 16 loads in flight at a time.
__device__ __forceinline__ double sum_squares(const float* __restrict__ x, int H) {
  constexpr int U = 16;
  double ss = 0.0;
  for (int h0 = threadIdx.x; h0 < H; h0 += 256 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x[min(h0 + 256 * u, H - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (h0 + 256 * u < H) ss = fma((double)v[u], (double)v[u], ss);
  }
  return ss;
}

// One workgroup per (expert, token): 256 threads stride over H in 8-element (16/32-byte) pieces
// with two fp64 accumulators each, then a fixed-order reduction.
template <typename XT>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ w, const XT* __restrict__ x, int T,
                                                       int E, int H, double* __restrict__ logits, int vec) {
  __shared__ double red[4];
  const int e = blockIdx.x, t = blockIdx.y;
  const uint16_t* wr = w + (int64_t)e * H;
  const XT* xr = x + (int64_t)t * H;
  double acc = router_dot(wr, xr, H, vec, [](double v) { return v; });
  acc = wave_sum_f64(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) logits[(int64_t)t * E + e] = (red[0] + red[1]) + (red[2] + red[3]);
}

// Top-k by (logit desc, id asc), by one workgroup; every thread calls it.  With a thread per expert
// it is topk_rank below; with more experts than threads it runs in two passes:
//  (a) g[e] = #{j in e's 64-expert block : L[j] > L[e]} (strict, one compare per pair, E * 64 pairs);
//  (b) the candidates are the experts with g < k.  Every expert of global rank < k is one (its
//      count within the block is at most its rank), and every expert ahead of such an expert has
//      smaller rank, so is one too;
//  (c) each candidate's rank among the candidates by (logit desc, id asc) is then its global rank
//      whenever that is below k, and a candidate of global rank >= k has the true top k ahead of
//      it, so its rank among candidates is >= k as well.  sel[rank] = id for ranks < k.
// Each task of (a) and (c) compares its 64 lanes with 16 values read at once (the passes are bound
// by LDS latency, not by the compares).  The partial counts are integers added with LDS atomics:
// exact in any order.  Candidates take list slots in atomic order, which changes nothing, as (c)
// orders them by logit and id alone.
// On entry (see topk_prepare): L holds the E logits and -inf up to E rounded to 64 (Ep); g and
// crank are zero; cl and cid hold -inf and INT_MAX (the padding that (c) compares against); ncand[0]
// is zero.  With Ep <= blockDim also: key, the keys below (0 for padding); ckey zero;
// skey[s] = key[s Ep / 64] (s < 64, a sample).
struct TopkScratch {
  int* g;            // [Ep]
  int* crank;        // [Ep]
  int* cid;          // [Ep]
  double* cl;        // [Ep]
  int* ncand;        // [1]
  uint32_t* key;     // [Ep], 16-byte aligned (one-pass form only, as the rest of this list)
  uint32_t* ckey;    // [Ep], 16-byte aligned
  uint32_t* skey;    // [64], 16-byte aligned
};
constexpr int kTopkChunk = 16;
__device__ __forceinline__ int topk_pad(int E) { return (E + 63) & ~63; }

// Order-preserving 32-bit image of a logit rounded to fp32, -0 taken as +0 (x + 0.0 is +0 for
// x = -0 and x otherwise): rounding to nearest is monotone, so key(a) > key(b) implies a > b and
// key(a) < key(b) implies a < b; equal keys decide nothing.  Finite and infinite logits map above 0,
// the key of the padding.
__device__ __forceinline__ uint32_t topk_key(double l) {
  const uint32_t b = __float_as_uint((float)(l + 0.0));
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Writes the state topk_select expects; src(e) gives logit e.  Every thread calls it; a barrier
// must follow.
template <typename Src>
__device__ void topk_prepare(double* L, int E, const TopkScratch& ts, Src src) {
  const int Ep = topk_pad(E);
  const bool one = Ep <= (int)blockDim.x;
  if (threadIdx.x == 0) ts.ncand[0] = 0;
  const int S = Ep >> 6;   // sample stride
  for (int e = threadIdx.x; e < Ep; e += blockDim.x) {
    const double l = e < E ? src(e) : -INFINITY;
    L[e] = l;
    ts.g[e] = 0;
    ts.crank[e] = 0;
    ts.cid[e] = INT_MAX;
    ts.cl[e] = -INFINITY;
    if (one) {
      const uint32_t key = e < E ? topk_key(l) : 0u;
      ts.key[e] = key;
      ts.ckey[e] = 0u;
      if (e % S == 0) ts.skey[e / S] = key;
    }
  }
}

// Experts with a thread each (Ep <= blockDim, blockDim >= 256).  The rank of e is
// #{j : L[j] > L[e], or L[j] = L[e] and j < e}; ranks are counted on the keys (above), and the
// fp64 logits and ids decide only between equal keys.
//  (1) tau = the k-th largest key of the sample skey (each sample key's count of greater sample
//      keys, then the smallest key among the samples with fewer than k above them).  At least k
//      keys are >= tau, so every expert of rank < k has a key >= tau.
//  (2) the candidates are the experts with key >= tau (about k E / 64 of them for unordered
//      logits; all E at worst), compacted in atomic order, which nothing below depends on.
//  (3) each candidate's rank: its count of greater candidate keys (every key above a candidate's
//      belongs to a candidate, so this is its count of greater keys overall), plus the candidates
//      of an equal key that come first by fp64 logit, then id.  Thread (i, p) counts part p of the
//      candidates (16 keys per step, the same for the whole wave, so every read is a broadcast;
//      equal keys are counted on the way, and only a part holding another candidate's equal key,
//      which is rare, compares logits and ids); the parts add with LDS atomics, exact.
//  (4) the ranks are distinct, so each candidate of rank r < k writes sel[r].
__device__ void topk_rank(const double* L, int E, int k, const TopkScratch& ts, int* sel) {
  const int Ep = topk_pad(E);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  if (wave < 4) {   // (1): wave w compares every sample key with sample keys 16 w .. 16 w + 15
    const uint32_t ks = ts.skey[lane];
    int c = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(ts.skey + 16 * wave + 4 * u);
      c += (int)(kv.x > ks) + (int)(kv.y > ks) + (int)(kv.z > ks) + (int)(kv.w > ks);
    }
    atomicAdd(&ts.g[lane], c);
  }
  __syncthreads();
  uint32_t tau = ts.g[lane] < k ? ts.skey[lane] : 0xffffffffu;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)tau, off, 64);
    tau = o < tau ? o : tau;
  }
  if (t < Ep) {   // (2): whole waves (Ep is a multiple of 64)
    const uint32_t ke = ts.key[t];
    const bool cand = t < E && ke >= tau;
    const uint64_t m = __ballot(cand);
    int base = 0;
    if (lane == 0 && m) base = atomicAdd(ts.ncand, __popcll(m));
    base = __shfl(base, 0, 64);
    if (cand) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      ts.cid[pos] = t;
      ts.ckey[pos] = ke;
      ts.cl[pos] = L[t];
    }
  }
  __syncthreads();
  const int C = __builtin_amdgcn_readfirstlane(*ts.ncand);
  const int Cp = (C + 63) & ~63;   // <= Ep <= blockDim; ckey is zero from C on
  const int np = __builtin_amdgcn_readfirstlane((int)blockDim.x / Cp);
  const int p = __builtin_amdgcn_readfirstlane(t / Cp);   // the same for a wave
  const int i = t - p * Cp;
  if (p < np && i < C) {   // (3)
    const int span = __builtin_amdgcn_readfirstlane(((Cp + np - 1) / np + 15) & ~15);
    const int j0 = p * span, j1 = j0 + span < Cp ? j0 + span : Cp;
    const uint32_t ki = ts.ckey[i];
    int c = 0, eq = 0;
    for (int j = j0; j < j1; j += 16) {
      u32x4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kv[u] = *reinterpret_cast<const u32x4*>(ts.ckey + j + 4 * u);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c += (int)(kv[u].x > ki) + (int)(kv[u].y > ki) + (int)(kv[u].z > ki) + (int)(kv[u].w > ki);
        eq += (int)(kv[u].x == ki) + (int)(kv[u].y == ki) + (int)(kv[u].z == ki) + (int)(kv[u].w == ki);
      }
    }
    if (i >= j0 && i < j1) --eq;   // its own key
    if (eq > 0) {   // another candidate of this part has the same key: the fp64 logit, then the id
      const double li = ts.cl[i];
      const int ei = ts.cid[i];
      for (int j = j0; j < j1; ++j)
        if (j != i && ts.ckey[j] == ki) c += (int)((ts.cl[j] > li) || (ts.cl[j] == li && ts.cid[j] < ei));
    }
    if (np == 1) ts.crank[i] = c;
    else atomicAdd(&ts.crank[i], c);
  }
  __syncthreads();
  for (int c = t; c < C; c += blockDim.x) {   // (4)
    const int r = ts.crank[c];
    if (r < k) sel[r] = ts.cid[c];
  }
}

__device__ void topk_select(const double* L, int E, int k, const TopkScratch& ts, int* sel) {
  if (topk_pad(E) <= (int)blockDim.x) {
    topk_rank(L, E, k, ts, sel);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  constexpr int Q = 64 / kTopkChunk;
  const int nb = topk_pad(E) >> 6;
  for (int task = wave; task < nb * Q; task += nw) {
    const int b = task / Q, q = task - b * Q;
    const int e = b * 64 + lane;
    const double le = L[e];
    const double* Lj = L + b * 64 + q * kTopkChunk;
    double v[kTopkChunk];
#pragma unroll
    for (int u = 0; u < kTopkChunk; ++u) v[u] = Lj[u];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kTopkChunk; ++u) c += v[u] > le;
    if (e < E) atomicAdd(&ts.g[e], c);
  }
  __syncthreads();
  for (int e0 = wave * 64; e0 < nb * 64; e0 += nw * 64) {
    const int e = e0 + lane;
    const bool cand = e < E && ts.g[e] < k;
    const uint64_t m = __ballot(cand);
    int base = 0;
    if (lane == 0 && m) base = atomicAdd(ts.ncand, __popcll(m));
    base = __shfl(base, 0, 64);
    if (cand) {
      const int p = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      ts.cid[p] = e;
      ts.cl[p] = L[e];
    }
  }
  __syncthreads();
  const int C = __builtin_amdgcn_readfirstlane(*ts.ncand);
  const int ncb = (C + 63) >> 6, nq = (C + kTopkChunk - 1) / kTopkChunk;
  for (int task = wave; task < ncb * nq; task += nw) {
    const int b = task / nq, q = task - b * nq;
    const int i = b * 64 + lane;
    const int ii = i < C ? i : C - 1;
    const int ei = ts.cid[ii];
    const double li = ts.cl[ii];
    double v[kTopkChunk];
    int id[kTopkChunk];
#pragma unroll
    for (int u = 0; u < kTopkChunk; ++u) {
      v[u] = ts.cl[q * kTopkChunk + u];
      id[u] = ts.cid[q * kTopkChunk + u];
    }
    int c = 0;
#pragma unroll
    for (int u = 0; u < kTopkChunk; ++u) c += (v[u] > li) || (v[u] == li && id[u] < ei);
    if (i < C) atomicAdd(&ts.crank[i], c);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += blockDim.x)
    if (ts.crank[i] < k) sel[ts.crank[i]] = ts.cid[i];
}

// Called by one whole wave: gates = softmax over the kept logits in fp64 (max subtracted), the
// denominator summed by a fixed shuffle tree over ranks; writes ids/gates[i] for i < k with
// want(i) true.
template <typename Want>
__device__ void topk_gates(const double* L, const int* sel, int k, int32_t* ids, float* gates, Want want) {
  const int i = threadIdx.x & 63;
  const double m = L[sel[0]];
  const double ex = i < k ? exp(L[sel[i]] - m) : 0.0;
  double z = ex;
  z = wave_sum_f64(z);
  if (i < k && want(i)) {
    ids[i] = sel[i];
    gates[i] = (float)(ex / z);
  }
}

__global__ __launch_bounds__(1024) void k_topk(const double* __restrict__ logits, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ gates) {
  __shared__ double L[kMaxExperts], cl[kMaxExperts];
  __shared__ int g[kMaxExperts], crank[kMaxExperts], cid[kMaxExperts];
  // the one-pass form's arrays (Ep <= the 1024 threads)
  __shared__ __attribute__((aligned(16))) uint32_t key[1024], ckey[1024], skey[64];
  __shared__ int sel[kMaxTopK], ncand[1];
  const int t = blockIdx.x;
  if (threadIdx.x < kMaxTopK) sel[threadIdx.x] = 0;
  const TopkScratch ts{g, crank, cid, cl, ncand, key, ckey, skey};
  topk_prepare(L, E, ts, [&](int e) { return logits[(int64_t)t * E + e]; });
  __syncthreads();
  topk_select(L, E, k, ts, sel);
  __syncthreads();
  if (threadIdx.x < 64) topk_gates(L, sel, k, ids + (int64_t)t * k, gates + (int64_t)t * k, [](int) { return true; });
}

// Pre-norm router for one token: every workgroup forms inv = 1/sqrt(mean(h^2) + eps) exactly as
// k_rmsnorm does (same per-thread strides and reduction order, fp64), then the logit of its expert
// on n = (float)(h * inv), again exactly as k_router_logits reads an fp32 n; workgroup e also writes
// its slice [e*ceil(H/E), ...) of n for the expert kernels.
__global__ __launch_bounds__(256) void k_router_norm_logits(const uint16_t* __restrict__ w, const float* __restrict__ h,
                                                            int E, int H, float eps, double* __restrict__ logits,
                                                            float* __restrict__ n, int vec) {
  __shared__ double red[4];
  __shared__ double red2[4];
  const int e = blockIdx.x;
  const int per = (H + E - 1) / E;
  constexpr int SU = 32;   // h values per thread for the sum of squares in one round of loads
  if (vec && H <= 256 * SU && H / 8 <= 256 * kRouterUnroll && per <= 256) {
    // The same sums in the same order as below, with every load issued before the first product:
    // the sum of squares's values (h = tid + 256 u), the router row's and h's 8-element pieces
    // (q = tid + 256 u, as router_dot), and the element of n this thread writes.  One round trip
    // to memory instead of four.
    const int tid = threadIdx.x;
    const uint16_t* wr = w + (int64_t)e * H;
    const int n8 = H / 8;
    float v[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) v[u] = h[min(tid + 256 * u, H - 1)];
    u32x4 wv[kRouterUnroll];
    RawX8<float> xv[kRouterUnroll];
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      const int q = min(tid + 256 * u, n8 - 1);
      wv[u] = *reinterpret_cast<const u32x4*>(wr + q * 8);
      xv[u].load(h + q * 8);
    }
    const int jn = min(e * per + tid, H - 1);
    const bool own = tid < per && e * per + tid < H;
    const float hn = h[jn];
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first product
    double ss = 0.0;
#pragma unroll
    for (int u = 0; u < SU; ++u)
      if (tid + 256 * u < H) ss = fma((double)v[u], (double)v[u], ss);
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    const double inv = 1.0 / sqrt(tot / (double)H + (double)eps);
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      if (tid + 256 * u < n8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a0 = fma(bf16_to_f64((uint16_t)(wv[u][j] & 0xffffu)), (double)(float)(xv[u].get(2 * j) * inv), a0);
          a1 = fma(bf16_to_f64((uint16_t)(wv[u][j] >> 16)), (double)(float)(xv[u].get(2 * j + 1) * inv), a1);
        }
      }
    }
    double acc = a0 + a1;
    acc = wave_sum_f64(acc);
    if ((tid & 63) == 0) red2[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) logits[e] = (red2[0] + red2[1]) + (red2[2] + red2[3]);
    if (own) n[jn] = (float)((double)hn * inv);
    return;
  }
  double ss = sum_squares(h, H);
  ss = wave_sum_f64(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double tot = (red[0] + red[1]) + (red[2] + red[3]);
  const double inv = 1.0 / sqrt(tot / (double)H + (double)eps);
  const uint16_t* wr = w + (int64_t)e * H;
  double acc = router_dot(wr, h, H, vec, [inv](double v) { return (double)(float)(v * inv); });
  acc = wave_sum_f64(acc);
  if ((threadIdx.x & 63) == 0) red2[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) logits[e] = (red2[0] + red2[1]) + (red2[2] + red2[3]);
  for (int j = e * per + (int)threadIdx.x; j < (e + 1) * per && j < H; j += 256) n[j] = (float)((double)h[j] * inv);
}

hipError_t launch_router_norm_logits(const uint16_t* w, const float* h, int E, int H, float eps, double* logits,
                                     float* n, hipStream_t stream) {
  const int vec = (H % 8 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0) &&
                  ((reinterpret_cast<uintptr_t>(h) & 15) == 0);
  hipLaunchKernelGGL(k_router_norm_logits, dim3((unsigned)E), dim3(256), 0, stream, w, h, E, H, eps, logits, n, vec);
  return hipGetLastError();
}

// Router logits of several tokens: workgroup (b, c) computes experts ET b .. ET b + ET-1 for tokens
// TT c .. TT c + TT-1, so each router row is read once per TT tokens and each token row once per ET
// experts.  Every (expert, token) sum takes exactly the steps of k_router_logits (router_dot's
// pieces q = tid, tid + 256, ... in increasing q, even elements into a0 and odd into a1, fp64
// fma; then a0 + a1, the same shuffle tree and the same four-wave sum), so the logits are those
// of one token at a time, bit for bit.  Needs H % 8 == 0 and 16-byte aligned rows; out-of-range
// experts and tokens load a valid row and are not written.
template <typename XT, int ET, int TT>
__global__ __launch_bounds__(256) void k_router_logits_tiles(const uint16_t* __restrict__ w, const XT* __restrict__ x,
                                                             int T, int E, int H, double* __restrict__ logits) {
  constexpr int U = 2;   // pieces per thread with loads in flight together
  __shared__ double red[ET * TT][4];
  const int e0 = blockIdx.x * ET, t0 = blockIdx.y * TT;
  const uint16_t* wr[ET];
  const XT* xr[TT];
#pragma unroll
  for (int i = 0; i < ET; ++i) wr[i] = w + (int64_t)min(e0 + i, E - 1) * H;
#pragma unroll
  for (int t = 0; t < TT; ++t) xr[t] = x + (int64_t)min(t0 + t, T - 1) * H;
  double a0[ET][TT], a1[ET][TT];
#pragma unroll
  for (int i = 0; i < ET; ++i)
#pragma unroll
    for (int t = 0; t < TT; ++t) a0[i][t] = a1[i][t] = 0.0;
  const int n8 = H / 8;
  for (int q0 = threadIdx.x; q0 < n8; q0 += 256 * U) {
    u32x4 wv[U][ET];
    RawX8<XT> xv[U][TT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + 256 * u, n8 - 1);
#pragma unroll
      for (int i = 0; i < ET; ++i) wv[u][i] = *reinterpret_cast<const u32x4*>(wr[i] + q * 8);
#pragma unroll
      for (int t = 0; t < TT; ++t) xv[u][t].load(xr[t] + q * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q0 + 256 * u < n8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int i = 0; i < ET; ++i) {
            const double we = bf16_to_f64((uint16_t)(wv[u][i][j] & 0xffffu));
            const double wo = bf16_to_f64((uint16_t)(wv[u][i][j] >> 16));
#pragma unroll
            for (int t = 0; t < TT; ++t) {
              a0[i][t] = fma(we, xv[u][t].get(2 * j), a0[i][t]);
              a1[i][t] = fma(wo, xv[u][t].get(2 * j + 1), a1[i][t]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < ET; ++i)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      double acc = a0[i][t] + a1[i][t];
      acc = wave_sum_f64(acc);
      if ((threadIdx.x & 63) == 0) red[i * TT + t][threadIdx.x >> 6] = acc;
    }
  __syncthreads();
  if (threadIdx.x < ET * TT) {
    const int i = threadIdx.x / TT, t = threadIdx.x % TT;
    const double* r = red[threadIdx.x];
    if (e0 + i < E && t0 + t < T) logits[(int64_t)(t0 + t) * E + e0 + i] = (r[0] + r[1]) + (r[2] + r[3]);
  }
}
constexpr int kRouterTileE = 4, kRouterTileT = 4;

hipError_t launch_router_logits(const uint16_t* w, const void* x, bool x_bf16, int T, int E, int H, double* logits,
                                hipStream_t stream) {
  const int vec = (H % 8 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0) &&
                  ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  if (T > 1 && vec) {
    const dim3 tiles((unsigned)cdiv(E, kRouterTileE), (unsigned)cdiv(T, kRouterTileT));
    if (x_bf16)
      hipLaunchKernelGGL((k_router_logits_tiles<uint16_t, kRouterTileE, kRouterTileT>), tiles, dim3(256), 0, stream, w,
                         static_cast<const uint16_t*>(x), T, E, H, logits);
    else
      hipLaunchKernelGGL((k_router_logits_tiles<float, kRouterTileE, kRouterTileT>), tiles, dim3(256), 0, stream, w,
                         static_cast<const float*>(x), T, E, H, logits);
    return hipGetLastError();
  }
  dim3 grid((unsigned)E, (unsigned)T);
  if (x_bf16)
    hipLaunchKernelGGL(k_router_logits<uint16_t>, grid, dim3(256), 0, stream, w, static_cast<const uint16_t*>(x), T,
                       E, H, logits, vec);
  else
    hipLaunchKernelGGL(k_router_logits<float>, grid, dim3(256), 0, stream, w, static_cast<const float*>(x), T, E, H,
                       logits, vec);
  return hipGetLastError();
}

hipError_t launch_router_topk(const uint16_t* w, const void* x, bool x_bf16, int T, int E, int H, int k, int32_t* ids,
                              float* gates, double* logits, hipStream_t stream) {
  const hipError_t err = launch_router_logits(w, x, x_bf16, T, E, H, logits, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_topk, dim3((unsigned)T), dim3(1024), 0, stream, logits, E, k, ids, gates);
  return hipGetLastError();
}

// =============================================================================================
// RMSNorm (unit weight), sum of squares accumulated in fp64, fixed reduction order.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, int H, float eps, float* out) {
  __shared__ double red[4];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * H;
  double ss = sum_squares(xr, H);
  ss = wave_sum_f64(ss);
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
//   gate/up:  grid k * 2 * ngu     -> part_gu[slot][m][part][row]   (rows of gate/up = I; ngu = nt_in
//             partials, one per K-tile, or fewer when a workgroup sums several K-tiles)
//   down:     grid k * nt_out * P  -> part_d[slot][tile][row]        (rows of down = H)
//             (each workgroup first rebuilds its 8*G entries of h = silu(g) * u from part_gu)
//   combine:  y[r] = residual[r] + sum_slot gate[slot] * sum_tile part_d[slot][tile][r]
template <bool F16, int BPW, int NT>
__device__ __forceinline__ void k_moe_gateup_body(BankArgs bank, const float* __restrict__ x,
                                                    const int32_t* __restrict__ ids, float* __restrict__ part_gu,
                                                    int32_t* __restrict__ status) {
  constexpr int G = Tile<F16>::kGroups;
  __shared__ __attribute__((aligned(16))) typename Tile<F16>::entry_t lut[kLutBytes / sizeof(typename Tile<F16>::entry_t)];
  __shared__ float vs[256];
  __shared__ float red[NT / 64];
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
  const int nrb = (int)cdiv(I, kSlabRows);
  const int nt16 = (int)cdiv(groups, kSlabGroups);
  const int i = threadIdx.x;
  const int k0 = tile * G * 8;
  // loads the tables need are issued before the code prefetch: waits on memory counters are in order
  const float v = (i < G * 8 && k0 + i < H) ? x[k0 + i] : 0.f;
  float cv[3][8];
  load_codebook_entry<F16>(cb, cv);
  RowStream<F16, BPW> rs;
  rs.begin(codes, nrb, nt16, tile, 0, nrb);
  if (i < G * 8) vs[i] = v;
  __syncthreads();
  const float out_scale = tile_tables<F16>(lut, cv, vs, v, red);
  rs.run(lut, out_scale, part_gu + (((int64_t)slot * 2 + m) * nt + tile) * pad_rows(I));
}

// ---------------------------------------------------------------------------------------------
// Wave-specialised table kernels (fp32 tables): one workgroup per CU, NSW streamer waves and 4
// builder waves.
//
// A workgroup owns ITEMS consecutive 16-group K-tiles of one matrix and a range of NSW * BPI row
// blocks.  The streamer waves stream those rows' codes through each K-tile's tables in turn and keep
// one running sum per row, so the workgroup writes one partial row vector.  The builder waves build
// the next K-tile's tables into the other half of a double buffer while the streamers gather.
//   gate/up (DOWN = false): work item b -> gm = b / nchunk (slot * 2 + matrix), K-tiles
//            ITEMS (b % nchunk) + [0, ITEMS), all 32 row blocks; partial row vector b of part_gu.
//   down    (DOWN = true):  work item b -> slot, row chunk rc, K-tile chunk kc (kc fastest); its
//            x operand is h = silu(g) * u, where g and u sum the `ngu` gate and up partials.
// (Work items are dealt to workgroups XCD by XCD; see the geometry below.)
// The roles exchange LDS counters with workgroup-scope release/acquire instead of barriers:
//   built[k%2] += 1 per builder wave when its share of item k's tables is written;
//                 streamers start item k at built[k%2] >= 4 (floor(k/2) + 1);
//   done[k%2]  += 1 per streamer wave when it has read item k's tables;
//                 builders overwrite buffer k%2 (item k >= 2) at done[k%2] >= NSW floor(k/2).
// The counts are per buffer so a sum cannot be reached early: a builder wave can only get to item
// k+2 once every streamer is past item k, hence when built[k%2] first reaches its target each
// builder wave has added exactly floor(k/2)+1 to it (and likewise for done).  Neither role waits on
// itself, so the waits end; each is still bounded (kSpinLimit polls, after which the kernel records
// RVQ_ERR_DEVICE_STALL rather than hang).
//
// The tables of one item are the product of the 768 x 8 codebook (3 stages x 256 entries) with the
// 8 x 16 matrix of the tile's x sub-vectors, computed with fp32 MFMAs: builder wave w owns 16-entry
// table tiles 12w .. 12w+11.  With lane l = 16q + i (q < 4), A holds codebook entry i of the table
// tile at dims 2q, 2q+1 (one per MFMA), B holds group i's x at the same dims, and D returns
// entries 4q..4q+3 of group i, written to rows 4q..4q+3 of the subtable's column of the skewed
// layout (see SkewLane; subtables 32..47 twice).  The codebook operands are the same for every
// item of the workgroup and are loaded once, before the start barrier.
//
// fp16 tables (F16): entries are stored scaled by 2^-e_k, e_k = f16_table_exponent(max |c| max |x_g|)
// over the codebook and the item's 16 groups (so no entry can overflow); the streamers scale each
// item's sums by 2^e_k before adding them to the row totals.  The two fp16 tables share one skewed
// array of 32-bit words, table k & 1 in half k & 1 of each word: the lookups keep the fp32
// layout's addresses (and its conflict-free banks), and both tables take 64 KiB.
constexpr int kPipeBuildWaves = 4;
constexpr int kPipeMaxItems = 8;
constexpr int kPipeMaxGu = 8;          // down: most gate/up partials per row
constexpr int kGuStreamWaves = 8, kGuBpi = 4;     // gate/up: 32 row blocks (I in (1984, 2048])
constexpr int kDnStreamWaves = 7, kDnBpi = 4;     // down: row chunks of 28 row blocks
constexpr int kSpinLimit = 1 << 22;
constexpr int kStatusStall = 8;        // RVQ_ERR_DEVICE_STALL

__device__ inline bool lds_wait_ge(int* flag, int target, int limit) {
  for (int i = 0; i < limit; ++i) {
    if (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Polls per bounded wait of the wave-specialised kernels: word kWaitLimitWord of the workspace
// header holds 0 for the default (kSpinLimit) or polls + 1 (set by rvq_workspace_set_wait_limit).
__device__ inline int wait_polls(const int32_t* header) {
  const int32_t w = header[kWaitLimitWord];
  return w <= 0 ? kSpinLimit : w - 1;
}

__global__ void k_set_word(int32_t* p, int32_t v) { *p = v; }

hipError_t launch_set_word(int32_t* p, int32_t v, hipStream_t stream) {
  hipLaunchKernelGGL(k_set_word, dim3(1), dim3(1), 0, stream, p, v);
  return hipGetLastError();
}

// Compute units of the current device (0 if the query fails), cached per device.
static int compute_units() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev >= 64) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  }
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cache[dev] = n;
  }
  return cache[dev];
}

struct PipeArgs {
  const float* x;         // gate/up: fp32 [H]
  const float* part_gu;   // down: gate/up partials [k][2][ngu][pad_rows(I)]
  float* out;             // gate/up: part_gu; down: part_d [k][nkc][pad_rows(H)]
  int nchunk;             // gate/up: workgroups per matrix; down: K-tile chunks per slot (nkc)
  int nrc;                // down: row chunks per slot
  int ngu;                // down: gate/up partials per row
  // gate/up with routing: when logits is set the workgroup picks its slot's expert itself (the
  // top-k of logits[0..E)), and the first workgroup of each slot writes ids/gates[slot]
  const double* logits;
  int32_t* ids_out;
  float* gates_out;
  int k;
  int gu_stride;          // down: partials stored per (slot, matrix) in part_gu (>= ngu)
};
constexpr int kRouteMaxExperts = 64 * (kGuStreamWaves + kPipeBuildWaves);   // a thread per expert

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

template <bool F16, bool DOWN, int NSW, int BPI, int ITEMS>
__global__ __launch_bounds__(64 * (NSW + kPipeBuildWaves)) void k_table_ws(BankArgs bank,
                                                                             const int32_t* __restrict__ ids,
                                                                             int32_t* __restrict__ status,
                                                                             PipeArgs pa) {
  constexpr int NB = 3;   // row blocks of codes held per streamer wave (deeper measured slower)
  constexpr int NBLK = ITEMS * BPI;
  constexpr int TPW = 48 / kPipeBuildWaves;                 // table tiles per builder wave
  // fp32: skewed 64-column tables (see SkewLane); fp16: 48 subtables S halves apart
  __shared__ __attribute__((aligned(16))) float lut[F16 ? 1 : 2][kSkewWords];
  // item k's table: fp32, buffer k & 1; fp16, half k & 1 of every word of the one buffer
  auto table = [&](int k) -> char* {
    return F16 ? reinterpret_cast<char*>(&lut[0][0]) + 2 * (k & 1) : reinterpret_cast<char*>(&lut[k & 1][0]);
  };
  __shared__ __attribute__((aligned(16))) float hs[DOWN ? ITEMS : 1][128];
  __shared__ int built[2], done[2], hready;
  __shared__ int cmax_bits;            // fp16: max squared codebook-entry norm (bits of a float >= 0)
  __shared__ float escale[ITEMS];      // fp16: 2^e_k of each item
  __shared__ int rsel[kMaxTopK];
  static_assert(DOWN || sizeof(lut) >= 36 * kRouteMaxExperts + 512, "top-k scratch must fit in the table buffers");
  static_assert(DOWN || 64 * (NSW + kPipeBuildWaves) >= kRouteMaxExperts, "the top-k takes a thread per expert");
  const int H = bank.H, I = bank.I;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wait_limit = wait_polls(status);   // status points at the workspace header
  // geometry of this workgroup.  Work item wi: the hardware deals workgroups to the 8 XCDs in turn,
  // so consecutive items are given to workgroups on one XCD (when the grid is a multiple of 8): the
  // workgroups of one slot and matrix then share an L2, which fetches their codebook (and, for
  // down, their gate/up partial sums) once.  Only where items run changes, never what they compute.
  const int nwg = (int)gridDim.x;
  const int wi = (nwg & 7) == 0 ? (int)(blockIdx.x & 7) * (nwg >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  int slot, m, t0, rb0;
  if constexpr (DOWN) {
    const int kc = wi % pa.nchunk;
    const int rc = (wi / pa.nchunk) % pa.nrc;
    slot = wi / (pa.nchunk * pa.nrc);
    m = 2;
    t0 = kc * ITEMS;
    rb0 = rc * NSW * BPI;
  } else {
    const int gm = wi / pa.nchunk;
    slot = gm >> 1;
    m = gm & 1;
    t0 = (wi - gm * pa.nchunk) * ITEMS;
    rb0 = 0;
  }
  const bool streamer = wave < NSW;
  const int bw = wave - NSW;
  // The loads of the prologue are issued in the order their results are needed: the expert id (or
  // this thread's router logit), then the operands that do not depend on the expert.  A wait for a
  // vector load also waits for every vector load issued before it.
  const bool route = !DOWN && pa.logits;
  const int e_given = route ? 0 : ids[slot];
  const double logit = route && (int)threadIdx.x < bank.E ? pa.logits[threadIdx.x] : 0.0;
  // down: builder wave bw computes h for items bw, bw + 4, ... (ITEMS <= 8, so at most two): lane l
  // takes entries l and 64 + l of the item's 128.  The gate/up partials depend on the slot only.
  constexpr int HI = DOWN ? (ITEMS + kPipeBuildWaves - 1) / kPipeBuildWaves : 1;
  constexpr int GU = DOWN ? kPipeMaxGu : 1;
  float gv[HI][2][GU], uv[HI][2][GU];
  if constexpr (DOWN) {
    if (!streamer) {
      const int64_t Ip = pad_rows(I);
      const float* pg = pa.part_gu + (int64_t)slot * 2 * pa.gu_stride * Ip;
      const float* pu = pg + (int64_t)pa.gu_stride * Ip;
#pragma unroll
      for (int n = 0; n < HI; ++n) {
        const int k = bw + n * kPipeBuildWaves < ITEMS ? bw + n * kPipeBuildWaves : ITEMS - 1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int64_t col = (int64_t)(t0 + k) * 128 + hh * 64 + lane;
#pragma unroll
          for (int p = 0; p < GU; ++p) {
            const int pp = p < pa.ngu ? p : 0;
            gv[n][hh][p] = pg[pp * Ip + col];
            uv[n][hh][p] = pu[pp * Ip + col];
          }
        }
      }
    }
  }
  // gate/up builders: this item range's x sub-vectors do not depend on the expert, so they are
  // requested first, ahead of the top-k
  f32x2 xb[DOWN ? 1 : ITEMS];
  const int q = lane >> 4, i16 = lane & 15;
  if constexpr (!DOWN) {
    if (!streamer) {
      const float* xt = pa.x + (int64_t)(slot / pa.k) * H;   // slot = token * k + i when batched
#pragma unroll
      for (int k = 0; k < ITEMS; ++k)
        xb[k] = *reinterpret_cast<const f32x2*>(xt + (int64_t)(t0 + k) * 128 + i16 * 8 + 2 * q);
    }
  }
  int e;
  if (route) {
    // top-k of the router logits, the same computation as k_topk.  Its scratch lies in the table
    // buffers, which nothing writes before the start barrier below; every read of it comes first.
    const int E = bank.E;
    char* scr = reinterpret_cast<char*>(&lut[0][0]);
    double* rl = reinterpret_cast<double*>(scr);
    constexpr int R = kRouteMaxExperts;   // a multiple of 64: every array below is 16-byte aligned
    const TopkScratch ts{reinterpret_cast<int*>(scr + 16 * R), reinterpret_cast<int*>(scr + 20 * R),
                         reinterpret_cast<int*>(scr + 24 * R), reinterpret_cast<double*>(scr + 8 * R),
                         reinterpret_cast<int*>(scr + 36 * R + 256), reinterpret_cast<uint32_t*>(scr + 28 * R),
                         reinterpret_cast<uint32_t*>(scr + 32 * R), reinterpret_cast<uint32_t*>(scr + 36 * R)};
    if (threadIdx.x < kMaxTopK) rsel[threadIdx.x] = 0;
    // a thread per expert (E <= kRouteMaxExperts = the workgroup size): logit j is thread j's
    topk_prepare(rl, E, ts, [&](int) { return logit; });
    __syncthreads();
    topk_select(rl, E, pa.k, ts, rsel);
    __syncthreads();
    e = rsel[slot];
    if (m == 0 && t0 == 0 && wave == 0)
      topk_gates(rl, rsel, pa.k, pa.ids_out, pa.gates_out, [&](int i) { return i == slot; });
  } else {
    e = e_given;
  }
  const bool bad = e < 0 || e >= bank.E;
  if constexpr (DOWN) {
    if (bad) return;  // the gate/up kernel records the status; combine skips the slot
  } else {
    if (bad) e = 0;   // recorded below; this slot's results are never read
  }
  const int rows = DOWN ? H : I;
  const int nrb = (int)cdiv(rows, kSlabRows);
  const int64_t tile_bytes = (int64_t)nrb * kSlabBytes;

  // the codebook operands of the builders, requested before the start barrier (ahead of the code
  // stream)
  f32x2 a[TPW];
  if (!streamer) {
    const float* cb = bank.cb + ((int64_t)e * 3 + m) * kCodebookFloats;
#pragma unroll
    for (int t = 0; t < TPW; ++t) a[t] = *reinterpret_cast<const f32x2*>(cb + ((bw * TPW + t) * 16 + i16) * 8 + 2 * q);
  } else if (threadIdx.x == 0) {
    built[0] = 0;
    built[1] = 0;
    done[0] = 0;
    done[1] = 0;
    hready = 0;
    cmax_bits = 0;
    if (!DOWN && bad) atomicExch(status, 6 /* RVQ_ERR_EXPERT_ID */);
  }
  __syncthreads();

  if (streamer) {
    // ----------------------------------------------------------------- streamers
    const uint8_t* codes = bank.codes + (int64_t)e * bank.stride + (int64_t)m * packed_bytes(I, H) +
                           (int64_t)t0 * tile_bytes + (int64_t)rb0 * kSlabBytes;
    float acc[BPI];
#pragma unroll
    for (int r = 0; r < BPI; ++r) acc[r] = 0.f;
    bool ok = true;
    SlabData buf[NB];
    const uint32_t lane_off = lane * 16;
    SkewLane sl;
    sl.init(lane);
    auto load_blk = [&](int i, int s) {
      const int k = s / BPI, r = s % BPI;
      load_slabs<false>(buf[i], codes + k * tile_bytes, codes + k * tile_bytes,
                        (uint32_t)(wave + NSW * r) * kSlabBytes + lane_off);
    };
#pragma unroll
    for (int i = 0; i < NB && i < NBLK; ++i) load_blk(i, i);   // never past the workgroup's blocks
    // Wave priority follows the finishing order of the previous item.  Two streamer waves share
    // each SIMD, and the SIMD's arbiter favours the older one, so without this the younger half
    // falls behind item by item and streams the workgroup's last blocks alone, with half the
    // loads in flight.  The later half of an item's finishers runs the next item at a higher
    // priority; the earlier half at the lowest.  Only the issue order changes.
    int pos = 0;   // lane 0: this wave's place among the item's finishers
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      ok &= lds_wait_ge(&built[k & 1], kPipeBuildWaves * (k / 2 + 1), wait_limit);
      if (k > 0) {
        if (__builtin_amdgcn_readfirstlane(pos) < NSW / 2) __builtin_amdgcn_s_setprio(0);
        else __builtin_amdgcn_s_setprio(2);
      }
#pragma unroll
      for (int r = 0; r < BPI; ++r) {
        const int s = k * BPI + r;
        float g = gather_skew<F16>(table(k), buf[s % NB], sl);
        // opaque use: without it the compiler interleaves the row blocks' gathers into one another
        // and spills
        asm volatile("" : : "v"(g));
        if constexpr (F16) g *= escale[k];
        acc[r] += g;
        if (s + NB < NBLK) load_blk(s % NB, s + NB);
      }
      if (lane == 0)
        pos = __hip_atomic_fetch_add(&done[k & 1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP) - NSW * (k / 2);
    }
    float* out = pa.out + (int64_t)wi * pad_rows(rows) + (int64_t)rb0 * kSlabRows;
    if constexpr (DOWN) out = pa.out + ((int64_t)slot * pa.nchunk + (wi % pa.nchunk)) * pad_rows(rows) +
                              (int64_t)rb0 * kSlabRows;
#pragma unroll
    for (int r = 0; r < BPI; ++r) out[(wave + NSW * r) * kSlabRows + lane] = acc[r];
    if (!ok && lane == 0) atomicExch(status, kStatusStall);
  } else {
    // ----------------------------------------------------------------- builders
    bool ok = true;
    float cmax2 = 0.f;
    if constexpr (DOWN) {
      // opaque copies: without them the compiler starts these sums before the expert id's load, and
      // the id, with it the whole prologue, waits for the partials
#pragma unroll
      for (int n = 0; n < HI; ++n)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int p = 0; p < GU; ++p) asm volatile("" : "+v"(gv[n][hh][p]), "+v"(uv[n][hh][p]));
    }
    if constexpr (F16) {
      // squared norm of codebook entry i16 of each table tile: the 4 lanes q hold 2 dims each
      float v = 0.f;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        float n2 = a[t].x * a[t].x + a[t].y * a[t].y;
        n2 += __shfl_xor(n2, 16, 64);
        n2 += __shfl_xor(n2, 32, 64);
        v = fmaxf(v, n2);
      }
      v = wave_max(v);
      if (lane == 0) atomicMax(&cmax_bits, __float_as_int(v));   // non-negative floats order as ints
    }
    if constexpr (DOWN) {
#pragma unroll
      for (int n = 0; n < HI; ++n) {
        const int k = bw + n * kPipeBuildWaves;
        if (k >= ITEMS) break;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float g = 0.f, u = 0.f;
#pragma unroll
          for (int p = 0; p < GU; ++p) {
            g += p < pa.ngu ? gv[n][hh][p] : 0.f;
            u += p < pa.ngu ? uv[n][hh][p] : 0.f;
          }
          hs[k][hh * 64 + lane] = g / (1.f + expf(-g)) * u;
        }
      }
    }
    if (DOWN || F16) {
      if (lane == 0) __hip_atomic_fetch_add(&hready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      ok &= lds_wait_ge(&hready, kPipeBuildWaves, wait_limit);
      if constexpr (F16) cmax2 = __int_as_float(cmax_bits);
    }
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      if (k >= 2) ok &= lds_wait_ge(&done[k & 1], NSW * (k / 2), wait_limit);
      // an opaque copy pins this item's products after the wait (otherwise the compiler may compute
      // every item's tables up front)
      f32x2 xk;
      if constexpr (DOWN) xk = *reinterpret_cast<const f32x2*>(&hs[k][i16 * 8 + 2 * q]);
      else xk = xb[k];
      asm volatile("" : "+v"(xk));
      float scale = 1.f;
      if constexpr (F16) {
        float n2 = xk.x * xk.x + xk.y * xk.y;   // squared norm of group i16's x
        n2 += __shfl_xor(n2, 16, 64);
        n2 += __shfl_xor(n2, 32, 64);
        const int ex = f16_table_exponent(sqrtf(cmax2) * sqrtf(wave_max(n2)));
        scale = ldexpf(1.f, -ex);
        if (bw == 0 && lane == 0) escale[k] = ldexpf(1.f, ex);
      }
      char* L = table(k);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ti = bw * TPW + t, st = ti >> 4, e0 = (ti & 15) * 16;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t].x, xk.x, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t].y, xk.y, d, 0, 0, 0);
        // skewed layout: entry c of subtable j at word 64 c + j; subtables 32..47 also at j + 16
        const int j = 3 * i16 + st, c0 = e0 + 4 * q;
        if constexpr (F16) {
          _Float16* col = reinterpret_cast<_Float16*>(L) + 2 * (kSkewCols * c0 + j);   // half k & 1 of the word
          const _Float16 h[4] = {(_Float16)(d.x * scale), (_Float16)(d.y * scale), (_Float16)(d.z * scale),
                                 (_Float16)(d.w * scale)};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            col[2 * kSkewCols * u] = h[u];
            if (j >= 32) col[2 * kSkewCols * u + 32] = h[u];
          }
        } else {
          float* col = reinterpret_cast<float*>(L) + kSkewCols * c0 + j;
          col[0] = d.x;
          col[kSkewCols] = d.y;
          col[2 * kSkewCols] = d.z;
          col[3 * kSkewCols] = d.w;
          if (j >= 32) {
            col[16] = d.x;
            col[kSkewCols + 16] = d.y;
            col[2 * kSkewCols + 16] = d.z;
            col[3 * kSkewCols + 16] = d.w;
          }
        }
      }
      if (lane == 0) __hip_atomic_fetch_add(&built[k & 1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (!ok && lane == 0) atomicExch(status, kStatusStall);
  }
}

// gate/up: 4-wave workgroups, three per CU (LDS-bound), so three workgroups' table builds and
// streams interleave on each CU.
constexpr int kGateUpThreads = 256;
template <int BPW>
__global__ __launch_bounds__(kGateUpThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_moe_gateup_f32(
    BankArgs bank, const float* __restrict__ x, const int32_t* __restrict__ ids, float* __restrict__ part_gu,
    int32_t* __restrict__ status) {
  k_moe_gateup_body<false, BPW, kGateUpThreads>(bank, x, ids, part_gu, status);
}
template <int BPW>
__global__ __launch_bounds__(kGateUpThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_moe_gateup_f16(
    BankArgs bank, const float* __restrict__ x, const int32_t* __restrict__ ids, float* __restrict__ part_gu,
    int32_t* __restrict__ status) {
  k_moe_gateup_body<true, BPW, kGateUpThreads>(bank, x, ids, part_gu, status);
}

template <bool F16, int BPW, int NT>
__device__ __forceinline__ void k_moe_down_body(BankArgs bank, const int32_t* __restrict__ ids,
                                                       const float* __restrict__ part_gu, float* __restrict__ part_d,
                                                       int nparts, int ngu) {
  constexpr int G = Tile<F16>::kGroups;
  constexpr int V = G * 8;              // entries of h this tile consumes
  constexpr int S = NT / V;             // threads cooperating on one entry's tile sums
  __shared__ __attribute__((aligned(16))) typename Tile<F16>::entry_t lut[kLutBytes / sizeof(typename Tile<F16>::entry_t)];
  __shared__ float vs[256];
  __shared__ float hg[S][V], hu[S][V];
  __shared__ float red[NT / 64];
  const int H = bank.H, I = bank.I;
  const int groups = I / 8;
  const int nt = (int)cdiv(groups, G);
  const int nt_in = ngu;   // gate/up partial sums per row
  const int p = blockIdx.x % nparts;
  const int tile = (blockIdx.x / nparts) % nt;
  const int slot = blockIdx.x / (nparts * nt);
  const int e = ids[slot];
  if (e < 0 || e >= bank.E) return;  // gate/up kernel records the status
  const int i = threadIdx.x;
  const int k0 = tile * V;
  const uint8_t* codes = bank.codes + (int64_t)e * bank.stride + 2 * packed_bytes(I, H);
  const float* cb = bank.cb + ((int64_t)e * 3 + 2) * kCodebookFloats;
  const int nrb = (int)cdiv(H, kSlabRows);
  const int nt16 = (int)cdiv(groups, kSlabGroups);
  const int per = (int)cdiv(nrb, nparts);
  const int rb0 = p * per;
  const int rb1 = rb0 + per < nrb ? rb0 + per : nrb;
  const int64_t Ip = pad_rows(I);
  // Loads the tables need (codebook entry, gate/up tile sums for h) are issued before the code
  // prefetch, since waits on the memory counter are in issue order.  Thread (ei, q) sums tiles
  // q, q+S, ... of entry ei; up to kHold tiles per thread are loaded at once (clamped addresses,
  // masked values, so the loads are unconditional).
  constexpr int kHold = 16;
  float cv[3][8];
  load_codebook_entry<F16>(cb, cv);
  const int ei = i % V, q = i / V;
  const bool live = k0 + ei < I;
  const float* pg = part_gu + ((int64_t)slot * 2 + 0) * nt_in * Ip + (live ? k0 + ei : 0);
  const float* pu = part_gu + ((int64_t)slot * 2 + 1) * nt_in * Ip + (live ? k0 + ei : 0);
  float gv[kHold], uv[kHold];
#pragma unroll
  for (int j = 0; j < kHold; ++j) {
    const int t = q + j * S;
    const int tt = t < nt_in ? t : nt_in - 1;
    gv[j] = pg[tt * Ip];
    uv[j] = pu[tt * Ip];
  }
  RowStream<F16, BPW> rs;
  rs.begin(codes, nrb, nt16, tile, rb0, rb1);
  float gs = 0.f, us = 0.f;
#pragma unroll
  for (int j = 0; j < kHold; ++j) {
    const bool in = q + j * S < nt_in;
    gs += in ? gv[j] : 0.f;
    us += in ? uv[j] : 0.f;
  }
  for (int t = q + kHold * S; t < nt_in; t += S) {  // only when H > 8 * G * S * kHold
    gs += pg[t * Ip];
    us += pu[t * Ip];
  }
  hg[q][ei] = live ? gs : 0.f;
  hu[q][ei] = live ? us : 0.f;
  __syncthreads();
  float v = 0.f;
  if (i < V) {
    float g = hg[0][i], u = hu[0][i];
#pragma unroll
    for (int qq = 1; qq < S; ++qq) {
      g += hg[qq][i];
      u += hu[qq][i];
    }
    if (k0 + i < I) v = g / (1.f + expf(-g)) * u;
    vs[i] = v;
  }
  __syncthreads();
  const float out_scale = tile_tables<F16>(lut, cv, vs, v, red);
  rs.run(lut, out_scale, part_d + ((int64_t)slot * nt + tile) * pad_rows(H));
}

// The down kernel runs one 16-wave workgroup per CU (256 workgroups = 16 experts x 16 tiles), so
// each (expert, tile) rebuilds its slice of h once.
constexpr int kDownThreads = 1024;
template <int BPW>
__global__ __launch_bounds__(kDownThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_moe_down_f32(
    BankArgs bank, const int32_t* __restrict__ ids, const float* __restrict__ part_gu, float* __restrict__ part_d,
    int nparts, int ngu) {
  k_moe_down_body<false, BPW, kDownThreads>(bank, ids, part_gu, part_d, nparts, ngu);
}
template <int BPW>
__global__ __launch_bounds__(kDownThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_moe_down_f16(
    BankArgs bank, const int32_t* __restrict__ ids, const float* __restrict__ part_gu, float* __restrict__ part_d,
    int nparts, int ngu) {
  k_moe_down_body<true, BPW, kDownThreads>(bank, ids, part_gu, part_d, nparts, ngu);
}

// Gated combine.  Workgroup = 64 rows x 16 waves; wave q sums slots q, q+16, ... over their
// `nt` partials (issued 8 at a time, so a slot costs few memory round trips), then wave 0 adds the
// 16 per-wave sums to the residual in a fixed order.
constexpr int kCombineWaves = 16;
__global__ __launch_bounds__(64 * kCombineWaves) void k_moe_combine(const float* __restrict__ part_d, int nt, int H,
                                                                    const int32_t* __restrict__ ids,
                                                                    const float* __restrict__ gates, int k, int E,
                                                                    const float* residual, float* y) {
  const int64_t Hp = pad_rows(H);
  __shared__ float red[kCombineWaves][64];
  // batched decode: token blockIdx.y owns slots [k t, k t + k) and rows t of residual and y
  const int tok = blockIdx.y;
  part_d += (int64_t)tok * k * nt * Hp;
  ids += tok * k;
  gates += tok * k;
  if (residual) residual += (int64_t)tok * H;
  y += (int64_t)tok * H;
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int r = blockIdx.x * 64 + lane;
  // every load is issued before the first use: the residual, and per slot the id, the gate and the
  // partial sums (their addresses do not depend on the id; an invalid id only drops the sum)
  const float res = (q == 0 && r < H && residual) ? residual[r] : 0.f;
  float acc = 0.f;
  if (r < H) {
    for (int slot = q; slot < k; slot += kCombineWaves) {
      const int e = ids[slot];
      const float g = gates[slot];
      const float* pd = part_d + (int64_t)slot * nt * Hp + r;
      float s = 0.f;
      for (int t = 0; t < nt; t += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = t + u < nt ? pd[(int64_t)(t + u) * Hp] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      if (e >= 0 && e < E) acc = fmaf(g, s, acc);
    }
  }
  red[q][lane] = acc;
  __syncthreads();
  if (q == 0 && r < H) {
    float o = res;
#pragma unroll
    for (int w = 0; w < kCombineWaves; ++w) o += red[w][lane];
    y[r] = o;
  }
}

static int down_parts(int H) {
  (void)H;
  return 1;
}

MoeWorkspace moe_workspace_layout(int H, int I, int k, bool f16) {
  const int G = f16 ? Tile<true>::kGroups : Tile<false>::kGroups;
  MoeWorkspace w;
  w.nt_in = (int)cdiv(H / 8, G);
  w.nt_out = (int)cdiv(I / 8, G);
  w.status_off = 0;
  w.part_gu_off = 256;
  // sized for 16-group K-tiles, the most partials any form of the kernels writes
  const size_t gu = (size_t)k * 2 * cdiv(H / 8, kSlabGroups) * pad_rows(I) * sizeof(float);
  w.part_d_off = w.part_gu_off + ((gu + 255) / 256) * 256;
  const size_t d = (size_t)k * cdiv(I / 8, kSlabGroups) * pad_rows(H) * sizeof(float);
  w.norm_off = w.part_d_off + ((d + 255) / 256) * 256;
  w.total = w.norm_off + ((H * sizeof(float) + 255) / 256) * 256;
  return w;
}

// Sums the gate/up partials of each (slot, matrix) row into partial 0, in ascending partial order
// (the order the down kernel's prologue adds them in), so that down reads one partial per row.  In
// place: each element is read and written by one thread.  part_gu: [P][2][stride][Ip].
__global__ __launch_bounds__(256) void k_sum_gu_partials(float* __restrict__ part_gu, int ngu, int stride, int64_t Ip) {
  constexpr int U = 32;   // partials in flight per thread
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Ip) return;
  float* p = part_gu + (int64_t)blockIdx.y * stride * Ip + i;
  float s = 0.f;
  for (int p0 = 0; p0 < ngu; p0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p0 + u < ngu ? p[(int64_t)(p0 + u) * Ip] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (p0 + u < ngu) s += v[u];
  }
  p[0] = s;
}

// T tokens of decode (T = 1 for the single-token entry points).  Pair p = t k + i (token t's i-th
// expert) is one "slot" of the kernels, which read x, residual and y at row p / k; the K-tile chunk
// sizes are chosen from one token's counts, so every pair sums the same K-tiles in the same order as
// in a single-token call (down's row split may differ with the pair count; it changes no sum).
// Shapes without both wave-specialised forms run the tokens one after another.
// status_hdr: where the status and wait-limit words are (the workspace header when null).
static hipError_t decode_tokens(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                                const float* x, int T, const int32_t* ids, const float* gates, int k,
                                const float* residual, float* y, bool f16, void* ws, hipStream_t stream, hipEvent_t* ev,
                                const Route* route, int32_t* status_hdr = nullptr) {
  const int P = T * k;
  const MoeWorkspace w = moe_workspace_layout(H, I, P, f16);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* status = status_hdr ? status_hdr : reinterpret_cast<int32_t*>(base + w.status_off);
  float* part_gu = reinterpret_cast<float*>(base + w.part_gu_off);
  float* part_d = reinterpret_cast<float*>(base + w.part_d_off);
  BankArgs bank{codes, cb, stride, E, H, I};
  const int nparts = down_parts(H);
  hipError_t err = hipSuccess;
  auto mark = [&](int i) {
    if (ev && err == hipSuccess) err = hipEventRecord(ev[i], stream);
  };
  mark(0);
  // The wave-specialised kernels: gate/up needs I in (1984, 2048] and whole
  // 16-group K-tiles; down needs I a multiple of 128 and H a multiple of 28 row blocks (more than
  // kPipeMaxGu gate/up partials are summed into one first).  Each sums `c` K-tiles per workgroup,
  // c chosen to fill the CUs in as few rounds as possible (ties: the larger c, i.e. fewer partials).
  const int ncu = compute_units();
  auto pick_chunk = [&](int ntiles, long per_chunk_groups) {
    int best_c = 0;
    long best = 0;
    for (int c = 1; c <= kPipeMaxItems; ++c) {
      if (ntiles % c != 0) continue;
      const long grid = per_chunk_groups * (ntiles / c);
      const long cost = (grid + ncu - 1) / ncu * c;
      if (best_c == 0 || cost <= best) best = cost, best_c = c;
    }
    return best_c;
  };
  // (their K-tiles are single slabs of 16 groups for either table precision)
  const int nt16_in = (int)cdiv(H / 8, kSlabGroups), nt16_out = (int)cdiv(I / 8, kSlabGroups);
  const int chunk = (ncu > 0 && (H / 8) % 16 == 0 && (int)cdiv(I, kSlabRows) == kGuStreamWaves * kGuBpi)
                        ? pick_chunk(nt16_in, 2L * k)
                        : 0;
  const int ngu = chunk ? nt16_in / chunk : w.nt_in;
  // down: row chunks of kDnBpi row blocks per streamer wave, or of one when few pairs would leave
  // CUs idle (only with 1 or 2 K-tiles per workgroup).  Only the rows a workgroup takes change, never
  // the K-tiles it sums, so every result is the same either way, and the choice is made from all P
  // pairs of the call.  The work estimate is rounds x K-tiles x row blocks per wave; ties keep kDnBpi.
  const int nrb_h = (int)cdiv(H, kSlabRows);
  int dn_bpi = kDnBpi;
  int nrc = nrb_h / (kDnStreamWaves * kDnBpi);
  // more gate/up partials than the down prologue reads (few slots: gate/up took few K-tiles per
  // workgroup to fill the CUs) are first summed into one
  const bool sum_gu = chunk && ngu > kPipeMaxGu;
  const int dchunk = (chunk && I % 128 == 0 && nrb_h % (kDnStreamWaves * kDnBpi) == 0)
                   ? pick_chunk(nt16_out, (long)k * nrc)
                   : 0;
  if (dchunk && dchunk <= 2 && ncu > 0) {
    const int nrc1 = nrb_h / kDnStreamWaves;
    auto cost = [&](int rows_per_wave, int chunks) {
      const long grid = (long)P * chunks * (nt16_out / dchunk);
      return (grid + ncu - 1) / ncu * dchunk * rows_per_wave;
    };
    if (cost(1, nrc1) < cost(kDnBpi, nrc)) dn_bpi = 1, nrc = nrc1;
  }
  const int nparts_d = dchunk ? nt16_out / dchunk : w.nt_out;
  if (T > 1 && !(chunk && dchunk)) {
    for (int t = 0; t < T; ++t) {
      const hipError_t e = decode_tokens(codes, cb, stride, E, H, I, x + (int64_t)t * H, 1, ids + t * k, gates + t * k,
                                         k, residual ? residual + (int64_t)t * H : nullptr, y + (int64_t)t * H, f16, ws,
                                         stream, nullptr, nullptr, status_hdr);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // routing: the gate/up kernel takes the top-k itself when it is the wave-specialised one;
  // otherwise k_topk writes ids/gates first
  const bool fused_route = route && chunk && E <= kRouteMaxExperts;
  if (route) {
    ids = route->ids;
    gates = route->gates;
    if (!fused_route)
      hipLaunchKernelGGL(k_topk, dim3(1), dim3(1024), 0, stream, route->logits, E, k, route->ids, route->gates);
  }
  const int bpw_gu = pick_bpw((int)cdiv(I, kSlabRows), 1, kGateUpThreads / 64);
  const int bpw_d = pick_bpw((int)cdiv(H, kSlabRows), nparts, kDownThreads / 64);
  if (chunk) {
    const dim3 grid((unsigned)(P * 2 * ngu));
    const PipeArgs pa{x,       nullptr, part_gu, ngu, 1, 0, fused_route ? route->logits : nullptr,
                      route ? route->ids : nullptr, route ? route->gates : nullptr, k, 0};
    switch (chunk) {
#define RVQ_WS_CASE(n)                                                                                             \
  case n:                                                                                                          \
    if (f16)                                                                                                       \
      hipLaunchKernelGGL((k_table_ws<true, false, kGuStreamWaves, kGuBpi, n>), grid, dim3(64 * (kGuStreamWaves + 4)),  \
                         0, stream, bank, ids, status, pa);                                                        \
    else                                                                                                           \
      hipLaunchKernelGGL((k_table_ws<false, false, kGuStreamWaves, kGuBpi, n>), grid, dim3(64 * (kGuStreamWaves + 4)), \
                         0, stream, bank, ids, status, pa);                                                        \
    break;
      RVQ_WS_CASE(1) RVQ_WS_CASE(2) RVQ_WS_CASE(3) RVQ_WS_CASE(4)
      RVQ_WS_CASE(5) RVQ_WS_CASE(6) RVQ_WS_CASE(7) RVQ_WS_CASE(8)
#undef RVQ_WS_CASE
    }
  } else if (f16) {
    RVQ_BPW_DISPATCH(bpw_gu, hipLaunchKernelGGL((k_moe_gateup_f16<B>), dim3(k * 2 * w.nt_in), dim3(kGateUpThreads), 0,
                                                stream, bank, x, ids, part_gu, status))
  } else {
    RVQ_BPW_DISPATCH(bpw_gu, hipLaunchKernelGGL((k_moe_gateup_f32<B>), dim3(k * 2 * w.nt_in), dim3(kGateUpThreads), 0,
                                                stream, bank, x, ids, part_gu, status))
  }
  mark(1);
  if (dchunk) {
    if (sum_gu)
      hipLaunchKernelGGL(k_sum_gu_partials, dim3((unsigned)cdiv(pad_rows(I), 256), (unsigned)(P * 2)), dim3(256), 0,
                         stream, part_gu, ngu, ngu, (int64_t)pad_rows(I));
    const int nkc = nt16_out / dchunk;
    const dim3 grid((unsigned)(P * nrc * nkc));
    const PipeArgs pa{nullptr, part_gu, part_d, nkc, nrc, sum_gu ? 1 : ngu, nullptr, nullptr, nullptr, k, ngu};
    if (dn_bpi == 1) {
#define RVQ_WS_CASE1(n)                                                                                            \
  case n:                                                                                                          \
    if (f16)                                                                                                       \
      hipLaunchKernelGGL((k_table_ws<true, true, kDnStreamWaves, 1, n>), grid, dim3(64 * (kDnStreamWaves + 4)), 0,   \
                         stream, bank, ids, status, pa);                                                           \
    else                                                                                                           \
      hipLaunchKernelGGL((k_table_ws<false, true, kDnStreamWaves, 1, n>), grid, dim3(64 * (kDnStreamWaves + 4)), 0,  \
                         stream, bank, ids, status, pa);                                                           \
    break;
      switch (dchunk) { RVQ_WS_CASE1(1) RVQ_WS_CASE1(2) }
#undef RVQ_WS_CASE1
    } else {
      switch (dchunk) {
#define RVQ_WS_CASE(n)                                                                                             \
  case n:                                                                                                          \
    if (f16)                                                                                                       \
      hipLaunchKernelGGL((k_table_ws<true, true, kDnStreamWaves, kDnBpi, n>), grid, dim3(64 * (kDnStreamWaves + 4)),   \
                         0, stream, bank, ids, status, pa);                                                        \
    else                                                                                                           \
      hipLaunchKernelGGL((k_table_ws<false, true, kDnStreamWaves, kDnBpi, n>), grid, dim3(64 * (kDnStreamWaves + 4)),  \
                         0, stream, bank, ids, status, pa);                                                        \
    break;
        RVQ_WS_CASE(1) RVQ_WS_CASE(2) RVQ_WS_CASE(3) RVQ_WS_CASE(4)
        RVQ_WS_CASE(5) RVQ_WS_CASE(6) RVQ_WS_CASE(7) RVQ_WS_CASE(8)
#undef RVQ_WS_CASE
      }
    }
  } else if (f16) {
    RVQ_BPW_DISPATCH(bpw_d, hipLaunchKernelGGL((k_moe_down_f16<B>), dim3(k * w.nt_out * nparts), dim3(kDownThreads), 0,
                                               stream, bank, ids, part_gu, part_d, nparts, ngu))
  } else {
    RVQ_BPW_DISPATCH(bpw_d, hipLaunchKernelGGL((k_moe_down_f32<B>), dim3(k * w.nt_out * nparts), dim3(kDownThreads), 0,
                                               stream, bank, ids, part_gu, part_d, nparts, ngu))
  }
  mark(2);
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)cdiv(H, 64), (unsigned)T), dim3(64 * kCombineWaves), 0, stream,
                     part_d, nparts_d, H, ids, gates, k, E, residual, y);
  mark(3);
  const hipError_t last = hipGetLastError();
  return err != hipSuccess ? err : last;
}

hipError_t launch_moe_decode(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                             const float* x, const int32_t* ids, const float* gates, int k, const float* residual,
                             float* y, bool f16, void* ws, hipStream_t stream, hipEvent_t* ev, const Route* route,
                             int32_t* status_hdr) {
  return decode_tokens(codes, cb, stride, E, H, I, x, 1, ids, gates, k, residual, y, f16, ws, stream, ev, route,
                       status_hdr);
}

hipError_t launch_moe_batch_decode(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                                   const float* x, int T, const int32_t* ids, const float* gates, int k,
                                   const float* residual, float* y, bool f16, void* ws, hipStream_t stream) {
  return decode_tokens(codes, cb, stride, E, H, I, x, T, ids, gates, k, residual, y, f16, ws, stream, nullptr, nullptr);
}

}  // namespace rvq

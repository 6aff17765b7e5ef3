// Device-side building blocks of the RVQ-LUT path for gfx950 (CDNA4).
//
// Method: a weight row is a run of 8-column groups, each coded by three bytes
// (one per residual stage) into 256-entry codebooks of 8-dim vectors; y = W x is
// computed from partial-dot tables T[g][s][c] = C_s[c] . x_g, three table reads
// and two adds per (row, group), never rebuilding W.  ("WASTE Inference Engine:
// Running Kimi K3 2.78T on Consumer Hardware", section "Residual Vector
// Quantization (RVQ)"; "Running a 2.78-Trillion-Parameter Model on a Laptop:
// Inside WASTE's NVMe-Streaming Engine", section "Technical Insight".)
//
// GPU mapping (one workgroup = 256 threads = 4 wave64):
//  * A workgroup owns one K-tile (16 groups with fp32 tables, 32 with fp16) of
//    one matrix.  It builds that tile's tables in LDS: thread c computes entry c
//    of all 3*groups subtables (48 KiB either way, so 3 workgroups fit a CU).
//  * Within a tile the table index of a code byte is simply its byte position
//    b = 3*g + s inside the row's run for the tile, so the stream loop never
//    decodes (g, s): byte b of the lane's registers reads subtable b at a
//    compile-time LDS offset, and the address VGPR is just code << 2 (or << 1).
//  * Codes are streamed in the packed layout: one 16-byte load per lane, 64
//    lanes = 1 KiB contiguous per load instruction, each lane owning one row, so
//    a row's partial sum for the tile needs no cross-lane reduction.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rvq {

constexpr int kSlabGroups = 16;                               // groups per packed slab
constexpr int kSlabRows = 64;                                 // rows per packed slab (one per lane)
constexpr int kSlabBytes = 3 * kSlabGroups * kSlabRows;       // 3072
constexpr int kEntries = 256;                                 // codebook entries per stage
constexpr int kCodebookFloats = 3 * kEntries * 8;             // 6144 floats per matrix
constexpr int kLutBytes = 49152;                              // per-workgroup table tile
constexpr int kThreads = 512;                                // threads of a table-path workgroup (8 waves)
constexpr int kWaves = kThreads / 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__host__ __device__ inline int64_t packed_bytes(int64_t rows, int64_t cols) {
  return cdiv(cols / 8, kSlabGroups) * cdiv(rows, kSlabRows) * kSlabBytes;
}

// Device view of an expert bank (see rvq_expert_bank_t in rvq.h).
struct BankArgs {
  const uint8_t* codes;
  const float* cb;
  int64_t stride;
  int E, H, I;
};

// Table precision traits: fp32 tables cover 16 groups (one slab), fp16 tables 32 (two slabs).
template <bool F16> struct Tile;
template <> struct Tile<false> {
  static constexpr int kGroups = 16;
  static constexpr int kSlabs = 1;
  typedef float entry_t;
};
template <> struct Tile<true> {
  static constexpr int kGroups = 32;
  static constexpr int kSlabs = 2;
  typedef f16 entry_t;
};

// ---------------------------------------------------------------------------------------------
// Reductions over one workgroup of 4 waves (fixed order: deterministic).
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
  const int nw = blockDim.x >> 6;
  for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Power-of-two exponent e with bound * 2^-e < 2^15 (so every fp16 table entry,
// bounded by `bound` through Cauchy-Schwarz, stays far below 65504).
__device__ inline int f16_table_exponent(float bound) {
  if (!(bound > 0.f)) return 0;
  if (!(bound < 3.0e38f)) return 113;
  int k;
  (void)frexpf(bound, &k);  // bound = m * 2^k, m in [0.5, 1)  =>  bound < 2^k
  int e = k - 15;
  return e < -100 ? -100 : (e > 113 ? 113 : e);
}

// ---------------------------------------------------------------------------------------------
// Table build.  `vs` (LDS) holds this tile's activation values, 8 per group, zero past the
// matrix's last group; `cv` holds this thread's codebook entry c = threadIdx.x for the 3 stages.
// Entry (g, s, c) goes to lut[(3g + s) * 256 + c], scaled by `scale` (a power of two; 1 for fp32).
template <bool F16>
__device__ __forceinline__ void load_codebook_entry(const float* __restrict__ cb, float (&cv)[3][8]) {
  const int c = threadIdx.x & (kEntries - 1);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(cb + (s * kEntries + c) * 8);
    const f32x4 b = *reinterpret_cast<const f32x4*>(cb + (s * kEntries + c) * 8 + 4);
    cv[s][0] = a.x; cv[s][1] = a.y; cv[s][2] = a.z; cv[s][3] = a.w;
    cv[s][4] = b.x; cv[s][5] = b.y; cv[s][6] = b.z; cv[s][7] = b.w;
  }
}

// Workgroups of 256*n threads: the n thread sets build interleaved groups.
template <bool F16>
__device__ __forceinline__ void build_tile(typename Tile<F16>::entry_t* lut, const float (&cv)[3][8],
                                           const float* vs, float scale) {
  const int c = threadIdx.x & (kEntries - 1);
  const int set = threadIdx.x >> 8;
  const int nsets = blockDim.x >> 8;
#pragma unroll 4
  for (int g = set; g < Tile<F16>::kGroups; g += nsets) {
    float xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = vs[g * 8 + j];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      float t = cv[s][0] * xv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) t = fmaf(cv[s][j], xv[j], t);
      if constexpr (F16) {
        lut[(3 * g + s) * kEntries + c] = (f16)(t * scale);
      } else {
        lut[(3 * g + s) * kEntries + c] = t;
      }
    }
  }
}

// Largest squared L2 norm over this thread's three codebook entries.
__device__ __forceinline__ float codebook_norm2(const float (&cv)[3][8]) {
  float m = 0.f;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    float n = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) n = fmaf(cv[s][j], cv[s][j], n);
    m = fmaxf(m, n);
  }
  return m;
}

// Squared norm of the 8-element group that element `i` (= this thread's element) belongs to:
// the 8 elements of a group sit in 8 consecutive lanes of one wave.
__device__ __forceinline__ float group_norm2(float v) {
  float n = v * v;
  n += __shfl_xor(n, 1, 64);
  n += __shfl_xor(n, 2, 64);
  n += __shfl_xor(n, 4, 64);
  return n;
}

// ---------------------------------------------------------------------------------------------
// Stream loop: each lane owns one row of a 64-row block; per slab it loads 48 code bytes as three
// 16-byte loads and adds the 48 table entries they select.
// STRIDE: floats between consecutive subtables (256, or more when padded against bank conflicts).
template <int BASE, int STRIDE = kEntries>
__device__ __forceinline__ float gather16_f32(const float* lut, u32x4 d, float acc) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = d[w];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += lut[(BASE + 4 * w + k) * STRIDE + ((v >> (8 * k)) & 0xffu)];
  }
  return acc;
}

// fp16 tables: two entries per v_dot2_f32_f16 against (1, 1), accumulating in fp32, so a pair of
// lookups costs one conversion-free add (measured 1 % faster per decode step than converting
// and adding each entry).
template <int BASE, int STRIDE = kEntries>
__device__ __forceinline__ float gather16_f16(const f16* lut, u32x4 d, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = d[w];
#pragma unroll
    for (int k = 0; k < 4; k += 2) {
      const h2 p = {lut[(BASE + 4 * w + k) * STRIDE + ((v >> (8 * k)) & 0xffu)],
                    lut[(BASE + 4 * w + k + 1) * STRIDE + ((v >> (8 * k + 8)) & 0xffu)]};
      acc = __builtin_amdgcn_fdot2(p, one, acc, false);
    }
  }
  return acc;
}

struct SlabData {
  u32x4 d[6];
};

// Loads one row block (48 code bytes per lane, or 96 with fp16 tables) of slab base(s) s0/s1 at
// byte offset `off` (< 4 GiB; lane part included): uniform 64-bit base + 32-bit lane offset, so
// the address costs one VGPR.
template <bool F16>
__device__ __forceinline__ void load_slabs(SlabData& s, const uint8_t* __restrict__ s0, const uint8_t* __restrict__ s1,
                                           uint32_t off) {
  // codes are read exactly once per token: non-temporal loads keep them from evicting what the
  // caches do reuse (codebooks, router weights, partial sums); measured 2 % faster per step
  const u32x4* a = reinterpret_cast<const u32x4*>(s0 + off);
  s.d[0] = __builtin_nontemporal_load(a);
  s.d[1] = __builtin_nontemporal_load(a + 64);
  s.d[2] = __builtin_nontemporal_load(a + 128);
  if constexpr (F16) {
    const u32x4* b = reinterpret_cast<const u32x4*>(s1 + off);
    s.d[3] = __builtin_nontemporal_load(b);
    s.d[4] = __builtin_nontemporal_load(b + 64);
    s.d[5] = __builtin_nontemporal_load(b + 128);
  }
}

// One slab (16 groups, three 16-byte code words per lane) through tables of either precision.
template <bool F16, int STRIDE>
__device__ __forceinline__ float gather_slab1(const void* lut, const SlabData& s) {
  float acc = 0.f;
  if constexpr (F16) {
    const f16* t = static_cast<const f16*>(lut);
    acc = gather16_f16<0, STRIDE>(t, s.d[0], acc);
    acc = gather16_f16<16, STRIDE>(t, s.d[1], acc);
    acc = gather16_f16<32, STRIDE>(t, s.d[2], acc);
  } else {
    const float* t = static_cast<const float*>(lut);
    acc = gather16_f32<0, STRIDE>(t, s.d[0], acc);
    acc = gather16_f32<16, STRIDE>(t, s.d[1], acc);
    acc = gather16_f32<32, STRIDE>(t, s.d[2], acc);
  }
  return acc;
}

template <bool F16, int STRIDE = kEntries>
__device__ __forceinline__ float gather_slabs(const void* lut, const SlabData& s) {
  float acc = 0.f;
  if constexpr (F16) {
    const f16* t = static_cast<const f16*>(lut);
    acc = gather16_f16<0>(t, s.d[0], acc);
    acc = gather16_f16<16>(t, s.d[1], acc);
    acc = gather16_f16<32>(t, s.d[2], acc);
    acc = gather16_f16<48>(t, s.d[3], acc);
    acc = gather16_f16<64>(t, s.d[4], acc);
    acc = gather16_f16<80>(t, s.d[5], acc);
  } else {
    const float* t = static_cast<const float*>(lut);
    acc = gather16_f32<0, STRIDE>(t, s.d[0], acc);
    acc = gather16_f32<16, STRIDE>(t, s.d[1], acc);
    acc = gather16_f32<32, STRIDE>(t, s.d[2], acc);
  }
  return acc;
}

// Streams row blocks [rb_begin, rb_end) of K-tile `tile` of one packed matrix through the tables in
// LDS, writing out[row] = out_scale * (sum over the tile) for every row of those blocks (`out` has
// its rows padded to a multiple of 64, so stores need no guard).  Waves take row blocks
// round-robin.  Each wave keeps NB row blocks of codes in registers: the buffer just gathered is
// refilled with the block NB steps ahead before the next buffer is gathered, so NB-1 blocks are
// always in flight; buffers rotate by unrolling, never by register copies.  begin() issues the
// first loads and may be called before the tables are built, so the first HBM round trip overlaps
// the build.
//
// BPW > 0: every wave streams exactly BPW row blocks (the launcher checked this), so the loop is
// straight-line code and the compiler's memory-counter waits are exact: a gather waits only for its
// own buffer.  BPW == 0: any range, with data-dependent loads (correct, but the waits are
// conservative, which costs overlap).
template <bool F16, int BPW>
struct RowStream {
  static constexpr int kDepth = F16 ? 2 : 3;   // 12 KiB / 9 KiB of codes per wave in registers
  static constexpr int NB = (BPW > 0 && BPW < kDepth) ? BPW : kDepth;
  SlabData buf[NB];
  const uint8_t* s0;       // slab bases of this tile (uniform)
  const uint8_t* s1;
  uint32_t lane_off;       // lane * 16
  int rb, step, rb_end;    // wave-uniform

  __device__ __forceinline__ void load(int i, int b) {
    load_slabs<F16>(buf[i], s0, s1, (uint32_t)b * kSlabBytes + lane_off);
  }

  __device__ __forceinline__ void begin(const uint8_t* __restrict__ codes, int nrb, int nt16, int tile, int rb_begin,
                                        int rb_end_) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lane_off = (threadIdx.x & 63) * 16;
    step = blockDim.x >> 6;
    rb = rb_begin + wave;
    rb_end = rb_end_;
    const int slab0 = tile * Tile<F16>::kSlabs;
    // the second slab of an fp16 tile may not exist (odd slab count): its tables are all zero then,
    // so any valid code bytes do; re-read slab0 to stay in bounds.
    const int slab1 = F16 ? (slab0 + 1 < nt16 ? slab0 + 1 : slab0) : slab0;
    s0 = codes + (int64_t)slab0 * nrb * kSlabBytes;
    s1 = codes + (int64_t)slab1 * nrb * kSlabBytes;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (BPW > 0) {
        load(i, rb + i * step);
      } else {
        if (rb + i * step < rb_end) load(i, rb + i * step);
      }
    }
  }

  __device__ __forceinline__ void run(const void* lut, float out_scale, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    if constexpr (BPW > 0) {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const float acc = gather_slabs<F16>(lut, buf[j % NB]);
        if (j + NB < BPW) load(j % NB, rb + (j + NB) * step);
        out[(rb + j * step) * kSlabRows + lane] = acc * out_scale;
      }
    } else {
      if (rb >= rb_end) return;
      for (;;) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const float acc = gather_slabs<F16>(lut, buf[i]);
          const int nb = rb + NB * step;
          if (nb < rb_end) load(i, nb);
          out[rb * kSlabRows + lane] = acc * out_scale;
          rb += step;
          if (rb >= rb_end) return;
        }
      }
    }
  }
};

// Row blocks per wave that have a straight-line specialisation.
__host__ __device__ constexpr bool fixed_bpw(int b) { return b == 1 || b == 2 || b == 4 || b == 7 || b == 8 || b == 14; }

}  // namespace rvq

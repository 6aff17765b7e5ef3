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
// GPU mapping.  Two families of table kernels use the helpers below.
//  * One-K-tile kernels (the single-matrix GEMV with kThreads = 512 threads = 8 waves; the fallback
//    MoE gate/up with 256 threads and down with 1024): a workgroup owns one K-tile (16 groups with
//    fp32 tables, 32 with fp16) of one matrix and builds that tile's plain tables in LDS
//    (kLutBytes = 48 KiB either way): thread c computes entry c of the 3 x groups subtables
//    (build_tile), then its waves stream row blocks through them (RowStream).  Within a tile the table
//    index of a code byte is its byte position b = 3g + s in the row's run, so the stream loop never
//    decodes (g, s).
//  * Wave-specialised kernels (k_table_ws in kernels.hip, the decode path's gate/up and down): one
//    workgroup per CU with NSW streamer waves and 4 builder waves (12 waves for gate/up, 11 for
//    down), several K-tiles per workgroup, tables double-buffered in the skewed 64 KiB layout below
//    (128 KiB for fp32 tables, one shared 64 KiB array for fp16), built with MFMAs while the
//    streamers gather from the other buffer.
//  * Codes are streamed in the packed layout: one 16-byte load per lane, 64 lanes = 1 KiB
//    contiguous per load instruction, each lane owning one row, so a row's partial sum for a tile
//    needs no cross-lane reduction.
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
// Reductions over one workgroup (fixed order: deterministic).
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

// ---------------------------------------------------------------------------------------------
// Skewed fp32 tables (the wave-specialised kernels).  The 64 lanes of a wave (one row each) gather
// from 48 subtables of 256 entries.  Read plainly, all lanes of an instruction share one subtable,
// so the 32 lanes of an LDS pass land on random banks (three to four passes' worth of conflicts
// per instruction).  Here entry c of table column j sits at byte 256 c + 4 j, so a column lies in
// one bank (j mod 32) whatever c is.  In step i, lane l reads column (l + i) mod 32 (subtables
// 0..31) and, for i = 32 + j, column 32 + (l + j) mod 16 + 16 ((l / 16) mod 2) (subtables 32..47,
// stored twice, at columns 32..47 and 48..63): the 32 lanes of every pass read 32 distinct banks.
// A lane thus needs its row's 48 code bytes in a rotated order: the first 32 left by l mod 32, the
// last 16 by l mod 16 (a select network over the dwords, v_alignbyte within them: about one VALU
// instruction per lookup); each lookup's address is then one v_perm (code byte above the lane's
// column offset).
constexpr int kSkewCols = 64;
constexpr int kSkewWords = kSkewCols * kEntries;   // 16384 floats (64 KiB) per table

// Per lane: the column offset (4 j) of each step; per wave: which lanes rotate by 1, 2 and 4 dwords
// (first 32 bytes) and by 1 and 2 dwords (last 16), as lane masks, and the byte shifts.
struct SkewLane {
  uint32_t col[48];
  uint64_t mA1, mA2, mA4, mB1, mB2;
  uint32_t shA, shB;
  __device__ __forceinline__ void init(int lane) {
    const int la = lane & 31, lb = lane & 15, hb = (lane >> 4) & 1;
#pragma unroll
    for (int i = 0; i < 32; ++i) col[i] = 4u * (uint32_t)((la + i) & 31);
#pragma unroll
    for (int j = 0; j < 16; ++j) col[32 + j] = 4u * (uint32_t)(32 + ((lb + j) & 15) + 16 * hb);
    mA1 = __ballot((la >> 2) & 1);
    mA2 = __ballot((la >> 3) & 1);
    mA4 = __ballot((la >> 4) & 1);
    mB1 = __ballot((lb >> 2) & 1);
    mB2 = __ballot((lb >> 3) & 1);
    shA = (uint32_t)(la & 3);
    shB = (uint32_t)(lb & 3);
  }
};

// b where the lane's bit of m is set, else a: one v_cndmask (issued as written, so the rotation
// below stays one select per dword per stage).
__device__ __forceinline__ uint32_t lane_select(uint32_t a, uint32_t b, uint64_t m) {
  uint32_t d;
  asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(m));
  return d;
}

// w[0..N) rotated left by whole dwords (the stages whose masks hold this lane), then by sh bytes.
template <int N>
__device__ __forceinline__ void rotate_stage(uint32_t (&w)[N], int bit, uint64_t m) {
  uint32_t t[N];
#pragma unroll
  for (int q = 0; q < N; ++q) t[q] = lane_select(w[q], w[(q + bit) % N], m);
#pragma unroll
  for (int q = 0; q < N; ++q) w[q] = t[q];
}
template <int N>
__device__ __forceinline__ void rotate_bytes_tail(uint32_t (&w)[N], uint32_t sh) {
  uint32_t t[N];
#pragma unroll
  for (int q = 0; q < N; ++q) t[q] = __builtin_amdgcn_alignbyte(w[(q + 1) % N], w[q], sh);
#pragma unroll
  for (int q = 0; q < N; ++q) w[q] = t[q];
}

// One row block's 48 lookups through a skewed table (lut: the table's first byte; the lane's codes
// in s.d[0..2] as loaded).
// F16: the table holds fp16 entries in one half of each 32-bit word (t already points at that
// half), and two lookups are added at a time with v_dot2 against (1, 1).
template <bool F16>
__device__ __forceinline__ float gather_skew(const char* t, const SlabData& s, const SkewLane& sl) {
  uint32_t lo[8] = {s.d[0][0], s.d[0][1], s.d[0][2], s.d[0][3], s.d[1][0], s.d[1][1], s.d[1][2], s.d[1][3]};
  uint32_t hi[4] = {s.d[2][0], s.d[2][1], s.d[2][2], s.d[2][3]};
  rotate_stage<8>(lo, 1, sl.mA1);
  rotate_stage<8>(lo, 2, sl.mA2);
  rotate_stage<8>(lo, 4, sl.mA4);
  rotate_bytes_tail<8>(lo, sl.shA);
  rotate_stage<4>(hi, 1, sl.mB1);
  rotate_stage<4>(hi, 2, sl.mB2);
  rotate_bytes_tail<4>(hi, sl.shB);
  const uint32_t r[12] = {lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7], hi[0], hi[1], hi[2], hi[3]};
  // bytes: [0] = column offset, [1] = code byte i, [2], [3] = 0  ->  256 c + 4 j
  auto addr = [&](int i) {
    return __builtin_amdgcn_perm(r[i >> 2], sl.col[i], 0x0c0c0000u | ((uint32_t)(4 + (i & 3)) << 8));
  };
  float acc = 0.f;
  if constexpr (F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int i = 0; i < 48; i += 2) {
      const h2 p = {*reinterpret_cast<const _Float16*>(t + addr(i)), *reinterpret_cast<const _Float16*>(t + addr(i + 1))};
      acc = __builtin_amdgcn_fdot2(p, one, acc, false);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 48; ++i) acc += *reinterpret_cast<const float*>(t + addr(i));
  }
  return acc;
}

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

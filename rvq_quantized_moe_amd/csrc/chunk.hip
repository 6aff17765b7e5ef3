// Multi-token (chunked prefill) MoE layer on gfx950: bucket the (token, expert) pairs of a chunk by
// expert, then for every expert decode its RVQ code groups straight into MFMA operands and multiply
// them with the expert's gathered tokens (fp32 accumulation).
//
// Why MFMA here: with T tokens every decoded weight is used by all the expert's tokens (about
// T*k/E of them: 32 at 512 tokens, top-16 of 256), so the work is a dense contraction; the pages'
// chunked prefill (news.hada.io topic 32035, K3 performance section: chunked 0.47 tok/s vs 0.29
// sequential) is the same observation on a CPU.  The table path stays the decode (T = 1) path.
//
// Operand fit: v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A[l%16][8(l/16) .. 8(l/16)+7] and
// B[8(l/16) .. +7][l%16]; D[4(l/16)+i][l%16] in its 4 accumulators.  One RVQ group (8 consecutive
// input columns of one weight row) is exactly one lane's A fragment, so a lane decodes its group
// (three codebook vectors summed) into registers and issues the MFMA; no weight tile is written.
// Which K columns form an MFMA step is free as long as A and B agree: in a 16-group K-tile, step kk
// gives lane slice q group 4q + kk, so a lane's four groups are 12 consecutive code bytes of its row
// (three aligned dwords), and each codebook address is one byte-select shift of a code dword.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device.hpp"
#include "launch.hpp"

namespace rvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunkRows = 64;            // weight rows per workgroup (one packed row block)
constexpr int kChunkTok = 48;             // pairs per MFMA pass (3 blocks of 16; 2 of the 256 experts of a
                                          // 512-token top-16 chunk take a second pass)
constexpr int kChunkBlocks = kChunkTok / 16;
constexpr int kChunkK = 128;              // K columns per staged tile (16 groups = one packed slab)
constexpr int kXStride = kChunkK + 8;     // staged token row length in 16-bit elements (pad: banks)

struct ChunkWs {
  size_t status_off, offsets_off, order_off, pair_token_off, pair_pos_off, hmax_off, h_off, y_off, x16_off, h16_off, total;
};

// Workspace layout of the chunk path (all 256-byte aligned):
//   status int32 | offsets int32[E+1] | order int32[E] | pair_token int32[P] | pair_pos int32[T*k]
//   | hmax uint32[P] (bit pattern of max|h| per pair) | h fp32 [P][I] (fp16 tiles) | y fp32 [P][H]
//   | x16 fp16 [T][H] (the chunk in fp16, for fp16 tiles) | h16 16-bit [P][I] (h as the down operand)
ChunkWs chunk_ws_layout(int E, int H, int I, int T, int k) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t P = (size_t)T * k;
  ChunkWs w;
  w.status_off = 0;
  w.offsets_off = 256;
  w.order_off = w.offsets_off + up((size_t)(E + 1) * 4);
  w.pair_token_off = w.order_off + up((size_t)E * 4);
  w.pair_pos_off = w.pair_token_off + up(P * 4);
  w.hmax_off = w.pair_pos_off + up(P * 4);
  w.h_off = w.hmax_off + up(P * 4);
  w.y_off = w.h_off + up(P * (size_t)I * 4);
  w.x16_off = w.y_off + up(P * (size_t)H * 4);
  w.h16_off = w.x16_off + up((size_t)T * H * 2);
  w.total = w.h16_off + up(P * (size_t)I * 2);
  return w;
}

size_t chunk_workspace_bytes(int E, int H, int I, int T, int k) { return chunk_ws_layout(E, H, I, T, k).total; }

// ---------------------------------------------------------------------------------------------
// Bucketing (one workgroup).  Pair (t, i) = token t's i-th selected expert e.  Pairs of expert e
// are placed at offsets[e] + (number of earlier tokens that also selected e): a per-expert token
// bitmap in LDS answers that with popcounts, so the order (token ascending within an expert) and
// every position are deterministic.  It also writes the order in which the expert kernels take the
// experts: by pair count, the largest first (in steps of 4 pairs, all counts from 252 up together),
// so that the longest work items start first.  Within a step the order is that of the atomics; it
// decides only when and where a work item runs, never what it computes.
__global__ __launch_bounds__(1024) void k_chunk_bucket(const int32_t* __restrict__ ids, int T, int k, int E,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ order,
                                                       int32_t* __restrict__ pair_token,
                                                       int32_t* __restrict__ pair_pos, int32_t* __restrict__ status) {
  extern __shared__ uint32_t sm[];
  const int words = (T + 31) / 32;
  uint32_t* bitmap = sm;                       // [E][words]
  int32_t* cnt = reinterpret_cast<int32_t*>(sm + (size_t)E * words);   // [E + 1]
  const int P = T * k;
  for (int i = threadIdx.x; i < E * words; i += blockDim.x) bitmap[i] = 0u;
  for (int i = threadIdx.x; i <= E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  // each thread's pairs 8 at a time, their ids loaded together (one memory round trip per 8)
  constexpr int kBatch = 8;
  for (int p0 = threadIdx.x; p0 < P; p0 += kBatch * blockDim.x) {
    int eb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + u * blockDim.x;
      eb[u] = p < P ? ids[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + u * blockDim.x;
      if (p >= P) continue;
      const int t = p / k, e = eb[u];
      if (e < 0 || e >= E) {
        atomicExch(status, 6 /* RVQ_ERR_EXPERT_ID */);
        continue;
      }
      atomicOr(&bitmap[(size_t)e * words + t / 32], 1u << (t % 32));
    }
  }
  __syncthreads();
  // counts per expert and their exclusive prefix: thread i takes experts [i per, (i + 1) per)
  // (per <= 4: E <= 4096 and 1024 threads), a shuffle scan within each wave, the 16 wave totals
  // through LDS.  Integer sums: exact in any grouping.
  __shared__ int wsum[1024 / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (E + (int)blockDim.x - 1) / (int)blockDim.x;
  const int e0 = threadIdx.x * per;
  int c[4];
  int own = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int cc = 0;
    if (j < per && e0 + j < E)
      for (int w = 0; w < words; ++w) cc += __popc(bitmap[(size_t)(e0 + j) * words + w]);
    c[j] = cc;
    own += cc;
  }
  int incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - own;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < per && e0 + j < E) {
      cnt[e0 + j] = run;
      offsets[e0 + j] = run;
      run += c[j];
    }
  }
  if (threadIdx.x == blockDim.x - 1) {   // the last thread's running sum is the total
    cnt[E] = run;
    offsets[E] = run;
  }
  __shared__ int obase[64], ofill[64];
  if (threadIdx.x < 64) {
    obase[threadIdx.x] = 0;
    ofill[threadIdx.x] = 0;
  }
  __syncthreads();
  auto bin_of = [](int cc) { return 63 - (cc >> 2 < 63 ? cc >> 2 : 63); };
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < per && e0 + j < E) atomicAdd(&obase[bin_of(c[j])], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int b = 0; b < 64; ++b) {
      const int n = obase[b];
      obase[b] = s;
      s += n;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < per && e0 + j < E) {
      const int b = bin_of(c[j]);
      order[obase[b] + atomicAdd(&ofill[b], 1)] = e0 + j;
    }
  for (int p0 = threadIdx.x; p0 < P; p0 += kBatch * blockDim.x) {
    int eb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + u * blockDim.x;
      eb[u] = p < P ? ids[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + u * blockDim.x;
      if (p >= P) continue;
      const int t = p / k, e = eb[u];
      if (e < 0 || e >= E) {
        pair_pos[p] = -1;
        continue;
      }
      const uint32_t* row = bitmap + (size_t)e * words;
      int r = 0;
      for (int w = 0; w < t / 32; ++w) r += __popc(row[w]);
      r += __popc(row[t / 32] & ((1u << (t % 32)) - 1u));
      const int pos = cnt[e] + r;
      pair_token[pos] = t;
      pair_pos[p] = pos;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Decode of one RVQ group into an MFMA A fragment.  Codebooks are held in LDS as fp16 [3][256][8]
// (12 KiB per matrix) for either tile precision: fp16 tiles sum the three vectors with packed fp16
// adds; bf16 tiles sum them in fp32 and round once (the fp16 codebook rounding, 2^-11, is far below
// bf16's 2^-8).
constexpr int kCbBytes = 3 * 256 * 8 * 2;

__device__ inline void load_codebooks(_Float16* d, const float* __restrict__ cb) {
  for (int i = threadIdx.x; i < 3 * 256 * 8 / 4; i += blockDim.x) {
    const f32x4 v = reinterpret_cast<const f32x4*>(cb)[i];
    d[4 * i] = (_Float16)v.x;
    d[4 * i + 1] = (_Float16)v.y;
    d[4 * i + 2] = (_Float16)v.z;
    d[4 * i + 3] = (_Float16)v.w;
  }
}

// LDS accesses by absolute address: each chunk kernel's LDS is the one dynamic array chunk_lds (no
// static LDS), which therefore starts at LDS address 0 (checked at kernel entry: lds_at_zero), so an
// address is an offset into it and constant parts go into the instruction's offset field.
extern __shared__ __attribute__((aligned(16))) uint8_t chunk_lds[];
typedef __attribute__((address_space(3))) const half8 lds_half8;
__device__ __forceinline__ half8 lds_h8(uint32_t a) { return *(lds_half8*)(uintptr_t)a; }
__device__ __forceinline__ bool lds_at_zero() {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)chunk_lds == 0u;
}

// 16 * (byte b of d), b a constant: one v_lshlrev_b32 whose source is the byte (SDWA byte select), the
// byte offset of a 16-byte codebook entry.
__device__ __forceinline__ uint32_t byte_x16(uint32_t d, int b) {
  uint32_t r;
  switch (b) {
    case 0: asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(d)); break;
    case 1: asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(d)); break;
    case 2: asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(d)); break;
    default: asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(d)); break;
  }
  return r;
}

// Stage s's entry of group kk (of the four in a lane's 12 code bytes d[0..2]): byte 3kk + s.
__device__ __forceinline__ uint32_t code_off(const uint32_t (&d)[3], int kk, int st) {
  const int b = 3 * kk + st;
  return byte_x16(d[b >> 2], b & 3);
}

template <bool F16>
struct Decoder;

// The three stage vectors of a group (read from LDS) summed into the A fragment.
template <>
struct Decoder<true> {
  typedef half8 frag_t;
  __device__ static frag_t sum(half8 a, half8 b, half8 d) { return a + b + d; }
};

// bf16: ((float)a + (float)b) + (float)d per element, then one rounding to bf16.  v_fma_mix_f32
// reads fp16 halves directly (op_sel_hi marks an fp16 source, op_sel picks its half) and computes
// x * 1 + y with one rounding, which is the fp32 sum of the two (x * 1 is exact): two instructions
// per element instead of three conversions and two additions.
__device__ __forceinline__ float mix_add_lo(uint32_t x, uint32_t y) {   // lo(x) + lo(y), both fp16
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,1]" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float mix_add_hi(uint32_t x, uint32_t y) {   // hi(x) + hi(y), both fp16
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float mix_add_lo_f32(uint32_t x, float y) {   // lo(x) (fp16) + y (fp32)
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float mix_add_hi_f32(uint32_t x, float y) {   // hi(x) (fp16) + y (fp32)
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(x), "v"(y));
  return r;
}

template <>
struct Decoder<false> {
  typedef bf16x8 frag_t;
  __device__ static frag_t sum(half8 a, half8 b, half8 d) {
    const u32x4 A = __builtin_bit_cast(u32x4, a), B = __builtin_bit_cast(u32x4, b), D = __builtin_bit_cast(u32x4, d);
    frag_t f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = (__bf16)mix_add_lo_f32(D[w], mix_add_lo(A[w], B[w]));
      f[2 * w + 1] = (__bf16)mix_add_hi_f32(D[w], mix_add_hi(A[w], B[w]));
    }
    return f;
  }
};

__device__ inline f32x4 mfma16(half8 a, half8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
__device__ inline f32x4 mfma16(bf16x8 a, half8 b, f32x4 c) { return mfma16(a, __builtin_bit_cast(bf16x8, b), c); }

// ---------------------------------------------------------------------------------------------
// Expert GEMM for NMAT products of one expert that share the activations: 64-row blocks of its
// matrices (gate/up: two row blocks of gate and of up, NMAT = 4, or one of each, NMAT = 2; down: two
// row blocks, NMAT = 2, or one).  Wave w owns rows [16w, 16w+16) of every product's block.
//   acc[m][tb] (lane l, i) = sum_k W_m[row0 + 16w + 4(l/16) + i][k] * act[pair tb*16 + l%16][k]
// Per 128-column K-tile, the 16-bit activations of up to 48 pairs sit in one half of a double
// buffer in LDS.  The next K-tile's activation loads are issued into registers before this tile's
// MFMAs and written to the other half after them, so one barrier per K-tile separates the halves
// and the load latency hides behind the compute.  Codes do not pass through LDS: each lane loads
// its own 12 code bytes per matrix (three dwords) one K-tile ahead.

// Activation rows of a product, already 16-bit (the MFMA operand type): the chunk's tokens
// gathered by pair (gate/up: rowmap = pair -> token) or the pairs' h (down: rowmap = null).
struct Act16 {
  const uint16_t* src;      // [rows][K]
  const int32_t* rowmap;
  int K;
};

__device__ inline int h_exponent(uint32_t maxbits) {
  const float m = __uint_as_float(maxbits);
  if (!(m > 0.f)) return 0;
  int e;
  (void)frexpf(m, &e);  // m < 2^e
  return e - 15;        // m * 2^-(e-15) < 2^15 < 65504
}

// Register staging of one K-tile's activations: every thread holds up to 3 16-byte pieces of the
// tile (48 rows x 16 pieces): piece u covers row (tid + 256u)/16, so piece u is exactly pair block u
// (rows 16u .. 16u+15).  A pass over NTB pair blocks stages pieces u < NTB only: the MFMAs read no
// other rows.
constexpr int kActPieces = kChunkTok * (kChunkK / 8) / 256;   // 3 (256-thread workgroups)
static_assert(kActPieces == kChunkBlocks, "staging piece u is pair block u");

struct StageRegs {
  u32x4 act[kActPieces];
};

struct TokenRows {  // per pass: the source row of each of this thread's activation rows (-1: none)
  int t[kActPieces];
};

template <int NTB>
__device__ inline void stage_issue(StageRegs& s, const Act16& a, const TokenRows& tr, int k0) {
#pragma unroll
  for (int u = 0; u < NTB; ++u) {
    const int c8 = (threadIdx.x + 256 * u) % (kChunkK / 8);
    const int t = tr.t[u];
    s.act[u] = (t >= 0 && k0 + c8 * 8 < a.K) ? *reinterpret_cast<const u32x4*>(a.src + (int64_t)t * a.K + k0 + c8 * 8)
                                             : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ inline uint32_t pack_h2(float lo, float hi) {
  const _Float16 l = (_Float16)lo, h = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}
__device__ inline uint32_t pack_b2(float lo, float hi) {
  const __bf16 l = (__bf16)lo, h = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

template <int NTB>
__device__ inline void stage_store(const StageRegs& s, uint16_t* x_lds) {
#pragma unroll
  for (int u = 0; u < NTB; ++u) {
    const int q = threadIdx.x + 256 * u, j = q / (kChunkK / 8), c8 = q % (kChunkK / 8);
    *reinterpret_cast<u32x4*>(x_lds + j * kXStride + c8 * 8) = s.act[u];
  }
}

// per pass: which source row each activation row of this thread reads
__device__ inline void pass_rows(TokenRows& tr, const Act16& a, int p0, int np) {
#pragma unroll
  for (int u = 0; u < kActPieces; ++u) {
    const int j = (threadIdx.x + 256 * u) / (kChunkK / 8);
    tr.t[u] = j < np ? (a.rowmap ? a.rowmap[p0 + j] : p0 + j) : -1;
  }
}

// Dynamic LDS of the chunk kernels: NCB fp16 codebooks (NCB = 1 where the products of a step share
// one, as down's two row blocks do), then two kChunkTok x kXStride activation tiles.
template <int NCB>
struct ChunkLds {
  static constexpr int kBuf = kChunkTok * kXStride * 2;
  __device__ static _Float16* cb() { return reinterpret_cast<_Float16*>(chunk_lds); }
  __device__ static uint16_t* act(int b) { return reinterpret_cast<uint16_t*>(chunk_lds + NCB * kCbBytes + b * kBuf); }
  static constexpr uint32_t act_addr(int b) { return NCB * kCbBytes + b * kBuf; }   // the same as an LDS address
};

// The K loop of one pass over NTB 16-pair blocks.  The body is straight-line code (no branch on the
// pair count, and the next tile's loads are issued unconditionally: the last iteration re-reads the
// last tile into the idle buffer), so the compiler's memory-counter waits stay exact and the
// prefetch is never drained early.
template <bool F16, int NMAT, int NTB, int NCB>
__device__ inline void k_loop(f32x4 (&acc)[NMAT][kChunkBlocks], const uint8_t* const (&mats)[NMAT], int ntile, int nrb, int rb,
                              const Act16& act, const TokenRows& tr) {
  typedef typename Decoder<F16>::frag_t frag_t;
  typedef ChunkLds<NCB> L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int r = 16 * wave + (lane & 15);
  // the lane's 12 code bytes (12q .. 12q+11 of row r's 48-byte run: groups 4q .. 4q+3) are three
  // dwords of the row block's slab in the bank (byte b of the run at (b/16)*1024 + 16r + b%16), read
  // once, straight into registers; its B operand rows start at pair lane%16, columns 32q (of the
  // group 4q + kk at step kk)
  uint32_t coff[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int b = 12 * q + 4 * i;
    coff[i] = (uint32_t)((b >> 4) * 1024 + r * 16 + (b & 15));
  }
  // ordinary loads: each 16-byte unit of a slab is read by up to three of the wave's dword loads,
  // and with non-temporal loads the L2 fetched its line again for each (8 % more HBM reads)
  auto load_codes = [&](uint32_t (&d)[NMAT][3], int kt) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < 3; ++i)
        d[m][i] = *reinterpret_cast<const uint32_t*>(mats[m] + ((int64_t)kt * nrb + rb) * kSlabBytes + coff[i]);
  };
  uint32_t dn[NMAT][3];   // the codes of the next K-tile
  load_codes(dn, 0);
  StageRegs st;
  stage_issue<NTB>(st, act, tr, 0);
  __syncthreads();  // the previous pass is done with both buffers (and the codebooks are stored)
  stage_store<NTB>(st, L::act(0));
  __syncthreads();
  const uint32_t bo = (uint32_t)(((lane & 15) * kXStride + 32 * q) * 2);
  const uint32_t boff[2] = {L::act_addr(0) + bo, L::act_addr(1) + bo};
  for (int kt = 0; kt < ntile; ++kt) {
    const int cur = kt & 1;
    const int nxt = kt + 1 < ntile ? kt + 1 : kt;
    uint32_t d[NMAT][3];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < 3; ++i) d[m][i] = dn[m][i];
    // the next K-tile's loads: activations (written to LDS at the end of this tile, the wait for
    // them leaves the code loads issued after them in flight), then codes, held in place here:
    // left to itself the scheduler sinks them to the end of the tile, where they arrive late
    stage_issue<NTB>(st, act, tr, nxt * kChunkK);
    load_codes(dn, nxt);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t ba = cur ? boff[1] : boff[0];
    // step kk's LDS reads (three codebook vectors per matrix, one B fragment per pair block) are
    // issued before step kk - 1's sums and MFMAs, so two steps' reads are in flight at a time
    half8 E[2][NMAT][3], Bq[2][NTB];
    auto fetch = [&](int kk, half8 (&e)[NMAT][3], half8 (&bq)[NTB]) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int st = 0; st < 3; ++st)
          e[m][st] = lds_h8((uint32_t)((m * NCB / NMAT) * kCbBytes + 4096 * st) + code_off(d[m], kk, st));
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) bq[tb] = lds_h8(ba + (uint32_t)((tb * 16 * kXStride + 8 * kk) * 2));
    };
    fetch(0, E[0], Bq[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < 4) fetch(kk + 1, E[c ^ 1], Bq[c ^ 1]);
      frag_t a[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) a[m] = Decoder<F16>::sum(E[c][m][0], E[c][m][1], E[c][m][2]);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m][tb] = mfma16(a[m], Bq[c][tb], acc[m][tb]);
    }
    stage_store<NTB>(st, L::act(cur ^ 1));
    __syncthreads();
  }
}

// One workgroup = (expert, row blocks [rb0, rb1)): loads the codebooks once, then per RBS row blocks
// loops over the expert's pairs kChunkTok at a time and over K.  Matrix m's slab of step rb is at
// mats[m] + (kt * nrb + rb) * kSlabBytes: RBS = 2 with mats = {W, W + one slab} takes row blocks rb
// and rb + 1 of one matrix W as the two products of a step (they share the staged activations).
template <bool F16, int NMAT, class Epi, int RBS = 1, int NCB = NMAT>
__device__ void expert_tile_gemm(const uint8_t* const (&mats)[NMAT], const float* const (&cbs)[NMAT], int K,
                                 int rb0, int rb1, int nrb, int p_begin, int n_pairs, const Act16& act, const Epi& epi) {
  typedef ChunkLds<NCB> L;
  _Float16* cb_lds = L::cb();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  for (int m = 0; m < NCB; ++m) load_codebooks(cb_lds + m * (kCbBytes / 2), cbs[m * NMAT / NCB]);
  const int ntile = (K / 8 + 15) / 16;
  for (int rb = rb0; rb < rb1; rb += RBS)
  for (int pb = 0; pb < n_pairs; pb += kChunkTok) {
    const int np = n_pairs - pb < kChunkTok ? n_pairs - pb : kChunkTok;
    TokenRows tr;
    pass_rows(tr, act, p_begin + pb, np);
    f32x4 acc[NMAT][kChunkBlocks];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int tb = 0; tb < kChunkBlocks; ++tb) acc[m][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    static_assert(kChunkBlocks == 3, "one case per pair-block count");
    switch ((np + 15) / 16) {
      case 1: k_loop<F16, NMAT, 1, NCB>(acc, mats, ntile, nrb, rb, act, tr); break;
      case 2: k_loop<F16, NMAT, 2, NCB>(acc, mats, ntile, nrb, rb, act, tr); break;
      default: k_loop<F16, NMAT, kChunkBlocks, NCB>(acc, mats, ntile, nrb, rb, act, tr); break;
    }
    epi(acc, p_begin + pb, np, rb * kChunkRows + 16 * wave + 4 * q, lane & 15);
  }
}

// Work index of this workgroup such that consecutive work items run on the same XCD: workgroups
// are dealt to the 8 XCDs round-robin, so work item w goes to workgroup (w % per) * 8 + w / per.
// An expert's workgroups then share one L2, which serves its activation rows to all of them.
// The grid is a multiple of 8; returns -1 for padding workgroups.
__device__ inline int xcd_major(int nwork) {
  const int per = gridDim.x >> 3;
  const int w = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  return w < nwork ? w : -1;
}

// This workgroup's expert and row-block group.  When the experts split evenly over the 8 XCDs, the
// order ranks are dealt out in groups of 8, one per XCD, forwards in even groups and backwards in
// odd ones: each XCD takes its experts in rank order (the heaviest first) and the XCDs' totals
// stay close.  All ngrp groups of one expert run together on one XCD.  Otherwise the experts go in
// id order, XCD-major.  Returns false for padding workgroups.
__device__ inline bool chunk_work(const int32_t* __restrict__ order, int E, int ngrp, int& e, int& grp) {
  if ((E & 7) == 0) {
    const int li = (int)(blockIdx.x >> 3);
    if (li >= (E >> 3) * ngrp) return false;
    const int g = li / ngrp, x = (int)(blockIdx.x & 7);
    grp = li % ngrp;
    e = order[g * 8 + ((g & 1) ? 7 - x : x)];
    return true;
  }
  const int w = xcd_major(E * ngrp);
  if (w < 0) return false;
  e = w / ngrp;
  grp = w % ngrp;
  return true;
}

// Gate/up: h[p][row] = silu(g) * u.  fp16 tiles: fp32 h (k_chunk_h16 scales it per pair); bf16
// tiles: bf16(h) straight into the down operand (the same rounding k_chunk_h16 would apply).
template <bool F16, int NB>
struct GateUpEpi {   // products {gate rb .. rb+NB-1, up rb .. rb+NB-1}: h of NB consecutive row blocks
  float* h;
  uint16_t* h16;
  int I;
  __device__ void operator()(const f32x4 (&acc)[2 * NB][kChunkBlocks], int p0, int np, int rloc, int col) const {
#pragma unroll
    for (int tb = 0; tb < kChunkBlocks; ++tb) {
      const int j = tb * 16 + col;
      if (j >= np) continue;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[b][tb][i], u = acc[NB + b][tb][i];
          hv[i] = g / (1.f + expf(-g)) * u;
        }
        const int r = rloc + b * kChunkRows;
        if constexpr (F16) {
          *reinterpret_cast<f32x4*>(h + (int64_t)(p0 + j) * I + r) = f32x4{hv[0], hv[1], hv[2], hv[3]};
        } else {
          *reinterpret_cast<u32x2*>(h16 + (int64_t)(p0 + j) * I + r) = u32x2{pack_b2(hv[0], hv[1]), pack_b2(hv[2], hv[3])};
        }
      }
    }
  }
};

// Down: y[p][row] = acc * 2^e(p) (undoing the fp16 scale of h).  NB products of consecutive row
// blocks (NB = 2: a step of two row blocks of the down matrix).
template <bool F16, int NB>
struct DownEpi {
  float* y;
  const uint32_t* hmax;
  int H;
  __device__ void operator()(const f32x4 (&acc)[NB][kChunkBlocks], int p0, int np, int rloc, int col) const {
#pragma unroll
    for (int tb = 0; tb < kChunkBlocks; ++tb) {
      const int j = tb * 16 + col;
      if (j >= np) continue;
      const float sc = F16 ? ldexpf(1.f, h_exponent(hmax[p0 + j])) : 1.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[(int64_t)(p0 + j) * H + rloc + b * kChunkRows + i] = acc[b][tb][i] * sc;
    }
  }
};

// An LDS layout other than the one the kernels address absolutely cannot happen (chunk_lds is their
// only LDS); if it ever did, the kernel reports it instead of computing.
__device__ inline bool chunk_lds_ok(int32_t* status) {
  if (lds_at_zero()) return true;
  if (threadIdx.x == 0) atomicExch(status, 8 /* RVQ_ERR_DEVICE_STALL: outputs invalid */);
  return false;
}

// PAIR: two row blocks of gate and up per step, four products sharing each B fragment (an even
// number of row blocks, groups of rpw even).
template <bool F16, bool PAIR>
__global__ __launch_bounds__(256) void k_chunk_gateup(BankArgs bank, const uint16_t* __restrict__ x16,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ order,
                                                      const int32_t* __restrict__ pair_token, float* __restrict__ h,
                                                      uint16_t* __restrict__ h16, int rpw, int32_t* __restrict__ status) {
  if (!chunk_lds_ok(status)) return;
  const int H = bank.H, I = bank.I;
  const int nrb = I / kChunkRows, ngrp = (nrb + rpw - 1) / rpw;
  int e, grp;
  if (!chunk_work(order, bank.E, ngrp, e, grp)) return;
  const int rb0 = grp * rpw;
  const int rb1 = rb0 + rpw < nrb ? rb0 + rpw : nrb;
  const int p_begin = offsets[e], n_pairs = offsets[e + 1] - p_begin;
  if (n_pairs == 0) return;
  const uint8_t* gate = bank.codes + (int64_t)e * bank.stride;
  const uint8_t* up = gate + packed_bytes(I, H);
  const float* gcb = bank.cb + ((int64_t)e * 3 + 0) * kCodebookFloats;
  const float* ucb = bank.cb + ((int64_t)e * 3 + 1) * kCodebookFloats;
  const Act16 act{x16, pair_token, H};
  if constexpr (PAIR) {
    const uint8_t* const mats[4] = {gate, gate + kSlabBytes, up, up + kSlabBytes};
    const float* const cbs[4] = {gcb, gcb, ucb, ucb};
    GateUpEpi<F16, 2> epi{h, h16, I};
    expert_tile_gemm<F16, 4, GateUpEpi<F16, 2>, 2, 2>(mats, cbs, H, rb0, rb1, nrb, p_begin, n_pairs, act, epi);
  } else {
    const uint8_t* const mats[2] = {gate, up};
    const float* const cbs[2] = {gcb, ucb};
    GateUpEpi<F16, 1> epi{h, h16, I};
    expert_tile_gemm<F16, 2>(mats, cbs, H, rb0, rb1, nrb, p_begin, n_pairs, act, epi);
  }
}

// PAIR: two row blocks per step (an even number of row blocks, groups of rpw even).
template <bool F16, bool PAIR>
__global__ __launch_bounds__(256) void k_chunk_down(BankArgs bank, const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ order,
                                                    const uint16_t* __restrict__ h16, const uint32_t* __restrict__ hmax,
                                                    float* __restrict__ y, int rpw, int32_t* __restrict__ status) {
  if (!chunk_lds_ok(status)) return;
  const int H = bank.H, I = bank.I;
  const int nrb = H / kChunkRows, ngrp = (nrb + rpw - 1) / rpw;
  int e, grp;
  if (!chunk_work(order, bank.E, ngrp, e, grp)) return;
  const int rb0 = grp * rpw;
  const int rb1 = rb0 + rpw < nrb ? rb0 + rpw : nrb;
  const int p_begin = offsets[e], n_pairs = offsets[e + 1] - p_begin;
  if (n_pairs == 0) return;
  const uint8_t* down = bank.codes + (int64_t)e * bank.stride + 2 * packed_bytes(I, H);
  const float* cb = bank.cb + ((int64_t)e * 3 + 2) * kCodebookFloats;
  const Act16 act{h16, nullptr, I};
  if constexpr (PAIR) {
    const uint8_t* const mats[2] = {down, down + kSlabBytes};
    const float* const cbs[2] = {cb, cb};
    DownEpi<F16, 2> epi{y, hmax, H};
    expert_tile_gemm<F16, 2, DownEpi<F16, 2>, 2, 1>(mats, cbs, I, rb0, rb1, nrb, p_begin, n_pairs, act, epi);
  } else {
    const uint8_t* const mats[1] = {down};
    const float* const cbs[1] = {cb};
    DownEpi<F16, 1> epi{y, hmax, H};
    expert_tile_gemm<F16, 1>(mats, cbs, I, rb0, rb1, nrb, p_begin, n_pairs, act, epi);
  }
}

// fp16 copy of the chunk's bf16 tokens, for fp16 tiles (exact for |x| inside the fp16 range): done
// once here instead of in every workgroup that stages the tokens.  8 elements per thread.
__global__ __launch_bounds__(256) void k_chunk_x16(const uint16_t* __restrict__ x, int64_t n8,
                                                   uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4 v = *reinterpret_cast<const u32x4*>(x + 8 * i);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) w[r] = pack_h2(__uint_as_float(w[r] << 16), __uint_as_float(w[r] & 0xffff0000u));
  *reinterpret_cast<u32x4*>(out + 8 * i) = u32x4{w[0], w[1], w[2], w[3]};
}

// h as the fp16 tiles' down operand, one workgroup per pair: fp16(h * 2^-e(p)), e(p) from the pair's
// max |h| (so no entry overflows; the down epilogue multiplies by 2^e(p)), written to hmax for it.
// 8 elements per thread and step (I is a multiple of 64).  (bf16 tiles take bf16(h) from the gate/up
// epilogue directly.)
__global__ __launch_bounds__(256) void k_chunk_h16(const float* __restrict__ h, uint32_t* __restrict__ hmax, int I,
                                                   uint16_t* __restrict__ out) {
  const int64_t p = blockIdx.x;
  const float* hp = h + p * I;
  uint16_t* op = out + p * I;
  __shared__ float red[4];
  float m = 0.f;
  for (int c = threadIdx.x * 8; c < I; c += 256 * 8) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(hp + c);
    const f32x4 b = *reinterpret_cast<const f32x4*>(hp + c + 4);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
    m = fmaxf(m, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (threadIdx.x == 0) hmax[p] = __float_as_uint(m);
  const float f = ldexpf(1.f, -h_exponent(__float_as_uint(m)));
  for (int c = threadIdx.x * 8; c < I; c += 256 * 8) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(hp + c);
    const f32x4 b = *reinterpret_cast<const f32x4*>(hp + c + 4);
    *reinterpret_cast<u32x4*>(op + c) =
        u32x4{pack_h2(a.x * f, a.y * f), pack_h2(a.z * f, a.w * f), pack_h2(b.x * f, b.y * f), pack_h2(b.z * f, b.w * f)};
  }
}

// out[t][r] = residual[t][r] + sum_i gates[t][i] * y[pair_pos[t][i]][r]   (fixed order in i)
__global__ __launch_bounds__(256) void k_chunk_combine(const float* __restrict__ y, const int32_t* __restrict__ pair_pos,
                                                       const float* __restrict__ gates, int k, int H,
                                                       const float* residual, float* out) {
  const int t = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= H) return;
  float acc = residual ? residual[(int64_t)t * H + r] : 0.f;
  // eight pairs' loads issued together (a dropped pair reads row 0, which exists, and is then
  // skipped), the sums still added in slot order
  for (int i0 = 0; i0 < k; i0 += 8) {
    int p[8];
    float g[8], v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      p[u] = i0 + u < k ? pair_pos[t * k + i0 + u] : -1;
      g[u] = i0 + u < k ? gates[t * k + i0 + u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = y[(int64_t)(p[u] < 0 ? 0 : p[u]) * H + r];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = p[u] < 0 ? acc : fmaf(g[u], v[u], acc);
  }
  out[(int64_t)t * H + r] = acc;
}

static size_t chunk_smem(bool f16, int ncb) {   // ncb codebooks in LDS
  (void)f16;
  return ncb * kCbBytes + 2 * ((size_t)kChunkTok * kXStride * 2);
}

hipError_t launch_moe_chunk(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                            const uint16_t* x, int T, const int32_t* ids, const float* gates, int k,
                            const float* residual, float* y, bool f16, void* ws, hipStream_t stream) {
  const ChunkWs w = chunk_ws_layout(E, H, I, T, k);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* status = reinterpret_cast<int32_t*>(base + w.status_off);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + w.offsets_off);
  int32_t* order = reinterpret_cast<int32_t*>(base + w.order_off);
  int32_t* pair_token = reinterpret_cast<int32_t*>(base + w.pair_token_off);
  int32_t* pair_pos = reinterpret_cast<int32_t*>(base + w.pair_pos_off);
  uint32_t* hmax = reinterpret_cast<uint32_t*>(base + w.hmax_off);
  float* h = reinterpret_cast<float*>(base + w.h_off);
  float* ybuf = reinterpret_cast<float*>(base + w.y_off);
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base + w.x16_off);
  uint16_t* h16 = reinterpret_cast<uint16_t*>(base + w.h16_off);
  BankArgs bank{codes, cb, stride, E, H, I};
  const size_t bucket_smem = ((size_t)E * ((T + 31) / 32) + E + 1) * 4;
  {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_chunk_bucket),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bucket_smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_chunk_bucket, dim3(1), dim3(1024), bucket_smem, stream, ids, T, k, E, offsets, order,
                     pair_token, pair_pos, status);
  // the gate/up operand: the tokens themselves (bf16 tiles) or their fp16 copy
  const int64_t nx8 = (int64_t)T * H / 8;
  if (f16) hipLaunchKernelGGL(k_chunk_x16, dim3((unsigned)cdiv(nx8, 256)), dim3(256), 0, stream, x, nx8, x16);
  const uint16_t* xg = f16 ? x16 : x;
  // row blocks per workgroup: the codebooks are loaded once per workgroup
  constexpr int rpw_gu = 2, rpw_dn = 4;
  static_assert(rpw_gu % 2 == 0 && rpw_dn % 2 == 0, "paired steps need an even number of row blocks per group");
  const unsigned g_gu = (unsigned)(cdiv(E * cdiv(I / kChunkRows, rpw_gu), 8) * 8);
  const unsigned g_dn = (unsigned)(cdiv(E * cdiv(H / kChunkRows, rpw_dn), 8) * 8);
  // down takes two row blocks per step when their number is even (rpw_dn is even, so every group
  // then is too); gate+up, and down in pairs, hold two codebooks next to the double-buffered token
  // tile: the attribute allows that allocation whatever the default limit
  const bool pair_dn = (H / kChunkRows) % 2 == 0, pair_gu = (I / kChunkRows) % 2 == 0;
  for (const void* f : {reinterpret_cast<const void*>(k_chunk_gateup<false, false>),
                        reinterpret_cast<const void*>(k_chunk_gateup<true, false>),
                        reinterpret_cast<const void*>(k_chunk_gateup<false, true>),
                        reinterpret_cast<const void*>(k_chunk_gateup<true, true>),
                        reinterpret_cast<const void*>(k_chunk_down<false, true>),
                        reinterpret_cast<const void*>(k_chunk_down<true, true>)}) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)chunk_smem(f16, 2));
    if (e != hipSuccess) return e;
  }
  const int64_t P = (int64_t)T * k;
  if (f16) {
    if (pair_gu)
      hipLaunchKernelGGL((k_chunk_gateup<true, true>), dim3(g_gu), dim3(256), chunk_smem(true, 2), stream, bank, xg,
                         offsets, order, pair_token, h, h16, rpw_gu, status);
    else
      hipLaunchKernelGGL((k_chunk_gateup<true, false>), dim3(g_gu), dim3(256), chunk_smem(true, 2), stream, bank, xg,
                         offsets, order, pair_token, h, h16, rpw_gu, status);
    hipLaunchKernelGGL(k_chunk_h16, dim3((unsigned)P), dim3(256), 0, stream, h, hmax, I, h16);
    if (pair_dn)
      hipLaunchKernelGGL((k_chunk_down<true, true>), dim3(g_dn), dim3(256), chunk_smem(true, 1), stream, bank, offsets, order,
                         h16, hmax, ybuf, rpw_dn, status);
    else
      hipLaunchKernelGGL((k_chunk_down<true, false>), dim3(g_dn), dim3(256), chunk_smem(true, 1), stream, bank, offsets, order,
                         h16, hmax, ybuf, rpw_dn, status);
  } else {
    if (pair_gu)
      hipLaunchKernelGGL((k_chunk_gateup<false, true>), dim3(g_gu), dim3(256), chunk_smem(false, 2), stream, bank, xg,
                         offsets, order, pair_token, h, h16, rpw_gu, status);
    else
      hipLaunchKernelGGL((k_chunk_gateup<false, false>), dim3(g_gu), dim3(256), chunk_smem(false, 2), stream, bank, xg,
                         offsets, order, pair_token, h, h16, rpw_gu, status);
    if (pair_dn)
      hipLaunchKernelGGL((k_chunk_down<false, true>), dim3(g_dn), dim3(256), chunk_smem(false, 1), stream, bank,
                         offsets, order, h16, hmax, ybuf, rpw_dn, status);
    else
      hipLaunchKernelGGL((k_chunk_down<false, false>), dim3(g_dn), dim3(256), chunk_smem(false, 1), stream, bank,
                         offsets, order, h16, hmax, ybuf, rpw_dn, status);
  }
  hipLaunchKernelGGL(k_chunk_combine, dim3((unsigned)cdiv(H, 256), (unsigned)T), dim3(256), 0, stream, ybuf, pair_pos,
                     gates, k, H, residual, y);
  return hipGetLastError();
}

}  // namespace rvq

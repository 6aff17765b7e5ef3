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
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device.hpp"
#include "launch.hpp"

namespace rvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kChunkRows = 64;            // weight rows per workgroup (one packed row block)
constexpr int kChunkTok = 64;             // tokens per MFMA pass (4 blocks of 16)
constexpr int kChunkK = 128;              // K columns per staged tile (16 groups = one packed slab)
constexpr int kXStride = kChunkK + 8;     // staged token row length in 16-bit elements (pad: banks)

struct ChunkWs {
  size_t status_off, offsets_off, pair_token_off, pair_pos_off, hmax_off, h_off, y_off, total;
};

// Workspace layout of the chunk path (all 256-byte aligned):
//   status int32 | offsets int32[E+1] | pair_token int32[P] | pair_pos int32[T*k]
//   | hmax uint32[P] (bit pattern of max|h| per pair) | h fp32 [P][I] | y fp32 [P][H]
ChunkWs chunk_ws_layout(int E, int H, int I, int T, int k) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t P = (size_t)T * k;
  ChunkWs w;
  w.status_off = 0;
  w.offsets_off = 256;
  w.pair_token_off = w.offsets_off + up((size_t)(E + 1) * 4);
  w.pair_pos_off = w.pair_token_off + up(P * 4);
  w.hmax_off = w.pair_pos_off + up(P * 4);
  w.h_off = w.hmax_off + up(P * 4);
  w.y_off = w.h_off + up(P * (size_t)I * 4);
  w.total = w.y_off + up(P * (size_t)H * 4);
  return w;
}

size_t chunk_workspace_bytes(int E, int H, int I, int T, int k) { return chunk_ws_layout(E, H, I, T, k).total; }

// ---------------------------------------------------------------------------------------------
// Bucketing (one workgroup).  Pair (t, i) = token t's i-th selected expert e.  Pairs of expert e
// are placed at offsets[e] + (number of earlier tokens that also selected e): a per-expert token
// bitmap in LDS answers that with popcounts, so the order (token ascending within an expert) and
// every position are deterministic.
__global__ __launch_bounds__(1024) void k_chunk_bucket(const int32_t* __restrict__ ids, int T, int k, int E,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ pair_token,
                                                       int32_t* __restrict__ pair_pos, uint32_t* __restrict__ hmax,
                                                       int32_t* __restrict__ status) {
  extern __shared__ uint32_t sm[];
  const int words = (T + 31) / 32;
  uint32_t* bitmap = sm;                       // [E][words]
  int32_t* cnt = reinterpret_cast<int32_t*>(sm + (size_t)E * words);   // [E + 1]
  const int P = T * k;
  for (int i = threadIdx.x; i < E * words; i += blockDim.x) bitmap[i] = 0u;
  for (int i = threadIdx.x; i <= E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int t = p / k;
    const int e = ids[p];
    hmax[p] = 0u;
    if (e < 0 || e >= E) {
      atomicExch(status, 6 /* RVQ_ERR_EXPERT_ID */);
      continue;
    }
    atomicOr(&bitmap[(size_t)e * words + t / 32], 1u << (t % 32));
  }
  __syncthreads();
  // counts per expert, then an exclusive prefix (one thread: E <= 4096 additions)
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
    for (int w = 0; w < words; ++w) c += __popc(bitmap[(size_t)e * words + w]);
    cnt[e] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int c = cnt[e];
      cnt[e] = run;
      offsets[e] = run;
      run += c;
    }
    cnt[E] = run;
    offsets[E] = run;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int t = p / k;
    const int e = ids[p];
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

// ---------------------------------------------------------------------------------------------
// Decode of one RVQ group into an MFMA A fragment.  Codes of the 64-row x 16-group tile are staged
// in LDS in the packed slab order (byte b of row r's 48-byte run at (b/16)*1024 + r*16 + b%16).
template <bool F16>
struct Decoder;

// fp16 tiles: codebooks held in LDS as fp16 [3][256][8]; the group is summed with packed fp16 adds.
template <>
struct Decoder<true> {
  typedef half8 frag_t;
  static constexpr int kCbBytes = 3 * 256 * 8 * 2;
  __device__ static void load_codebooks(uint8_t* dst, const float* __restrict__ cb) {
    _Float16* d = reinterpret_cast<_Float16*>(dst);
    for (int i = threadIdx.x; i < 3 * 256 * 8; i += blockDim.x) d[i] = (_Float16)cb[i];
  }
  __device__ static frag_t decode(const uint8_t* cbs, int c0, int c1, int c2) {
    const half8* t = reinterpret_cast<const half8*>(cbs);
    return t[c0] + t[256 + c1] + t[512 + c2];
  }
};

// bf16 tiles: codebooks held in LDS as fp32; the group is summed in fp32 and rounded once.
template <>
struct Decoder<false> {
  typedef bf16x8 frag_t;
  static constexpr int kCbBytes = 3 * 256 * 8 * 4;
  __device__ static void load_codebooks(uint8_t* dst, const float* __restrict__ cb) {
    float* d = reinterpret_cast<float*>(dst);
    for (int i = threadIdx.x; i < 3 * 256 * 8; i += blockDim.x) d[i] = cb[i];
  }
  __device__ static frag_t decode(const uint8_t* cbs, int c0, int c1, int c2) {
    const f32x4* t = reinterpret_cast<const f32x4*>(cbs);
    const f32x4 a0 = t[2 * c0], a1 = t[2 * c0 + 1];
    const f32x4 b0 = t[2 * (256 + c1)], b1 = t[2 * (256 + c1) + 1];
    const f32x4 d0 = t[2 * (512 + c2)], d1 = t[2 * (512 + c2) + 1];
    const f32x4 s0 = a0 + b0 + d0, s1 = a1 + b1 + d1;
    frag_t f;
    f[0] = (__bf16)s0.x; f[1] = (__bf16)s0.y; f[2] = (__bf16)s0.z; f[3] = (__bf16)s0.w;
    f[4] = (__bf16)s1.x; f[5] = (__bf16)s1.y; f[6] = (__bf16)s1.z; f[7] = (__bf16)s1.w;
    return f;
  }
};

__device__ inline f32x4 mfma16(half8 a, half8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

// Stages one packed slab (64 rows x 16 groups, 3072 bytes) into LDS.
__device__ inline void stage_slab(uint8_t* dst, const uint8_t* __restrict__ src) {
  for (int i = threadIdx.x; i < kSlabBytes / 16; i += blockDim.x)
    reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
}

// The three code bytes of group g (0..15) of row r (0..63) of a staged slab.
__device__ inline void slab_codes(const uint8_t* slab, int r, int g, int& c0, int& c1, int& c2) {
  const int b = 3 * g;
  c0 = slab[(b / 16) * 1024 + r * 16 + b % 16];
  c1 = slab[((b + 1) / 16) * 1024 + r * 16 + (b + 1) % 16];
  c2 = slab[((b + 2) / 16) * 1024 + r * 16 + (b + 2) % 16];
}

// ---------------------------------------------------------------------------------------------
// Expert GEMM for one 64-row block of NMAT matrices of one expert (NMAT = 2: gate and up, which
// share the activations; NMAT = 1: down).  Activations for the expert's pairs are staged per
// 128-column K-tile as 16-bit rows; wave w owns rows [16w, 16w+16) of every matrix.
//   acc[m][tb] (lane l, i) = sum_k W_m[row0 + 16w + 4(l/16) + i][k] * act[pair tb*16 + l%16][k]
template <bool F16, int NMAT>
struct ExpertTile {
  typedef typename Decoder<F16>::frag_t frag_t;
  f32x4 acc[NMAT][4];
};

// Activation source for the gate/up product: bf16 token rows of the chunk, gathered by pair.
struct ActTokens {
  const uint16_t* x;      // bf16 [T][K]
  const int32_t* pair_token;
  int K;
};
// Activation source for the down product: fp32 h rows [P][K] (per pair), scaled by 2^-e for fp16.
struct ActH {
  const float* h;
  const uint32_t* hmax;
  int K;
};

__device__ inline int h_exponent(uint32_t maxbits) {
  const float m = __uint_as_float(maxbits);
  if (!(m > 0.f)) return 0;
  int e;
  (void)frexpf(m, &e);  // m < 2^e
  return e - 15;        // m * 2^-(e-15) < 2^15 < 65504
}

template <bool F16>
__device__ inline void stage_act(uint16_t* xs, const ActTokens& a, int p0, int np, int k0) {
  // 64 token rows x 128 columns; thread q copies 8 columns (16 bytes) at a time.
  for (int q = threadIdx.x; q < kChunkTok * (kChunkK / 8); q += blockDim.x) {
    const int j = q / (kChunkK / 8), c8 = q % (kChunkK / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < np && k0 + c8 * 8 < a.K) {
      const int t = a.pair_token[p0 + j];
      v = *reinterpret_cast<const u32x4*>(a.x + (int64_t)t * a.K + k0 + c8 * 8);
      if constexpr (F16) {
        // bf16 -> fp16 (exact for |x| below the fp16 range)
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float lo = __uint_as_float(w[r] << 16), hi = __uint_as_float(w[r] & 0xffff0000u);
          const _Float16 hl = (_Float16)lo, hh = (_Float16)hi;
          w[r] = (uint32_t)__builtin_bit_cast(uint16_t, hl) | ((uint32_t)__builtin_bit_cast(uint16_t, hh) << 16);
        }
        v = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
    *reinterpret_cast<u32x4*>(xs + j * kXStride + c8 * 8) = v;
  }
}

template <bool F16>
__device__ inline void stage_act(uint16_t* xs, const ActH& a, int p0, int np, int k0) {
  for (int q = threadIdx.x; q < kChunkTok * (kChunkK / 8); q += blockDim.x) {
    const int j = q / (kChunkK / 8), c8 = q % (kChunkK / 8);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (j < np && k0 + c8 * 8 < a.K) {
      const float* src = a.h + (int64_t)(p0 + j) * a.K + k0 + c8 * 8;
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(src + 4);
      const float v[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      if constexpr (F16) {
        const float sc = ldexpf(1.f, -h_exponent(a.hmax[p0 + j]));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const _Float16 lo = (_Float16)(v[2 * r] * sc), hi = (_Float16)(v[2 * r + 1] * sc);
          w[r] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const __bf16 lo = (__bf16)v[2 * r], hi = (__bf16)v[2 * r + 1];
          w[r] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
      }
    }
    *reinterpret_cast<u32x4*>(xs + j * kXStride + c8 * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// One workgroup = (expert, 64-row block); loops over the expert's pairs 64 at a time and over K.
template <bool F16, int NMAT, class Act, class Epi>
__device__ void expert_tile_gemm(const uint8_t* const (&mats)[NMAT], const float* const (&cbs)[NMAT], int K,
                                 int rb, int nrb, int p_begin, int n_pairs, const Act& act, const Epi& epi,
                                 uint8_t* smem) {
  typedef typename Decoder<F16>::frag_t frag_t;
  constexpr int CB = Decoder<F16>::kCbBytes;
  uint8_t* cb_lds = smem;                                         // NMAT codebooks
  uint8_t* code_lds = smem + NMAT * CB;                           // NMAT slabs
  uint16_t* x_lds = reinterpret_cast<uint16_t*>(code_lds + NMAT * kSlabBytes);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int m = 0; m < NMAT; ++m) Decoder<F16>::load_codebooks(cb_lds + m * CB, cbs[m]);
  const int ntile = (K / 8 + 15) / 16;
  for (int pb = 0; pb < n_pairs; pb += kChunkTok) {
    const int np = n_pairs - pb < kChunkTok ? n_pairs - pb : kChunkTok;
    f32x4 acc[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[m][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < ntile; ++kt) {
      __syncthreads();  // previous tile's LDS contents are consumed
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        stage_slab(code_lds + m * kSlabBytes, mats[m] + ((int64_t)kt * nrb + rb) * kSlabBytes);
      stage_act<F16>(x_lds, act, p_begin + pb, np, kt * kChunkK);
      __syncthreads();
      const int r = 16 * wave + (lane & 15);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int g = 4 * kk + (lane >> 4);
        frag_t a[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          int c0, c1, c2;
          slab_codes(code_lds + m * kSlabBytes, r, g, c0, c1, c2);
          a[m] = Decoder<F16>::decode(cb_lds + m * CB, c0, c1, c2);
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          if (tb * 16 < np) {
            const frag_t b =
                *reinterpret_cast<const frag_t*>(x_lds + (tb * 16 + (lane & 15)) * kXStride + 32 * kk + 8 * (lane >> 4));
#pragma unroll
            for (int m = 0; m < NMAT; ++m) acc[m][tb] = mfma16(a[m], b, acc[m][tb]);
          }
        }
      }
    }
    epi(acc, p_begin + pb, np, 16 * wave + 4 * (lane >> 4), lane & 15);
  }
}

// Gate/up: h[p][row] = silu(g) * u (fp32), and the per-pair max |h| (fp16 tiles scale h by it).
template <bool F16>
struct GateUpEpi {
  float* h;
  uint32_t* hmax;
  int I, row0;
  __device__ void operator()(const f32x4 (&acc)[2][4], int p0, int np, int rloc, int col) const {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int j = tb * 16 + col;
      if (j >= np) continue;
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[0][tb][i], u = acc[1][tb][i];
        const float hv = g / (1.f + expf(-g)) * u;
        h[(int64_t)(p0 + j) * I + row0 + rloc + i] = hv;
        m = fmaxf(m, fabsf(hv));
      }
      if constexpr (F16) atomicMax(&hmax[p0 + j], __float_as_uint(m));
    }
  }
};

// Down: y[p][row] = acc * 2^e(p) (undoing the fp16 scale of h).
template <bool F16>
struct DownEpi {
  float* y;
  const uint32_t* hmax;
  int H, row0;
  __device__ void operator()(const f32x4 (&acc)[1][4], int p0, int np, int rloc, int col) const {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int j = tb * 16 + col;
      if (j >= np) continue;
      const float sc = F16 ? ldexpf(1.f, h_exponent(hmax[p0 + j])) : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[(int64_t)(p0 + j) * H + row0 + rloc + i] = acc[0][tb][i] * sc;
    }
  }
};

template <bool F16>
__global__ __launch_bounds__(256) void k_chunk_gateup(BankArgs bank, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ pair_token, float* __restrict__ h,
                                                      uint32_t* __restrict__ hmax) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_gu[];
  const int H = bank.H, I = bank.I;
  const int nrb = I / kChunkRows;
  const int e = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int p_begin = offsets[e], n_pairs = offsets[e + 1] - p_begin;
  if (n_pairs == 0) return;
  const uint8_t* rec = bank.codes + (int64_t)e * bank.stride;
  const uint8_t* const mats[2] = {rec, rec + packed_bytes(I, H)};
  const float* const cbs[2] = {bank.cb + ((int64_t)e * 3 + 0) * kCodebookFloats,
                               bank.cb + ((int64_t)e * 3 + 1) * kCodebookFloats};
  ActTokens act{x, pair_token, H};
  GateUpEpi<F16> epi{h, hmax, I, rb * kChunkRows};
  expert_tile_gemm<F16, 2>(mats, cbs, H, rb, nrb, p_begin, n_pairs, act, epi, smem_gu);
}

template <bool F16>
__global__ __launch_bounds__(256) void k_chunk_down(BankArgs bank, const int32_t* __restrict__ offsets,
                                                    const float* __restrict__ h, const uint32_t* __restrict__ hmax,
                                                    float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_dn[];
  const int H = bank.H, I = bank.I;
  const int nrb = H / kChunkRows;
  const int e = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int p_begin = offsets[e], n_pairs = offsets[e + 1] - p_begin;
  if (n_pairs == 0) return;
  const uint8_t* rec = bank.codes + (int64_t)e * bank.stride;
  const uint8_t* const mats[1] = {rec + 2 * packed_bytes(I, H)};
  const float* const cbs[1] = {bank.cb + ((int64_t)e * 3 + 2) * kCodebookFloats};
  ActH act{h, hmax, I};
  DownEpi<F16> epi{y, hmax, H, rb * kChunkRows};
  expert_tile_gemm<F16, 1>(mats, cbs, I, rb, nrb, p_begin, n_pairs, act, epi, smem_dn);
}

// out[t][r] = residual[t][r] + sum_i gates[t][i] * y[pair_pos[t][i]][r]   (fixed order in i)
__global__ __launch_bounds__(256) void k_chunk_combine(const float* __restrict__ y, const int32_t* __restrict__ pair_pos,
                                                       const float* __restrict__ gates, int k, int H,
                                                       const float* residual, float* out) {
  const int t = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= H) return;
  float acc = residual ? residual[(int64_t)t * H + r] : 0.f;
  for (int i = 0; i < k; ++i) {
    const int p = pair_pos[t * k + i];
    if (p < 0) continue;
    acc = fmaf(gates[t * k + i], y[(int64_t)p * H + r], acc);
  }
  out[(int64_t)t * H + r] = acc;
}

static size_t chunk_smem(bool f16, int nmat) {
  const size_t cb = f16 ? Decoder<true>::kCbBytes : Decoder<false>::kCbBytes;
  return nmat * cb + nmat * kSlabBytes + (size_t)kChunkTok * kXStride * 2;
}

hipError_t launch_moe_chunk(const uint8_t* codes, const float* cb, int64_t stride, int E, int H, int I,
                            const uint16_t* x, int T, const int32_t* ids, const float* gates, int k,
                            const float* residual, float* y, bool f16, void* ws, hipStream_t stream) {
  const ChunkWs w = chunk_ws_layout(E, H, I, T, k);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* status = reinterpret_cast<int32_t*>(base + w.status_off);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + w.offsets_off);
  int32_t* pair_token = reinterpret_cast<int32_t*>(base + w.pair_token_off);
  int32_t* pair_pos = reinterpret_cast<int32_t*>(base + w.pair_pos_off);
  uint32_t* hmax = reinterpret_cast<uint32_t*>(base + w.hmax_off);
  float* h = reinterpret_cast<float*>(base + w.h_off);
  float* ybuf = reinterpret_cast<float*>(base + w.y_off);
  BankArgs bank{codes, cb, stride, E, H, I};
  const size_t bucket_smem = ((size_t)E * ((T + 31) / 32) + E + 1) * 4;
  hipLaunchKernelGGL(k_chunk_bucket, dim3(1), dim3(1024), bucket_smem, stream, ids, T, k, E, offsets, pair_token,
                     pair_pos, hmax, status);
  const unsigned g_gu = (unsigned)(E * (I / kChunkRows)), g_dn = (unsigned)(E * (H / kChunkRows));
  // bf16 tiles keep fp32 codebooks in LDS (over 64 KiB for gate+up): allow the larger allocation
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_chunk_gateup<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)chunk_smem(false, 2));
  if (f16) {
    hipLaunchKernelGGL(k_chunk_gateup<true>, dim3(g_gu), dim3(256), chunk_smem(true, 2), stream, bank, x, offsets,
                       pair_token, h, hmax);
    hipLaunchKernelGGL(k_chunk_down<true>, dim3(g_dn), dim3(256), chunk_smem(true, 1), stream, bank, offsets, h, hmax,
                       ybuf);
  } else {
    hipLaunchKernelGGL(k_chunk_gateup<false>, dim3(g_gu), dim3(256), chunk_smem(false, 2), stream, bank, x, offsets,
                       pair_token, h, hmax);
    hipLaunchKernelGGL(k_chunk_down<false>, dim3(g_dn), dim3(256), chunk_smem(false, 1), stream, bank, offsets, h,
                       hmax, ybuf);
  }
  hipLaunchKernelGGL(k_chunk_combine, dim3((unsigned)cdiv(H, 256), (unsigned)T), dim3(256), 0, stream, ybuf, pair_pos,
                     gates, k, H, residual, y);
  return hipGetLastError();
}

}  // namespace rvq

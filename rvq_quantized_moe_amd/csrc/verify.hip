// Expert-record check: the CRC-32 of every expert record's code payload, at HBM speed.
//
// news.hada.io topic 32035, disk-streaming architecture section: the engine checks each record's
// magic, expert id and offset range on every read, and a crc32 of the record payload on request
// (codebooks carry no checksum).  Here the bank is resident in HBM and the check is one pass over
// it: rvq_bank_crc32 returns, per expert, the CRC-32 of IEEE 802.3 (preset all ones, bits least
// significant first, final complement) of its 3 packed code matrices.
//
// The CRC is linear over GF(2), so it is computed in pieces and recombined exactly:
//  * lane j of a wave takes span j (1 KiB) of a 64 KiB block and runs the table-driven remainder
//    over it from a zero register (four 256-entry tables in LDS, one 32-bit word per step);
//  * a remainder r followed by n more bytes becomes r * x^(8n) mod P, so the wave multiplies each
//    lane's remainder by x^(8 * bytes after its span) and XORs them: the block's remainder;
//  * a second kernel does the same over a record's blocks, then applies the preset register
//    (all ones, carried through the whole payload: 0xFFFFFFFF * x^(8 L)) and the final complement.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rvq.h"
#include "device.hpp"
#include "launch.hpp"

namespace rvq {

constexpr uint32_t kCrcPoly = 0xEDB88320u;   // generator x^32 + ... + 1, bit-reversed, x^32 implied
constexpr int kCrcSpan = 1024;               // bytes per lane
constexpr int kCrcSpansPerBlock = 64;        // one wave per block
constexpr uint32_t kGfOne = 0x80000000u;     // x^0: bit 31 holds the coefficient of x^0

// Polynomials mod P in the bit-reversed register: bit 31 - i holds the coefficient of x^i.
__host__ __device__ inline uint32_t gf_mul_x(uint32_t a) { return (a & 1u) ? (a >> 1) ^ kCrcPoly : a >> 1; }

__host__ __device__ inline uint32_t gf_mul(uint32_t a, uint32_t b) {
  uint32_t r = 0;
  for (int i = 0; i < 32; ++i) {   // r += a_i * (b x^i)
    if (a & (kGfOne >> i)) r ^= b;
    b = gf_mul_x(b);
  }
  return r;
}

struct CrcConsts {
  uint32_t span_shift[kCrcSpansPerBlock];   // x^(8 * kCrcSpan * j)
  uint32_t pow2[32];                        // x^(8 * kCrcSpan * 2^k)
};

// x^(8 * kCrcSpan * m) from the powers of two of m.
__device__ inline uint32_t shift_spans(int64_t m, const uint32_t (&pow2)[32]) {
  uint32_t r = kGfOne;
  for (int k = 0; m != 0; ++k, m >>= 1)
    if (m & 1) r = gf_mul(r, pow2[k]);
  return r;
}

__device__ inline uint32_t wave_xor(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

// One wave per 64 KiB block of one record: blk[e * nblocks + b] = zero-preset remainder of block b.
__global__ __launch_bounds__(256) void k_crc_blocks(const uint8_t* __restrict__ codes, int64_t stride, int64_t nspans,
                                                    int nblocks, int E, uint32_t* __restrict__ blk, CrcConsts cc) {
  __shared__ uint32_t tab[4][256];
  {
    // tab[0][n]: register after byte n from zero (8 steps of x); tab[k][n]: tab[k-1][n] followed by
    // one zero byte
    const int n = threadIdx.x;
    uint32_t r = (uint32_t)n;
#pragma unroll
    for (int b = 0; b < 8; ++b) r = gf_mul_x(r);
    tab[0][n] = r;
  }
  __syncthreads();
  {
    const int n = threadIdx.x;
    uint32_t r = tab[0][n];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      r = tab[0][r & 0xffu] ^ (r >> 8);
      tab[k][n] = r;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)E * nblocks) return;   // (no barrier follows)
  const int e = (int)(w / nblocks), b = (int)(w % nblocks);
  const int64_t s0 = (int64_t)b * kCrcSpansPerBlock;
  const int nsp = (int)(nspans - s0 < kCrcSpansPerBlock ? nspans - s0 : kCrcSpansPerBlock);
  uint32_t r = 0;
  if (lane < nsp) {
    // each lane walks its own span, so one load instruction touches 64 lines, each 16 bytes of it:
    // ordinary (cached) loads keep the line for the lane's next 7 loads (non-temporal loads here
    // measured 2.1x slower, the line fetched again for every piece)
    const u32x4* p = reinterpret_cast<const u32x4*>(codes + (int64_t)e * stride + (s0 + lane) * kCrcSpan);
    for (int t = 0; t < kCrcSpan / 16; t += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[t + u];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          r ^= v[u][q];   // four bytes, least significant first
          r = tab[3][r & 0xffu] ^ tab[2][(r >> 8) & 0xffu] ^ tab[1][(r >> 16) & 0xffu] ^ tab[0][r >> 24];
        }
    }
    r = gf_mul(r, cc.span_shift[nsp - 1 - lane]);
  }
  r = wave_xor(r);
  if (lane == 0) blk[w] = r;
}

// One wave per record: fold its blocks, then the preset register and the final complement.  With a
// status word the CRC is not stored but compared with `expect`: a mismatch stores the record-error
// code and `tag` into status[0..1].
__global__ __launch_bounds__(64) void k_crc_finish(const uint32_t* __restrict__ blk, int64_t nspans, int nblocks,
                                                   uint32_t* __restrict__ crc, CrcConsts cc, uint32_t expect,
                                                   int32_t tag, int32_t* __restrict__ status) {
  const int e = blockIdx.x, lane = threadIdx.x;
  uint32_t acc = 0;
  for (int b = lane; b < nblocks; b += 64) {
    const int64_t end = (int64_t)(b + 1) * kCrcSpansPerBlock;
    const int64_t after = nspans - (end < nspans ? end : nspans);
    acc ^= gf_mul(blk[(int64_t)e * nblocks + b], shift_spans(after, cc.pow2));
  }
  acc = wave_xor(acc);
  if (lane == 0) {
    const uint32_t c = ~(acc ^ gf_mul(0xFFFFFFFFu, shift_spans(nspans, cc.pow2)));
    if (!status) {
      crc[e] = c;
    } else if (c != expect) {
      status[0] = RVQ_ERR_RECORD;
      status[1] = tag;
    }
  }
}

static CrcConsts crc_consts() {
  CrcConsts c;
  uint32_t span = kGfOne;   // x^(8 * kCrcSpan)
  for (int i = 0; i < 8 * kCrcSpan; ++i) span = gf_mul_x(span);
  c.span_shift[0] = kGfOne;
  for (int j = 1; j < kCrcSpansPerBlock; ++j) c.span_shift[j] = gf_mul(c.span_shift[j - 1], span);
  c.pow2[0] = span;
  for (int k = 1; k < 32; ++k) c.pow2[k] = gf_mul(c.pow2[k - 1], c.pow2[k - 1]);
  return c;
}

int64_t crc_payload_bytes(int H, int I) { return 2 * (int64_t)packed_bytes(I, H) + (int64_t)packed_bytes(H, I); }

size_t crc_workspace_bytes(int E, int H, int I) {
  const int64_t nblocks = cdiv(crc_payload_bytes(H, I) / kCrcSpan, kCrcSpansPerBlock);
  return (size_t)((E * nblocks * 4 + 255) / 256 * 256);
}

static hipError_t crc_records(const uint8_t* codes, int64_t stride, int E, int H, int I, uint32_t* crc, void* ws,
                              uint32_t expect, int32_t tag, int32_t* status, hipStream_t stream) {
  static const CrcConsts cc = crc_consts();
  const int64_t payload = crc_payload_bytes(H, I);   // a multiple of the 3072-byte slab, so of kCrcSpan
  const int64_t nspans = payload / kCrcSpan;
  const int nblocks = (int)cdiv(nspans, kCrcSpansPerBlock);
  uint32_t* blk = static_cast<uint32_t*>(ws);
  const int64_t waves = (int64_t)E * nblocks;
  hipLaunchKernelGGL(k_crc_blocks, dim3((unsigned)cdiv(waves, 4)), dim3(256), 0, stream, codes, stride, nspans, nblocks,
                     E, blk, cc);
  hipLaunchKernelGGL(k_crc_finish, dim3((unsigned)E), dim3(64), 0, stream, blk, nspans, nblocks, crc, cc, expect, tag,
                     status);
  return hipGetLastError();
}

hipError_t launch_bank_crc32(const uint8_t* codes, int64_t stride, int E, int H, int I, uint32_t* crc, void* ws,
                             hipStream_t stream) {
  return crc_records(codes, stride, E, H, I, crc, ws, 0, 0, nullptr, stream);
}

hipError_t launch_record_crc_check(const uint8_t* codes, int H, int I, uint32_t expect, int32_t tag, int32_t* status,
                                   void* ws, hipStream_t stream) {
  return crc_records(codes, 0, 1, H, I, nullptr, ws, expect, tag, status, stream);
}

}  // namespace rvq

// Expert pool: an LRU set of HBM slots over experts held in pinned host memory (extern "C" entry
// points of include/rvq.h, "Expert pool" section).
//
// The pages' engine keeps only the trunk resident and streams each token's experts from NVMe into
// an LRU cache held at one token's working set, overlapping the reads with compute and prefetching
// the experts that the next layer's router, run early on the current residual, predicts
// ("Running a 2.78-Trillion-Parameter Model on a Laptop", Technical Insight; news.hada.io topic
// 32035, read-ahead and router-prediction section).  Here host DRAM plays the NVMe role and HBM the
// RAM cache: records are copied host-to-device by the DMA engines on streams of the pool's own (one
// for the copies an acquire needs, one for look-ahead copies, so that a demand copy never queues
// behind a prefetch), and the caller's compute stream waits only for the copies it needs.
//
// Ordering without host synchronisation:
//  * every acquire records an event on the compute stream before returning slots; the kernels of
//    earlier acquires were enqueued before it, so once the copy stream has waited for it, any slot
//    that the current acquire does not hand out may be overwritten;
//  * a slot handed out by the latest acquire may still be read by kernels in flight, so neither a
//    later prefetch nor anything but the next acquire (after its own event) evicts it;
//  * a slot's copy records an event on its copy stream; the compute stream waits for it once, the
//    first time the slot is handed out after the copy, and the slot's next copy (on either copy
//    stream) waits for it too.
//
// Record stores: the host store may instead hold self-describing expert records (header, codebooks,
// codes in one 4 KiB-aligned block, as the pages' container does); each record's header is then
// checked on the host before any copy from it, and with verify on, the CRC-32 of each slot's codes
// is compared on the device with the header's.  The checks run on streams of the pool's own (one
// per copy stream, so that a demand copy's check never waits behind a look-ahead copy), and the copy
// engine goes on to the next copy meanwhile; the slot's `loaded` event is then recorded after its
// check.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/rvq.h"
#include "device.hpp"
#include "launch.hpp"

struct rvq_expert_pool {
  const uint8_t* host_codes = nullptr;
  const float* host_cb = nullptr;
  int64_t stride = 0, payload = 0;       // host record stride; code bytes per expert
  int64_t slot_stride = 0;               // bytes between slot records in dev_codes
  const uint8_t* host_records = nullptr; // record store (else host_codes / host_cb)
  int32_t layer = 0;
  bool verify = false;
  uint8_t* verify_ws = nullptr;          // status words, then the CRC workspace of each check stream
  hipStream_t check[2] = {nullptr, nullptr};   // payload checks after demand / look-ahead copies
  hipEvent_t copied[2] = {nullptr, nullptr};   // end of the latest copy on each copy stream
  int E = 0, H = 0, I = 0, S = 0;
  uint8_t* dev_codes = nullptr;
  float* dev_cb = nullptr;
  hipStream_t copy = nullptr;            // copies an acquire needs
  hipStream_t ahead = nullptr;           // look-ahead copies (never queued in front of the former)
  hipEvent_t compute_mark = nullptr;     // recorded on the compute stream at each acquire
  std::vector<int> slot_of;              // [E] slot holding the expert, or -1
  std::vector<int> expert_in;            // [S] expert held, or -1
  std::vector<int64_t> last_use;         // [S] index of the acquire that last handed the slot out
  std::vector<int64_t> stamp;            // [S] recency (larger = more recent)
  std::vector<hipEvent_t> loaded;        // [S] end of the slot's latest copy
  std::vector<char> unwaited;            // [S] the compute stream has not yet waited for that copy
  int64_t acquires = 0, clock = 0;
  int64_t hits = 0, misses = 0, prefetches = 0, bytes = 0;
  bool mark_waited[2] = {false, false};  // each copy stream already waits for this acquire's mark
};

namespace {

constexpr int64_t kCbBytes = 3 * (int64_t)rvq::kCodebookFloats * sizeof(float);   // one expert's codebooks
constexpr int64_t kRecordAlign = 4096;
constexpr int64_t kHeaderPage = 4096;                   // header + zero fill
constexpr int64_t kRecordCodesOffset = kHeaderPage + kCbBytes;

// Verify workspace: [0, 256) two int32 status words; then, per check stream, the CRC block partials
// of one record.
int64_t crc_region_bytes(int H, int I) { return (int64_t)rvq::crc_workspace_bytes(1, H, I); }
int64_t verify_ws_bytes(int H, int I) { return 256 + 2 * crc_region_bytes(H, I); }

const rvq_record_header_t* header_of(const rvq_expert_pool& p, int e) {
  return reinterpret_cast<const rvq_record_header_t*>(p.host_records + (int64_t)e * p.stride);
}

// The read-time check of the record holding expert e (record stores only).
bool record_ok(const rvq_expert_pool& p, int e) {
  return !p.host_records ||
         rvq_record_check(p.host_records + (int64_t)e * p.stride, p.stride, p.layer, e, p.H, p.I) == RVQ_OK;
}

// Least recently stamped slot that the latest acquire has not handed out (empty slots first); -1 if
// every slot is in use by it.
int pick_victim(const rvq_expert_pool& p, int64_t busy_acquire) {
  int best = -1;
  for (int s = 0; s < p.S; ++s) {
    if (p.last_use[s] == busy_acquire) continue;
    if (p.expert_in[s] < 0) return s;
    if (best < 0 || p.stamp[s] < p.stamp[best]) best = s;
  }
  return best;
}

// Copies expert e into slot s (after the latest compute mark) on the demand stream, or on the
// look-ahead stream (lookahead).
hipError_t load_slot(rvq_expert_pool& p, int s, int e, bool lookahead) {
  hipError_t err = hipSuccess;
  hipStream_t st = lookahead ? p.ahead : p.copy;
  if (!p.mark_waited[lookahead]) {
    err = hipStreamWaitEvent(st, p.compute_mark, 0);
    if (err != hipSuccess) return err;
    p.mark_waited[lookahead] = true;
  }
  // the slot's previous copy may still be in flight on the other copy stream
  err = hipStreamWaitEvent(st, p.loaded[s], 0);
  if (err != hipSuccess) return err;
  if (p.expert_in[s] >= 0) p.slot_of[p.expert_in[s]] = -1;
  p.expert_in[s] = e;
  p.slot_of[e] = s;
  const uint8_t* src_codes = p.host_codes + (int64_t)e * p.stride;
  const uint8_t* src_cb = reinterpret_cast<const uint8_t*>(p.host_cb) + (int64_t)e * kCbBytes;
  uint32_t crc = 0;
  if (p.host_records) {   // offsets from the header that record_ok accepted
    const rvq_record_header_t* h = header_of(p, e);
    src_codes = p.host_records + (int64_t)e * p.stride + h->codes_offset;
    src_cb = p.host_records + (int64_t)e * p.stride + h->codebook_offset;
    crc = h->payload_crc32;
  }
  uint8_t* dst_codes = p.dev_codes + (int64_t)s * p.slot_stride;
  err = hipMemcpyAsync(dst_codes, src_codes, p.payload, hipMemcpyHostToDevice, st);
  if (err == hipSuccess)
    err = hipMemcpyAsync(reinterpret_cast<uint8_t*>(p.dev_cb) + (int64_t)s * kCbBytes, src_cb, kCbBytes,
                         hipMemcpyHostToDevice, st);
  if (err == hipSuccess && p.verify) {   // the check, on its own stream, after this copy
    err = hipEventRecord(p.copied[lookahead], st);
    hipStream_t ck = p.check[lookahead];
    if (err == hipSuccess) err = hipStreamWaitEvent(ck, p.copied[lookahead], 0);
    if (err == hipSuccess)
      err = rvq::launch_record_crc_check(dst_codes, p.H, p.I, crc, e, reinterpret_cast<int32_t*>(p.verify_ws),
                                         p.verify_ws + 256 + lookahead * crc_region_bytes(p.H, p.I), ck);
    if (err == hipSuccess) err = hipEventRecord(p.loaded[s], ck);
  } else if (err == hipSuccess) {
    err = hipEventRecord(p.loaded[s], st);
  }
  p.unwaited[s] = 1;
  p.bytes += p.payload + kCbBytes;
  return err;
}

// Shared part of the two constructors: the fields already set on p, then the maps, streams, events
// and (verify) the cleared status words.
int finish_create(rvq_expert_pool* p, int32_t num_experts, int32_t hidden, int32_t inter, void* slot_codes,
                  float* slot_codebooks, int32_t slots, rvq_expert_pool_t** out) {
  p->E = num_experts;
  p->H = hidden;
  p->I = inter;
  p->S = slots;
  p->dev_codes = static_cast<uint8_t*>(slot_codes);
  p->dev_cb = slot_codebooks;
  p->slot_of.assign(num_experts, -1);
  p->expert_in.assign(slots, -1);
  p->last_use.assign(slots, -1);
  p->stamp.assign(slots, 0);
  p->unwaited.assign(slots, 0);
  p->loaded.assign(slots, nullptr);
  bool ok = hipStreamCreateWithFlags(&p->copy, hipStreamNonBlocking) == hipSuccess &&
            hipStreamCreateWithFlags(&p->ahead, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&p->compute_mark, hipEventDisableTiming) == hipSuccess;
  for (int s = 0; ok && s < slots; ++s) ok = hipEventCreateWithFlags(&p->loaded[s], hipEventDisableTiming) == hipSuccess;
  if (ok && p->verify)
    ok = hipStreamCreateWithFlags(&p->check[0], hipStreamNonBlocking) == hipSuccess &&
         hipStreamCreateWithFlags(&p->check[1], hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&p->copied[0], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&p->copied[1], hipEventDisableTiming) == hipSuccess;
  if (ok && p->verify) {
    const int32_t zero[2] = {RVQ_OK, -1};
    ok = hipMemcpy(p->verify_ws, zero, sizeof zero, hipMemcpyHostToDevice) == hipSuccess;
  }
  if (!ok) {
    rvq_pool_destroy(p);
    return RVQ_ERR_HIP;
  }
  *out = p;
  return RVQ_OK;
}

bool slots_aligned(const void* slot_codes, const float* slot_codebooks) {
  return (reinterpret_cast<uintptr_t>(slot_codes) & 255) == 0 && (reinterpret_cast<uintptr_t>(slot_codebooks) & 15) == 0;
}

}  // namespace

extern "C" {

size_t rvq_record_bytes(int32_t hidden, int32_t inter) {
  const size_t codes = rvq_bank_record_bytes(hidden, inter);
  if (codes == 0) return 0;
  return (size_t)((kRecordCodesOffset + (int64_t)codes + kRecordAlign - 1) / kRecordAlign * kRecordAlign);
}

int rvq_record_header_init(rvq_record_header_t* h, int32_t layer, int32_t expert, int32_t hidden, int32_t inter,
                           uint32_t payload_crc32) {
  if (!h) return RVQ_ERR_NULL;
  const size_t codes = rvq_bank_record_bytes(hidden, inter);
  if (codes == 0 || layer < 0 || expert < 0) return RVQ_ERR_SHAPE;
  memset(h, 0, sizeof *h);
  h->magic = RVQ_RECORD_MAGIC;
  h->version = RVQ_RECORD_VERSION;
  h->layer = layer;
  h->expert = expert;
  h->hidden = hidden;
  h->inter = inter;
  h->codebook_offset = kHeaderPage;
  h->codebook_bytes = kCbBytes;
  h->codes_offset = kRecordCodesOffset;
  h->codes_bytes = (int64_t)codes;
  h->payload_crc32 = payload_crc32;
  return RVQ_OK;
}

int rvq_record_check(const void* record, int64_t record_bytes, int32_t layer, int32_t expert, int32_t hidden,
                     int32_t inter) {
  if (!record) return RVQ_ERR_NULL;
  const size_t codes = rvq_bank_record_bytes(hidden, inter);
  if (codes == 0 || layer < 0 || expert < 0) return RVQ_ERR_SHAPE;
  rvq_record_header_t h;
  if (record_bytes < (int64_t)sizeof h) return RVQ_ERR_RECORD;
  memcpy(&h, record, sizeof h);
  if (h.magic != RVQ_RECORD_MAGIC || h.version != RVQ_RECORD_VERSION) return RVQ_ERR_RECORD;
  if (h.layer != layer || h.expert != expert || h.hidden != hidden || h.inter != inter) return RVQ_ERR_RECORD;
  if (h.codebook_bytes != kCbBytes || h.codes_bytes != (int64_t)codes) return RVQ_ERR_RECORD;
  // regions: past the header, 16-byte aligned, inside the record (no overflow: sizes are known and
  // positive, offsets compared before subtracting), and disjoint
  const auto inside = [&](int64_t off, int64_t n) {
    return off >= (int64_t)sizeof h && off % 16 == 0 && off <= record_bytes && n <= record_bytes - off;
  };
  if (!inside(h.codebook_offset, h.codebook_bytes) || !inside(h.codes_offset, h.codes_bytes)) return RVQ_ERR_RECORD;
  if (h.codebook_offset < h.codes_offset + h.codes_bytes && h.codes_offset < h.codebook_offset + h.codebook_bytes)
    return RVQ_ERR_RECORD;
  return RVQ_OK;
}

int rvq_pool_create(const void* host_codes, const float* host_codebooks, int64_t record_stride, int32_t num_experts,
                    int32_t hidden, int32_t inter, void* slot_codes, float* slot_codebooks, int32_t slots,
                    rvq_expert_pool_t** out) {
  if (!out) return RVQ_ERR_NULL;
  *out = nullptr;
  if (!host_codes || !host_codebooks || !slot_codes || !slot_codebooks) return RVQ_ERR_NULL;
  const size_t rec = rvq_bank_record_bytes(hidden, inter);
  if (rec == 0 || num_experts < 1 || slots < 1 || record_stride < (int64_t)rec) return RVQ_ERR_SHAPE;
  if (record_stride % 256 != 0 || !slots_aligned(slot_codes, slot_codebooks)) return RVQ_ERR_ALIGN;
  rvq_expert_pool* p = new (std::nothrow) rvq_expert_pool;
  if (!p) return RVQ_ERR_HIP;
  p->host_codes = static_cast<const uint8_t*>(host_codes);
  p->host_cb = host_codebooks;
  p->stride = record_stride;
  p->slot_stride = record_stride;
  p->payload = (int64_t)rec;
  return finish_create(p, num_experts, hidden, inter, slot_codes, slot_codebooks, slots, out);
}

size_t rvq_pool_verify_workspace_bytes(int32_t hidden, int32_t inter) {
  if (rvq_bank_record_bytes(hidden, inter) == 0) return 0;
  return (size_t)verify_ws_bytes(hidden, inter);
}

int rvq_pool_create_records(const void* host_records, int64_t record_bytes, int32_t layer, int32_t num_experts,
                            int32_t hidden, int32_t inter, void* slot_codes, float* slot_codebooks,
                            int64_t slot_stride, int32_t slots, int32_t verify, void* verify_workspace,
                            size_t verify_workspace_bytes, rvq_expert_pool_t** out) {
  if (!out) return RVQ_ERR_NULL;
  *out = nullptr;
  if (!host_records || !slot_codes || !slot_codebooks || (verify && !verify_workspace)) return RVQ_ERR_NULL;
  const size_t rec = rvq_record_bytes(hidden, inter);
  const size_t payload = rvq_bank_record_bytes(hidden, inter);
  if (rec == 0 || layer < 0 || num_experts < 1 || slots < 1 || record_bytes < (int64_t)rec ||
      slot_stride < (int64_t)payload)
    return RVQ_ERR_SHAPE;
  if (record_bytes % kRecordAlign != 0 || slot_stride % 256 != 0 || !slots_aligned(slot_codes, slot_codebooks) ||
      (verify && (reinterpret_cast<uintptr_t>(verify_workspace) & 255) != 0))
    return RVQ_ERR_ALIGN;
  if (verify && verify_workspace_bytes < rvq_pool_verify_workspace_bytes(hidden, inter)) return RVQ_ERR_WORKSPACE;
  rvq_expert_pool* p = new (std::nothrow) rvq_expert_pool;
  if (!p) return RVQ_ERR_HIP;
  p->host_records = static_cast<const uint8_t*>(host_records);
  p->stride = record_bytes;
  p->slot_stride = slot_stride;
  p->payload = (int64_t)payload;
  p->layer = layer;
  p->verify = verify != 0;
  p->verify_ws = static_cast<uint8_t*>(verify_workspace);
  return finish_create(p, num_experts, hidden, inter, slot_codes, slot_codebooks, slots, out);
}

int rvq_pool_verify_status(rvq_expert_pool_t* p, int32_t* bad_expert) {
  if (!p || !bad_expert) return RVQ_ERR_NULL;
  *bad_expert = -1;
  if (hipStreamSynchronize(p->copy) != hipSuccess || hipStreamSynchronize(p->ahead) != hipSuccess) return RVQ_ERR_HIP;
  if (!p->verify) return RVQ_OK;
  if (hipStreamSynchronize(p->check[0]) != hipSuccess || hipStreamSynchronize(p->check[1]) != hipSuccess)
    return RVQ_ERR_HIP;
  int32_t st[2];
  if (hipMemcpy(st, p->verify_ws, sizeof st, hipMemcpyDeviceToHost) != hipSuccess) return RVQ_ERR_HIP;
  if (st[0] == RVQ_OK) return RVQ_OK;
  *bad_expert = st[1];
  const int32_t zero[2] = {RVQ_OK, -1};
  if (hipMemcpy(p->verify_ws, zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return RVQ_ERR_HIP;
  return RVQ_ERR_RECORD;
}

int rvq_pool_destroy(rvq_expert_pool_t* p) {
  if (!p) return RVQ_ERR_NULL;
  int st = RVQ_OK;
  if (p->copy && hipStreamSynchronize(p->copy) != hipSuccess) st = RVQ_ERR_HIP;
  if (p->ahead && hipStreamSynchronize(p->ahead) != hipSuccess) st = RVQ_ERR_HIP;
  for (hipStream_t c : p->check)
    if (c && hipStreamSynchronize(c) != hipSuccess) st = RVQ_ERR_HIP;
  for (hipEvent_t e : p->loaded)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->copied)
    if (e) (void)hipEventDestroy(e);
  for (hipStream_t c : p->check)
    if (c) (void)hipStreamDestroy(c);
  if (p->compute_mark) (void)hipEventDestroy(p->compute_mark);
  if (p->copy) (void)hipStreamDestroy(p->copy);
  if (p->ahead) (void)hipStreamDestroy(p->ahead);
  delete p;
  return st;
}

int rvq_pool_acquire(rvq_expert_pool_t* p, const int32_t* ids, int32_t k, int32_t* slot_ids, hipStream_t stream) {
  if (!p || !ids || !slot_ids) return RVQ_ERR_NULL;
  if (k < 1 || k > p->S) return RVQ_ERR_SHAPE;
  for (int i = 0; i < k; ++i)
    if (ids[i] < 0 || ids[i] >= p->E) return RVQ_ERR_EXPERT_ID;
  for (int i = 0; i < k; ++i)   // every record this call would read, before any state changes
    if (p->slot_of[ids[i]] < 0 && !record_ok(*p, ids[i])) return RVQ_ERR_RECORD;
  const int64_t a = ++p->acquires;
  hipError_t err = hipEventRecord(p->compute_mark, stream);
  if (err != hipSuccess) return RVQ_ERR_HIP;
  p->mark_waited[0] = p->mark_waited[1] = false;
  // resident experts first, so that no eviction below can take a slot this acquire needs
  for (int i = 0; i < k; ++i) {
    const int s = p->slot_of[ids[i]];
    if (s < 0) continue;
    if (p->last_use[s] != a) ++p->hits;
    p->last_use[s] = a;
    p->stamp[s] = ++p->clock;
  }
  for (int i = 0; i < k; ++i) {
    int s = p->slot_of[ids[i]];
    if (s < 0) {
      s = pick_victim(*p, a);   // exists: at most k - 1 < S slots carry this acquire's mark
      ++p->misses;
      err = load_slot(*p, s, ids[i], false);
      if (err != hipSuccess) return RVQ_ERR_HIP;
      p->last_use[s] = a;
      p->stamp[s] = ++p->clock;
    }
    slot_ids[i] = s;
  }
  for (int i = 0; i < k; ++i) {
    const int s = slot_ids[i];
    if (p->unwaited[s]) {
      if (hipStreamWaitEvent(stream, p->loaded[s], 0) != hipSuccess) return RVQ_ERR_HIP;
      p->unwaited[s] = 0;
    }
  }
  return RVQ_OK;
}

int rvq_pool_prefetch(rvq_expert_pool_t* p, const int32_t* ids, int32_t k) {
  if (!p || !ids) return RVQ_ERR_NULL;
  if (k < 0) return RVQ_ERR_SHAPE;
  for (int i = 0; i < k; ++i) {
    const int e = ids[i];
    if (e < 0 || e >= p->E) return RVQ_ERR_EXPERT_ID;
    if (p->slot_of[e] >= 0) continue;
    if (!record_ok(*p, e)) return RVQ_ERR_RECORD;
    const int s = pick_victim(*p, p->acquires);
    if (s < 0) break;   // every slot is held by the latest acquire
    if (load_slot(*p, s, e, true) != hipSuccess) return RVQ_ERR_HIP;
    p->stamp[s] = ++p->clock;
    ++p->prefetches;
  }
  return RVQ_OK;
}

int rvq_pool_stats(const rvq_expert_pool_t* p, int64_t* hits, int64_t* misses, int64_t* prefetches,
                   int64_t* bytes_copied) {
  if (!p || !hits || !misses || !prefetches || !bytes_copied) return RVQ_ERR_NULL;
  *hits = p->hits;
  *misses = p->misses;
  *prefetches = p->prefetches;
  *bytes_copied = p->bytes;
  return RVQ_OK;
}

}  // extern "C"

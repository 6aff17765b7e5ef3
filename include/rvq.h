/* rvq.h - C ABI of librvq.so: the RVQ-LUT Mixture-of-Experts expert forward
 * on MI355X (gfx950).
 *
 * The method (from the WASTE engine pages):
 *  - Expert weights are stored with three-stage residual vector quantization:
 *    every run of 8 consecutive columns of a weight row (a "group") is coded by
 *    three bytes, one per stage, each choosing an 8-dim vector from that stage's
 *    256-entry codebook; the decoded sub-vector is the sum of the three chosen
 *    vectors.  3 bytes per 8 weights = exactly 3.00 bits per weight.
 *    ("WASTE Inference Engine: Running Kimi K3 2.78T on Consumer Hardware",
 *    section "Residual Vector Quantization (RVQ)"; news.hada.io topic 32035,
 *    quantization-and-accuracy section.)
 *  - The product W x is computed without rebuilding W: per codebook stage and
 *    per group position a table of partial dot products
 *        T[g][s][c] = C_s[c] . x[8g .. 8g+7]
 *    is built from the activation, and each row then needs, per group, three
 *    table reads and two additions.  ("Running a 2.78-Trillion-Parameter Model
 *    on a Laptop: Inside WASTE's NVMe-Streaming Engine", section "Technical
 *    Insight".)
 *  - An expert is a gate, an up and a down matrix stored next to each other
 *    (same page, same section); the router picks 16 experts per layer
 *    (news.hada.io topic 32035, read-ahead and router-prediction section).
 *
 * Conventions for every entry point:
 *  - Data pointers are DEVICE pointers unless stated otherwise; the caller
 *    owns every buffer.  The library never allocates device memory.  It does
 *    not synchronise, except rvq_check_device_status (which synchronises
 *    `stream`) and the expert pool's verify_status and destroy (which wait for
 *    the pool's own streams); the expert pool is the one object the library
 *    creates (host memory, streams and events of its own, freed by destroy).
 *  - Work is enqueued on `stream` (0 = the null stream).  The library keeps no
 *    global mutable state: calls on distinct streams with distinct workspaces
 *    may run concurrently (the expert pool is an object of the caller's).
 *  - Return value: RVQ_OK (0) or an rvq_status_t error.  Every host-visible
 *    argument is validated before anything is enqueued: a call that returns an
 *    error other than RVQ_ERR_HIP has enqueued nothing.
 *  - Descriptor structs are read during the call only.
 *  - Sizes are element counts unless named *_bytes.
 *  - Every sum is taken in a fixed order, so results repeat bit for bit on a
 *    given device.  How the table kernels split K into partial sums is chosen
 *    from the device's compute-unit count (to fill it), so a device with
 *    another count may round differently, within the stated tolerances.
 */
#ifndef RVQ_H_
#define RVQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RVQ_OK = 0,
  RVQ_ERR_NULL = 1,        /* a required pointer is NULL */
  RVQ_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  RVQ_ERR_DTYPE = 3,       /* unsupported dtype for this argument */
  RVQ_ERR_ALIGN = 4,       /* a pointer or stride violates the stated alignment */
  RVQ_ERR_WORKSPACE = 5,   /* workspace smaller than the size query returned */
  RVQ_ERR_EXPERT_ID = 6,   /* (device status) an expert id outside [0, num_experts) was seen */
  RVQ_ERR_HIP = 7,         /* a HIP runtime call failed */
  RVQ_ERR_DEVICE_STALL = 8, /* (device status) a kernel's bounded internal wait gave up; outputs invalid */
  RVQ_ERR_RECORD = 9       /* an expert record failed its header check, or its payload its CRC-32 */
} rvq_status_t;

typedef enum { RVQ_F32 = 0, RVQ_F16 = 1, RVQ_BF16 = 2 } rvq_dtype_t;

/* Human-readable name of a status code (static storage; never NULL). */
const char *rvq_status_string(int status);

/* ------------------------------------------------------------------------
 * Code layout.
 *
 * Canonical codes (what a converter produces and what the synthetic
 * generators emit): uint8 [rows][cols/8][3], stage-minor, row-major, i.e. the
 * three stage bytes of group g of row r sit at byte 3*(r*(cols/8) + g).
 *
 * Packed codes (what the kernels stream; a pure byte permutation, same 3.00
 * bits per weight):  the matrix is cut into slabs of 64 rows x 16 groups
 * (3072 bytes).  Slab (t, b) covers groups [16t, 16t+16) of rows
 * [64b, 64b+64); slabs are ordered t-major: slab index = t*ceil(rows/64) + b.
 * Inside a slab, byte 1024*j + 16*l + i (j < 3, l < 64, i < 16) is byte
 * 16*j + i of row 64b+l's 48-byte run for those 16 groups (so one 16-byte
 * load per lane, 64 lanes, reads one contiguous KiB).  Rows past `rows` and
 * groups past cols/8 are zero-filled.
 * ------------------------------------------------------------------------ */

/* Bytes of the packed form of a rows x cols matrix:
 * ceil(cols/8 / 16) * ceil(rows / 64) * 3072.  Equals 3*rows*cols/8 when rows
 * is a multiple of 64 and cols of 128.  Returns 0 for invalid sizes. */
size_t rvq_packed_bytes(int32_t rows, int32_t cols);

/* Canonical -> packed.  src: [rows][cols/8][3] uint8 (device, any alignment);
 * dst: rvq_packed_bytes(rows, cols) bytes, 16-byte aligned; src and dst must
 * not overlap.  rows >= 1, cols >= 8, cols % 8 == 0. */
int rvq_pack_codes(const uint8_t *src, int32_t rows, int32_t cols, uint8_t *dst, hipStream_t stream);

/* One RVQ matrix W [rows x cols] in packed layout with its codebooks. */
typedef struct {
  const uint8_t *codes;      /* packed codes, 16-byte aligned */
  const float *codebooks;    /* [3 stages][256 entries][8] fp32, 16-byte aligned */
  int32_t rows, cols;        /* cols % 8 == 0 */
} rvq_matrix_t;

/* ------------------------------------------------------------------------
 * Partial-dot tables (the "lookup tables per codebook and position").
 *
 * lut[g][s][c] = sum_{j<8} codebooks[s][c][j] * x[8g+j],  g < cols/8.
 * lut_dtype RVQ_F32: float lut[cols/8][3][256]; *log2_scale is set to 0.
 * lut_dtype RVQ_F16: _Float16 lut[cols/8][3][256] holding
 *   fp16_rne(lut * 2^-e) with one power-of-two exponent e for the whole table,
 *   chosen from the bound |lut| <= max_{s,c} ||C_s[c]||_2 * max_g ||x_g||_2 so
 *   that no entry overflows; e is written to *log2_scale (device int32).
 * x: fp32 [cols]; lut: 16-byte aligned, 4*cols/8*768 (F32) or 2*cols/8*768
 * (F16) bytes; log2_scale: device int32.  No workspace.
 * ------------------------------------------------------------------------ */
int rvq_lut_build(const float *x, int32_t cols, const float *codebooks, int32_t lut_dtype, void *lut,
                  int32_t *log2_scale, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Single-matrix LUT GEMV: y = W x through the table path, tables built on
 * chip per K-tile (16 groups for RVQ_F32, 32 groups for RVQ_F16 tables, each
 * F16 tile with its own power-of-two scale), W never rebuilt.
 * x: fp32 [cols]; y: fp32 [rows].  workspace: device, 256-byte aligned, at
 * least rvq_expert_gemv_workspace_bytes(rows, cols, lut_dtype) bytes; its
 * contents need no initialisation.
 * ------------------------------------------------------------------------ */
size_t rvq_expert_gemv_workspace_bytes(int32_t rows, int32_t cols, int32_t lut_dtype);
int rvq_expert_gemv(const rvq_matrix_t *W, const float *x, int32_t lut_dtype, float *y, void *workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Router: logits[t][e] = sum_h w_router[e][h] * x[t][h], accumulated in fp64
 * (bf16 x fp32 products are exact in fp64), then the k experts with the
 * largest logits in the order (logit descending, expert id ascending) and
 * gates = softmax over those k logits (= softmax over all E renormalised to
 * the selected k).  The pages fix only that 16 experts are chosen per layer
 * and that none of them is dropped (news.hada.io topic 32035, read-ahead and
 * router-prediction section; "Running a 2.78-Trillion-Parameter Model on a
 * Laptop", Technical Insight); the linear router without bias, the tie order
 * and the renormalised softmax gates are this library's reading, the
 * plainest router consistent with them.
 * w_router: bf16 [E][H]; x: [T][H] of x_dtype RVQ_F32 or RVQ_BF16;
 * ids: int32 [T][k]; gates: fp32 [T][k]; logits: double [T][E], written, and
 * required (not NULL): the selection kernel reads the logits back from it, and
 * the call takes no workspace to hold them otherwise.
 * 1 <= k <= E <= 4096, k <= 64, H >= 1, T >= 1.  No workspace.
 * ------------------------------------------------------------------------ */
int rvq_router_topk(const void *w_router_bf16, const void *x, int32_t x_dtype, int32_t T, int32_t E, int32_t H,
                    int32_t k, int32_t *ids, float *gates, double *logits, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Expert bank: E SwiGLU experts sharing (hidden H, inter I).  Record e starts
 * at codes + e*record_stride and holds, back to back, the packed gate [I x H],
 * packed up [I x H] and packed down [H x I] codes (each of
 * rvq_packed_bytes(...) bytes).  codebooks: fp32 [E][3 (gate, up, down)][3][256][8].
 * record_stride: multiple of 256, >= rvq_bank_record_bytes(H, I).
 * ------------------------------------------------------------------------ */
typedef struct {
  const uint8_t *codes;
  const float *codebooks;
  int64_t record_stride;
  int32_t num_experts, hidden, inter;
} rvq_expert_bank_t;

size_t rvq_bank_record_bytes(int32_t hidden, int32_t inter);

/* ------------------------------------------------------------------------
 * MoE layer forward for T tokens:
 *   y[t] = residual[t] + sum_{i<k} gates[t][i] * down( silu(gate x_t) * (up x_t) )
 * of expert ids[t][i], silu(z) = z / (1 + exp(-z)).
 * T == 1 (decode): table path; compute_dtype RVQ_F32 or RVQ_F16 (table
 * precision; accumulation is fp32); x_dtype RVQ_F32 (4-byte aligned).
 * 2 <= T <= 4096 (chunked prefill): each expert's tokens are gathered and
 * multiplied against its codes decoded to matrix-core operands;
 * compute_dtype RVQ_F16 or RVQ_BF16 (operand precision; accumulation fp32);
 * x_dtype RVQ_BF16 (16-byte aligned); H and I multiples of 64; and
 * num_experts * (ceil(T/32) + 1) + 1 <= 16384 (the bucketing bitmap).
 * No events may be passed for T > 1 (RVQ_ERR_SHAPE).
 * ids, gates: device [T][k] (as written by rvq_router_topk); residual: fp32
 * [T][H] or NULL; y: fp32 [T][H] (may alias residual).
 * An id outside [0, num_experts) contributes zero and sets the sticky device
 * status RVQ_ERR_EXPERT_ID in the workspace (see rvq_check_device_status).
 * workspace: 256-byte aligned, >= rvq_moe_layer_workspace_bytes(...) for
 * the same T, k and compute_dtype, and zero-filled once by
 * rvq_workspace_init before its first use: its header holds the sticky device
 * status (and, for T == 1, the wait limit below), which must start at zero;
 * the rest needs no initialisation.
 * ------------------------------------------------------------------------ */
size_t rvq_moe_layer_workspace_bytes(const rvq_expert_bank_t *bank, int32_t T, int32_t k, int32_t compute_dtype);
int rvq_moe_layer_forward(const rvq_expert_bank_t *bank, const void *x, int32_t x_dtype, int32_t T,
                          const int32_t *ids, const float *gates, int32_t k, const float *residual, float *y,
                          int32_t compute_dtype, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Same as rvq_moe_layer_forward, and records events[0..3] on `stream`
 * around its kernels: [0] before the gate/up table kernel, [1] between it
 * and the SwiGLU+down stage (with few experts, k = 1 for instance, that stage
 * first sums the gate/up partial sums in a small kernel of its own), [2]
 * before the gated combine, [3] after it, so a caller can time each stage
 * with hipEventElapsedTime.  events: host array of 4 caller-created events
 * (none NULL). */
int rvq_moe_layer_forward_timed(const rvq_expert_bank_t *bank, const void *x, int32_t x_dtype, int32_t T,
                                const int32_t *ids, const float *gates, int32_t k, const float *residual, float *y,
                                int32_t compute_dtype, void *workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t *events);

/* ------------------------------------------------------------------------
 * One routed decode step for one token: the router and top-k of
 * rvq_router_topk (T = 1, x_dtype RVQ_F32) followed by rvq_moe_layer_forward
 * (T = 1) on the selected experts, with the same results as calling the two.
 * Where the gate/up kernel can (fp32 tables, the shapes its wave-specialised
 * form takes, num_experts <= 768), each of its workgroups takes the top-k
 * itself instead of a separate selection kernel.
 * w_router: bf16 [E][H]; x: fp32 [H]; residual: fp32 [H] or NULL; y: fp32
 * [H] (may alias residual); ids: int32 [k], gates: fp32 [k], logits: fp64
 * [E]: all written.  compute_dtype: RVQ_F32 or RVQ_F16 (table precision).
 * workspace: as for rvq_moe_layer_forward with T = 1 and the same k and
 * compute_dtype.  1 <= k <= min(64, E), E <= 4096.
 * ------------------------------------------------------------------------ */
int rvq_moe_decode_routed(const rvq_expert_bank_t *bank, const void *w_router_bf16, const float *x, int32_t k,
                          const float *residual, float *y, int32_t *ids, float *gates, double *logits,
                          int32_t compute_dtype, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * rvq_moe_decode_routed without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture that may not call
 * hipMalloc, tight serving loops, harnesses that forbid allocation).  Same
 * kernels, same results bit for bit; the gate/up and down partial sums live
 * in a static array of the library, 24 MiB (25,165,824 bytes) per GPU, held
 * from the library's first use on that GPU until the process ends.  The call
 * allocates nothing: no hipMalloc, hipFree or allocating library routine.
 * Its layout must fit: the layout of rvq_moe_layer_workspace_bytes(bank, 1,
 * k, compute_dtype) (22,050,560 bytes at hidden 7168, inter 2048, k = 16) may
 * not exceed 24 MiB, else RVQ_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's array: two calls that overlap on
 * one GPU (on different streams) race and give undefined results; calls
 * ordered on one stream, or on streams ordered by events, are safe.
 * status: DEVICE int32[2] (at least 8 bytes, 256-byte aligned), zero-filled
 * by the caller before its first use: word 0 collects the sticky device
 * status as a workspace header does (read and clear it with
 * rvq_check_device_status(status, stream)), word 1 is the wait limit (0 = the
 * default; a status buffer of 256 bytes may be passed to
 * rvq_workspace_set_wait_limit).  Other arguments as for
 * rvq_moe_decode_routed.
 * ------------------------------------------------------------------------ */
int rvq_moe_decode_routed_scratch(const rvq_expert_bank_t *bank, const void *w_router_bf16, const float *x, int32_t k,
                                  const float *residual, float *y, int32_t *ids, float *gates, double *logits,
                                  int32_t compute_dtype, int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One pre-norm residual MoE block for one token (a layer of the stack):
 *   n = RMSNorm(h) (unit weight, as rvq_rmsnorm);  h_out = h + MoE(n)
 * with the router, top-k and expert forward of rvq_moe_decode_routed on n.
 * Results equal rvq_rmsnorm followed by rvq_moe_decode_routed(x = n,
 * residual = h) bit for bit: the normalisation is folded into the router
 * kernel (each of its workgroups forms the same fp64 mean square), which also
 * stores n for the expert kernels, so no separate normalisation kernel runs.
 * h, h_out: fp32 [H] (may alias); eps >= 0; other arguments and the
 * workspace as for rvq_moe_decode_routed (n lives in the workspace).
 * ------------------------------------------------------------------------ */
int rvq_moe_block_decode(const rvq_expert_bank_t *bank, const void *w_router_bf16, const float *h, int32_t k,
                         float eps, float *h_out, int32_t *ids, float *gates, double *logits, int32_t compute_dtype,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * A small batch of T decode tokens through the table (LUT) path: for every
 * token t, y[t] = [residual[t] +] sum_i gates[t][i] * expert_{ids[t][i]}(x[t]),
 * each token with its own partial-dot tables, as in rvq_moe_layer_forward
 * with T = 1.  The pages' engine decodes one token at a time ("Running a
 * 2.78-Trillion-Parameter Model on a Laptop", section "Gotcha": no batching)
 * and reports chunked prefill faster than sequential (news.hada.io topic
 * 32035, prefill figures); this entry point is the per-token side of that
 * comparison: its cost grows with T (every token streams its experts' codes),
 * while the chunk path (rvq_moe_layer_forward, T > 1) decodes each touched
 * expert once for all its tokens.  The benchmark reports the crossover.
 * All T tokens run in the same three launches (pair t*k + i is one work item
 * of the gate/up and down kernels, chunked exactly as for one token), so each
 * y[t] equals a single-token rvq_moe_layer_forward call bit for bit; shapes
 * without the wave-specialised kernels run the tokens one after another.
 * x, residual, y: fp32 [T][H] (y may alias residual); ids: int32 [T][k];
 * gates: fp32 [T][k]; 1 <= T <= 256; 1 <= k <= 64; table_dtype RVQ_F32 or
 * RVQ_F16; workspace 256-byte aligned, >= the query below, zero-filled once
 * by rvq_workspace_init.  Errors as rvq_moe_layer_forward.
 * ------------------------------------------------------------------------ */
size_t rvq_moe_batch_decode_workspace_bytes(const rvq_expert_bank_t *bank, int32_t T, int32_t k, int32_t table_dtype);
int rvq_moe_batch_decode(const rvq_expert_bank_t *bank, const float *x, int32_t T, const int32_t *ids,
                         const float *gates, int32_t k, const float *residual, float *y, int32_t table_dtype,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RVQ encoding (checkpoint conversion; the pages convert offline, news.hada.io
 * topic 32035, conversion section): codes[r][g][s] for W fp32 [rows][cols]
 * (cols % 8 == 0, 16-byte aligned, rows >= 1) against codebooks fp32
 * [3][256][8] (16-byte aligned), written in the canonical layout
 * [rows][cols/8][3] (pack with rvq_pack_codes).  Stage by stage, each 8-column
 * sub-vector takes the entry nearest in squared Euclidean distance to what the
 * earlier stages left, which is then subtracted; the distance is accumulated in
 * fp32 over the 8 dims in order with no fused operations and ties go to the
 * lower index, so the result is reproducible bit for bit.  The codebooks
 * themselves can be fitted with rvq_fit (below).
 * ------------------------------------------------------------------------ */
int rvq_encode(const float *W, int32_t rows, int32_t cols, const float *codebooks, uint8_t *codes,
               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Codebook fitting: the three stage codebooks of a matrix and its codes.
 *
 * The pages' codebooks come from their offline converter (K3's experts were
 * trained for the format; news.hada.io topic 32035, conversion section names
 * an encoder without its method).  The plainest fit of the residual form
 * ("Running a 2.78-Trillion-Parameter Model on a Laptop", Technical Insight:
 * 3 stages x 256 entries x 8 dims) is computed: residual k-means.  For stage
 * s = 0, 1, 2: the 256 centroids start at the sub-vectors init_idx[s][c] of
 * what stages < s left (stage 0: W); `iters` Lloyd iterations follow, each
 * assigning every sub-vector to its nearest centroid (exactly the decision of
 * rvq_encode: fp32 squared distance, no fused operations, ties to the lower
 * index) and replacing every centroid that has members by their mean (one
 * with none keeps its value); then every sub-vector is assigned once more,
 * that is its stage-s code, and its centroid is subtracted (fp32).  The mean
 * is an fp64 sum in a fixed order: within each run of 2048 consecutive
 * sub-vectors (row-major sub-vector index r*(cols/8) + g) over its members in
 * ascending index, then the run sums in ascending run order; divided by the
 * member count, rounded to fp32.  So the result is reproducible bit for bit,
 * and codes equal rvq_encode(W, codebooks).
 *
 * W: fp32 [rows][cols] (device, 4-byte aligned, not modified); cols % 8 == 0,
 * rows * cols / 8 <= INT32_MAX.  init_idx: HOST int32 [3][256], each in
 * [0, rows*cols/8) (random starts are the caller's: pass them in).
 * 0 <= iters <= 10000.  codebooks out: fp32 [3][256][8] (16-byte aligned);
 * codes out: uint8 [rows][cols/8][3] canonical.  workspace: device,
 * 256-byte aligned, rvq_fit_workspace_bytes(rows, cols) bytes (about 41
 * bytes per sub-vector: the residual, the current assignment, the run sums).
 * Errors: RVQ_ERR_NULL, RVQ_ERR_SHAPE (shape, iters, or an index out of
 * range), RVQ_ERR_ALIGN, RVQ_ERR_WORKSPACE, RVQ_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t rvq_fit_workspace_bytes(int32_t rows, int32_t cols);
int rvq_fit(const float *W, int32_t rows, int32_t cols, int32_t iters, const int32_t *init_idx, float *codebooks,
            uint8_t *codes, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Integrity check of a resident bank (news.hada.io topic 32035, disk-
 * streaming architecture section: each expert record's payload carries an
 * optional crc32, checked on request; codebooks carry none).
 * crc[e] (device uint32 [num_experts], 4-byte aligned) = CRC-32 of IEEE
 * 802.3 (the zlib / PNG CRC: preset all ones, bits least significant first,
 * final complement) of expert e's code payload: its gate, up and down
 * matrices in the packed layout, 2 * rvq_packed_bytes(inter, hidden) +
 * rvq_packed_bytes(hidden, inter) bytes from codes + e * record_stride.
 * One pass over the bank at HBM speed; compare against CRCs recorded when
 * the bank was written.  workspace: 256-byte aligned, >= the query below
 * (no zero-fill needed).
 * ------------------------------------------------------------------------ */
size_t rvq_bank_crc32_workspace_bytes(const rvq_expert_bank_t *bank);
int rvq_bank_crc32(const rvq_expert_bank_t *bank, uint32_t *crc, void *workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Expert records: the self-describing host form of one expert.
 *
 * The pages' container stores each expert as one 4 KiB-aligned block holding
 * gate, up and down next to each other with their RVQ codebooks and a CRC32
 * header, read with a single read call ("Running a 2.78-Trillion-Parameter
 * Model on a Laptop", Technical Insight); every read checks the record's
 * magic, expert id and offset range, so that a truncated or wrongly joined
 * bank is refused instead of answering with wrong weights, and a crc32 of the
 * payload is checked on request; codebooks carry no checksum (news.hada.io
 * topic 32035, disk-streaming architecture section).
 *
 * Layout of a record of rvq_record_bytes(hidden, inter) bytes (all integers
 * little-endian, as the structure below on this ABI):
 *   [0, 64)            rvq_record_header_t; the rest of the first 4 KiB is 0
 *   [4096, +73728)     codebooks, fp32 [3 matrices: gate, up, down][3][256][8]
 *   [77824, +P)        codes, the packed bank record (P = rvq_bank_record_bytes)
 *   then zero padding to a multiple of 4096.
 * The header's offsets and sizes state that layout; a reader trusts only
 * what rvq_record_check has accepted.
 * ------------------------------------------------------------------------ */
#define RVQ_RECORD_MAGIC 0x45515652u /* bytes 'R' 'V' 'Q' 'E' */
#define RVQ_RECORD_VERSION 1u

typedef struct {
  uint32_t magic;           /* RVQ_RECORD_MAGIC */
  uint32_t version;         /* RVQ_RECORD_VERSION */
  int32_t layer;            /* layer of the expert */
  int32_t expert;           /* expert id within the layer */
  int32_t hidden, inter;    /* expert shape H, I */
  int64_t codebook_offset;  /* bytes from the record start */
  int64_t codebook_bytes;   /* 73,728 */
  int64_t codes_offset;     /* bytes from the record start */
  int64_t codes_bytes;      /* rvq_bank_record_bytes(hidden, inter) */
  uint32_t payload_crc32;   /* CRC-32 (IEEE 802.3, as rvq_bank_crc32) of the codes */
  uint32_t reserved;        /* 0 */
} rvq_record_header_t;      /* 64 bytes */

/* Bytes of one record: 77,824 + rvq_bank_record_bytes, rounded up to 4096
 * (16,592,896 at hidden 7168, inter 2048); 0 for an invalid shape. */
size_t rvq_record_bytes(int32_t hidden, int32_t inter);

/* Fills *header (host memory) with the standard layout above.
 * Errors: RVQ_ERR_NULL, RVQ_ERR_SHAPE (invalid shape, negative layer or id). */
int rvq_record_header_init(rvq_record_header_t *header, int32_t layer, int32_t expert, int32_t hidden,
                           int32_t inter, uint32_t payload_crc32);

/* The check the pages apply on every read, on a record in HOST memory of
 * record_bytes bytes: magic and version; layer, expert id and shape equal to
 * the expected ones; codebook and code sizes those of the shape; both regions
 * 16-byte aligned, past the header, disjoint and inside the record.  Reads
 * only the header; returns RVQ_OK or RVQ_ERR_RECORD (RVQ_ERR_NULL, or
 * RVQ_ERR_SHAPE for an invalid expected shape).  Needs no GPU. */
int rvq_record_check(const void *record, int64_t record_bytes, int32_t layer, int32_t expert, int32_t hidden,
                     int32_t inter);

/* ------------------------------------------------------------------------
 * Expert pool: experts held in pinned host memory, an LRU set of `slots`
 * device records as the cache (the pages' engine streams experts from NVMe
 * into an LRU cache sized to one token's working set and prefetches what the
 * next layer's router predicts: "Running a 2.78-Trillion-Parameter Model on a
 * Laptop", Technical Insight; news.hada.io topic 32035, read-ahead and
 * router-prediction section).  Host DRAM stands in for the NVMe tier here.
 *
 * rvq_pool_create: host_codes: num_experts records of record_stride bytes in
 * the packed layout (as in rvq_expert_bank_t), host_codebooks: fp32
 * [num_experts][3][3][256][8]; both pinned host memory (hipHostMalloc or a
 * pinned torch tensor) that outlives the pool.  slot_codes (256-byte aligned,
 * slots * record_stride bytes) and slot_codebooks (16-byte aligned, fp32
 * [slots][3][3][256][8]) are device memory the caller owns; an
 * rvq_expert_bank_t over them with num_experts = slots is the bank that the
 * decode entry points use with slot ids.  The pool creates streams of its
 * own (default priority): one for the copies acquire needs, one for
 * look-ahead copies, and with verify (below) one per copy stream for the
 * payload checks.
 * rvq_pool_acquire: makes the k experts ids[0..k) (host int32, 1 <= k <=
 * slots) resident and writes their slot ids to slot_ids (host int32 [k]).
 * Missing experts are copied (LRU victim among the slots this call does not
 * use), after all work already enqueued on `stream` (earlier decodes may
 * still read the victims); `stream` is made to wait for the copies of the
 * slots it gets, so work enqueued on it afterwards sees them.  The slots
 * stay valid for work enqueued on `stream` until the next acquire.  Never
 * blocks the host.
 * rvq_pool_prefetch: starts copies of the listed experts that are not
 * resident (look-ahead), into slots that the latest acquire did not hand
 * out; stops when none is free.  Does not touch any stream but the pool's.
 * rvq_pool_stats: hits and misses of the acquires (distinct experts per
 * call), prefetch copies started, bytes copied host to device.
 * rvq_pool_destroy: waits for the pool's copies, frees its stream and events.
 * Errors: RVQ_ERR_NULL, RVQ_ERR_SHAPE, RVQ_ERR_ALIGN, RVQ_ERR_EXPERT_ID (an
 * id outside [0, num_experts): nothing is copied), RVQ_ERR_HIP.  A pool is
 * not thread-safe: one host thread drives it.
 * ------------------------------------------------------------------------ */
typedef struct rvq_expert_pool rvq_expert_pool_t;
int rvq_pool_create(const void *host_codes, const float *host_codebooks, int64_t record_stride, int32_t num_experts,
                    int32_t hidden, int32_t inter, void *slot_codes, float *slot_codebooks, int32_t slots,
                    rvq_expert_pool_t **out);
int rvq_pool_acquire(rvq_expert_pool_t *pool, const int32_t *ids, int32_t k, int32_t *slot_ids, hipStream_t stream);
int rvq_pool_prefetch(rvq_expert_pool_t *pool, const int32_t *ids, int32_t k);
int rvq_pool_stats(const rvq_expert_pool_t *pool, int64_t *hits, int64_t *misses, int64_t *prefetches,
                   int64_t *bytes_copied);
int rvq_pool_destroy(rvq_expert_pool_t *pool);

/* Pool over a host store of expert records (the layout above): num_experts
 * records of record_bytes bytes each (>= rvq_record_bytes(hidden, inter),
 * multiple of 4096) in pinned host memory, record e holding expert e of
 * `layer`.  Every copy into a slot (acquire miss or prefetch) first checks
 * that record with rvq_record_check; acquire returns RVQ_ERR_RECORD for a
 * record that fails, having copied nothing and changed no state, and
 * prefetch stops at it with RVQ_ERR_RECORD.  slot_stride: bytes between slot
 * records in slot_codes (multiple of 256, >= rvq_bank_record_bytes).
 * verify != 0 adds the pages' optional payload check: after each copy the
 * CRC-32 of the slot's codes is computed on the device, on a check stream of
 * the pool's (one per copy stream) while the next copy proceeds, and compared
 * with the header's (the compute stream and the slot's next copy wait for
 * the check); a
 * mismatch is recorded in verify_workspace (device,
 * rvq_pool_verify_workspace_bytes(hidden, inter) bytes, 256-byte aligned,
 * owned by the caller; NULL when verify == 0).  The decode still runs on the
 * copied bytes: the check reports, it does not repair.
 * rvq_pool_verify_status: waits for the pool's copies and checks, returns
 * RVQ_ERR_RECORD and the id of an expert whose payload failed (in
 * *bad_expert, -1 if none) and clears the record, else RVQ_OK; RVQ_OK with
 * -1 for a pool without verify.  Synchronises the pool's streams. */
size_t rvq_pool_verify_workspace_bytes(int32_t hidden, int32_t inter);
int rvq_pool_create_records(const void *host_records, int64_t record_bytes, int32_t layer, int32_t num_experts,
                            int32_t hidden, int32_t inter, void *slot_codes, float *slot_codebooks,
                            int64_t slot_stride, int32_t slots, int32_t verify, void *verify_workspace,
                            size_t verify_workspace_bytes, rvq_expert_pool_t **out);
int rvq_pool_verify_status(rvq_expert_pool_t *pool, int32_t *bad_expert);

/* Zero-fill a workspace (with a kernel, so the call can be graph-captured).
 * This also resets the wait limit below to the default. */
int rvq_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Testing aid for the failure path of the T == 1 table kernels (decode,
 * routed decode, pre-norm block, batch decode).  Stores in the header of
 * `workspace` how many times each bounded wait between the kernels' wave
 * roles polls before it gives up (which sets RVQ_ERR_DEVICE_STALL in that
 * workspace's status and leaves the output invalid, but lets every kernel
 * finish).  polls < 0 restores the default (4,194,304, about a tenth of a
 * second).  Enqueued on `stream` (a one-thread kernel, graph-capturable);
 * applies to kernels that use this workspace and run after it.  The value
 * lives in the workspace, not in the library: other workspaces are not
 * affected.  workspace: 256-byte aligned, >= 256 bytes.  Errors: RVQ_ERR_NULL,
 * RVQ_ERR_ALIGN, RVQ_ERR_WORKSPACE, RVQ_ERR_SHAPE (polls == INT32_MAX). */
int rvq_workspace_set_wait_limit(void *workspace, size_t workspace_bytes, int32_t polls, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RMSNorm with unit weight: out[t] = x[t] / sqrt(mean(x[t]^2) + eps).
 * The pages mention norms only inside the model's trunk and give no formula;
 * this normalisation is the one the stacked-layer decode puts between MoE
 * layers (pre-norm residual blocks, see rvq_moe_block_decode), a reading of
 * this library, not a passage of the pages.
 * x, out: fp32 [T][H] (may alias).  T >= 1, H >= 1, eps >= 0.
 * ------------------------------------------------------------------------ */
int rvq_rmsnorm(const float *x, int32_t T, int32_t H, float eps, float *out, hipStream_t stream);

/* Measurement aid: copies nbytes (multiple of 16) from src to dst (16-byte
 * aligned, non-overlapping) with the same non-temporal 16-byte global loads
 * the code stream uses, so its duration gives the achievable streaming rate
 * and its memory-traffic counters scale those of the table kernels. */
int rvq_stream_copy(const void *src, void *dst, size_t nbytes, hipStream_t stream);

/* Measurement aid: reads nbytes (multiple of 16) from src (16-byte aligned)
 * with the same non-temporal 16-byte global loads as the code stream (one
 * workgroup per compute unit, each reading one contiguous part with 64 KiB per
 * compute unit in flight, the fastest read pattern measured) and writes nothing
 * but, in practice never, one word to sink (device uint32): its duration gives
 * the achievable read-only streaming rate, the bound of the table kernels' code
 * stream. */
int rvq_stream_read(const void *src, size_t nbytes, uint32_t *sink, hipStream_t stream);

/* Synchronises `stream`, returns the sticky device status held in the
 * workspace of rvq_moe_layer_forward (RVQ_OK, RVQ_ERR_EXPERT_ID, or
 * RVQ_ERR_DEVICE_STALL if a kernel's bounded wait between its wave roles gave
 * up, which leaves y invalid) and clears it.  Returns RVQ_ERR_HIP if the synchronisation or copy fails. */
int rvq_check_device_status(void *workspace, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* RVQ_H_ */

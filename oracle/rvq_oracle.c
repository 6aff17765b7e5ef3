/* fp64 CPU oracle for the RVQ-LUT MoE expert forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the GPU path.
 *
 * It computes the plain definitions, slowly and in double precision:
 *  - RVQ decode: a weight sub-vector of 8 consecutive columns of one row is
 *    the sum of three code vectors, one from each of three 256-entry stage
 *    codebooks, chosen by that group's three code bytes (stage-minor).
 *    (WASTE Inference Engine: Running Kimi K3 2.78T on Consumer Hardware,
 *    section "Residual Vector Quantization (RVQ)"; news.hada.io topic 32035,
 *    section on quantization and accuracy: 3 stages x 256 entries x 8 dims.)
 *  - Expert output: y = W x with W rebuilt element by element (never the
 *    table form), then down(silu(gate x) * (up x)).
 *  - Partial-dot tables (for checking only): T[g][s][c] = C_s[c] . x[8g:8g+8],
 *    the per-codebook, per-position tables of "Running a 2.78-Trillion-
 *    Parameter Model on a Laptop: Inside WASTE's NVMe-Streaming Engine",
 *    section "Technical Insight".
 *  - Router: logits = W_r x with bf16 weights widened exactly; top-k by
 *    (logit descending, expert id ascending); gates = softmax over the k
 *    selected logits (news.hada.io topic 32035, read-ahead section: 16
 *    experts per layer).
 *  - RMSNorm: h / sqrt(mean(h^2) + eps), unit weight.
 *  - RVQ encoding (for checking the GPU encoder): each 8-column sub-vector
 *    is quantised stage by stage, each stage choosing the entry nearest (in
 *    squared Euclidean distance) to what the earlier stages left, and that
 *    entry is subtracted: the residual form of the RVQ decode above.  The
 *    plain definition, in double precision: the fp32 weights and entries are
 *    widened, differences, squares, sums and the residual are fp64; exact
 *    ties go to the lower index.  Beside each code it can report the best and
 *    second-best squared distances and the squared norm of the residual the
 *    stage was applied to, so that a caller can tell a decision taken in a
 *    lower precision from a wrong one (two entries within rounding of each
 *    other are both correct answers).
 *  - Record check: CRC-32 of an expert record's code payload (news.hada.io
 *    topic 32035, disk-streaming architecture section: an optional crc32 of
 *    each record's payload), computed bit by bit from its definition.
 *  - Codebook fitting (the converter's side of the RVQ form; the pages name
 *    the offline conversion but not its method): residual k-means.  Stage by
 *    stage, 256 centroids start at the residual sub-vectors the caller names
 *    (rounded to fp32, the codebooks' type), then Lloyd iterations: every
 *    sub-vector goes to its nearest centroid (the encoding decision above, in
 *    fp64), every centroid with members becomes their mean (a centroid without
 *    members keeps its value); after the last iteration the sub-vectors are
 *    assigned once more, those codes are the stage's codes, and the chosen
 *    centroids are subtracted (fp64 residual).  The mean is one fp64 sum over
 *    the members in ascending sub-vector index, divided by the member count
 *    and rounded to fp32.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- threads */
typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void *ctx; int64_t lo, hi; } range_job;

static void *range_worker(void *arg) {
  range_job *j = (range_job *)arg;
  j->fn(j->ctx, j->lo, j->hi);
  return 0;
}

static void parallel_for(int64_t n, int threads, range_fn fn, void *ctx) {
  if (threads < 1) threads = 1;
  if (threads > 128) threads = 128;
  if (threads == 1 || n < 2) { fn(ctx, 0, n); return; }
  pthread_t th[128];
  range_job jobs[128];
  int64_t per = (n + threads - 1) / threads;
  int used = 0;
  for (int t = 0; t < threads; ++t) {
    int64_t lo = t * per, hi = lo + per;
    if (lo >= n) break;
    if (hi > n) hi = n;
    jobs[t].fn = fn; jobs[t].ctx = ctx; jobs[t].lo = lo; jobs[t].hi = hi;
    pthread_create(&th[t], 0, range_worker, &jobs[t]);
    ++used;
  }
  for (int t = 0; t < used; ++t) pthread_join(th[t], 0);
}

/* ---------------------------------------------------------------- RVQ decode */
/* One row of W, rebuilt in double: W[r][8g+j] = C0[c0][j] + C1[c1][j] + C2[c2][j]. */
static void decode_row(const uint8_t *codes, const float *cb, int64_t cols, int64_t r, double *w) {
  int64_t groups = cols / 8;
  const uint8_t *row = codes + r * groups * 3;
  for (int64_t g = 0; g < groups; ++g) {
    const float *v0 = cb + (0 * 256 + row[3 * g + 0]) * 8;
    const float *v1 = cb + (1 * 256 + row[3 * g + 1]) * 8;
    const float *v2 = cb + (2 * 256 + row[3 * g + 2]) * 8;
    for (int j = 0; j < 8; ++j) w[8 * g + j] = (double)v0[j] + (double)v1[j] + (double)v2[j];
  }
}

void orc_dequant(const uint8_t *codes, const float *cb, int64_t rows, int64_t cols, double *W) {
  for (int64_t r = 0; r < rows; ++r) decode_row(codes, cb, cols, r, W + r * cols);
}

/* ---------------------------------------------------------------- matvec */
typedef struct {
  const uint8_t *codes; const float *cb; int64_t rows, cols;
  const double *X; int64_t ntok;            /* X[t][cols] */
  const int64_t *rowsel;                    /* NULL = all rows */
  double *Y;                                /* Y[t][nrows_out] */
  int64_t nout;
} gemv_ctx;

static void gemv_range(void *vctx, int64_t lo, int64_t hi) {
  gemv_ctx *c = (gemv_ctx *)vctx;
  double *w = (double *)malloc(sizeof(double) * c->cols);
  for (int64_t i = lo; i < hi; ++i) {
    int64_t r = c->rowsel ? c->rowsel[i] : i;
    decode_row(c->codes, c->cb, c->cols, r, w);
    for (int64_t t = 0; t < c->ntok; ++t) {
      const double *x = c->X + t * c->cols;
      double acc = 0.0;
      for (int64_t k = 0; k < c->cols; ++k) acc += w[k] * x[k];
      c->Y[t * c->nout + i] = acc;
    }
  }
  free(w);
}

/* Y[t][i] = sum_k W[row_i][k] X[t][k] for the selected rows (all rows if rowsel == NULL). */
void orc_gemv_batch(const uint8_t *codes, const float *cb, int64_t rows, int64_t cols,
                    const double *X, int64_t ntok, const int64_t *rowsel, int64_t nsel,
                    double *Y, int threads) {
  gemv_ctx c = {codes, cb, rows, cols, X, ntok, rowsel, Y, rowsel ? nsel : rows};
  parallel_for(c.nout, threads, gemv_range, &c);
}

void orc_gemv(const uint8_t *codes, const float *cb, int64_t rows, int64_t cols, const double *x,
              const int64_t *rowsel, int64_t nsel, double *y, int threads) {
  orc_gemv_batch(codes, cb, rows, cols, x, 1, rowsel, nsel, y, threads);
}

/* ---------------------------------------------------------------- partial-dot tables */
/* T[g][s][c] = sum_j C_s[c][j] * x[8g+j]  (groups = cols/8). */
void orc_lut(const float *cb, const double *x, int64_t cols, double *T) {
  int64_t groups = cols / 8;
  for (int64_t g = 0; g < groups; ++g)
    for (int s = 0; s < 3; ++s)
      for (int c = 0; c < 256; ++c) {
        double acc = 0.0;
        for (int j = 0; j < 8; ++j) acc += (double)cb[(s * 256 + c) * 8 + j] * x[8 * g + j];
        T[(g * 3 + s) * 256 + c] = acc;
      }
}

/* The table form of the same product: y[r] = sum_g sum_s T[g][s][codes[r][g][s]]. */
void orc_gemv_via_lut(const uint8_t *codes, const double *T, int64_t rows, int64_t cols, double *y) {
  int64_t groups = cols / 8;
  for (int64_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int64_t g = 0; g < groups; ++g)
      for (int s = 0; s < 3; ++s) acc += T[(g * 3 + s) * 256 + codes[(r * groups + g) * 3 + s]];
    y[r] = acc;
  }
}

/* ---------------------------------------------------------------- SwiGLU expert */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Y[t] = down( silu(gate X[t]) * (up X[t]) ) for ntok tokens; output rows of down
 * restricted to rowsel if given.  gate/up are [inter x hidden], down is [hidden x inter]. */
void orc_expert_batch(const uint8_t *gate_codes, const float *gate_cb,
                      const uint8_t *up_codes, const float *up_cb,
                      const uint8_t *down_codes, const float *down_cb,
                      int64_t hidden, int64_t inter, const double *X, int64_t ntok,
                      const int64_t *rowsel, int64_t nsel, double *Y, int threads) {
  double *g = (double *)malloc(sizeof(double) * ntok * inter);
  double *u = (double *)malloc(sizeof(double) * ntok * inter);
  orc_gemv_batch(gate_codes, gate_cb, inter, hidden, X, ntok, 0, 0, g, threads);
  orc_gemv_batch(up_codes, up_cb, inter, hidden, X, ntok, 0, 0, u, threads);
  for (int64_t i = 0; i < ntok * inter; ++i) g[i] = orc_silu(g[i]) * u[i];
  orc_gemv_batch(down_codes, down_cb, hidden, inter, g, ntok, rowsel, nsel, Y, threads);
  free(g);
  free(u);
}

/* ---------------------------------------------------------------- router */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

typedef struct { const uint16_t *w; const double *X; int64_t ntok, E, H; double *L; } router_ctx;

static void router_range(void *vctx, int64_t lo, int64_t hi) {
  router_ctx *c = (router_ctx *)vctx;
  for (int64_t e = lo; e < hi; ++e)
    for (int64_t t = 0; t < c->ntok; ++t) {
      double acc = 0.0;
      for (int64_t k = 0; k < c->H; ++k) acc += bf16_to_double(c->w[e * c->H + k]) * c->X[t * c->H + k];
      c->L[t * c->E + e] = acc;
    }
}

/* L[t][e] = sum_k Wr[e][k] X[t][k], Wr given as bf16 bit patterns. */
void orc_router_logits(const uint16_t *w_bf16, const double *X, int64_t ntok, int64_t E, int64_t H,
                       double *L, int threads) {
  router_ctx c = {w_bf16, X, ntok, E, H, L};
  parallel_for(E, threads, router_range, &c);
}

/* Selection by sorting the whole list with the key (logit descending, id ascending),
 * then keeping the first k.  gates = exp(l - l_max) / sum over the k kept.
 * gap_out[0] = l[k-th] - l[(k+1)-th] (inf if k == E); gap_out[1] = smallest
 * difference between consecutive kept logits (inf if k == 1). */
static const double *g_sort_logits;
static int cmp_rank(const void *a, const void *b) {
  int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
  double li = g_sort_logits[i], lj = g_sort_logits[j];
  if (li > lj) return -1;
  if (li < lj) return 1;
  return (i < j) ? -1 : (i > j);
}

void orc_topk(const double *logits, int64_t E, int64_t k, int32_t *ids, double *gates, double *gap_out) {
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * E);
  for (int64_t e = 0; e < E; ++e) order[e] = (int32_t)e;
  g_sort_logits = logits;
  qsort(order, (size_t)E, sizeof(int32_t), cmp_rank);
  double m = logits[order[0]];
  double z = 0.0;
  for (int64_t i = 0; i < k; ++i) {
    ids[i] = order[i];
    gates[i] = exp(logits[order[i]] - m);
    z += gates[i];
  }
  for (int64_t i = 0; i < k; ++i) gates[i] /= z;
  if (gap_out) {
    gap_out[0] = (k < E) ? logits[order[k - 1]] - logits[order[k]] : INFINITY;
    double mg = INFINITY;
    for (int64_t i = 1; i < k; ++i) {
      double d = logits[order[i - 1]] - logits[order[i]];
      if (d < mg) mg = d;
    }
    gap_out[1] = mg;
  }
  free(order);
}

/* ---------------------------------------------------------------- RMSNorm */
void orc_rmsnorm(const double *h, int64_t H, double eps, double *out) {
  double ss = 0.0;
  for (int64_t k = 0; k < H; ++k) ss += h[k] * h[k];
  double inv = 1.0 / sqrt(ss / (double)H + eps);
  for (int64_t k = 0; k < H; ++k) out[k] = h[k] * inv;
}

/* ---------------------------------------------------------------- CRC-32
 * The CRC-32 of IEEE 802.3 (as in zlib and PNG): the message bits, least
 * significant bit of each byte first, are divided by the generator
 * x^32 + x^26 + x^23 + x^22 + x^16 + x^12 + x^11 + x^10 + x^8 + x^7 + x^5 +
 * x^4 + x^2 + x + 1 with the register preset to all ones and the remainder
 * complemented.  In the bit-reversed register the generator's low 32 terms
 * read 0xEDB88320, and each message bit is one shift-and-conditional-subtract
 * step: no table, no combination of partial results. */
uint32_t orc_crc32(const uint8_t *data, int64_t n) {
  uint32_t r = 0xFFFFFFFFu;
  for (int64_t i = 0; i < n; ++i) {
    r ^= data[i];
    for (int b = 0; b < 8; ++b) r = (r & 1u) ? (r >> 1) ^ 0xEDB88320u : (r >> 1);
  }
  return ~r;
}

/* ---------------------------------------------------------------- RVQ encode */
/* Nearest entry of C (fp32 [256][8]) to v (fp64): squared distances in fp64, ties to the lower
 * index.  d_best / d_second receive the smallest and second-smallest distances. */
static int nearest_entry(const double *v, const float *C, double *d_best, double *d_second) {
  int best = 0;
  double b1 = INFINITY, b2 = INFINITY;
  for (int c = 0; c < 256; ++c) {
    double d = 0.0;
    for (int j = 0; j < 8; ++j) {
      const double t = v[j] - (double)C[c * 8 + j];
      d += t * t;
    }
    if (d < b1) {
      b2 = b1;
      b1 = d;
      best = c;
    } else if (d < b2) {
      b2 = d;
    }
  }
  if (d_best) *d_best = b1;
  if (d_second) *d_second = b2;
  return best;
}

/* W: fp32 [rows][cols] (cols % 8 == 0); cb: fp32 [3][256][8]; codes: [rows][cols/8][3].
 * margins (or NULL): fp64 [rows][cols/8][3][3] = (best distance, second-best distance, squared norm
 * of the residual the stage was applied to) for every decision. */
void orc_rvq_encode(const float *W, int64_t rows, int64_t cols, const float *cb, uint8_t *codes,
                    double *margins) {
  const int64_t G = cols / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < G; ++g) {
      double v[8];
      for (int j = 0; j < 8; ++j) v[j] = (double)W[r * cols + 8 * g + j];
      for (int s = 0; s < 3; ++s) {
        const float *C = cb + (int64_t)s * 256 * 8;
        double d1, d2, vv = 0.0;
        for (int j = 0; j < 8; ++j) vv += v[j] * v[j];
        const int best = nearest_entry(v, C, &d1, &d2);
        for (int j = 0; j < 8; ++j) v[j] = v[j] - (double)C[best * 8 + j];
        codes[(r * G + g) * 3 + s] = (uint8_t)best;
        if (margins) {
          double *m = margins + ((r * G + g) * 3 + s) * 3;
          m[0] = d1;
          m[1] = d2;
          m[2] = vv;
        }
      }
    }
}

/* ---------------------------------------------------------------- RVQ codebook fit
 * W: fp32 [rows][cols]; init: [3][256] sub-vector indices (row-major sub-vector order,
 * each in [0, rows*cols/8)); cb out: fp32 [3][256][8]; codes out: [rows][cols/8][3]. */
typedef struct { const double *R; const float *C; int32_t *code; } assign_ctx;

static void assign_range(void *p, int64_t lo, int64_t hi) {
  assign_ctx *a = (assign_ctx *)p;
  for (int64_t i = lo; i < hi; ++i) a->code[i] = nearest_entry(a->R + i * 8, a->C, 0, 0);
}

void orc_rvq_fit(const float *W, int64_t rows, int64_t cols, int iters, const int32_t *init, float *cb,
                 uint8_t *codes, int threads) {
  const int64_t N = rows * (cols / 8);
  double *R = (double *)malloc((size_t)N * 8 * sizeof(double));   /* what the earlier stages left */
  int32_t *code = (int32_t *)malloc((size_t)N * sizeof(int32_t));
  for (int64_t i = 0; i < N * 8; ++i) R[i] = (double)W[i];       /* sub-vector i = W[8i .. 8i+8) */
  for (int s = 0; s < 3; ++s) {
    float *C = cb + (int64_t)s * 256 * 8;
    for (int c = 0; c < 256; ++c)
      for (int j = 0; j < 8; ++j) C[c * 8 + j] = (float)R[(int64_t)init[s * 256 + c] * 8 + j];
    assign_ctx a = {R, C, code};
    for (int it = 0; it <= iters; ++it) {
      parallel_for(N, threads, assign_range, &a);
      if (it == iters) break;
      double sum[256][8];
      int64_t n[256];
      memset(sum, 0, sizeof sum);
      memset(n, 0, sizeof n);
      for (int64_t i = 0; i < N; ++i) {
        n[code[i]] += 1;
        for (int j = 0; j < 8; ++j) sum[code[i]][j] += R[i * 8 + j];
      }
      for (int c = 0; c < 256; ++c)
        if (n[c] > 0)
          for (int j = 0; j < 8; ++j) C[c * 8 + j] = (float)(sum[c][j] / (double)n[c]);
    }
    for (int64_t i = 0; i < N; ++i) {
      codes[i * 3 + s] = (uint8_t)code[i];
      for (int j = 0; j < 8; ++j) R[i * 8 + j] = R[i * 8 + j] - (double)C[code[i] * 8 + j];
    }
  }
  free(code);
  free(R);
}

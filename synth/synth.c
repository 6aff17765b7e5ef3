/* Seeded synthetic inputs shared by the GPU path's tests/benchmarks and the
 * fp64 oracle.  This file holds random-number generation only: no part of
 * the RVQ method's arithmetic lives here.
 *
 * Generator: SplitMix64 used in counter mode.  A stream is keyed by
 * (seed, tensor id); its i-th 64-bit word is mix64(key + (i+1)*GAMMA),
 * which is exactly SplitMix64's (i+1)-th output from state `key`, so any
 * slice of any tensor can be regenerated independently.
 *   key(seed, tid) = mix64(mix64(seed) ^ tid)
 * Bytes: word i supplies bytes 8i..8i+7, little-endian.
 * Normals: Box-Muller on word pairs (2p, 2p+1):
 *   u1 = ((w_{2p} >> 11) + 1) * 2^-53  in (0, 1]
 *   u2 =  (w_{2p+1} >> 11)    * 2^-53  in [0, 1)
 *   z_{2p} = sqrt(-2 ln u1) cos(2 pi u2), z_{2p+1} = sqrt(-2 ln u1) sin(2 pi u2)
 * computed in double, scaled by std in double, rounded to float (RNE).
 * bf16 values are the float rounded to nearest-even on the upper 16 bits.
 */
#include <stdint.h>
#include <math.h>
#include <pthread.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tid) { return mix64(mix64(seed + GAMMA) ^ tid); }

static inline uint64_t word(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* n 64-bit words starting at word index `first`. */
void synth_words(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, uint64_t *out) {
  uint64_t key = synth_key(seed, tid);
  for (uint64_t i = 0; i < n; ++i) out[i] = word(key, first + i);
}

/* Uniform bytes [first, first+n) of the stream. */
typedef struct { uint64_t key, first, n; uint8_t *out; } bytes_job;

static void bytes_range(uint64_t key, uint64_t first, uint64_t n, uint8_t *out) {
  uint64_t b = first, end = first + n;
  while (b < end) {
    uint64_t w = word(key, b >> 3);
    unsigned j = (unsigned)(b & 7);
    if (j == 0 && end - b >= 8) {
      memcpy(out + (b - first), &w, 8);  /* little-endian host */
      b += 8;
    } else {
      out[b - first] = (uint8_t)(w >> (8 * j));
      ++b;
    }
  }
}

static void *bytes_worker(void *arg) {
  bytes_job *j = (bytes_job *)arg;
  bytes_range(j->key, j->first, j->n, j->out);
  return 0;
}

void synth_bytes(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, uint8_t *out, int threads) {
  uint64_t key = synth_key(seed, tid);
  if (threads <= 1 || n < (1u << 20)) { bytes_range(key, first, n, out); return; }
  if (threads > 64) threads = 64;
  pthread_t th[64];
  bytes_job jobs[64];
  uint64_t chunk = ((n / threads) + 7) & ~7ULL;
  int used = 0;
  for (int t = 0; t < threads; ++t) {
    uint64_t s = (uint64_t)t * chunk;
    if (s >= n) break;
    uint64_t len = (s + chunk > n) ? n - s : chunk;
    jobs[t].key = key; jobs[t].first = first + s; jobs[t].n = len; jobs[t].out = out + s;
    pthread_create(&th[t], 0, bytes_worker, &jobs[t]);
    ++used;
  }
  for (int t = 0; t < used; ++t) pthread_join(th[t], 0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = (double)((word(key, 2 * p) >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(word(key, 2 * p + 1) >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* Normal(0, std) elements [first, first+n) as float. */
void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, double std, float *out) {
  uint64_t key = synth_key(seed, tid);
  for (uint64_t k = 0; k < n; ++k) out[k] = (float)(std * normal_at(key, first + k));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* Normal(0, std) elements as bf16 bit patterns (float first, then RNE to bf16). */
void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t first, uint64_t n, double std, uint16_t *out) {
  uint64_t key = synth_key(seed, tid);
  for (uint64_t k = 0; k < n; ++k) out[k] = f32_to_bf16_rne((float)(std * normal_at(key, first + k)));
}

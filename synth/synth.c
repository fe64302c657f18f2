/*
 * synth.c - seeded, counter-based synthetic inputs (weights, KV cache, token
 * ids, lengths) for the decode workloads.
 *
 * This module is shared by the oracle side and the HIP side and holds none of
 * the decoder's arithmetic: it only turns (seed, tensor key, element index)
 * into numbers.  Every element is a pure function of that triple, so any slice
 * of any tensor can be regenerated independently and in any thread order.
 *
 * Definitions (stated here so that an independent re-implementation can
 * reproduce every byte):
 *   mix64(z)          = SplitMix64 finaliser of (z + 0x9E3779B97F4A7C15):
 *                         z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                         z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
 *   draw(seed,key,i)  = mix64(mix64(mix64(seed) ^ key) ^ i)
 *   key(name)         = 64-bit FNV-1a of the tensor name's bytes
 *   unit53(u)         = (u >> 11) * 2^-53                    in [0, 1)
 *   unit24(u)         = (u >> 40) * 2^-24                    in [0, 1)
 *   normal pair j     : u1 = 1 - unit24(draw(..,2j)) in (0,1], u2 = unit24(draw(..,2j+1))
 *                       r = sqrtf(-2 logf(u1)); a = 2 pi u2 (float);
 *                       element 2j = r cosf(a), element 2j+1 = r sinf(a)
 *                       (Box-Muller in single precision: every value is
 *                       rounded to bf16 afterwards)
 *   bf16 value        = round-to-nearest-even of the float sigma*z
 *   uniform int       = lo + floor(unit53(draw(seed,key,i)) * (hi - lo + 1))
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

static inline uint64_t draw(uint64_t seed, uint64_t key, uint64_t i) { return mix64(mix64(mix64(seed) ^ key) ^ i); }

uint64_t synth_draw(uint64_t seed, uint64_t key, uint64_t i) { return draw(seed, key, i); }

uint64_t synth_key(const char* name) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (const unsigned char* p = (const unsigned char*)name; *p; ++p) {
    h ^= *p;
    h *= 0x100000001b3ull;
  }
  return h;
}

static inline double unit53(uint64_t u) { return (double)(u >> 11) * (1.0 / 9007199254740992.0); }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  if ((x & 0x7f800000u) == 0x7f800000u) return (uint16_t)((x >> 16) | ((x & 0xffffu) ? 0x40u : 0u)); /* inf / nan */
  uint32_t lsb = (x >> 16) & 1u;
  x += 0x7fffu + lsb;
  return (uint16_t)(x >> 16);
}

static inline float unit24(uint64_t u) { return (float)(u >> 40) * (1.0f / 16777216.0f); }

static inline void normal_pair(uint64_t seed, uint64_t key, uint64_t pair, float* z0, float* z1) {
  float u1 = 1.0f - unit24(draw(seed, key, 2 * pair));
  float u2 = unit24(draw(seed, key, 2 * pair + 1));
  float r = sqrtf(-2.0f * logf(u1));
  float a = 6.28318530717958647692f * u2;
  *z0 = r * cosf(a);
  *z1 = r * sinf(a);
}

double synth_normal(uint64_t seed, uint64_t key, uint64_t idx) {
  float z0, z1;
  normal_pair(seed, key, idx >> 1, &z0, &z1);
  return (idx & 1) ? z1 : z0;
}

typedef struct {
  uint16_t* out;
  int64_t begin, end; /* element range of this worker, relative to out */
  int64_t start;      /* global element index of out[0] */
  uint64_t seed, key;
  float sigma;
} normal_job;

static void* normal_worker(void* arg) {
  normal_job* j = (normal_job*)arg;
  int64_t i = j->begin;
  /* elements come in Box-Muller pairs; compute both halves of a pair at once */
  while (i < j->end) {
    uint64_t g = (uint64_t)(j->start + i);
    float z0, z1;
    normal_pair(j->seed, j->key, g >> 1, &z0, &z1);
    if ((g & 1) == 0 && i + 1 < j->end) {
      j->out[i] = f32_to_bf16_rne(j->sigma * z0);
      j->out[i + 1] = f32_to_bf16_rne(j->sigma * z1);
      i += 2;
    } else {
      j->out[i] = f32_to_bf16_rne(j->sigma * ((g & 1) ? z1 : z0));
      i += 1;
    }
  }
  return 0;
}

/* out[i] = bf16(sigma * N(seed, key, start + i)) for i in [0, n). Returns 0. */
int synth_fill_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t key, int64_t start, double sigma,
                           int nthreads) {
  if (n <= 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < (int64_t)nthreads * 4096) nthreads = 1;
  pthread_t th[256];
  normal_job jobs[256];
  int64_t per = (n + nthreads - 1) / nthreads;
  per = (per + 1) & ~(int64_t)1;
  int launched = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = (int64_t)t * per, e = b + per;
    if (b >= n) break;
    if (e > n) e = n;
    jobs[t] = (normal_job){out, b, e, start, seed, key, (float)sigma};
    if (nthreads == 1) {
      normal_worker(&jobs[t]);
    } else {
      pthread_create(&th[t], 0, normal_worker, &jobs[t]);
      ++launched;
    }
  }
  for (int t = 0; t < launched; ++t) pthread_join(th[t], 0);
  return 0;
}

/* out[i] = uniform integer in [lo, hi] for global index start + i. */
int synth_fill_uniform_i32(int32_t* out, int64_t n, uint64_t seed, uint64_t key, int64_t start, int32_t lo,
                           int32_t hi) {
  if (hi < lo) return -1;
  double span = (double)hi - (double)lo + 1.0;
  for (int64_t i = 0; i < n; ++i) {
    int64_t v = (int64_t)lo + (int64_t)floor(unit53(draw(seed, key, (uint64_t)(start + i))) * span);
    if (v > hi) v = hi;
    out[i] = (int32_t)v;
  }
  return 0;
}

/* out[i] = bf16(value) */
int synth_fill_const_bf16(uint16_t* out, int64_t n, float value) {
  uint16_t b = f32_to_bf16_rne(value);
  for (int64_t i = 0; i < n; ++i) out[i] = b;
  return 0;
}

/*
 * Seeded, counter-based synthetic inputs shared by the GPU path's tests and
 * bench and by the CPU oracle.  Nothing here computes any part of the scan:
 * it only draws numbers and rounds them to a storage type.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast Splittable
 * Pseudorandom Number Generators", OOPSLA 2014).  The i-th output of a stream
 * is mix(key + (i + 1) * GAMMA), so every element is a pure function of
 * (seed, stream, flat index) and any slice can be regenerated on its own.
 *
 *   uniform(i)  = (mix(...) >> 11) * 2^-53                  in [0, 1)
 *   normal(i)   = Box-Muller on uniform(2i), uniform(2i+1):
 *                 sqrt(-2 ln(1 - u1)) * cos(2 pi u2)
 *
 * Storage rounding: the fp64 value is cast to fp32 (round to nearest even),
 * and for bf16 the fp32 bit pattern is rounded to its upper 16 bits with
 * round-to-nearest-even (NaN kept quiet).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of stream `stream` under `seed`: two rounds of the mixer so that
 * nearby (seed, stream) pairs give unrelated keys. */
uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return sm64_mix(sm64_mix(seed * SM64_GAMMA + 0x2545F4914F6CDD1DULL) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t sm64_at(uint64_t key, uint64_t i) { return sm64_mix(key + (i + 1) * SM64_GAMMA); }

static inline double u01(uint64_t key, uint64_t i) { return (double)(sm64_at(key, i) >> 11) * 0x1.0p-53; }

static inline double normal01(uint64_t key, uint64_t i) {
  double u1 = u01(key, 2 * i), u2 = u01(key, 2 * i + 1);
  return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586476925286766559 * u2);
}

uint16_t synth_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* Distribution kinds.  p0, p1 are parameters; `period` is used by IDX. */
enum {
  SYN_NORMAL = 0,        /* p0 + p1 * N(0,1)                                  */
  SYN_UNIFORM = 1,       /* U(p0, p1)                                         */
  SYN_SOFTPLUS_NORMAL = 2, /* softplus(p0 + p1 * N(0,1)) = log(1 + e^v)       */
  SYN_NEG_EXP_UNIFORM = 3, /* -exp(U(p0, p1))                                 */
  SYN_NEG_IDX = 4,       /* -(1 + (i mod period)) : A = -(1..N) per channel   */
  SYN_CONST = 5          /* p0                                                */
};

static double draw(int kind, double p0, double p1, int64_t period, uint64_t key, uint64_t i) {
  switch (kind) {
    case SYN_NORMAL: return p0 + p1 * normal01(key, i);
    case SYN_UNIFORM: return p0 + (p1 - p0) * u01(key, i);
    case SYN_SOFTPLUS_NORMAL: {
      double v = p0 + p1 * normal01(key, i);
      return v > 0 ? v + log1p(exp(-v)) : log1p(exp(v));
    }
    case SYN_NEG_EXP_UNIFORM: return -exp(p0 + (p1 - p0) * u01(key, i));
    case SYN_NEG_IDX: return -(double)(1 + (int64_t)(i % (uint64_t)period));
    default: return p0;
  }
}

typedef struct {
  int kind, out_bf16;
  double p0, p1;
  int64_t period;
  uint64_t key, start, n;
  void* out;
} job_t;

static void* run_job(void* arg) {
  job_t* j = (job_t*)arg;
  for (uint64_t k = 0; k < j->n; ++k) {
    float f = (float)draw(j->kind, j->p0, j->p1, j->period, j->key, j->start + k);
    if (j->out_bf16) ((uint16_t*)j->out)[k] = synth_f32_to_bf16(f);
    else ((float*)j->out)[k] = f;
  }
  return 0;
}

/* Fill out[0..n) with elements start..start+n of stream (seed, stream).
 * out_bf16 = 0: float32 output; 1: bf16 bit patterns (uint16). */
int synth_fill(void* out, uint64_t n, uint64_t start, int out_bf16, int kind, double p0, double p1,
               int64_t period, uint64_t seed, uint64_t stream, int nthreads) {
  if (period <= 0) period = 1;
  uint64_t key = synth_key(seed, stream);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < (uint64_t)nthreads * 65536) nthreads = 1;
  job_t jobs[256];
  pthread_t th[256];
  uint64_t per = (n + nthreads - 1) / nthreads;
  size_t esz = out_bf16 ? 2 : 4;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t s = (uint64_t)t * per, e = s + per < n ? s + per : n;
    jobs[t] = (job_t){kind, out_bf16, p0, p1, period, key, start + s, e > s ? e - s : 0, (char*)out + s * esz};
  }
  for (int t = 1; t < nthreads; ++t)
    if (pthread_create(&th[t], 0, run_job, &jobs[t])) { run_job(&jobs[t]); th[t] = 0; }
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t)
    if (th[t]) pthread_join(th[t], 0);
  return 0;
}

/* Raw 64-bit outputs, for checking the mixer against its published definition. */
void synth_raw(uint64_t* out, uint64_t n, uint64_t start, uint64_t seed, uint64_t stream) {
  uint64_t key = synth_key(seed, stream);
  for (uint64_t k = 0; k < n; ++k) out[k] = sm64_at(key, start + k);
}

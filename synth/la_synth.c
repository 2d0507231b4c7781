/*
 * la_synth.c -- seeded synthetic inputs for LayerAdam runs.
 *
 * Holds none of the update's arithmetic: it only draws numbers. Both the
 * oracle side and the HIP side of every test and benchmark take their inputs
 * from here.
 *
 * Generator: counter-based SplitMix64 (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014). Stream s of seed
 * k has key = mix(k XOR mix(s + GAMMA)); its i-th draw is
 * mix(key + (i + 1) * GAMMA), i.e. the i-th output of a SplitMix64 generator
 * whose state starts at key. Uniforms use the top 53 bits. Normals use the
 * Box-Muller transform on draw pairs (2k, 2k+1): radius sqrt(-2 ln(1 - U0)),
 * angle 2*pi*U1; element 2k takes the cosine branch, element 2k+1 the sine
 * branch. A value depends only on (seed, stream, index), never on the thread
 * count.
 *
 * Narrow formats: the FP32 sample is converted to BF16 or FP16 by rounding
 * toward zero (truncation of the significand), with FP16 subnormals, and
 * FP16 overflow saturating to the largest finite value.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix(seed ^ mix(stream + GAMMA));
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix(key + (i + 1) * GAMMA);
}

static inline double uniform01(uint64_t bits) {
  return (double)(bits >> 11) * 0x1.0p-53; /* [0, 1) */
}

/* Standard normals of the pair k: elements 2k (cosine) and 2k+1 (sine). */
static inline void normal_pair(uint64_t key, uint64_t k, double *z0, double *z1) {
  double u0 = uniform01(draw(key, 2 * k));
  double u1 = uniform01(draw(key, 2 * k + 1));
  double radius = sqrt(-2.0 * log(1.0 - u0));
  double angle = 6.283185307179586476925 * u1;
  *z0 = radius * cos(angle);
  *z1 = radius * sin(angle);
}

static inline uint32_t f32_bits(float x) {
  uint32_t b;
  memcpy(&b, &x, 4);
  return b;
}

static inline uint16_t to_bf16_rtz(float x) {
  uint32_t b = f32_bits(x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  return (uint16_t)(b >> 16);
}

static inline uint16_t to_fp16_rtz(float x) {
  uint32_t b = f32_bits(x);
  uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
  uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7E00u;
  if (a == 0x7F800000u) return sign | 0x7C00u;
  int e = (int)(a >> 23) - 127;
  if (e > 15) return sign | 0x7BFFu;
  if (e >= -14) return sign | (uint16_t)((e + 15) << 10) | (uint16_t)((a >> 13) & 0x3FFu);
  if (e < -25 || a == 0) return sign;
  uint32_t significand = 0x800000u | (a & 0x7FFFFFu);
  return sign | (uint16_t)(significand >> (-e - 1));
}

/* ---------------------------------------------------------------------- */
/* Threaded fills.                                                         */
/* ---------------------------------------------------------------------- */
enum { KIND_NORMAL_F32, KIND_UNIFORM_F32, KIND_NORMAL_HALF };

typedef struct {
  int kind;
  uint64_t key, outlier_key;
  void *out;
  int64_t begin, end;
  double a, b;         /* normal: mean, std; uniform: lo, hi */
  double scale;        /* half: multiplier applied before rounding to FP32 */
  double outlier_prob; /* half: per-element probability of an outlier */
  float outlier_mult;  /* half: outlier multiplier, applied in FP32 */
  int half_format;     /* 0 BF16, 1 FP16 */
} job;

static inline void put(const job *j, int64_t i, double z) {
  if (j->kind == KIND_NORMAL_F32) {
    ((float *)j->out)[i] = (float)(j->a + j->b * z);
  } else {
    float x = (float)(j->b * j->scale * z);
    if (j->outlier_prob > 0.0 &&
        uniform01(draw(j->outlier_key, (uint64_t)i)) < j->outlier_prob)
      x = x * j->outlier_mult;
    ((uint16_t *)j->out)[i] = j->half_format ? to_fp16_rtz(x) : to_bf16_rtz(x);
  }
}

static void run_job(const job *j) {
  if (j->kind == KIND_UNIFORM_F32) {
    for (int64_t i = j->begin; i < j->end; ++i) {
      double u = uniform01(draw(j->key, (uint64_t)i));
      ((float *)j->out)[i] = (float)(j->a + (j->b - j->a) * u);
    }
    return;
  }
  for (int64_t k = j->begin >> 1; 2 * k < j->end; ++k) {
    double z0, z1;
    normal_pair(j->key, (uint64_t)k, &z0, &z1);
    if (2 * k >= j->begin) put(j, 2 * k, z0);
    if (2 * k + 1 < j->end) put(j, 2 * k + 1, z1);
  }
}

static void *thread_main(void *arg) {
  run_job((const job *)arg);
  return NULL;
}

static void run_threaded(const job *proto, int64_t n, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < 65536) nthreads = 1;
  job jobs[256];
  pthread_t tids[256];
  int64_t per = (n + nthreads - 1) / nthreads;
  per = (per + 1) & ~(int64_t)1; /* keep Box-Muller pairs within one thread */
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *proto;
    jobs[t].begin = (int64_t)t * per;
    jobs[t].end = jobs[t].begin + per < n ? jobs[t].begin + per : n;
    if (jobs[t].begin >= n) break;
    if (nthreads == 1 || pthread_create(&tids[t], NULL, thread_main, &jobs[t]) != 0) {
      run_job(&jobs[t]);
      tids[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (nthreads > 1 && tids[t]) pthread_join(tids[t], NULL);
}

void las_fill_normal_f32(uint64_t seed, uint64_t stream, float *out, int64_t n,
                         double mean, double std, int nthreads) {
  job j = {0};
  j.kind = KIND_NORMAL_F32;
  j.key = stream_key(seed, stream);
  j.out = out;
  j.a = mean;
  j.b = std;
  run_threaded(&j, n, nthreads);
}

void las_fill_uniform_f32(uint64_t seed, uint64_t stream, float *out, int64_t n,
                          double lo, double hi, int nthreads) {
  job j = {0};
  j.kind = KIND_UNIFORM_F32;
  j.key = stream_key(seed, stream);
  j.out = out;
  j.a = lo;
  j.b = hi;
  run_threaded(&j, n, nthreads);
}

void las_fill_normal_half(uint64_t seed, uint64_t stream, uint16_t *out,
                          int64_t n, double std, double scale,
                          uint64_t outlier_stream, double outlier_prob,
                          double outlier_mult, int half_format, int nthreads) {
  job j = {0};
  j.kind = KIND_NORMAL_HALF;
  j.key = stream_key(seed, stream);
  j.outlier_key = stream_key(seed, outlier_stream);
  j.out = out;
  j.b = std;
  j.scale = scale;
  j.outlier_prob = outlier_prob;
  j.outlier_mult = (float)outlier_mult;
  j.half_format = half_format;
  run_threaded(&j, n, nthreads);
}

/* One uniform draw, for per-tensor constants. */
double las_uniform_at(uint64_t seed, uint64_t stream, int64_t i) {
  return uniform01(draw(stream_key(seed, stream), (uint64_t)i));
}

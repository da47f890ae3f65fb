/*
 * Seeded, counter-based input generator for the KDA workloads.
 *
 * Test and benchmark infrastructure shared by the fp64 oracle and the HIP
 * path.  It draws the synthetic inputs the workloads describe and holds none
 * of the delta-rule arithmetic: only random numbers, the distributions the
 * workloads name (normal, L2-normalised normal rows, scaled sigmoid of a
 * normal, uniform integers) and the rounding of fp64 values to the stored
 * fp32 / bf16 formats.
 *
 * Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The i-th output of the
 * generator seeded with s is mix(s + (i + 1) * GAMMA), so any output can be
 * computed from its index alone: every (tensor, element) draws independently
 * of every other and slices regenerate identically in any order.
 *
 * Streams: the base of a stream is out(out(seed, tensor_id), sub) where
 * out(s, i) is the i-th SplitMix64 output of seed s; `sub` is 0 for prefill
 * tensors and step + 1 for the inputs of decode step `step`.
 * Element n of a stream uses outputs 2n and 2n + 1 of the stream base as two
 * uniforms in (0, 1], turned into one standard normal by the cosine branch of
 * the Box-Muller transform (Box & Muller, Ann. Math. Stat. 1958).
 *
 * Rounding: fp64 -> fp32 by the C conversion (IEEE round-to-nearest-even),
 * fp32 -> bf16 by round-to-nearest-even on the bit pattern.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th output (0-based) of SplitMix64 seeded with s */
static inline uint64_t sm_out(uint64_t s, uint64_t i) { return mix64(s + (i + 1) * GAMMA); }

/* uniform double in (0, 1] from the top 53 bits */
static inline double u01(uint64_t x) { return (double)((x >> 11) + 1) * (1.0 / 9007199254740992.0); }

uint64_t dg_stream_base(uint64_t seed, uint64_t tensor_id, uint64_t sub) {
  return sm_out(sm_out(seed, tensor_id), sub);
}

static inline double normal_at(uint64_t base, uint64_t n) {
  double u1 = u01(sm_out(base, 2 * n));
  double u2 = u01(sm_out(base, 2 * n + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* dtype: 0 = fp32, 1 = bf16 (stored as uint16 bit patterns), 2 = fp64 */
static inline void store(void* out, int dtype, uint64_t i, double x) {
  if (dtype == 0) ((float*)out)[i] = (float)x;
  else if (dtype == 1) ((uint16_t*)out)[i] = f32_to_bf16_rne((float)x);
  else ((double*)out)[i] = x;
}

enum { K_NORMAL = 0, K_UNIT_ROWS = 1, K_SIGMOID = 2 };

typedef struct {
  int kind, dtype;
  uint64_t base;
  uint64_t r0, r1;   /* row range [r0, r1) handled by this worker */
  int dim;           /* row length */
  double scale;
  void* out;
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  double* row = (double*)malloc(sizeof(double) * (size_t)j->dim);
  for (uint64_t r = j->r0; r < j->r1; ++r) {
    uint64_t n0 = r * (uint64_t)j->dim;
    for (int c = 0; c < j->dim; ++c) row[c] = normal_at(j->base, n0 + (uint64_t)c);
    if (j->kind == K_UNIT_ROWS) {
      double ss = 0.0;
      for (int c = 0; c < j->dim; ++c) ss += row[c] * row[c];
      double inv = 1.0 / sqrt(ss);
      for (int c = 0; c < j->dim; ++c) store(j->out, j->dtype, n0 + c, row[c] * inv);
    } else if (j->kind == K_SIGMOID) {
      for (int c = 0; c < j->dim; ++c) store(j->out, j->dtype, n0 + c, j->scale / (1.0 + exp(-row[c])));
    } else {
      for (int c = 0; c < j->dim; ++c) store(j->out, j->dtype, n0 + c, j->scale * row[c]);
    }
  }
  free(row);
  return NULL;
}

/*
 * Fill `rows` x `dim` elements of stream (seed, tensor_id, sub):
 *   kind 0: scale * N(0,1)
 *   kind 1: N(0,1) rows L2-normalised in fp64 (scale ignored)
 *   kind 2: scale * sigmoid(N(0,1))
 * then rounded to `dtype`.  Returns 0 on success.
 */
int dg_fill(uint64_t seed, uint64_t tensor_id, uint64_t sub, int kind, double scale, int dtype, uint64_t rows,
            int dim, void* out, int nthreads) {
  if (!out || dim <= 0 || kind < 0 || kind > 2 || dtype < 0 || dtype > 2) return 1;
  if (rows == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if ((uint64_t)nthreads > rows) nthreads = (int)rows;
  uint64_t base = dg_stream_base(seed, tensor_id, sub);
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  uint64_t per = (rows + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t r0 = (uint64_t)t * per, r1 = r0 + per;
    if (r0 >= rows) break;
    if (r1 > rows) r1 = rows;
    jobs[t] = (job_t){kind, dtype, base, r0, r1, dim, scale, out};
    if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) { run_job(&jobs[t]); th[t] = 0; }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
  free(jobs);
  free(th);
  return 0;
}

/* n integers uniform in [lo, hi] (inclusive) from stream (seed, tensor_id, 0):
 * out[i] = lo + floor(u * (hi - lo + 1)) with u = output i as a uniform in [0, 1). */
int dg_uniform_ints(uint64_t seed, uint64_t tensor_id, int n, int lo, int hi, int32_t* out) {
  if (!out || n < 0 || hi < lo) return 1;
  uint64_t base = dg_stream_base(seed, tensor_id, 0);
  uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
  for (int i = 0; i < n; ++i) {
    double u = (double)(sm_out(base, (uint64_t)i) >> 11) * (1.0 / 9007199254740992.0);
    uint64_t off = (uint64_t)(u * (double)span);
    if (off >= span) off = span - 1;
    out[i] = (int32_t)((int64_t)lo + (int64_t)off);
  }
  return 0;
}

/* raw access for tests: i-th SplitMix64 output of seed s, and one normal */
uint64_t dg_splitmix_out(uint64_t s, uint64_t i) { return sm_out(s, i); }
double dg_normal_at(uint64_t seed, uint64_t tensor_id, uint64_t sub, uint64_t n) {
  return normal_at(dg_stream_base(seed, tensor_id, sub), n);
}

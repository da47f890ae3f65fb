/*
 * fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the KDA library itself never does.
 * It shares no code, header or helper with the HIP path.
 *
 * What it computes is the plain definition of the KDA recurrence, token by
 * token, in fp64, for each (sequence, head) independently:
 *
 *   S_t  = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t  = S_t^T q_t                      (read out after the update)
 *   alpha_t = exp(g_t), elementwise over the d_k key channels
 *
 * Passages followed (Kimi K3 pages):
 *  - Kimi Delta Attention is a gated delta-rule linear attention on a
 *    fixed-size recurrent state (technical-report page, "Quick answer" and
 *    FAQ "What is Kimi Delta Attention?"; architecture blog, "Why the
 *    attention stack is the story");
 *  - the delta rule removes the value currently stored under a key before
 *    writing the new one (architecture blog, "Kimi Delta Attention: the linear
 *    core", second paragraph) -- the (I - beta k k^T) factor;
 *  - the forget gate decays the state per channel rather than with one scalar
 *    (same section, third paragraph; technical-report page, "Architecture at a
 *    glance") -- Diag(alpha_t) acting on the key rows of S;
 *  - the log-decay is bounded below through a scaled sigmoid (technical-report
 *    page, "Architecture at a glance"): here g is taken as the already-bounded
 *    log-decay, used as given.
 * The pages never print the recurrence as an equation; the form above is the
 * standard gated delta rule they name, with the decay applied first and the
 * delta correction taken against the decayed state (the factor order of the
 * equation), and no query scaling.
 *
 * One step, written out:
 *   1. S[c][:] *= exp(g[c])                 for every key channel c
 *   2. p[j] = sum_c S[c][j] * k[c]          (value currently stored under k)
 *   3. u[j] = beta * (v[j] - p[j])
 *   4. S[c][j] += k[c] * u[j]
 *   5. o[j] = sum_c S[c][j] * q[c]
 *
 * Inputs are the stored values (fp32, or bf16 bit patterns) decoded exactly to
 * fp64, so the oracle measures the arithmetic of an implementation, not the
 * rounding of its inputs; fp64 arrays are also accepted, for inputs that the
 * caller has transformed in fp64 (gate from its pre-activation, normalised
 * q and k).  Layouts (row-major): q, k, g [.., T, H, d_k];
 * v [.., T, H, d_v]; beta [.., T, H]; states [.., H, d_k, d_v].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* exact decode of a stored element: dtype 0 = fp32, 1 = bf16 bits, 2 = fp64 (inputs already
   transformed in fp64, e.g. from gate pre-activations) */
static inline double ld(const void* p, int dtype, size_t i) {
  if (dtype == 0) return (double)((const float*)p)[i];
  if (dtype == 2) return ((const double*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

typedef struct {
  const void *q, *k, *v, *g, *beta;
  int dtype, H, dk, dv;
} inputs_t;

typedef struct {
  size_t row0;        /* (token, head) row index of the unit's first token */
  long T;             /* tokens in the unit's sequence */
  const double* h0;   /* d_k x d_v initial state, or NULL for zero */
  double* o;          /* output of token 0, or NULL */
  size_t o_stride;    /* elements between consecutive tokens' outputs */
  double* hT;         /* d_k x d_v final state, or NULL */
} unit_t;

/* Run the recurrence of one (sequence, head) unit. */
static void run_unit(const inputs_t* in, const unit_t* u) {
  const int dk = in->dk, dv = in->dv;
  double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
  double* kk = (double*)malloc(sizeof(double) * dk);
  double* qq = (double*)malloc(sizeof(double) * dk);
  double* p = (double*)malloc(sizeof(double) * dv);
  if (u->h0)
    memcpy(S, u->h0, sizeof(double) * (size_t)dk * dv);
  for (long t = 0; t < u->T; ++t) {
    size_t row = u->row0 + (size_t)t * (size_t)in->H;
    for (int c = 0; c < dk; ++c) {
      kk[c] = ld(in->k, in->dtype, row * dk + c);
      qq[c] = ld(in->q, in->dtype, row * dk + c);
    }
    double b = ld(in->beta, in->dtype, row);
    /* 1. decay each key row of the state */
    for (int c = 0; c < dk; ++c) {
      double a = exp(ld(in->g, in->dtype, row * dk + c));
      for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;
    }
    /* 2. value stored under k in the decayed state */
    for (int j = 0; j < dv; ++j) p[j] = 0.0;
    for (int c = 0; c < dk; ++c)
      for (int j = 0; j < dv; ++j) p[j] += S[(size_t)c * dv + j] * kk[c];
    /* 3.-4. delta-rule write: replace it, in proportion beta, by v */
    for (int j = 0; j < dv; ++j) p[j] = b * (ld(in->v, in->dtype, row * dv + j) - p[j]);
    for (int c = 0; c < dk; ++c)
      for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kk[c] * p[j];
    /* 5. read out the updated state */
    if (u->o) {
      double* o = u->o + (size_t)t * u->o_stride;
      for (int j = 0; j < dv; ++j) o[j] = 0.0;
      for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) o[j] += S[(size_t)c * dv + j] * qq[c];
    }
  }
  if (u->hT) memcpy(u->hT, S, sizeof(double) * (size_t)dk * dv);
  free(S);
  free(kk);
  free(qq);
  free(p);
}

typedef struct {
  const inputs_t* in;
  const unit_t* units;
  int n_units;
  int next;
  pthread_mutex_t mu;
} pool_t;

static void* worker(void* arg) {
  pool_t* P = (pool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&P->mu);
    int i = P->next++;
    pthread_mutex_unlock(&P->mu);
    if (i >= P->n_units) break;
    run_unit(P->in, &P->units[i]);
  }
  return NULL;
}

static void run_all(const inputs_t* in, const unit_t* units, int n_units, int nthreads) {
  if (n_units <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_units) nthreads = n_units;
  pool_t P;
  P.in = in;
  P.units = units;
  P.n_units = n_units;
  P.next = 0;
  pthread_mutex_init(&P.mu, NULL);
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  int* ok = (int*)calloc((size_t)nthreads, sizeof(int));
  for (int t = 0; t < nthreads; ++t) ok[t] = pthread_create(&th[t], NULL, worker, &P) == 0;
  worker(&P); /* the calling thread works too; it also finishes all units if no thread started */
  for (int t = 0; t < nthreads; ++t)
    if (ok[t]) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&P.mu);
  free(th);
  free(ok);
}

static int bad_dims(int H, int dk, int dv, int dtype) { return H <= 0 || dk <= 0 || dv <= 0 || dtype < 0 || dtype > 2; }

/*
 * Batched forward.  o: [B,T,H,dv] fp64 (or NULL); hT: [B,H,dk,dv] fp64 (or NULL);
 * h0: [B,H,dk,dv] fp64 (or NULL for a zero start; an fp32 state converts
 * exactly).  Returns 0 on success.
 */
int kda_oracle_forward(const void* q, const void* k, const void* v, const void* g, const void* beta, int dtype,
                       const double* h0, double* o, double* hT, int B, long T, int H, int dk, int dv, int nthreads) {
  if (B < 0 || T < 0 || bad_dims(H, dk, dv, dtype)) return 1;
  inputs_t in = {q, k, v, g, beta, dtype, H, dk, dv};
  int n = B * H;
  unit_t* units = (unit_t*)calloc((size_t)(n > 0 ? n : 1), sizeof(unit_t));
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      unit_t* u = &units[b * H + h];
      size_t sidx = (size_t)(b * H + h) * dk * dv;
      u->row0 = (size_t)b * (size_t)T * H + h;
      u->T = T;
      u->h0 = h0 ? h0 + sidx : NULL;
      u->o = o ? o + ((size_t)b * (size_t)T * H + h) * dv : NULL;
      u->o_stride = (size_t)H * dv;
      u->hT = hT ? hT + sidx : NULL;
    }
  run_all(&in, units, n, nthreads);
  free(units);
  return 0;
}

/*
 * Forward on a subset of (b, h) units, for sampled checks of large workloads.
 * unit_ids[i] = b * H + h.  o: [n_units, T, dv]; hT: [n_units, dk, dv] (either NULL).
 */
int kda_oracle_forward_units(const void* q, const void* k, const void* v, const void* g, const void* beta, int dtype,
                             const double* h0, double* o, double* hT, int B, long T, int H, int dk, int dv,
                             const int* unit_ids, int n_units, int nthreads) {
  if (B < 0 || T < 0 || n_units < 0 || bad_dims(H, dk, dv, dtype)) return 1;
  inputs_t in = {q, k, v, g, beta, dtype, H, dk, dv};
  unit_t* units = (unit_t*)calloc((size_t)(n_units > 0 ? n_units : 1), sizeof(unit_t));
  for (int i = 0; i < n_units; ++i) {
    int id = unit_ids[i];
    if (id < 0 || id >= B * H) { free(units); return 1; }
    int b = id / H, h = id % H;
    unit_t* u = &units[i];
    u->row0 = (size_t)b * (size_t)T * H + h;
    u->T = T;
    u->h0 = h0 ? h0 + (size_t)id * dk * dv : NULL;
    u->o = o ? o + (size_t)i * (size_t)T * dv : NULL;
    u->o_stride = (size_t)dv;
    u->hT = hT ? hT + (size_t)i * dk * dv : NULL;
  }
  run_all(&in, units, n_units, nthreads);
  free(units);
  return 0;
}

/*
 * Packed variable-length forward: N sequences concatenated along the token
 * axis of [T_total, H, d] tensors, sequence n covering tokens
 * [cu_seqlens[n], cu_seqlens[n+1]).  No state crosses a sequence boundary.
 * h0, hT: [N, H, dk, dv]; o: [T_total, H, dv].
 */
int kda_oracle_forward_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              int dtype, const int32_t* cu_seqlens, int N, const double* h0, double* o, double* hT,
                              int H, int dk, int dv, int nthreads) {
  if (N < 0 || !cu_seqlens || bad_dims(H, dk, dv, dtype)) return 1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n] || cu_seqlens[0] != 0) return 1;
  inputs_t in = {q, k, v, g, beta, dtype, H, dk, dv};
  int nu = N * H;
  unit_t* units = (unit_t*)calloc((size_t)(nu > 0 ? nu : 1), sizeof(unit_t));
  for (int n = 0; n < N; ++n)
    for (int h = 0; h < H; ++h) {
      unit_t* u = &units[n * H + h];
      size_t sidx = (size_t)(n * H + h) * dk * dv;
      u->row0 = (size_t)cu_seqlens[n] * H + h;
      u->T = cu_seqlens[n + 1] - cu_seqlens[n];
      u->h0 = h0 ? h0 + sidx : NULL;
      u->o = o ? o + ((size_t)cu_seqlens[n] * H + h) * dv : NULL;
      u->o_stride = (size_t)H * dv;
      u->hT = hT ? hT + sidx : NULL;
    }
  run_all(&in, units, nu, nthreads);
  free(units);
  return 0;
}

/*
 * One decode step for B sequences: the same single-token update applied to a
 * persistent fp64 state [B, H, dk, dv], in place.  q, k, g: [B, H, dk];
 * v: [B, H, dv]; beta: [B, H]; o: [B, H, dv] fp64.
 */
typedef struct {
  const inputs_t* in;
  double* state;
  double* o;
  int n, next;
  pthread_mutex_t mu;
} dpool_t;

static void decode_unit(const inputs_t* in, size_t row, double* S, double* o) {
  const int dk = in->dk, dv = in->dv;
  double* p = (double*)malloc(sizeof(double) * dv);
  double b = ld(in->beta, in->dtype, row);
  for (int c = 0; c < dk; ++c) {
    double a = exp(ld(in->g, in->dtype, row * dk + c));
    for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;
  }
  for (int j = 0; j < dv; ++j) p[j] = 0.0;
  for (int c = 0; c < dk; ++c) {
    double kc = ld(in->k, in->dtype, row * dk + c);
    for (int j = 0; j < dv; ++j) p[j] += S[(size_t)c * dv + j] * kc;
  }
  for (int j = 0; j < dv; ++j) p[j] = b * (ld(in->v, in->dtype, row * dv + j) - p[j]);
  for (int c = 0; c < dk; ++c) {
    double kc = ld(in->k, in->dtype, row * dk + c);
    for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kc * p[j];
  }
  for (int j = 0; j < dv; ++j) o[j] = 0.0;
  for (int c = 0; c < dk; ++c) {
    double qc = ld(in->q, in->dtype, row * dk + c);
    for (int j = 0; j < dv; ++j) o[j] += S[(size_t)c * dv + j] * qc;
  }
  free(p);
}

static void* dworker(void* arg) {
  dpool_t* P = (dpool_t*)arg;
  const inputs_t* in = P->in;
  for (;;) {
    pthread_mutex_lock(&P->mu);
    int i = P->next++;
    pthread_mutex_unlock(&P->mu);
    if (i >= P->n) break;
    decode_unit(in, (size_t)i, P->state + (size_t)i * in->dk * in->dv, P->o + (size_t)i * in->dv);
  }
  return NULL;
}

int kda_oracle_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta, int dtype,
                           double* state, double* o, int B, int H, int dk, int dv, int nthreads) {
  if (B < 0 || !state || !o || bad_dims(H, dk, dv, dtype)) return 1;
  inputs_t in = {q, k, v, g, beta, dtype, H, dk, dv};
  dpool_t P;
  P.in = &in;
  P.state = state;
  P.o = o;
  P.n = B * H;
  P.next = 0;
  pthread_mutex_init(&P.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > P.n) nthreads = P.n > 0 ? P.n : 1;
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  int* ok = (int*)calloc((size_t)nthreads, sizeof(int));
  for (int t = 0; t < nthreads; ++t) ok[t] = pthread_create(&th[t], NULL, dworker, &P) == 0;
  dworker(&P);
  for (int t = 0; t < nthreads; ++t)
    if (ok[t]) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&P.mu);
  free(th);
  free(ok);
  return 0;
}

/*
 * Backward (reverse mode) of the recurrence above, for training: given the
 * adjoints do = dL/do [.., T, H, d_v] and dhT = dL/dhT [.., H, d_k, d_v] (or
 * none), it returns dL/dq, dL/dk, dL/dg [.., T, H, d_k], dL/dv [.., T, H, d_v],
 * dL/dbeta [.., T, H] and dL/dh0 [.., H, d_k, d_v], all fp64.  The pages give
 * no backward (training with KDA is stated on the technical-report page,
 * "Training"); this is the chain rule applied to the five steps of one token,
 * taken in reverse order, with dS the adjoint of the state after the token:
 *
 *   5. o = S^T q            dq[c]  = sum_j S[c][j] do[j];      dS[c][j] += q[c] do[j]
 *   4. S = S' + k u^T       dk[c] += sum_j dS[c][j] u[j];      du[j] = sum_c dS[c][j] k[c];  dS' = dS
 *   3. u = beta (v - p)     dbeta  = sum_j du[j] (v[j] - p[j]); dv[j] = beta du[j];  dp[j] = -beta du[j]
 *   2. p = S'^T k           dk[c] += sum_j S'[c][j] dp[j];     dS'[c][j] += k[c] dp[j]
 *   1. S' = Diag(a) S_prev  dg[c]  = sum_j dS'[c][j] S'[c][j] (a = exp(g), da/dg = a);
 *                           dS_prev[c][j] = a[c] dS'[c][j]
 *
 * and dh0 is dS once every token has been undone.  The forward states are
 * recomputed from checkpoints kept every BWD_BLOCK tokens: one block's states
 * at a time are held, so memory is (T / BWD_BLOCK + BWD_BLOCK) states per unit.
 */
#define BWD_BLOCK 64

typedef struct {
  size_t row0;
  long T;
  const double* h0;   /* or NULL */
  const double* dO;   /* adjoint of o at token 0 (stride o_stride) */
  size_t o_stride;
  const double* dhT;  /* or NULL */
  double *dq, *dk, *dg, *dv, *dbeta; /* token 0's rows; q/k/g rows advance by H dk, v rows by H dv, beta by H */
  double* dh0;
} bunit_t;

/* one forward token step on S (in place); keeps S' (decayed state), p and u for the backward */
static void fwd_token(const inputs_t* in, size_t row, double* S, double* Sd, double* p, double* u) {
  const int dk = in->dk, dv = in->dv;
  const double b = ld(in->beta, in->dtype, row);
  for (int c = 0; c < dk; ++c) {
    double a = exp(ld(in->g, in->dtype, row * dk + c));
    for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;
  }
  if (Sd) memcpy(Sd, S, sizeof(double) * (size_t)dk * dv);
  for (int j = 0; j < dv; ++j) p[j] = 0.0;
  for (int c = 0; c < dk; ++c) {
    double kc = ld(in->k, in->dtype, row * dk + c);
    for (int j = 0; j < dv; ++j) p[j] += S[(size_t)c * dv + j] * kc;
  }
  for (int j = 0; j < dv; ++j) u[j] = b * (ld(in->v, in->dtype, row * dv + j) - p[j]);
  for (int c = 0; c < dk; ++c) {
    double kc = ld(in->k, in->dtype, row * dk + c);
    for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kc * u[j];
  }
}

static void backward_unit(const inputs_t* in, const bunit_t* u) {
  const int dk = in->dk, dv = in->dv, H = in->H;
  const size_t ss = (size_t)dk * dv;
  const long T = u->T, nblk = (T + BWD_BLOCK - 1) / BWD_BLOCK;
  double* ckpt = (double*)malloc(sizeof(double) * ss * (size_t)(nblk > 0 ? nblk : 1)); /* state before block */
  double* blk = (double*)malloc(sizeof(double) * ss * (BWD_BLOCK + 1)); /* states before each token, + after */
  double* Sd = (double*)malloc(sizeof(double) * ss);
  double* dS = (double*)malloc(sizeof(double) * ss);
  double* p = (double*)malloc(sizeof(double) * dv);
  double* uu = (double*)malloc(sizeof(double) * dv);
  double* du = (double*)malloc(sizeof(double) * dv);
  double* S = (double*)calloc(ss, sizeof(double));
  if (u->h0) memcpy(S, u->h0, sizeof(double) * ss);
  for (long n = 0; n < nblk; ++n) {
    memcpy(ckpt + (size_t)n * ss, S, sizeof(double) * ss);
    for (long t = n * BWD_BLOCK; t < T && t < (n + 1) * BWD_BLOCK; ++t)
      fwd_token(in, u->row0 + (size_t)t * H, S, NULL, p, uu);
  }
  if (u->dhT) memcpy(dS, u->dhT, sizeof(double) * ss);
  else memset(dS, 0, sizeof(double) * ss);
  for (long n = nblk - 1; n >= 0; --n) {
    const long t0 = n * BWD_BLOCK, t1 = (t0 + BWD_BLOCK < T) ? t0 + BWD_BLOCK : T;
    /* recompute the states before every token of the block */
    memcpy(blk, ckpt + (size_t)n * ss, sizeof(double) * ss);
    for (long t = t0; t < t1; ++t) {
      memcpy(blk + (size_t)(t - t0 + 1) * ss, blk + (size_t)(t - t0) * ss, sizeof(double) * ss);
      fwd_token(in, u->row0 + (size_t)t * H, blk + (size_t)(t - t0 + 1) * ss, NULL, p, uu);
    }
    for (long t = t1 - 1; t >= t0; --t) {
      const size_t row = u->row0 + (size_t)t * H;
      const double* Sprev = blk + (size_t)(t - t0) * ss;
      const double* Snew = blk + (size_t)(t - t0 + 1) * ss;
      const double b = ld(in->beta, in->dtype, row);
      const double* dO = u->dO + (size_t)t * u->o_stride;
      double* dq = u->dq + (size_t)t * H * dk;
      double* dkk = u->dk + (size_t)t * H * dk;
      double* dg = u->dg + (size_t)t * H * dk;
      double* dvv = u->dv + (size_t)t * H * dv;
      /* forward quantities of this token: S' (decayed state), p, u */
      memcpy(S, Sprev, sizeof(double) * ss);
      fwd_token(in, row, S, Sd, p, uu);
      /* 5. readout */
      for (int c = 0; c < dk; ++c) {
        double acc = 0.0, qc = ld(in->q, in->dtype, row * dk + c);
        for (int j = 0; j < dv; ++j) {
          acc += Snew[(size_t)c * dv + j] * dO[j];
          dS[(size_t)c * dv + j] += qc * dO[j];
        }
        dq[c] = acc;
      }
      /* 4. write k u^T */
      for (int j = 0; j < dv; ++j) du[j] = 0.0;
      for (int c = 0; c < dk; ++c) {
        double acc = 0.0, kc = ld(in->k, in->dtype, row * dk + c);
        for (int j = 0; j < dv; ++j) {
          acc += dS[(size_t)c * dv + j] * uu[j];
          du[j] += dS[(size_t)c * dv + j] * kc;
        }
        dkk[c] = acc;
      }
      /* 3. u = beta (v - p) */
      double db = 0.0;
      for (int j = 0; j < dv; ++j) {
        double vj = ld(in->v, in->dtype, row * dv + j);
        db += du[j] * (vj - p[j]);
        dvv[j] = b * du[j];
        du[j] = -b * du[j]; /* now dp */
      }
      u->dbeta[(size_t)t * H] = db;
      /* 2. p = S'^T k */
      for (int c = 0; c < dk; ++c) {
        double acc = 0.0, kc = ld(in->k, in->dtype, row * dk + c);
        for (int j = 0; j < dv; ++j) {
          acc += Sd[(size_t)c * dv + j] * du[j];
          dS[(size_t)c * dv + j] += kc * du[j];
        }
        dkk[c] += acc;
      }
      /* 1. decay */
      for (int c = 0; c < dk; ++c) {
        double acc = 0.0, a = exp(ld(in->g, in->dtype, row * dk + c));
        for (int j = 0; j < dv; ++j) {
          acc += dS[(size_t)c * dv + j] * Sd[(size_t)c * dv + j];
          dS[(size_t)c * dv + j] *= a;
        }
        dg[c] = acc;
      }
    }
  }
  if (u->dh0) memcpy(u->dh0, dS, sizeof(double) * ss);
  free(ckpt); free(blk); free(Sd); free(dS); free(p); free(uu); free(du); free(S);
}

typedef struct {
  const inputs_t* in;
  const bunit_t* units;
  int n, next;
  pthread_mutex_t mu;
} bpool_t;

static void* bworker(void* arg) {
  bpool_t* P = (bpool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&P->mu);
    int i = P->next++;
    pthread_mutex_unlock(&P->mu);
    if (i >= P->n) break;
    backward_unit(P->in, &P->units[i]);
  }
  return NULL;
}

static void bwd_run(const inputs_t* in, const bunit_t* units, int n, int nthreads) {
  if (n <= 0) return;
  bpool_t P;
  P.in = in;
  P.units = units;
  P.n = n;
  P.next = 0;
  pthread_mutex_init(&P.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = n;
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  int* ok = (int*)calloc((size_t)nthreads, sizeof(int));
  for (int t = 0; t < nthreads; ++t) ok[t] = pthread_create(&th[t], NULL, bworker, &P) == 0;
  bworker(&P);
  for (int t = 0; t < nthreads; ++t)
    if (ok[t]) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&P.mu);
  free(th);
  free(ok);
}

/*
 * Batched backward.  dO: [B,T,H,dv] fp64; dhT: [B,H,dk,dv] fp64 or NULL (zero);
 * h0 as in the forward.  Outputs (fp64, all required): dq, dk, dg [B,T,H,dk],
 * dv [B,T,H,dv], dbeta [B,T,H], dh0 [B,H,dk,dv].  Returns 0 on success.
 */
int kda_oracle_backward(const void* q, const void* k, const void* v, const void* g, const void* beta, int dtype,
                        const double* h0, const double* dO, const double* dhT, double* dq, double* dk, double* dg,
                        double* dv, double* dbeta, double* dh0, int B, long T, int H, int dk_, int dv_, int nthreads) {
  if (B < 0 || T < 0 || bad_dims(H, dk_, dv_, dtype) || !dO || !dq || !dk || !dg || !dv || !dbeta || !dh0) return 1;
  inputs_t in = {q, k, v, g, beta, dtype, H, dk_, dv_};
  int n = B * H;
  bunit_t* units = (bunit_t*)calloc((size_t)(n > 0 ? n : 1), sizeof(bunit_t));
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      bunit_t* u = &units[b * H + h];
      size_t sidx = (size_t)(b * H + h) * dk_ * dv_, r0 = (size_t)b * (size_t)T * H + h;
      u->row0 = r0;
      u->T = T;
      u->h0 = h0 ? h0 + sidx : NULL;
      u->dO = dO + r0 * dv_;
      u->o_stride = (size_t)H * dv_;
      u->dhT = dhT ? dhT + sidx : NULL;
      u->dq = dq + r0 * dk_;
      u->dk = dk + r0 * dk_;
      u->dg = dg + r0 * dk_;
      u->dv = dv + r0 * dv_;
      u->dbeta = dbeta + r0;
      u->dh0 = dh0 + sidx;
    }
  bwd_run(&in, units, n, nthreads);
  free(units);
  return 0;
}

/*
 * A plain C client of libkda.so: it includes include/kda.h, allocates device memory through the
 * HIP runtime's C API and calls the library with no Python in the way.  Built and linked by
 * tests/test_c_client.py (gcc, host only); run on a GPU it checks that a prefill and a decode
 * step complete, that the final state matches a prefill split in two (state hand-off through the
 * C ABI), and that invalid calls are rejected.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

/* the few HIP runtime entry points used here, declared by hand to stay plain C */
typedef int hipError_t;
extern hipError_t hipMalloc(void** ptr, size_t size);
extern hipError_t hipFree(void* ptr);
extern hipError_t hipMemcpy(void* dst, const void* src, size_t size, int kind);
extern hipError_t hipDeviceSynchronize(void);
enum { H2D = 1, D2H = 2 };

static uint64_t rng = 88172645463325252ull;
static float urand(void) { /* xorshift64, in [-0.5, 0.5) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (float)((rng >> 11) * (1.0 / 9007199254740992.0)) - 0.5f;
}

#define CHECK(x)                                                       \
  do {                                                                 \
    kda_status s_ = (x);                                               \
    if (s_ != KDA_OK) {                                                \
      fprintf(stderr, "%s -> %s\n", #x, kda_status_string(s_));        \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static void* dev_upload(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != 0) return NULL;
  if (host && bytes) hipMemcpy(d, host, bytes, H2D);
  return d;
}

int main(int argc, char** argv) {
  const int compile_only = argc > 1 && strcmp(argv[1], "--version") == 0;
  printf("libkda version %d\n", kda_version());
  if (compile_only) return 0;

  const int B = 1, T = 160, H = 2, D = 64, C = 32;
  const size_t nk = (size_t)B * T * H * D, nb = (size_t)B * T * H, ns = (size_t)B * H * D * D;
  float *q = malloc(nk * 4), *k = malloc(nk * 4), *v = malloc(nk * 4), *g = malloc(nk * 4), *beta = malloc(nb * 4);
  for (size_t r = 0; r < nb; ++r) {
    double nq = 0, nkk = 0;
    for (int c = 0; c < D; ++c) {
      q[r * D + c] = urand();
      k[r * D + c] = urand();
      v[r * D + c] = 2.f * urand();
      g[r * D + c] = -2.5f - 5.f * urand(); /* in (-5, 0] */
      nq += q[r * D + c] * q[r * D + c];
      nkk += k[r * D + c] * k[r * D + c];
    }
    for (int c = 0; c < D; ++c) {
      q[r * D + c] /= (float)sqrt(nq);
      k[r * D + c] /= (float)sqrt(nkk);
    }
    beta[r] = 0.5f + urand();
  }
  void *dq = dev_upload(q, nk * 4), *dk = dev_upload(k, nk * 4), *dv = dev_upload(v, nk * 4);
  void *dg = dev_upload(g, nk * 4), *db = dev_upload(beta, nb * 4), *dout = dev_upload(NULL, nk * 4);
  float *dh = dev_upload(NULL, ns * 4), *dh2 = dev_upload(NULL, ns * 4);
  if (!dq || !dk || !dv || !dg || !db || !dout || !dh || !dh2) {
    fprintf(stderr, "device allocation failed\n");
    return 1;
  }

  /* one call over all T tokens */
  size_t wsb = kda_chunked_forward_workspace_bytes(B, T, H, D, D, C, KDA_F32);
  void* ws = dev_upload(NULL, wsb);
  CHECK(kda_chunked_forward(dq, dk, dv, dg, db, NULL, dout, dh, B, T, H, D, D, C, KDA_F32, ws, wsb, NULL));

  /* the same tokens in two calls, the first's final state handed to the second: inputs of the
     second half start T/2 tokens in (B = 1, so token t of head h is row t H + h) */
  const int T1 = T / 2, T2 = T - T1;
  const size_t off_k = (size_t)T1 * H * D, off_b = (size_t)T1 * H;
  CHECK(kda_chunked_forward(dq, dk, dv, dg, db, NULL, dout, dh2, B, T1, H, D, D, C, KDA_F32, ws, wsb, NULL));
  CHECK(kda_chunked_forward((char*)dq + off_k * 4, (char*)dk + off_k * 4, (char*)dv + off_k * 4,
                            (char*)dg + off_k * 4, (char*)db + off_b * 4, dh2, (char*)dout + off_k * 4, dh2, B, T2, H,
                            D, D, C, KDA_F32, ws, wsb, NULL));
  if (hipDeviceSynchronize() != 0) return 1;
  float *h_one = malloc(ns * 4), *h_two = malloc(ns * 4);
  hipMemcpy(h_one, dh, ns * 4, D2H);
  hipMemcpy(h_two, dh2, ns * 4, D2H);
  double num = 0, den = 0;
  for (size_t i = 0; i < ns; ++i) {
    num = fmax(num, fabs((double)h_one[i] - h_two[i]));
    den = fmax(den, fabs((double)h_one[i]));
  }
  printf("state hand-off: max |one call - two calls| / max |state| = %.3e\n", num / den);
  if (!(num / den < 1e-4) || !isfinite(num)) return 1;

  /* one decode step on the final state */
  CHECK(kda_decode_step(dq, dk, dv, dg, db, dh, dout, B, H, D, D, KDA_F32, NULL));
  if (hipDeviceSynchronize() != 0) return 1;

  /* invalid calls are rejected before anything runs */
  if (kda_chunked_forward(dq, dk, dv, dg, db, NULL, dout, dh, B, T, H, 96, D, C, KDA_F32, ws, wsb, NULL) !=
      KDA_ERR_UNSUPPORTED)
    return 1;
  if (kda_chunked_forward(dq, dk, dv, dg, db, NULL, dout, dh, B, T, H, D, D, C, KDA_F32, ws, wsb - 1, NULL) !=
      KDA_ERR_WORKSPACE)
    return 1;
  printf("c client ok\n");
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dg); hipFree(db); hipFree(dout); hipFree(dh); hipFree(dh2);
  hipFree(ws);
  free(q); free(k); free(v); free(g); free(beta); free(h_one); free(h_two);
  return 0;
}

/*
 * Drives every entry point of the fp64 oracle on small shapes (ragged lengths, windows,
 * Q-Cal, K above the chunk count, shared landmark heads, given selections with padding),
 * built with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize.py:
 * any out-of-bounds access, leak or undefined operation aborts the run.  Values come
 * from a small linear congruential generator; every output is checked to be finite.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/hils_oracle.h"

static unsigned long long g_state = 12345;
static double urand(void) {
  g_state = g_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return ((g_state >> 11) * (1.0 / 9007199254740992.0)) * 2.0 - 1.0;
}
static double* vec(size_t n) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}
static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run_case(int B, int Hq, int Hkv, int Hl, int d, int N, int K, int r, int W) {
  hr_shape s = {B, Hq, Hkv, Hl, d, 64, K, N, r, W};
  const int C = N / 64;
  double* k = vec((size_t)B * Hkv * N * d);
  double* v = vec((size_t)B * Hkv * N * d);
  double* lmk = vec((size_t)B * Hl * (C ? C : 1) * d);
  double* D = r ? vec((size_t)Hq * r * d) : NULL;
  double* U = r ? vec((size_t)Hq * d * r) : NULL;
  double* kc = (double*)malloc(sizeof(double) * ((size_t)B * Hl * (C ? C : 1) * d));
  double* bc = (double*)malloc(sizeof(double) * ((size_t)B * Hl * (C ? C : 1)));
  hr_compress(&s, k, HR_F64, lmk, HR_F64, kc, bc);
  if (!finite_all(kc, (size_t)B * Hl * C * d) || !finite_all(bc, (size_t)B * Hl * C)) return 1;
  /* every row of every (b, h) */
  const int64_t n = (int64_t)B * Hq * N;
  int32_t* rb = (int32_t*)malloc(sizeof(int32_t) * n);
  int32_t* rh = (int32_t*)malloc(sizeof(int32_t) * n);
  int32_t* rp = (int32_t*)malloc(sizeof(int32_t) * n);
  int64_t t = 0;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h)
      for (int i = 0; i < N; ++i, ++t) {
        rb[t] = b;
        rh[t] = h;
        rp[t] = i;
      }
  double* q = vec((size_t)n * d);
  double* o = (double*)malloc(sizeof(double) * n * d);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * n * K);
  double* ssc = (double*)malloc(sizeof(double) * n * K);
  double* gap = (double*)malloc(sizeof(double) * n);
  double* lse = (double*)malloc(sizeof(double) * n);
  int32_t* nsel = (int32_t*)malloc(sizeof(int32_t) * n);
  for (int mode = HR_LANDMARK; mode <= HR_EXACT; ++mode) {
    hr_attend(&s, mode, n, rb, rh, rp, q, HR_F64, k, v, HR_F64, kc, bc, D, U, HR_F64, NULL, o, sel, ssc, gap, lse,
              nsel);
    if (!finite_all(o, (size_t)n * d) || !finite_all(lse, (size_t)n)) return 2;
  }
  /* given selections: the landmark selection with one slot of each row cleared to -1 */
  for (int64_t x = 0; x < n; ++x) sel[x * K + (x % K)] = -1;
  hr_attend(&s, HR_GIVEN, n, rb, rh, rp, q, HR_F64, k, v, HR_F64, kc, bc, D, U, HR_F64, sel, o, NULL, NULL, NULL, NULL,
            NULL);
  if (!finite_all(o, (size_t)n * d)) return 3;
  double* sc = (double*)malloc(sizeof(double) * (C > 0 ? C : 1));
  for (int64_t x = 0; x < n; x += 7) {
    hr_row_scores(&s, HR_LANDMARK, rb[x], rh[x], rp[x], q + x * d, HR_F64, k, HR_F64, kc, bc, D, U, HR_F64, sc);
    hr_row_scores(&s, HR_EXACT, rb[x], rh[x], rp[x], q + x * d, HR_F64, k, HR_F64, kc, bc, D, U, HR_F64, sc);
  }
  hr_dense(&s, n, rb, rh, rp, q, HR_F64, k, v, HR_F64, o);
  if (!finite_all(o, (size_t)n * d)) return 4;
  if (Hl == Hq) {   /* the backward pass needs one landmark head per query head */
    hr_attend(&s, HR_LANDMARK, n, rb, rh, rp, q, HR_F64, k, v, HR_F64, kc, bc, D, U, HR_F64, NULL, o, sel, ssc, gap,
              lse, nsel);
    double* dO = vec((size_t)n * d);
    double* dq = (double*)malloc(sizeof(double) * n * d);
    double* dk = (double*)malloc(sizeof(double) * ((size_t)B * Hkv * N * d));
    double* dv = (double*)malloc(sizeof(double) * ((size_t)B * Hkv * N * d));
    double* dkc = (double*)malloc(sizeof(double) * ((size_t)B * Hl * (C ? C : 1) * d));
    double* dbc = (double*)malloc(sizeof(double) * ((size_t)B * Hl * (C ? C : 1)));
    double* dl = (double*)malloc(sizeof(double) * ((size_t)B * Hl * (C ? C : 1) * d));
    double* dD = r ? (double*)malloc(sizeof(double) * ((size_t)Hq * r * d)) : NULL;
    double* dU = r ? (double*)malloc(sizeof(double) * ((size_t)Hq * d * r)) : NULL;
    hr_attend_backward(&s, n, rb, rh, rp, q, HR_F64, k, v, HR_F64, kc, bc, lmk, HR_F64, D, U, HR_F64, sel, dO, dq, dk,
                       dv, dkc, dbc, dl, dD, dU);
    if (!finite_all(dq, (size_t)n * d) || !finite_all(dk, (size_t)B * Hkv * N * d)) return 5;
    free(dO), free(dq), free(dk), free(dv), free(dkc), free(dbc), free(dl), free(dD), free(dU);
  }
  free(k), free(v), free(lmk), free(D), free(U), free(kc), free(bc), free(rb), free(rh), free(rp), free(q), free(o);
  free(sel), free(ssc), free(gap), free(lse), free(nsel), free(sc);
  return 0;
}

int main(void) {
  /* B, Hq, Hkv, Hl, d, N, K, r, W */
  const int cases[][9] = {
      {1, 2, 1, 2, 64, 300, 3, 0, 0},      /* ragged tail, K < C */
      {2, 4, 2, 4, 64, 640, 16, 4, 0},     /* K above the chunk count, Q-Cal */
      {1, 4, 2, 2, 128, 515, 4, 0, 192},   /* shared landmark heads, a window */
      {1, 2, 2, 2, 64, 40, 2, 2, 0},       /* no complete chunk */
      {1, 1, 1, 1, 64, 700, 5, 3, 704},    /* a window longer than the sequence */
  };
  for (unsigned c = 0; c < sizeof cases / sizeof cases[0]; ++c) {
    const int* x = cases[c];
    const int rc = run_case(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7], x[8]);
    if (rc) {
      printf("case %u failed (%d)\n", c, rc);
      return 1;
    }
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}

/*
 * HiLS-Attention forward pass: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY (see hils_oracle.h).  Every function follows the
 * steps in the order the pages give them; comments cite the page and section.
 * Plain loops in double precision, libm exp/log, the C library's qsort as the
 * sorting step.  No blocking, fusion or reordering.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - the landmark softmax and the intra-chunk softmax use the same scale
 *     1/sqrt(d) as the chunk score;
 *   - a landmark query attends the S keys of its own chunk only;
 *   - query i scores the complete past chunks c < floor(i/S); its own chunk
 *     floor(i/S) is always attended with a causal mask and takes its exact
 *     log-sum-exp as its score; the own chunk is not part of the top-K budget;
 *   - the local sliding window (aitrends.kr "Technical details": window 512
 *     with S = 64 and top-K = 32; the pages do not say how it joins the
 *     fusion) is taken at chunk granularity: it holds the W/S most recent
 *     chunks, the own one included, keys j <= i only.  It is one fusion entry
 *     whose score is its exact log-sum-exp, and the top-K candidates are the
 *     complete chunks before it, so every key j <= i is in exactly one entry.
 *     W = S is the method without a window;
 *   - with fewer than K past chunks, all of them are selected;
 *   - ties in the chunk score go to the lower chunk index;
 *   - Q-Cal: q^ = q + U_h (D_h q) scores chunks; the raw q attends.
 */
#include "hils_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double ld(const void* p, int dt, int64_t i) {
  if (dt == HR_F64) return ((const double*)p)[i];
  if (dt == HR_F32) return (double)((const float*)p)[i];
  /* bf16: the upper half of an IEEE float */
  uint32_t x = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &x, 4);
  return (double)f;
}

/*
 * Landmark compression (aitrends.kr, "Key contributions" first item and
 * "Methodology"; "Technical details"): the landmark query of chunk c attends
 * the chunk's S keys; the attention weights a_j give the compressed key
 * k'_c = sum_j a_j k_j and the entropy bias b'_c = -sum_j a_j log a_j.
 */
void hr_compress(const hr_shape* s, const void* k, int kdt, const void* lmk, int ldt, double* kc,
                 double* bc) {
  const int B = s->B, Hl = s->Hl, Hkv = s->Hkv, d = s->d, S = s->S, N = s->N;
  const int C = N / S;
  const double tau = 1.0 / sqrt((double)d);
  const int lm_per_kv = Hl / Hkv;
#pragma omp parallel for collapse(3) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int l = 0; l < Hl; ++l)
      for (int c = 0; c < C; ++c) {
        const int kvh = l / lm_per_kv;
        const int64_t lbase = (((int64_t)b * Hl + l) * C + c) * d;
        const int64_t kbase = (((int64_t)b * Hkv + kvh) * N + (int64_t)c * S) * d;
        double* z = (double*)malloc(sizeof(double) * S);
        double m = -INFINITY;
        for (int j = 0; j < S; ++j) {
          double acc = 0.0;
          for (int e = 0; e < d; ++e) acc += ld(lmk, ldt, lbase + e) * ld(k, kdt, kbase + (int64_t)j * d + e);
          z[j] = tau * acc;
          if (z[j] > m) m = z[j];
        }
        double Z = 0.0;
        for (int j = 0; j < S; ++j) Z += exp(z[j] - m);
        double* out = kc + lbase;
        for (int e = 0; e < d; ++e) out[e] = 0.0;
        double ent = 0.0;
        for (int j = 0; j < S; ++j) {
          double a = exp(z[j] - m) / Z;
          for (int e = 0; e < d; ++e) out[e] += a * ld(k, kdt, kbase + (int64_t)j * d + e);
          if (a > 0.0) ent -= a * log(a);
        }
        bc[((int64_t)b * Hl + l) * C + c] = ent;
        free(z);
      }
}

/*
 * Q-Cal (aitrends.kr, "Methodology": a low-rank down/up projection of the
 * query q_i gives q^_i, used only to calibrate the chunk-level score).
 * D_h is [r, d], U_h is [d, r].
 */
void hr_qcal(const hr_shape* s, int h, const double* q, const void* D, const void* U, int wdt,
             double* qhat) {
  const int d = s->d, r = s->r;
  for (int e = 0; e < d; ++e) qhat[e] = q[e];
  if (r <= 0 || !D || !U) return;
  double* t = (double*)malloc(sizeof(double) * r);
  for (int a = 0; a < r; ++a) {
    double acc = 0.0;
    for (int e = 0; e < d; ++e) acc += ld(D, wdt, ((int64_t)h * r + a) * d + e) * q[e];
    t[a] = acc;
  }
  for (int e = 0; e < d; ++e) {
    double acc = 0.0;
    for (int a = 0; a < r; ++a) acc += ld(U, wdt, ((int64_t)h * d + e) * r + a) * t[a];
    qhat[e] += acc;
  }
  free(t);
}

/* chunks in the local window (the own chunk counts) */
static int window_chunks(const hr_shape* s) { return s->W > s->S ? s->W / s->S : 1; }

/* candidate chunks of the query at position pos: complete chunks before the window */
static int candidates(const hr_shape* s, int pos) {
  const int C = s->N / s->S;
  int P = pos / s->S - (window_chunks(s) - 1);
  if (P > C) P = C;
  return P > 0 ? P : 0;
}

/* softmax attention of q over keys [j0, j1) of one KV head: o (normalised) and the LSE */
static double attend_range(const hr_shape* s, const double* q, const void* k, const void* v, int kvdt,
                           int64_t kvbase_row, int j0, int j1, double* o) {
  const int d = s->d;
  const double tau = 1.0 / sqrt((double)d);
  const int n = j1 - j0;
  double* t = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
  double m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    const int64_t kb = (kvbase_row + j0 + j) * d;
    for (int e = 0; e < d; ++e) acc += q[e] * ld(k, kvdt, kb + e);
    t[j] = tau * acc;
    if (t[j] > m) m = t[j];
  }
  double l = 0.0;
  for (int j = 0; j < n; ++j) l += exp(t[j] - m);
  for (int e = 0; e < d; ++e) o[e] = 0.0;
  for (int j = 0; j < n; ++j) {
    double p = exp(t[j] - m) / l;
    const int64_t vb = (kvbase_row + j0 + j) * d;
    for (int e = 0; e < d; ++e) o[e] += p * ld(v, kvdt, vb + e);
  }
  free(t);
  return m + log(l);
}

/*
 * Chunk score (aitrends.kr, "Methodology", the formula with its worked
 * example): s_ic = q^_i . k'_c / sqrt(d) + b'_c.  In HR_EXACT mode the score
 * is the exact log-sum-exp of the chunk, log sum_j exp(q_i . k_j / sqrt(d)),
 * the quantity the surrogate linearises ("Technical details").
 */
int hr_row_scores(const hr_shape* s, int mode, int b, int h, int pos, const void* qrow, int qdt,
                  const void* k, int kvdt, const double* kc, const double* bc, const void* D,
                  const void* U, int wdt, double* out) {
  const int d = s->d, S = s->S, C = s->N / s->S;
  const double tau = 1.0 / sqrt((double)d);
  const int P = candidates(s, pos);
  double* q = (double*)malloc(sizeof(double) * d);
  double* qh = (double*)malloc(sizeof(double) * d);
  for (int e = 0; e < d; ++e) q[e] = ld(qrow, qdt, e);
  if (mode == HR_EXACT) {
    const int kvh = h / (s->Hq / s->Hkv);
    const int64_t row0 = ((int64_t)b * s->Hkv + kvh) * s->N;
    double* tmp = (double*)malloc(sizeof(double) * d);
    for (int c = 0; c < P; ++c) out[c] = attend_range(s, q, k, k, kvdt, row0, c * S, c * S + S, tmp);
    free(tmp);
  } else {
    hr_qcal(s, h, q, D, U, wdt, qh);
    const int lm = h / (s->Hq / s->Hl);
    for (int c = 0; c < P; ++c) {
      const double* kp = kc + (((int64_t)b * s->Hl + lm) * C + c) * d;
      double acc = 0.0;
      for (int e = 0; e < d; ++e) acc += qh[e] * kp[e];
      out[c] = tau * acc + bc[((int64_t)b * s->Hl + lm) * C + c];
    }
  }
  free(q);
  free(qh);
  return P;
}

typedef struct {
  double score;
  int32_t idx;
} cand;

/* order: higher score first; equal scores -> lower chunk index first */
static int by_score_desc(const void* x, const void* y) {
  const cand* a = (const cand*)x;
  const cand* b = (const cand*)y;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->idx > b->idx) - (a->idx < b->idx);
}

static int by_idx_asc(const void* x, const void* y) {
  const cand* a = (const cand*)x;
  const cand* b = (const cand*)y;
  return (a->idx > b->idx) - (a->idx < b->idx);
}

/*
 * One query through the hierarchical factorisation (hotpaper.ai abstract;
 * aitrends.kr "Methodology" calculation flow and "Key contributions"
 * second item; ai-papers.net "How HiLS Attention works", Fig. 1):
 *   1. score every candidate chunk with the surrogate, keep the top K;
 *   2. attend independently inside each selected chunk (intra-chunk softmax);
 *   3. the local window (the own, partial chunk and the W/S - 1 chunks before
 *      it) is attended causally with one softmax; its score is its exact LSE;
 *   4. fuse the per-chunk outputs with a softmax over the chunk scores.
 */
void hr_attend(const hr_shape* s, int mode, int64_t nrows, const int32_t* row_b,
               const int32_t* row_h, const int32_t* row_pos, const void* qrows, int qdt,
               const void* k, const void* v, int kvdt, const double* kc, const double* bc,
               const void* D, const void* U, int wdt, const int32_t* sel_in, double* o,
               int32_t* sel_idx, double* sel_score, double* gap, double* lse_own, int32_t* nsel) {
  const int d = s->d, S = s->S, K = s->K;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < nrows; ++n) {
    const int b = row_b[n], h = row_h[n], pos = row_pos[n];
    const int kvh = h / (s->Hq / s->Hkv);
    const int64_t row0 = ((int64_t)b * s->Hkv + kvh) * s->N;
    const int P = candidates(s, pos);
    const void* qn = (const char*)qrows + (size_t)n * d * (qdt == HR_F64 ? 8 : qdt == HR_F32 ? 4 : 2);

    /* step 1: scores of all past chunks and the top-K */
    double* sc = (double*)malloc(sizeof(double) * (P > 0 ? P : 1));
    hr_row_scores(s, mode == HR_EXACT ? HR_EXACT : HR_LANDMARK, b, h, pos, qn, qdt, k, kvdt, kc, bc, D,
                  U, wdt, sc);
    cand* cs = (cand*)malloc(sizeof(cand) * (P > 0 ? P : 1));
    for (int c = 0; c < P; ++c) {
      cs[c].score = sc[c];
      cs[c].idx = c;
    }
    int ns = 0;
    double g = INFINITY;
    if (mode == HR_GIVEN) {
      cand* chosen = (cand*)malloc(sizeof(cand) * (K > 0 ? K : 1));
      for (int t = 0; t < K; ++t) {
        int c = sel_in[n * K + t];
        if (c >= 0 && c < P) {
          chosen[ns].idx = c;
          chosen[ns].score = sc[c];
          ++ns;
        }
      }
      memcpy(cs, chosen, sizeof(cand) * ns);
      free(chosen);
    } else {
      qsort(cs, P, sizeof(cand), by_score_desc);
      ns = P < K ? P : K;
      if (P > K) g = cs[K - 1].score - cs[K].score;
    }
    qsort(cs, ns, sizeof(cand), by_idx_asc);

    /* steps 2-4 */
    double* q = (double*)malloc(sizeof(double) * d);
    for (int e = 0; e < d; ++e) q[e] = ld(qn, qdt, e);
    double* oc = (double*)malloc(sizeof(double) * d * (ns + 1));
    double* sig = (double*)malloc(sizeof(double) * (ns + 1));
    for (int t = 0; t < ns; ++t) {
      const int c = cs[t].idx;
      attend_range(s, q, k, v, kvdt, row0, c * S, c * S + S, oc + (int64_t)t * d);
      sig[t] = cs[t].score;
    }
    int w0 = (pos / S - (window_chunks(s) - 1)) * S; /* first key of the window */
    if (w0 < 0) w0 = 0;
    const double lse = attend_range(s, q, k, v, kvdt, row0, w0, pos + 1, oc + (int64_t)ns * d);
    sig[ns] = lse;
    double M = -INFINITY;
    for (int t = 0; t <= ns; ++t)
      if (sig[t] > M) M = sig[t];
    double Zs = 0.0;
    for (int t = 0; t <= ns; ++t) Zs += exp(sig[t] - M);
    double* on = o + n * d;
    for (int e = 0; e < d; ++e) on[e] = 0.0;
    for (int t = 0; t <= ns; ++t) {
      const double w = exp(sig[t] - M) / Zs;
      for (int e = 0; e < d; ++e) on[e] += w * oc[(int64_t)t * d + e];
    }

    if (sel_idx)
      for (int t = 0; t < K; ++t) sel_idx[n * K + t] = t < ns ? cs[t].idx : -1;
    if (sel_score)
      for (int t = 0; t < K; ++t) sel_score[n * K + t] = t < ns ? cs[t].score : -INFINITY;
    if (gap) gap[n] = g;
    if (lse_own) lse_own[n] = lse;
    if (nsel) nsel[n] = ns;
    free(sc);
    free(cs);
    free(q);
    free(oc);
    free(sig);
  }
}

/*
 * Dense causal attention, the baseline the pages measure the sparse method
 * against (hotpaper.ai abstract; ai-papers.net "Results"): query n of head
 * row_h[n] at position row_pos[n] attends every key 0..pos of its KV head with
 * one softmax over all of them.
 */
void hr_dense(const hr_shape* s, int64_t nrows, const int32_t* row_b, const int32_t* row_h,
              const int32_t* row_pos, const void* qrows, int qdt, const void* k, const void* v, int kvdt,
              double* o) {
  const int d = s->d;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t n = 0; n < nrows; ++n) {
    double* q = (double*)malloc(sizeof(double) * d);
    for (int e = 0; e < d; ++e) q[e] = ld(qrows, qdt, n * d + e);
    const int kvh = row_h[n] / (s->Hq / s->Hkv);
    const int64_t base = ((int64_t)row_b[n] * s->Hkv + kvh) * s->N;
    attend_range(s, q, k, v, kvdt, base, 0, row_pos[n] + 1, o + n * d);
    free(q);
  }
}

/*
 * Backward pass: the gradients of the forward pass above with respect to every
 * input, for end-to-end retrieval learning (hotpaper.ai abstract and "Key
 * contributions": the training signal reaches the landmark queries and the
 * query calibration through the chunk scores; aitrends.kr "Key contributions").
 * The selection is held fixed (top-K is piecewise constant in its inputs), so
 * this is the exact gradient wherever the selection does not change.
 *
 * For query rows n (row_b/row_h/row_pos, query vectors qrows) with their
 * selections sel_idx [n, K] (-1 padded; the forward's) and output gradients
 * dO [n, d], the chain rule runs through the forward's steps in reverse:
 *   4. fusion:  w = softmax(sigma), o = sum_e w_e o_e  ->
 *      dsigma_e = w_e (dO.o_e - dO.o), do_e = w_e dO;
 *   3. each entry's softmax attention (a selected chunk, or the window with its
 *      exact LSE as the score): logits t_j = tau q.k_j, p = softmax(t) ->
 *      dt_j = p_j (do_e.v_j - do_e.o_e) (+ dsigma_e p_j for the window, whose
 *      score is log sum_j exp t_j), dq += tau sum_j dt_j k_j,
 *      dk_j += tau dt_j q, dv_j += p_j do_e;
 *   2. chunk score s_c = tau q^.k'_c + b'_c -> dq^ += tau dsigma_c k'_c,
 *      dk'_c += tau dsigma_c q^, db'_c += dsigma_c;
 *      Q-Cal q^ = q + U (D q) -> dq += dq^ + D^T (U^T dq^),
 *      dU += dq^ (D q)^T, dD += (U^T dq^) q^T;
 *   1. compression (every chunk with a nonzero dk'_c or db'_c):
 *      a = softmax(z), z_j = tau L_c.k_j, k' = sum a_j k_j, b' = -sum a_j log a_j
 *      -> da_j = dk'.k_j - db' (log a_j + 1), dz_j = a_j (da_j - sum_m a_m da_m),
 *      dL_c = tau sum_j dz_j k_j, dk_j += a_j dk'_c + tau dz_j L_c.
 * Outputs (all overwritten): dq [n, d]; dk, dv [B,Hkv,N,d]; dkc [B,Hl,C,d],
 * dbc [B,Hl,C]; dlmk [B,Hl,C,d]; dD [Hq,r,d], dU [Hq,d,r] (may be NULL when
 * r == 0).  Plain serial loops, fp64.
 */
void hr_attend_backward(const hr_shape* s, int64_t nrows, const int32_t* row_b, const int32_t* row_h,
                        const int32_t* row_pos, const void* qrows, int qdt, const void* k, const void* v,
                        int kvdt, const double* kc, const double* bc, const void* lmk, int ldt, const void* D,
                        const void* U, int wdt, const int32_t* sel_idx, const double* dO, double* dq,
                        double* dk, double* dv, double* dkc, double* dbc, double* dlmk, double* dD, double* dU) {
  const int d = s->d, S = s->S, K = s->K, r = s->r, C = s->N / s->S;
  const double tau = 1.0 / sqrt((double)d);
  const int64_t kv_elems = (int64_t)s->B * s->Hkv * s->N * d;
  const int64_t lm_elems = (int64_t)s->B * s->Hl * C * d;
  memset(dq, 0, sizeof(double) * nrows * d);
  memset(dk, 0, sizeof(double) * kv_elems);
  memset(dv, 0, sizeof(double) * kv_elems);
  memset(dkc, 0, sizeof(double) * lm_elems);
  memset(dbc, 0, sizeof(double) * s->B * s->Hl * C);
  memset(dlmk, 0, sizeof(double) * lm_elems);
  if (r > 0 && dD) memset(dD, 0, sizeof(double) * s->Hq * r * d);
  if (r > 0 && dU) memset(dU, 0, sizeof(double) * s->Hq * d * r);
  double* q = (double*)malloc(sizeof(double) * d);
  double* qh = (double*)malloc(sizeof(double) * d);
  double* dqh = (double*)malloc(sizeof(double) * d);
  double* oe = (double*)malloc(sizeof(double) * d * (K + 1));
  double* o = (double*)malloc(sizeof(double) * d);
  double* sig = (double*)malloc(sizeof(double) * (K + 1));
  int* ent_c = (int*)malloc(sizeof(int) * (K + 1));
  double* t = (double*)malloc(sizeof(double) * (s->N > 0 ? s->N : 1));
  double* tr = (double*)malloc(sizeof(double) * (r > 0 ? r : 1));
  double* ur = (double*)malloc(sizeof(double) * (r > 0 ? r : 1));
  for (int64_t n = 0; n < nrows; ++n) {
    const int b = row_b[n], h = row_h[n], pos = row_pos[n];
    const int kvh = h / (s->Hq / s->Hkv), lm = h / (s->Hq / s->Hl);
    const int64_t row0 = ((int64_t)b * s->Hkv + kvh) * s->N;
    const int P = candidates(s, pos);
    const size_t qsz = qdt == HR_F64 ? 8 : qdt == HR_F32 ? 4 : 2;
    for (int e = 0; e < d; ++e) q[e] = ld((const char*)qrows + (size_t)n * d * qsz, qdt, e);
    hr_qcal(s, h, q, D, U, wdt, qh);
    /* forward, entry by entry: the selected chunks, then the window */
    int ns = 0;
    for (int x = 0; x < K; ++x) {
      const int c = sel_idx[n * K + x];
      if (c < 0 || c >= P) continue;
      const double* kp = kc + (((int64_t)b * s->Hl + lm) * C + c) * d;
      double acc = 0.0;
      for (int e = 0; e < d; ++e) acc += qh[e] * kp[e];
      sig[ns] = tau * acc + bc[((int64_t)b * s->Hl + lm) * C + c];
      attend_range(s, q, k, v, kvdt, row0, c * S, c * S + S, oe + (int64_t)ns * d);
      ent_c[ns++] = c;
    }
    int w0 = (pos / S - (window_chunks(s) - 1)) * S;
    if (w0 < 0) w0 = 0;
    sig[ns] = attend_range(s, q, k, v, kvdt, row0, w0, pos + 1, oe + (int64_t)ns * d);
    double M = -INFINITY, Z = 0.0;
    for (int x = 0; x <= ns; ++x)
      if (sig[x] > M) M = sig[x];
    for (int x = 0; x <= ns; ++x) Z += exp(sig[x] - M);
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    for (int x = 0; x <= ns; ++x)
      for (int e = 0; e < d; ++e) o[e] += exp(sig[x] - M) / Z * oe[(int64_t)x * d + e];
    /* 4. fusion */
    const double* g = dO + n * d;
    double go = 0.0;
    for (int e = 0; e < d; ++e) go += g[e] * o[e];
    for (int e = 0; e < d; ++e) dqh[e] = 0.0;
    double* dqn = dq + n * d;
    for (int x = 0; x <= ns; ++x) {
      const double w = exp(sig[x] - M) / Z;
      const double* ox = oe + (int64_t)x * d;
      double gx = 0.0;
      for (int e = 0; e < d; ++e) gx += g[e] * ox[e];
      const double dsig = w * (gx - go);
      /* 3. the entry's softmax attention; do_e = w g, do_e.o_e = w gx */
      const int window = x == ns;
      const int j0 = window ? w0 : ent_c[x] * S, j1 = window ? pos + 1 : ent_c[x] * S + S;
      double m = -INFINITY;
      for (int j = j0; j < j1; ++j) {
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc += q[e] * ld(k, kvdt, (row0 + j) * d + e);
        t[j - j0] = tau * acc;
        if (t[j - j0] > m) m = t[j - j0];
      }
      double l = 0.0;
      for (int j = j0; j < j1; ++j) l += exp(t[j - j0] - m);
      for (int j = j0; j < j1; ++j) {
        const double p = exp(t[j - j0] - m) / l;
        double gv = 0.0;
        for (int e = 0; e < d; ++e) gv += g[e] * ld(v, kvdt, (row0 + j) * d + e);
        double dt = p * (w * gv - w * gx);
        if (window) dt += dsig * p;
        for (int e = 0; e < d; ++e) {
          dqn[e] += tau * dt * ld(k, kvdt, (row0 + j) * d + e);
          dk[(row0 + j) * d + e] += tau * dt * q[e];
          dv[(row0 + j) * d + e] += p * w * g[e];
        }
      }
      /* 2. the chunk score */
      if (!window) {
        const int64_t ci = ((int64_t)b * s->Hl + lm) * C + ent_c[x];
        for (int e = 0; e < d; ++e) {
          dqh[e] += tau * dsig * kc[ci * d + e];
          dkc[ci * d + e] += tau * dsig * qh[e];
        }
        dbc[ci] += dsig;
      }
    }
    /* Q-Cal */
    for (int e = 0; e < d; ++e) dqn[e] += dqh[e];
    if (r > 0 && D && U) {
      for (int a = 0; a < r; ++a) {
        double acc = 0.0, acc2 = 0.0;
        for (int e = 0; e < d; ++e) {
          acc += ld(D, wdt, ((int64_t)h * r + a) * d + e) * q[e];
          acc2 += ld(U, wdt, ((int64_t)h * d + e) * r + a) * dqh[e];
        }
        tr[a] = acc;   /* D q */
        ur[a] = acc2;  /* U^T dq^ */
      }
      for (int e = 0; e < d; ++e)
        for (int a = 0; a < r; ++a) {
          dqn[e] += ld(D, wdt, ((int64_t)h * r + a) * d + e) * ur[a];
          if (dU) dU[((int64_t)h * d + e) * r + a] += dqh[e] * tr[a];
          if (dD) dD[((int64_t)h * r + a) * d + e] += ur[a] * q[e];
        }
    }
  }
  /* 1. compression */
  double* z = (double*)malloc(sizeof(double) * S);
  double* a = (double*)malloc(sizeof(double) * S);
  double* da = (double*)malloc(sizeof(double) * S);
  for (int b = 0; b < s->B; ++b)
    for (int l = 0; l < s->Hl; ++l)
      for (int c = 0; c < C; ++c) {
        const int64_t ci = ((int64_t)b * s->Hl + l) * C + c;
        int nz = dbc[ci] != 0.0;
        for (int e = 0; e < d && !nz; ++e) nz = dkc[ci * d + e] != 0.0;
        if (!nz) continue;
        const int kvh = l / (s->Hl / s->Hkv);
        const int64_t kb = ((int64_t)b * s->Hkv + kvh) * s->N + (int64_t)c * S;
        double m = -INFINITY, Zc = 0.0;
        for (int j = 0; j < S; ++j) {
          double acc = 0.0;
          for (int e = 0; e < d; ++e) acc += ld(lmk, ldt, ci * d + e) * ld(k, kvdt, (kb + j) * d + e);
          z[j] = tau * acc;
          if (z[j] > m) m = z[j];
        }
        for (int j = 0; j < S; ++j) Zc += exp(z[j] - m);
        double sda = 0.0;
        for (int j = 0; j < S; ++j) {
          a[j] = exp(z[j] - m) / Zc;
          double acc = 0.0;
          for (int e = 0; e < d; ++e) acc += dkc[ci * d + e] * ld(k, kvdt, (kb + j) * d + e);
          da[j] = acc - (a[j] > 0.0 ? dbc[ci] * (log(a[j]) + 1.0) : 0.0);
          sda += a[j] * da[j];
        }
        for (int j = 0; j < S; ++j) {
          const double dz = a[j] * (da[j] - sda);
          for (int e = 0; e < d; ++e) {
            dlmk[ci * d + e] += tau * dz * ld(k, kvdt, (kb + j) * d + e);
            dk[(kb + j) * d + e] += a[j] * dkc[ci * d + e] + tau * dz * ld(lmk, ldt, ci * d + e);
          }
        }
      }
  free(z);
  free(a);
  free(da);
  free(q);
  free(qh);
  free(dqh);
  free(oe);
  free(o);
  free(sig);
  free(ent_c);
  free(t);
  free(tr);
  free(ur);
}

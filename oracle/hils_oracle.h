/*
 * HiLS-Attention forward pass: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code; the product path
 * never does.  It shares no code, header or table with the GPU library.
 *
 * Source: "Hierarchical Sparse Attention Done Right: Toward Infinite Context
 * Modeling" (arXiv 2607.02980), as summarised on the aitrends.kr article
 * (sections "Methodology" and "Technical details"), the hotpaper.ai summary
 * and abstract, and the ai-papers.net article (section "How HiLS Attention
 * works", Fig. 1).
 */
#ifndef HILS_ORACLE_H
#define HILS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type codes of the input arrays */
enum { HR_F32 = 0, HR_BF16 = 1, HR_F64 = 2 };

/* score modes of hr_attend */
enum {
  HR_LANDMARK = 0, /* chunk score = landmark surrogate s_ic = q^.k'_c/sqrt(d) + b'_c  */
  HR_EXACT = 1,    /* chunk score = exact LSE of the query's logits over the chunk    */
  HR_GIVEN = 2     /* selection supplied by the caller; scores are the surrogate      */
};

typedef struct {
  int32_t B, Hq, Hkv, Hl; /* batch, query heads, KV heads, landmark heads           */
  int32_t d, S, K;        /* head dim, chunk size, top-K                           */
  int32_t N;              /* token rows of k/v (prefill length or cache capacity) */
  int32_t r;              /* Q-Cal rank (0: no Q-Cal)                             */
  int32_t W;              /* local window in tokens, a multiple of S (0: S)        */
} hr_shape;

/* Landmark compression of every complete chunk c < N/S:
 *   kc [B,Hl,C,d] (fp64), bc [B,Hl,C] (fp64). */
void hr_compress(const hr_shape* s, const void* k, int kdt, const void* lmk, int ldt, double* kc,
                 double* bc);

/* q^ = q + U_h (D_h q) for one d-vector q of head h (q^ = q when r == 0). */
void hr_qcal(const hr_shape* s, int h, const double* q, const void* D, const void* U, int wdt,
             double* qhat);

/* The scores of every candidate chunk of one query (head h, batch b, position
 * pos): out[c] for c < pos/S - (W/S - 1) (the complete chunks before the local
 * window), in the given mode (HR_LANDMARK or HR_EXACT).  Returns the number of
 * scores written. */
int hr_row_scores(const hr_shape* s, int mode, int b, int h, int pos, const void* qrow, int qdt,
                  const void* k, int kvdt, const double* kc, const double* bc, const void* D,
                  const void* U, int wdt, double* out);

/* The full forward pass for nrows queries.  Query n is the d-vector
 * qrows[n*d ...] of head row_h[n] in batch row_b[n] at position row_pos[n];
 * it attends keys/values k, v [B,Hkv,N,d].
 * Outputs: o [nrows,d]; sel_idx [nrows,K] ascending chunk ids, -1 padded;
 * sel_score [nrows,K] the chunk scores in the same order (-inf padded);
 * gap [nrows] = K-th minus (K+1)-th best score (+inf if no (K+1)-th);
 * lse_own [nrows] (the LSE of the local window, the own chunk when W = S);
 * nsel [nrows].  Any output pointer may be NULL except o. */
void hr_attend(const hr_shape* s, int mode, int64_t nrows, const int32_t* row_b,
               const int32_t* row_h, const int32_t* row_pos, const void* qrows, int qdt,
               const void* k, const void* v, int kvdt, const double* kc, const double* bc,
               const void* D, const void* U, int wdt, const int32_t* sel_in, double* o,
               int32_t* sel_idx, double* sel_score, double* gap, double* lse_own, int32_t* nsel);

/* Backward pass (gradients of hr_attend's output o with the selection held
 * fixed): given the rows of hr_attend, their selections sel_idx [n, K] and the
 * output gradients dO [n, d] (fp64), writes dq [n, d]; dk, dv [B,Hkv,N,d];
 * dkc [B,Hl,C,d], dbc [B,Hl,C] (gradients of k', b'); dlmk [B,Hl,C,d];
 * dD [Hq,r,d], dU [Hq,d,r] (NULL allowed when r == 0).  Surrogate scores only;
 * kc/bc are the forward's compression of k and lmk. */
void hr_attend_backward(const hr_shape* s, int64_t nrows, const int32_t* row_b, const int32_t* row_h,
                        const int32_t* row_pos, const void* qrows, int qdt, const void* k, const void* v,
                        int kvdt, const double* kc, const double* bc, const void* lmk, int ldt, const void* D,
                        const void* U, int wdt, const int32_t* sel_idx, const double* dO, double* dq,
                        double* dk, double* dv, double* dkc, double* dbc, double* dlmk, double* dD, double* dU);

/* Dense causal attention of nrows queries (as in hr_attend) over keys
 * 0..row_pos[n] of their KV head: o [nrows,d]. */
void hr_dense(const hr_shape* s, int64_t nrows, const int32_t* row_b, const int32_t* row_h,
              const int32_t* row_pos, const void* qrows, int qdt, const void* k, const void* v, int kvdt,
              double* o);

#ifdef __cplusplus
}
#endif
#endif

/*
 * hils.h — C ABI of the HiLS-Attention forward pass on AMD Instinct MI355X (gfx950).
 *
 * HiLS ("Hierarchical Landmark Sparse") attention, from "Hierarchical Sparse
 * Attention Done Right: Toward Infinite Context Modeling" (arXiv 2607.02980):
 *   (1) a landmark query per chunk of S keys gives softmax weights a_j over the
 *       chunk; k'_c = sum_j a_j k_j and b'_c = -sum_j a_j log a_j
 *       (aitrends.kr article, "Key contributions" and "Methodology");
 *   (2) query i scores every complete past chunk c < floor(i/S) with
 *       s_ic = q^_i . k'_c / sqrt(d) + b'_c (q^ = Q-Cal-calibrated query) and keeps
 *       the top K; ties go to the lower chunk index ("Methodology", the formula
 *       and its worked example);
 *   (3) the query attends each selected chunk with an independent softmax, and
 *       its own partial chunk causally; the own chunk's score is its exact
 *       log-sum-exp (hotpaper.ai abstract; "Methodology" calculation flow);
 *   (4) the per-chunk outputs are fused with a softmax over the chunk scores
 *       (abstract; aitrends.kr "Key contributions", hierarchical softmax).
 *
 * Local window (aitrends.kr "Technical details": a local sliding window of 512
 * tokens beside S = 64 and top-K = 32; the pages do not say how it joins the
 * fusion).  dims.window = W > S widens the own chunk of (3) to the W/S most
 * recent chunks, the own one included (keys floor(i/S)*S - (W - S) .. i, at
 * least 0): one causal softmax over them, scored by its exact log-sum-exp.
 * The candidates of (2) are then the complete chunks c < floor(i/S) - (W/S - 1)
 * before the window, so every key j <= i lies in exactly one fused entry.
 * W = S (or 0) is the method without a window.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer allocated by the caller, except
 *     `dims`, which is a host pointer.  The library allocates no memory and keeps
 *     no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *     work is enqueued asynchronously on it; no call synchronises (except the
 *     measurement variant hils_attn_prefill_timed).
 *   - Every call validates all arguments before enqueuing anything; on a non-OK
 *     return nothing was enqueued (except HILS_E_HIP, returned when a launch
 *     failed).  hils_last_error() then holds a message (thread-local).
 *   - Layouts are dense row-major ("head-major", as torch SDPA):
 *       q, o       [B, Hq, N, d]        (decode: [B, Hq, d])
 *       k, v       [B, Hkv, N, d]       (decode: the KV cache, N = capacity)
 *       lmk_q      [B, Hlmk, C, d]      landmark queries, C = floor(N / S)
 *       kc         [B, Hlmk, C, d]      fp32, compressed keys k'
 *       bc         [B, Hlmk, C]         fp32, entropy biases b'
 *       qcal_D     [Hq, r, d]           Q-Cal down projection (r = qcal_rank)
 *       qcal_U     [Hq, d, r]           Q-Cal up projection
 *       sel_idx    [B, Hq, N, K] int32  selected chunk ids (decode: [B, Hq, K])
 *       sel_score  [B, Hq, N, K] fp32   their scores s_ic
 *     Query head h uses KV head h / (Hq / Hkv) and landmark head h / (Hq / Hlmk).
 *   - A selection list holds a row's K best chunks (of equal scores the lower chunk
 *     id is kept) in ascending chunk id order; sel_score holds the score of the
 *     chunk in the same slot.  Rows with fewer than K past chunks select all of
 *     them and pad with id -1 and score -inf after them.
 *   - q, k, v, o, lmk_q, qcal_D, qcal_U all have the element type `io`;
 *     kc, bc and sel_score are always fp32.
 *   - The tensor arguments (q, k, v, o, the caches, lmk_q, kc, qcal_D, qcal_U and the
 *     gradients) must be 16-byte aligned, as hipMalloc and torch allocations are: the
 *     kernels move their rows with 16-byte accesses.  A misaligned one returns
 *     HILS_E_INVAL.
 */
#ifndef HILS_H
#define HILS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { HILS_F32 = 0, HILS_BF16 = 1 } hils_dtype_t;

enum {
  HILS_OK = 0,
  HILS_E_INVAL = -1,       /* a required pointer is NULL or a size is inconsistent      */
  HILS_E_UNSUPPORTED = -2, /* legal but not implemented (d, S, K, dtype, head layout)    */
  HILS_E_WORKSPACE = -3,   /* ws_bytes < hils_workspace_bytes(dims, op)                  */
  HILS_E_HIP = -4          /* a HIP launch failed; the runtime's message is kept         */
};

/* op codes of hils_workspace_bytes */
enum {
  HILS_OP_COMPRESS = 0,
  HILS_OP_SCORE_TOPK = 1,
  HILS_OP_PREFILL = 2,
  HILS_OP_DECODE = 3,
  HILS_OP_BACKWARD = 4,
  HILS_OP_DECODE_MIRROR = 5, /* the decode calls over the landmark mirror */
  HILS_OP_DENSE_DECODE = 6   /* hils_dense_decode */
};

typedef struct {
  int32_t B;         /* batch (sequences)                                              */
  int32_t Hq;        /* query heads                                                    */
  int32_t Hkv;       /* KV heads; Hq % Hkv == 0                                        */
  int32_t Hlmk;      /* landmark heads, Hq % Hlmk == 0 and Hlmk % Hkv == 0: Hq (one per */
                     /* query head) or Hkv (one per KV group, shared by its query      */
                     /* heads); the backward pass needs Hlmk == Hq                      */
  int32_t d;         /* head dimension: 64 or 128                                      */
  int32_t S;         /* chunk size: 64                                                 */
  int32_t K;         /* top-K chunks per query: 1 <= K <= 64                            */
  int32_t N;         /* prefill: tokens; decode: KV-cache capacity (row stride of k/v) */
  int32_t qcal_rank; /* Q-Cal rank r, 0 <= r <= 32 (0: no Q-Cal, q^ = q)                */
  int32_t io;        /* hils_dtype_t of q, k, v, o, lmk_q, qcal_D, qcal_U              */
  int32_t window;    /* local window W in tokens, a multiple of S, W <= 32*S; 0 or S:   */
                     /* the own chunk only (see "Local window" above)                   */
} hils_dims_t;

/* Bytes of device workspace the call `op` needs for these dims (0 if none).
 * Returns (size_t)-1 if dims is invalid or unsupported. */
size_t hils_workspace_bytes(const hils_dims_t* dims, int op);

/*
 * Landmark compression, step (1), of chunks c_begin <= c < c_end of every
 * (batch, landmark head):  z_j = lmk_q[b,l,c] . k[b, l/(Hlmk/Hkv), c*S + j] / sqrt(d),
 * a = softmax_j(z), kc[b,l,c] = sum_j a_j k_j, bc[b,l,c] = -sum_j a_j log a_j.
 * Chunks outside [c_begin, c_end) are left untouched, so a decode cache can be
 * extended one completed chunk at a time.  0 <= c_begin <= c_end <= floor(N/S);
 * an empty range does nothing and then k, lmk_q, kc and bc may be NULL.
 * Needs no workspace.
 */
int hils_landmark_compress(const hils_dims_t* dims, const void* k, const void* lmk_q, int32_t c_begin,
                           int32_t c_end, float* kc, float* bc, void* stream);

/*
 * Chunk scoring and top-K, step (2), for a block of Nq queries per (batch, query
 * head): q [B,Hq,Nq,d]; query i of batch b sits at position p = q_pos0[b] + i
 * (q_pos0: [B] int32 on the device, 0 <= q_pos0[b] < 2^30; NULL: every block starts
 * at position 0, as in a prefill of the whole sequence).  It scores the complete
 * chunks c < floor(p/S) - (W/S - 1) of the context held in kc/bc
 * ([B,Hlmk,floor(N/S),d] / [B,Hlmk,floor(N/S)], N = dims.N) with
 * s_ic = q^_i . kc[c] / sqrt(d) + bc[c], q^ = q + U_h (D_h q) when qcal_rank > 0
 * (qcal_D/qcal_U may be NULL only if qcal_rank == 0), and keeps the K best.
 * Writes sel_idx and sel_score [B,Hq,Nq,K] (ascending ids, padded).  0 <= Nq <= N;
 * Nq == 0 does nothing (the arrays may then be NULL).  Needs a workspace of
 * hils_workspace_bytes(dims, HILS_OP_SCORE_TOPK) bytes (sized for Nq = N).
 */
int hils_chunk_score_topk(const hils_dims_t* dims, int32_t Nq, const void* q, const int32_t* q_pos0,
                          const void* qcal_D, const void* qcal_U, const float* kc, const float* bc, int32_t* sel_idx,
                          float* sel_score, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole prefill forward pass, steps (1)-(4), for all N queries of every
 * (batch, query head); writes o [B,Hq,N,d].
 *   lmk_q != NULL: landmark compression runs first in the same call and writes
 *                  kc/bc (which may then be NULL: the workspace holds them);
 *   lmk_q == NULL: kc/bc are inputs (precomputed by hils_landmark_compress).
 * When N < S there is no complete chunk and lmk_q, kc and bc may all be NULL.
 * sel_idx_out/sel_score_out (nullable) receive the selection of step (2).
 * Range: with bf16 I/O each (query, chunk) output travels between kernels as fp16;
 * it is a convex combination of v rows, so it is finite whenever every |v| <= 65504
 * (fp16's largest finite value).  Larger |v| overflow to infinity.  fp32 I/O keeps
 * fp32 outputs and has no such limit.
 */
int hils_attn_prefill(const hils_dims_t* dims, const void* q, const void* k, const void* v, const void* lmk_q,
                      float* kc, float* bc, const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out,
                      float* sel_score_out, void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * hils_attn_prefill for measurement: the same work, plus the GPU time of each
 * stage in milliseconds, taken with HIP events on `stream`, in
 * stage_ms[HILS_PREFILL_STAGES] (a HOST array): [0] landmark compression (0 if
 * lmk_q == NULL), [1] k' preparation and the threshold pass of the top-K,
 * [2] scoring and top-K selection, [3] bucketing of (query, chunk) pairs,
 * [4] intra-chunk attention of the selected chunks, [5] own-chunk attention,
 * [6] fusion.  Unlike every other call it synchronises with the stream before
 * returning.
 */
#define HILS_PREFILL_STAGES 7
int hils_attn_prefill_timed(const hils_dims_t* dims, const void* q, const void* k, const void* v, const void* lmk_q,
                            float* kc, float* bc, const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out,
                            float* sel_score_out, void* o, void* ws, size_t ws_bytes, void* stream,
                            float* stage_ms);

/*
 * One decode step: for every sequence b and query head h, the single query
 * q[b,h] at position seq_lens[b]-1 runs steps (2)-(4) against the KV cache
 * (k_cache/v_cache [B,Hkv,N,d], N = capacity).  seq_lens [B] int32 lives on the
 * device and counts the cached tokens including the current one
 * (1 <= seq_lens[b] <= N; the caller appends the new token's k/v first).
 * kc/bc [B,Hlmk,floor(N/S),d] must hold the compressed keys of every complete
 * chunk c < floor((seq_lens[b]-1)/S) (see hils_landmark_compress).
 * Writes o [B,Hq,d]; sel_idx_out (nullable) [B,Hq,K].
 * Limits of the library: N/S <= 65536 for decode (4M tokens at S = 64), N/S <= 16384
 * for prefill and hils_chunk_score_topk; prefill also needs
 * B*Hq*N*K < 2^32 and N*K < 2^26 (the latter only binds for K > 32).
 */
int hils_attn_decode(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* seq_lens, const float* kc, const float* bc, const void* qcal_D,
                     const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * hils_attn_decode for measurement: the same work, plus the GPU time of each
 * stage in milliseconds (HIP events on `stream`) in stage_ms[HILS_DECODE_STAGES]
 * (a HOST array): [0] chunk scoring scan (with each split's best chunks), [1]
 * the merge into the top-K, [2] chunk gather-attention and fusion.  With bf16 I/O and
 * B*Hq at least the device's compute-unit count the merge runs inside the attention
 * kernel: [1] is then 0 and [2] includes it.  Synchronises with the stream before
 * returning.
 */
#define HILS_DECODE_STAGES 3
int hils_attn_decode_timed(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, const float* kc, const float* bc, const void* qcal_D,
                           const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes,
                           void* stream, float* stage_ms);

/*
 * The landmark mirror: an 8-bit copy of the landmark cache that cuts the bytes the
 * decode scan streams to about a quarter (a decode step reads every past chunk's
 * compressed key for step (2): aitrends.kr "Technical details" on the decode cost;
 * "Methodology" for the score).  kc_mirror: B*Hlmk*floor(N/S)*(d + 8) bytes (device,
 * caller-owned, 16-byte aligned), two planes.  First the codes [B, Hlmk, floor(N/S), d]
 * int8: with m = max_e |kc[b,l,c,e]|, code_e = rint(kc[b,l,c,e] * fl(127 / m)) in
 * [-127, 127] (0 when m = 0; rint rounds half to even).  Then for each (b, l, c) the
 * pair (bc[b,l,c], fl(m / 127)) as fp32 [B, Hlmk, floor(N/S), 2].
 *
 * hils_landmark_mirror writes the mirror of chunks c_begin <= c < c_end from kc/bc
 * (call it wherever kc/bc of those chunks change, e.g. after hils_landmark_compress
 * of the chunk a decode step completes); other chunks are untouched.  Same range rules
 * as hils_landmark_compress; no workspace; asynchronous on `stream`.
 *
 * hils_attn_decode_mirror: hils_attn_decode with the scan over kc_mirror.  Its result
 * is the same as hils_attn_decode's, bit for bit (selection, scores and o): from a
 * chunk's codes the scan takes a lower and an upper bound of its exact fp32 score
 * (the codes' error is at most s/2 per element, so the dot product's is at most
 * (s/2) ||q^||_1; q^ enters as two 8-bit parts, hi + lo/254, whose error adds about
 * 1%, and a margin covers the fp32 sums); each split of 1024 chunks keeps the chunks
 * whose upper bound reaches its own K-th largest lower bound, and per (sequence, head)
 * every kept chunk whose upper bound reaches the K-th largest kept lower bound is
 * rescored exactly from kc/bc in hils_attn_decode's arithmetic; the top K is taken
 * from those.  kc_mirror must hold every chunk that hils_attn_decode would score
 * (c < floor((seq_lens[b]-1)/S), as kc/bc); it may be NULL only when N < S.
 * Workspace: hils_workspace_bytes(dims, HILS_OP_DECODE_MIRROR) (the decode workspace plus
 * the scan's survivor lists); limits as hils_attn_decode.  When many scores lie
 * within the bounds' width of the K-th one (e.g. all equal), the rescoring reads more
 * of kc: the result stays exact, the step gets slower.
 * hils_attn_decode_mirror_timed: the same with stage times as hils_attn_decode_timed
 * ([0] the mirror scan with the rescoring, [1] the top-K merge, [2] attention and
 * fusion).
 */
int hils_landmark_mirror(const hils_dims_t* dims, const float* kc, const float* bc, int32_t c_begin, int32_t c_end,
                         uint8_t* kc_mirror, void* stream);
int hils_attn_decode_mirror(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const float* kc, const float* bc, const uint8_t* kc_mirror,
                            const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws,
                            size_t ws_bytes, void* stream);
int hils_attn_decode_mirror_timed(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* seq_lens, const float* kc, const float* bc,
                                  const uint8_t* kc_mirror, const void* qcal_D, const void* qcal_U,
                                  int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes, void* stream,
                                  float* stage_ms);

/*
 * hils_attn_decode for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same decode step
 * and results, with no workspace argument.  Its scratch memory is a device array inside
 * the library, HILS_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held until the process
 * ends; its address is looked up once per device on the first call.  The call allocates
 * nothing.  Dims whose decode workspace (hils_workspace_bytes(dims, HILS_OP_DECODE))
 * exceeds HILS_NOALLOC_SCRATCH_BYTES return HILS_E_UNSUPPORTED.  Every call on one GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams, other host
 * threads) race and give wrong results; order them on one stream.
 */
#define HILS_NOALLOC_SCRATCH_BYTES (16u << 20)
int hils_attn_decode_noalloc(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, const float* kc, const float* bc, const void* qcal_D,
                             const void* qcal_U, int32_t* sel_idx_out, void* o, void* stream);

/*
 * Chunk-paged KV cache (the pages' chunks are the natural page: ai-papers.net
 * "How HiLS Attention works"; aitrends.kr "Technical details" on decode cost).
 * A page holds one S-token chunk of every KV head: k_pages / v_pages
 * [num_pages, Hkv, S, d] (io dtype, device).  block_table [B, max_blocks] int32
 * (device) gives the page of chunk c of sequence b; only chunks a call reads
 * need valid entries.  dims.N must equal max_blocks * S (the capacity); page ids
 * outside [0, num_pages) are clamped into the pool (wrong values, never an
 * access outside it).  The landmark cache kc/bc stays contiguous
 * [B, Hlmk, max_blocks, d] / [B, Hlmk, max_blocks].
 *
 * hils_landmark_compress_paged: hils_landmark_compress for chunks
 * [c_begin, c_end) of every sequence, reading keys from the pages; call it for
 * the chunk that a decode step completes (incremental compression).
 * hils_attn_decode_paged: hils_attn_decode on the paged cache (same workspace,
 * HILS_OP_DECODE).  hils_attn_decode_paged_mirror: the same step scanning the landmark
 * mirror (hils_landmark_mirror, built from the contiguous kc/bc), with
 * hils_attn_decode_paged's result bit for bit.  All are asynchronous on `stream`.
 */
int hils_landmark_compress_paged(const hils_dims_t* dims, const void* k_pages, const int32_t* block_table,
                                 int32_t max_blocks, int32_t num_pages, const void* lmk_q, int32_t c_begin,
                                 int32_t c_end, float* kc, float* bc, void* stream);
int hils_attn_decode_paged(const hils_dims_t* dims, const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* block_table, int32_t max_blocks, int32_t num_pages, const int32_t* seq_lens,
                           const float* kc, const float* bc, const void* qcal_D, const void* qcal_U,
                           int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes, void* stream);
int hils_attn_decode_paged_mirror(const hils_dims_t* dims, const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* block_table, int32_t max_blocks, int32_t num_pages,
                                  const int32_t* seq_lens, const float* kc, const float* bc, const uint8_t* kc_mirror,
                                  const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * Backward pass of hils_attn_prefill (end-to-end retrieval learning: the training
 * signal reaches the landmark queries and the query calibration through the chunk
 * scores; hotpaper.ai abstract and "Key contributions", aitrends.kr "Key
 * contributions").  Given the forward's inputs, its compressed keys kc, its
 * selection (sel_idx, sel_score: the forward's sel_idx_out / sel_score_out), its
 * output o and the output gradient dO [B,Hq,N,d], writes the gradients of
 * sum(o * dO) with the selection held fixed (top-K is piecewise constant):
 *   dq [B,Hq,N,d], dk, dv [B,Hkv,N,d], dlmk [B,Hlmk,C,d] (landmark queries, through
 *   k' and b'), dD [Hq,r,d], dU [Hq,d,r] (Q-Cal; may be NULL when qcal_rank == 0).
 * bf16 I/O only (HILS_E_UNSUPPORTED otherwise).  Workspace:
 * hils_workspace_bytes(dims, HILS_OP_BACKWARD).  dq is the sum of one bf16 partial per
 * (row, selected chunk) (its attention term and its score term) and the window's fp32
 * term, added in a fixed order and rounded to bf16 once: deterministic.  dk, dv, the
 * landmark and Q-Cal gradients are accumulated in fp32 with float atomics and rounded
 * once, so their low bits depend on timing.
 * lmk_q, kc and dlmk may be NULL when N < S.  Same limits as hils_attn_prefill.
 * Asynchronous on `stream`.
 */
int hils_attn_prefill_backward(const hils_dims_t* dims, const void* q, const void* k, const void* v, const void* lmk_q,
                               const float* kc, const void* qcal_D, const void* qcal_U, const int32_t* sel_idx,
                               const float* sel_score, const void* o, const void* dO, void* dq, void* dk, void* dv,
                               void* dlmk, void* dD, void* dU, void* ws, size_t ws_bytes, void* stream);

/*
 * Dense causal attention, the baseline the pages measure the sparse method
 * against (hotpaper.ai abstract; ai-papers.net "Results"): for every (b, h) and
 * row i, o[b,h,i] = sum_{j <= i} softmax_j(q[b,h,i].k[b,kvh,j] / sqrt(d)) v[b,kvh,j]
 * with kvh = h / (Hq/Hkv).  It uses the same MFMA tiles as the sparse pass.
 * q, o [B,Hq,N,d]; k, v [B,Hkv,N,d] (device, io dtype, contiguous).  dims is
 * validated as for the other calls (S, K, Hlmk and qcal_rank are not used).
 * No workspace; asynchronous on `stream`.
 */
int hils_dense_attention(const hils_dims_t* dims, const void* q, const void* k, const void* v, void* o,
                         void* stream);

/*
 * Dense decode, the baseline of the decode step (the pages compare decode latency with
 * full attention: hotpaper.ai abstract, ai-papers.net "Results"): for every sequence b
 * and query head h, o[b,h] = sum_{j < L_b} softmax_j(q[b,h].k[b,kvh,j] / sqrt(d))
 * v[b,kvh,j], kvh = h / (Hq/Hkv), L_b = seq_lens[b] (clamped to N) -- every cached key,
 * nothing selected.  q, o [B,Hq,d]; k_cache, v_cache [B,Hkv,N,d]; seq_lens [B] (device).
 * bf16 I/O and Hq/Hkv in {1, 2, 4, 8} (HILS_E_UNSUPPORTED otherwise); S, K, Hlmk,
 * qcal_rank and window are not used.  The keys are split into runs of 2048, each read
 * once for the KV group's query heads; the runs' partial softmax sums are merged per
 * (b, h).  Workspace: hils_workspace_bytes(dims, HILS_OP_DENSE_DECODE).  Asynchronous on
 * `stream`.
 */
int hils_dense_decode(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, void* o, void* ws, size_t ws_bytes, void* stream);

/* Message of the last non-OK return on this thread ("" if none). */
const char* hils_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HILS_H */

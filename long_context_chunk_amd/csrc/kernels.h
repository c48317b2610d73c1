// Internal launchers of the HiLS kernels (host side).  io: 0 = fp32, 1 = bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hils {

// Geometry of one call, validated by the ABI layer.
struct Geom {
  int B, Hq, Hkv, Hl, d, S, K, N, r, io;
  int nw = 1;  // chunks in the local window (the own chunk and the nw - 1 before it)
  int C() const { return N / S; }
  int G() const { return Hq / Hkv; }
};

// Where the keys/values of chunk c of (sequence b, KV head kvh) live.  Contiguous caches
// ([B,Hkv,N,d]) have table == nullptr.  Paged caches hold one chunk of every KV head per
// page ([pages,Hkv,64,d]); chunk c of sequence b is page table[b * max_blocks + c].
// Either way the chunk's 64 rows are consecutive d-vectors.
struct KvPages {
  const int32_t* table = nullptr;
  int max_blocks = 0, num_pages = 0;
  // first row of the chunk, in d-vectors from the base pointer; page ids outside the pool
  // are clamped into it (a bad table gives wrong values, never an access outside the pool)
  __device__ __forceinline__ int64_t chunk_row(int b, int kvh, int Hkv, int N, int c) const {
    if (table == nullptr) return ((int64_t)b * Hkv + kvh) * N + (int64_t)c * 64;
    const int p = min(max(table[(int64_t)b * max_blocks + c], 0), num_pages - 1);
    return ((int64_t)p * Hkv + kvh) * 64;
  }
};

hipError_t launch_compress(int io, const void* k, const void* lmk, float* kc, float* bc, int B, int Hkv, int Hl,
                           int N, int d, int c_begin, int c_end, hipStream_t st, KvPages pg = KvPages());

// Bucketing of the (query row, selected chunk) pairs of a prefill selection by bucket
// (b, query head, chunk), numbered head-major: pairs[boff[bk] .. boff[bk+1]) are the pair
// ids (linear indices into sel_idx) of bucket bk; toff[bk] is its first work item of
// BUCKET_ITEM_ROWS pairs, toff[nbk] the total.  counts and cursor hold nbk words each and
// are contiguous (counts first); tmp holds B*Hq*N*K words.
constexpr int BUCKET_ITEM_ROWS = 1024;
struct BucketBufs {
  uint32_t *counts, *cursor, *boff, *toff, *pairs, *tmp;
  uint32_t* imap;  // work item -> bucket (bucket_items_bound entries)
};
void launch_bucket_pairs(const Geom& g, const int32_t* sel, BucketBufs bb, hipStream_t st);
int64_t bucket_items_bound(const Geom& g);  // host bound on the work items (0 if no pairs)

// Backward pass of the prefill forward (bf16 I/O), the selection held fixed.
struct BwdArgs {
  const void *q, *k, *v, *lmk, *D, *U, *o, *dO;
  const float *kc, *sel_score;
  const int32_t* sel_idx;
  void *dq, *dk, *dv, *dlmk, *dD, *dU;
};
size_t backward_workspace_bytes(const Geom& g);
hipError_t launch_backward(const Geom& g, const BwdArgs& a, void* ws, size_t ws_bytes, hipStream_t st);

// Chunk scores and per-row top-K for a block of Nq <= N queries of every (b, h), query i of
// batch b at position pos0[b] + i (pos0 nullable: 0); q, sel_idx, sel_score hold Nq rows per (b, h).
size_t score_workspace_bytes(const Geom& g);
// ev (nullable): two events recorded after the threshold pass and after the selection pass.
hipError_t launch_score_topk(const Geom& g, int Nq, const int32_t* pos0, const void* q, const void* D, const void* U,
                             const float* kc, const float* bc, int32_t* sel_idx, float* sel_score, void* ws,
                             size_t ws_bytes, hipStream_t st, hipEvent_t* ev = nullptr);

// Intra-chunk attention and fusion for prefill, given the selection.
size_t attend_workspace_bytes(const Geom& g);
// ev (nullable): four events recorded after bucketing, chunk attention, own-chunk attention and fusion.
hipError_t launch_prefill_attend(const Geom& g, const void* q, const void* k, const void* v, const int32_t* sel_idx,
                                 const float* sel_score, void* o, void* ws, size_t ws_bytes, hipStream_t st,
                                 hipEvent_t* ev = nullptr);

// One decode step.
// mirror: the workspace of the step over the landmark mirror (it adds the scan's survivor lists)
size_t decode_workspace_bytes(const Geom& g, bool mirror = false);
// kcm (nullable): the 8-bit mirror of kc/bc (launch_mirror); when given, the scan reads it
// and the survivors of its score bounds are rescored exactly from kc/bc.
// ev (nullable): four events recorded before the scan, after it, after the top-K merge, and
// after chunk attention and fusion.
hipError_t launch_decode(const Geom& g, const void* q, const void* kcache, const void* vcache, const int32_t* seq_lens,
                         const float* kc, const float* bc, const uint8_t* kcm, const void* D, const void* U,
                         int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes, hipStream_t st,
                         hipEvent_t* ev = nullptr, KvPages pg = KvPages());
// The mirror of chunks [c_begin, c_end): in a buffer of B*Hlmk*C*(d + 8) bytes, the 8-bit
// codes of k' [B*Hlmk*C, d], then per row b' and the codes' scale as fp32 pairs.
hipError_t launch_mirror(const Geom& g, const float* kc, const float* bc, uint8_t* kcm, int c_begin, int c_end,
                         hipStream_t st);

// Dense causal attention (the baseline).
hipError_t launch_dense(const Geom& g, const void* q, const void* k, const void* v, void* o, hipStream_t st);
size_t dense_decode_workspace_bytes(const Geom& g);
hipError_t launch_dense_decode(const Geom& g, const void* q, const void* k, const void* v, const int32_t* seq_lens,
                               void* o, void* ws, hipStream_t st);

}  // namespace hils

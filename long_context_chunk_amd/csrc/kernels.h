// Internal launchers of the HiLS kernels (host side).  io: 0 = fp32, 1 = bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hils {

// Geometry of one call, validated by the ABI layer.
struct Geom {
  int B, Hq, Hkv, Hl, d, S, K, N, r, io;
  int C() const { return N / S; }
  int G() const { return Hq / Hkv; }
};

hipError_t launch_compress(int io, const void* k, const void* lmk, float* kc, float* bc, int B, int Hkv, int Hl,
                           int N, int d, int c_begin, int c_end, hipStream_t st);

// Chunk scores and per-row top-K for all N queries of every (b, h).
size_t score_workspace_bytes(const Geom& g);
// ev (nullable): two events recorded after the threshold pass and after the selection pass.
hipError_t launch_score_topk(const Geom& g, const void* q, const void* D, const void* U, const float* kc,
                             const float* bc, int32_t* sel_idx, float* sel_score, void* ws, size_t ws_bytes,
                             hipStream_t st, hipEvent_t* ev = nullptr);

// Intra-chunk attention and fusion for prefill, given the selection.
size_t attend_workspace_bytes(const Geom& g);
// ev (nullable): four events recorded after bucketing, chunk attention, own-chunk attention and fusion.
hipError_t launch_prefill_attend(const Geom& g, const void* q, const void* k, const void* v, const int32_t* sel_idx,
                                 const float* sel_score, void* o, void* ws, size_t ws_bytes, hipStream_t st,
                                 hipEvent_t* ev = nullptr);

// One decode step.
size_t decode_workspace_bytes(const Geom& g);
// ev (nullable): four events recorded before the scan, after it, after the top-K merge, and
// after chunk attention and fusion.
hipError_t launch_decode(const Geom& g, const void* q, const void* kcache, const void* vcache, const int32_t* seq_lens,
                         const float* kc, const float* bc, const void* D, const void* U, int32_t* sel_idx_out,
                         void* o, void* ws, size_t ws_bytes, hipStream_t st, hipEvent_t* ev = nullptr);

// Dense causal attention (the baseline).
hipError_t launch_dense(const Geom& g, const void* q, const void* k, const void* v, void* o, hipStream_t st);

}  // namespace hils

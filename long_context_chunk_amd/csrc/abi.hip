// The C ABI of include/hils.h: argument validation, workspace layout and
// dispatch to the kernel launchers.  Nothing is enqueued unless every argument
// is valid.
#include <stdarg.h>
#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <stdio.h>
#include <string.h>

#include "../../include/hils.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(HILS_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The kernels move rows of the tensor arguments with 16-byte vector accesses.  NULL (an
// optional argument left out) passes.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15u) return false;
  return true;
}
int misaligned() { return fail(HILS_E_INVAL, "tensor arguments must be 16-byte aligned device pointers"); }

// Validates dims; on success fills g.  Returns HILS_OK or an error code.
int check_dims(const hils_dims_t* dims, hils::Geom& g) {
  if (!dims) return fail(HILS_E_INVAL, "dims is NULL");
  const hils_dims_t& s = *dims;
  if (s.B < 1 || s.Hq < 1 || s.Hkv < 1 || s.Hlmk < 1 || s.N < 1)
    return fail(HILS_E_INVAL, "B, Hq, Hkv, Hlmk and N must be >= 1 (B=%d Hq=%d Hkv=%d Hlmk=%d N=%d)", s.B, s.Hq,
                s.Hkv, s.Hlmk, s.N);
  if (s.Hq % s.Hkv != 0) return fail(HILS_E_INVAL, "Hq (%d) must be a multiple of Hkv (%d)", s.Hq, s.Hkv);
  if (s.Hq % s.Hlmk != 0 || s.Hlmk % s.Hkv != 0)
    return fail(HILS_E_INVAL, "need Hq %% Hlmk == 0 and Hlmk %% Hkv == 0 (Hq=%d Hlmk=%d Hkv=%d)", s.Hq, s.Hlmk, s.Hkv);
  if (s.K < 1) return fail(HILS_E_INVAL, "K must be >= 1 (K=%d)", s.K);
  if (s.qcal_rank < 0) return fail(HILS_E_INVAL, "qcal_rank must be >= 0 (%d)", s.qcal_rank);
  if (s.d < 1 || s.S < 1) return fail(HILS_E_INVAL, "d and S must be >= 1 (d=%d S=%d)", s.d, s.S);
  if (s.io != HILS_F32 && s.io != HILS_BF16) return fail(HILS_E_UNSUPPORTED, "io dtype %d not supported", s.io);
  if (s.d != 64 && s.d != 128) return fail(HILS_E_UNSUPPORTED, "head dim %d not supported (64 or 128)", s.d);
  if (s.S != 64) return fail(HILS_E_UNSUPPORTED, "chunk size %d not supported (64)", s.S);
  if (s.K > 64) return fail(HILS_E_UNSUPPORTED, "K=%d not supported (K <= 64)", s.K);
  if (s.qcal_rank > 32) return fail(HILS_E_UNSUPPORTED, "qcal_rank=%d not supported (<= 32)", s.qcal_rank);
  if (s.window < 0 || s.window % s.S != 0)
    return fail(HILS_E_INVAL, "window must be a non-negative multiple of S (window=%d S=%d)", s.window, s.S);
  if (s.window > 32 * s.S) return fail(HILS_E_UNSUPPORTED, "window=%d not supported (<= 32*S)", s.window);
  g = hils::Geom{s.B, s.Hq, s.Hkv, s.Hlmk, s.d, s.S, s.K, s.N, s.qcal_rank, s.io, std::max(1, s.window / s.S)};
  return HILS_OK;
}

// Paged K/V: the capacity N must be max_blocks chunks; the table and pool sizes >= 1.
int check_pages(const hils::Geom& g, const int32_t* table, int32_t max_blocks, int32_t num_pages,
                hils::KvPages& pg) {
  if (!table) return fail(HILS_E_INVAL, "block_table must be non-NULL");
  if (max_blocks < 1 || num_pages < 1)
    return fail(HILS_E_INVAL, "max_blocks and num_pages must be >= 1 (%d, %d)", max_blocks, num_pages);
  if ((int64_t)max_blocks * g.S != g.N)
    return fail(HILS_E_INVAL, "dims.N (%d) must equal max_blocks * S (%d * %d)", g.N, max_blocks, g.S);
  pg.table = table;
  pg.max_blocks = max_blocks;
  pg.num_pages = num_pages;
  return HILS_OK;
}

// Prefill-only limits: (row, slot) pair ids are 32-bit, the bucket histograms hold at
// most 16384 chunks, and a bucketing key holds an entry index of one (b, h) below 2^26.
int check_prefill(const hils::Geom& g) {
  if ((int64_t)g.B * g.Hq * (int64_t)g.N * g.K >= ((int64_t)1 << 32))
    return fail(HILS_E_UNSUPPORTED, "prefill needs B*Hq*N*K < 2^32");
  if ((int64_t)g.N * g.K >= ((int64_t)1 << 26))
    return fail(HILS_E_UNSUPPORTED, "prefill needs N*K < 2^26 (N=%d K=%d)", g.N, g.K);
  if (g.C() > 16384) return fail(HILS_E_UNSUPPORTED, "prefill needs N/S <= 16384 (N=%d)", g.N);
  return HILS_OK;
}

// prefill workspace: [kc | bc | sel_idx | sel_score | score workspace | attend workspace]
struct PrefillWs {
  size_t kc, bc, sel_idx, sel_score, score, attend, total;
};
PrefillWs prefill_ws(const hils::Geom& g) {
  PrefillWs w;
  const size_t C = (size_t)g.C(), rows = (size_t)g.B * g.Hq * g.N;
  size_t off = 0;
  w.kc = off;
  off += align_up((size_t)g.B * g.Hl * C * g.d * 4);
  w.bc = off;
  off += align_up((size_t)g.B * g.Hl * C * 4);
  w.sel_idx = off;
  off += align_up(rows * g.K * 4);
  w.sel_score = off;
  off += align_up(rows * g.K * 4);
  w.score = off;
  off += align_up(hils::score_workspace_bytes(g));
  w.attend = off;
  off += align_up(hils::attend_workspace_bytes(g));
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

const char* hils_last_error(void) { return g_err; }

size_t hils_workspace_bytes(const hils_dims_t* dims, int op) {
  hils::Geom g;
  if (check_dims(dims, g) != HILS_OK) return (size_t)-1;
  switch (op) {
    case HILS_OP_COMPRESS:
      return 0;
    case HILS_OP_SCORE_TOPK:
      return hils::score_workspace_bytes(g);
    case HILS_OP_PREFILL:
      if (check_prefill(g) != HILS_OK) return (size_t)-1;
      return prefill_ws(g).total;
    case HILS_OP_BACKWARD:
      if (check_prefill(g) != HILS_OK) return (size_t)-1;
      return hils::backward_workspace_bytes(g);
    case HILS_OP_DENSE_DECODE:
      return hils::dense_decode_workspace_bytes(g);
    case HILS_OP_DECODE:
      if (g.C() > 65536) {
        fail(HILS_E_UNSUPPORTED, "decode needs N/S <= 65536 (N=%d)", g.N);
        return (size_t)-1;
      }
      return hils::decode_workspace_bytes(g);
    case HILS_OP_DECODE_MIRROR:
      if (g.C() > 65536) {
        fail(HILS_E_UNSUPPORTED, "decode needs N/S <= 65536 (N=%d)", g.N);
        return (size_t)-1;
      }
      return hils::decode_workspace_bytes(g, true);
    default:
      fail(HILS_E_INVAL, "unknown op %d", op);
      return (size_t)-1;
  }
}

int hils_landmark_compress(const hils_dims_t* dims, const void* k, const void* lmk_q, int32_t c_begin,
                           int32_t c_end, float* kc, float* bc, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (c_begin < 0 || c_end < c_begin || c_end > g.C())
    return fail(HILS_E_INVAL, "need 0 <= c_begin <= c_end <= N/S (c_begin=%d c_end=%d N/S=%d)", c_begin, c_end, g.C());
  if (c_end == c_begin) {  // nothing to compress: the arrays may be empty (NULL)
    g_err[0] = 0;
    return HILS_OK;
  }
  if (!k || !lmk_q || !kc || !bc) return fail(HILS_E_INVAL, "k, lmk_q, kc and bc must be non-NULL");
  if (!aligned16({k, lmk_q, kc})) return misaligned();
  hipError_t e = hils::launch_compress(g.io, k, lmk_q, kc, bc, g.B, g.Hkv, g.Hl, g.N, g.d, c_begin, c_end,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hils_landmark_compress");
  g_err[0] = 0;
  return HILS_OK;
}

int hils_chunk_score_topk(const hils_dims_t* dims, int32_t Nq, const void* q, const int32_t* q_pos0,
                          const void* qcal_D, const void* qcal_U, const float* kc, const float* bc, int32_t* sel_idx,
                          float* sel_score, void* ws, size_t ws_bytes, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (g.C() > 16384) return fail(HILS_E_UNSUPPORTED, "scoring needs N/S <= 16384 (N=%d)", g.N);
  if (Nq < 0 || Nq > g.N) return fail(HILS_E_INVAL, "need 0 <= Nq <= N (Nq=%d N=%d)", Nq, g.N);
  if (Nq == 0) {  // no query: nothing to do, the arrays may be empty (NULL)
    g_err[0] = 0;
    return HILS_OK;
  }
  if (!q || !sel_idx || !sel_score) return fail(HILS_E_INVAL, "q, sel_idx and sel_score must be non-NULL");
  if (g.C() > 0 && (!kc || !bc)) return fail(HILS_E_INVAL, "kc and bc must be non-NULL");
  if (!aligned16({q, kc, qcal_D, qcal_U})) return misaligned();
  if (g.r > 0 && (!qcal_D || !qcal_U)) return fail(HILS_E_INVAL, "qcal_rank > 0 needs qcal_D and qcal_U");
  const size_t need = hils::score_workspace_bytes(g);
  if (!ws && need > 0) return fail(HILS_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(HILS_E_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
  hipError_t e = hils::launch_score_topk(g, Nq, q_pos0, q, qcal_D, qcal_U, kc, bc, sel_idx, sel_score, ws, ws_bytes,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hils_chunk_score_topk");
  g_err[0] = 0;
  return HILS_OK;
}

}  // extern "C"

namespace {

// hils_attn_prefill with optional stage timing (stage_ms: HILS_PREFILL_STAGES host floats, or NULL)
int run_prefill(const hils_dims_t* dims, const void* q, const void* k, const void* v, const void* lmk_q, float* kc,
                float* bc, const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out, float* sel_score_out, void* o,
                void* ws, size_t ws_bytes, void* stream, float* stage_ms) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if ((rc = check_prefill(g))) return rc;
  if (!q || !k || !v || !o) return fail(HILS_E_INVAL, "q, k, v and o must be non-NULL");
  if (g.C() > 0 && !lmk_q && (!kc || !bc)) return fail(HILS_E_INVAL, "without lmk_q, kc and bc are required inputs");
  if (!aligned16({q, k, v, o, lmk_q, kc, qcal_D, qcal_U})) return misaligned();
  if (g.r > 0 && (!qcal_D || !qcal_U)) return fail(HILS_E_INVAL, "qcal_rank > 0 needs qcal_D and qcal_U");
  const PrefillWs w = prefill_ws(g);
  if (!ws && w.total > 0) return fail(HILS_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", w.total);
  if (ws_bytes < w.total) return fail(HILS_E_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, w.total);
  char* base = (char*)ws;
  float* kcp = kc ? kc : (float*)(base + w.kc);
  float* bcp = bc ? bc : (float*)(base + w.bc);
  int32_t* sel = sel_idx_out ? sel_idx_out : (int32_t*)(base + w.sel_idx);
  float* scr = sel_score_out ? sel_score_out : (float*)(base + w.sel_score);
  hipStream_t st = (hipStream_t)stream;
  constexpr int NS = HILS_PREFILL_STAGES;
  hipEvent_t ev[NS + 1] = {};
  hipError_t e = hipSuccess;
  if (stage_ms) {
    for (int i = 0; i <= NS && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    if (e == hipSuccess) e = hipEventRecord(ev[0], st);
  }
  if (e == hipSuccess && lmk_q && g.C() > 0) {
    e = hils::launch_compress(g.io, k, lmk_q, kcp, bcp, g.B, g.Hkv, g.Hl, g.N, g.d, 0, g.C(), st);
  }
  if (e == hipSuccess && stage_ms) e = hipEventRecord(ev[1], st);
  if (e == hipSuccess)
    e = hils::launch_score_topk(g, g.N, nullptr, q, qcal_D, qcal_U, kcp, bcp, sel, scr, base + w.score,
                                w.attend - w.score, st,
                                stage_ms ? ev + 2 : nullptr);
  if (e == hipSuccess)
    e = hils::launch_prefill_attend(g, q, k, v, sel, scr, o, base + w.attend, w.total - w.attend, st,
                                    stage_ms ? ev + 4 : nullptr);
  if (stage_ms) {
    if (e == hipSuccess) e = hipEventSynchronize(ev[NS]);
    for (int i = 0; i < NS && e == hipSuccess; ++i) e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    for (int i = 0; i <= NS; ++i)
      if (ev[i]) hipEventDestroy(ev[i]);
  }
  if (e != hipSuccess) return hip_fail(e, "hils_attn_prefill");
  g_err[0] = 0;
  return HILS_OK;
}

int run_decode(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* seq_lens, const float* kc, const float* bc, const void* qcal_D, const void* qcal_U,
               int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes, void* stream, float* stage_ms,
               hils::KvPages pg = hils::KvPages(), const uint8_t* kcm = nullptr) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !seq_lens || !o)
    return fail(HILS_E_INVAL, "q, k_cache, v_cache, seq_lens and o must be non-NULL");
  if (g.C() > 0 && (!kc || !bc)) return fail(HILS_E_INVAL, "kc and bc must be non-NULL");
  if (!aligned16({q, k_cache, v_cache, o, kc, qcal_D, qcal_U, kcm})) return misaligned();
  if (g.C() > 65536) return fail(HILS_E_UNSUPPORTED, "decode needs N/S <= 65536 (N=%d)", g.N);
  if (g.r > 0 && (!qcal_D || !qcal_U)) return fail(HILS_E_INVAL, "qcal_rank > 0 needs qcal_D and qcal_U");
  const size_t need = hils::decode_workspace_bytes(g, kcm != nullptr);
  if (!ws && need > 0) return fail(HILS_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(HILS_E_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  constexpr int NS = HILS_DECODE_STAGES;
  hipEvent_t ev[NS + 1] = {};
  hipError_t e = hipSuccess;
  if (stage_ms)
    for (int i = 0; i <= NS && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
  if (e == hipSuccess)
    e = hils::launch_decode(g, q, k_cache, v_cache, seq_lens, kc, bc, kcm, qcal_D, qcal_U, sel_idx_out, o, ws,
                            ws_bytes, st, stage_ms ? ev : nullptr, pg);
  if (stage_ms) {
    if (e == hipSuccess) e = hipEventSynchronize(ev[NS]);
    for (int i = 0; i < NS && e == hipSuccess; ++i) e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    for (int i = 0; i <= NS; ++i)
      if (ev[i]) hipEventDestroy(ev[i]);
  }
  if (e != hipSuccess) return hip_fail(e, "hils_attn_decode");
  g_err[0] = 0;
  return HILS_OK;
}

// The mirror decode calls need the mirror whenever the cache has a complete chunk.
int check_mirror(const hils_dims_t* dims, const uint8_t* kcm) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (g.C() > 0 && !kcm) return fail(HILS_E_INVAL, "kc_mirror must be non-NULL");
  return HILS_OK;
}

// Scratch memory of hils_attn_decode_noalloc: a file-scope device array, one copy per GPU,
// held until the process ends.  Host code never uses the array's name as an address: its
// device address is looked up once per device (with that device current) and cached.
static __device__ __align__(256) unsigned char scratch[HILS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hils_attn_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HILS_E_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hils_attn_decode_noalloc: hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HILS_OK;
}

}  // namespace

extern "C" {

int hils_attn_prefill(const hils_dims_t* dims, const void* q, const void* k, const void* v, const void* lmk_q,
                      float* kc, float* bc, const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out,
                      float* sel_score_out, void* o, void* ws, size_t ws_bytes, void* stream) {
  return run_prefill(dims, q, k, v, lmk_q, kc, bc, qcal_D, qcal_U, sel_idx_out, sel_score_out, o, ws, ws_bytes, stream,
                     nullptr);
}

int hils_attn_prefill_timed(const hils_dims_t* dims, const void* q, const void* k, const void* v, const void* lmk_q,
                            float* kc, float* bc, const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out,
                            float* sel_score_out, void* o, void* ws, size_t ws_bytes, void* stream,
                            float* stage_ms) {
  if (!stage_ms) return fail(HILS_E_INVAL, "stage_ms must be non-NULL");
  return run_prefill(dims, q, k, v, lmk_q, kc, bc, qcal_D, qcal_U, sel_idx_out, sel_score_out, o, ws, ws_bytes, stream,
                     stage_ms);
}

int hils_attn_decode(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* seq_lens, const float* kc, const float* bc, const void* qcal_D,
                     const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes,
                     void* stream) {
  return run_decode(dims, q, k_cache, v_cache, seq_lens, kc, bc, qcal_D, qcal_U, sel_idx_out, o, ws, ws_bytes, stream,
                    nullptr);
}

int hils_attn_decode_timed(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, const float* kc, const float* bc, const void* qcal_D,
                           const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes,
                           void* stream, float* stage_ms) {
  if (!stage_ms) return fail(HILS_E_INVAL, "stage_ms must be non-NULL");
  return run_decode(dims, q, k_cache, v_cache, seq_lens, kc, bc, qcal_D, qcal_U, sel_idx_out, o, ws, ws_bytes, stream,
                    stage_ms);
}

int hils_landmark_mirror(const hils_dims_t* dims, const float* kc, const float* bc, int32_t c_begin, int32_t c_end,
                         uint8_t* kc_mirror, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (c_begin < 0 || c_end < c_begin || c_end > g.C())
    return fail(HILS_E_INVAL, "need 0 <= c_begin <= c_end <= N/S (c_begin=%d c_end=%d N/S=%d)", c_begin, c_end, g.C());
  if (c_end == c_begin) {
    g_err[0] = 0;
    return HILS_OK;
  }
  if (!kc || !bc || !kc_mirror) return fail(HILS_E_INVAL, "kc, bc and kc_mirror must be non-NULL");
  hipError_t e = hils::launch_mirror(g, kc, bc, kc_mirror, c_begin, c_end, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hils_landmark_mirror");
  g_err[0] = 0;
  return HILS_OK;
}

int hils_attn_decode_mirror(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const float* kc, const float* bc, const uint8_t* kc_mirror,
                            const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws,
                            size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_mirror(dims, kc_mirror))) return rc;
  return run_decode(dims, q, k_cache, v_cache, seq_lens, kc, bc, qcal_D, qcal_U, sel_idx_out, o, ws, ws_bytes, stream,
                    nullptr, hils::KvPages(), kc_mirror);
}

int hils_attn_decode_mirror_timed(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* seq_lens, const float* kc, const float* bc,
                                  const uint8_t* kc_mirror, const void* qcal_D, const void* qcal_U,
                                  int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes, void* stream,
                                  float* stage_ms) {
  if (!stage_ms) return fail(HILS_E_INVAL, "stage_ms must be non-NULL");
  int rc;
  if ((rc = check_mirror(dims, kc_mirror))) return rc;
  return run_decode(dims, q, k_cache, v_cache, seq_lens, kc, bc, qcal_D, qcal_U, sel_idx_out, o, ws, ws_bytes, stream,
                    stage_ms, hils::KvPages(), kc_mirror);
}

int hils_attn_decode_noalloc(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, const float* kc, const float* bc, const void* qcal_D,
                             const void* qcal_U, int32_t* sel_idx_out, void* o, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (g.C() > 65536) return fail(HILS_E_UNSUPPORTED, "decode needs N/S <= 65536 (N=%d)", g.N);
  const size_t need = hils::decode_workspace_bytes(g);
  if (need > (size_t)HILS_NOALLOC_SCRATCH_BYTES)
    return fail(HILS_E_UNSUPPORTED, "hils_attn_decode_noalloc: these dims need %zu bytes of scratch, above its %zu",
                need, (size_t)HILS_NOALLOC_SCRATCH_BYTES);
  if (!q || !k_cache || !v_cache || !seq_lens || !o)
    return fail(HILS_E_INVAL, "q, k_cache, v_cache, seq_lens and o must be non-NULL");
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return run_decode(dims, q, k_cache, v_cache, seq_lens, kc, bc, qcal_D, qcal_U, sel_idx_out, o, ws,
                    (size_t)HILS_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int hils_landmark_compress_paged(const hils_dims_t* dims, const void* k_pages, const int32_t* block_table,
                                 int32_t max_blocks, int32_t num_pages, const void* lmk_q, int32_t c_begin,
                                 int32_t c_end, float* kc, float* bc, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  hils::KvPages pg;
  if ((rc = check_pages(g, block_table, max_blocks, num_pages, pg))) return rc;
  if (c_begin < 0 || c_end < c_begin || c_end > g.C())
    return fail(HILS_E_INVAL, "need 0 <= c_begin <= c_end <= N/S (c_begin=%d c_end=%d N/S=%d)", c_begin, c_end, g.C());
  if (c_end == c_begin) {
    g_err[0] = 0;
    return HILS_OK;
  }
  if (!k_pages || !lmk_q || !kc || !bc) return fail(HILS_E_INVAL, "k_pages, lmk_q, kc and bc must be non-NULL");
  hipError_t e = hils::launch_compress(g.io, k_pages, lmk_q, kc, bc, g.B, g.Hkv, g.Hl, g.N, g.d, c_begin, c_end,
                                       (hipStream_t)stream, pg);
  if (e != hipSuccess) return hip_fail(e, "hils_landmark_compress_paged");
  g_err[0] = 0;
  return HILS_OK;
}

int hils_attn_decode_paged(const hils_dims_t* dims, const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* block_table, int32_t max_blocks, int32_t num_pages, const int32_t* seq_lens,
                           const float* kc, const float* bc, const void* qcal_D, const void* qcal_U,
                           int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  hils::KvPages pg;
  if ((rc = check_pages(g, block_table, max_blocks, num_pages, pg))) return rc;
  return run_decode(dims, q, k_pages, v_pages, seq_lens, kc, bc, qcal_D, qcal_U, sel_idx_out, o, ws, ws_bytes, stream,
                    nullptr, pg);
}

int hils_attn_decode_paged_mirror(const hils_dims_t* dims, const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* block_table, int32_t max_blocks, int32_t num_pages,
                                  const int32_t* seq_lens, const float* kc, const float* bc, const uint8_t* kc_mirror,
                                  const void* qcal_D, const void* qcal_U, int32_t* sel_idx_out, void* o, void* ws,
                                  size_t ws_bytes, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if ((rc = check_mirror(dims, kc_mirror))) return rc;
  hils::KvPages pg;
  if ((rc = check_pages(g, block_table, max_blocks, num_pages, pg))) return rc;
  return run_decode(dims, q, k_pages, v_pages, seq_lens, kc, bc, qcal_D, qcal_U, sel_idx_out, o, ws, ws_bytes, stream,
                    nullptr, pg, kc_mirror);
}

int hils_dense_decode(const hils_dims_t* dims, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, void* o, void* ws, size_t ws_bytes, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !seq_lens || !o)
    return fail(HILS_E_INVAL, "q, k_cache, v_cache, seq_lens and o must be non-NULL");
  if (!aligned16({q, k_cache, v_cache, o})) return misaligned();
  if (g.io != HILS_BF16) return fail(HILS_E_UNSUPPORTED, "the dense decode baseline needs bf16 I/O");
  const int G = g.Hq / g.Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(HILS_E_UNSUPPORTED, "the dense decode baseline needs Hq/Hkv in {1, 2, 4, 8} (%d)", G);
  const size_t need = hils::dense_decode_workspace_bytes(g);
  if (!ws || ws_bytes < need) return fail(HILS_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if ((int64_t)g.B * g.Hkv * ((g.N + 2047) / 2048) > 0x7fffffff)
    return fail(HILS_E_UNSUPPORTED, "B*Hkv*ceil(N/2048) must fit a 31-bit grid");
  const hipError_t e = hils::launch_dense_decode(g, q, k_cache, v_cache, seq_lens, o, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hils_dense_decode");
  g_err[0] = 0;
  return HILS_OK;
}

int hils_dense_attention(const hils_dims_t* dims, const void* q, const void* k, const void* v, void* o,
                         void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if (!q || !k || !v || !o) return fail(HILS_E_INVAL, "q, k, v and o must be non-NULL");
  if (!aligned16({q, k, v, o})) return misaligned();
  if ((int64_t)g.B * g.Hq * ((g.N + 127) / 128) > 0x7fffffff)
    return fail(HILS_E_UNSUPPORTED, "B*Hq*ceil(N/128) must fit a 31-bit grid");
  const hipError_t e = hils::launch_dense(g, q, k, v, o, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hils_dense_attention");
  g_err[0] = 0;
  return HILS_OK;
}

int hils_attn_prefill_backward(const hils_dims_t* dims, const void* q, const void* k, const void* v, const void* lmk_q,
                               const float* kc, const void* qcal_D, const void* qcal_U, const int32_t* sel_idx,
                               const float* sel_score, const void* o, const void* dO, void* dq, void* dk, void* dv,
                               void* dlmk, void* dD, void* dU, void* ws, size_t ws_bytes, void* stream) {
  hils::Geom g;
  int rc = check_dims(dims, g);
  if (rc) return rc;
  if ((rc = check_prefill(g))) return rc;
  if (g.io != HILS_BF16) return fail(HILS_E_UNSUPPORTED, "the backward pass needs bf16 I/O");
  if (!q || !k || !v || !o || !dO || !dq || !dk || !dv || !sel_idx || !sel_score)
    return fail(HILS_E_INVAL, "q, k, v, o, dO, dq, dk, dv, sel_idx and sel_score must be non-NULL");
  if (g.C() > 0 && (!lmk_q || !kc || !dlmk))
    return fail(HILS_E_INVAL, "lmk_q, kc and dlmk must be non-NULL when N >= S");
  if (g.r > 0 && (!qcal_D || !qcal_U || !dD || !dU))
    return fail(HILS_E_INVAL, "qcal_D, qcal_U, dD and dU must be non-NULL when qcal_rank > 0");
  if (!aligned16({q, k, v, o, dO, dq, dk, dv, lmk_q, kc, dlmk, qcal_D, qcal_U, dD, dU})) return misaligned();
  const size_t need = hils::backward_workspace_bytes(g);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(HILS_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  const hils::BwdArgs a{q, k, v, lmk_q, qcal_D, qcal_U, o, dO, kc, sel_score, sel_idx, dq, dk, dv, dlmk, dD, dU};
  const hipError_t e = hils::launch_backward(g, a, ws, ws_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hils_attn_prefill_backward");
  g_err[0] = 0;
  return HILS_OK;
}

}  // extern "C"

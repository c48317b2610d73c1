// One decode step: every sequence b has one new query per head at position
// L_b - 1 (L_b = seq_lens[b], the cache length including the current token).
//
//   1. decode_scan    s_c = q^ . k'_c / sqrt(d) + b'_c for every candidate chunk
//                     c < floor((L_b - 1)/S) - (nw - 1), the complete chunks before the
//                     local window of nw chunks  (fp32 GEMV streaming k' from HBM:
//                     the dominant traffic of a decode step).  Each workgroup keeps
//                     the best 32 of its 1024 chunks (64-bit selection keys, bitonic
//                     lane networks); decode_merge merges the splits of a (b, h) into
//                     the exact top-K (ties to the lower chunk id).
//   2. decode_attend  one workgroup per (b, h, selected chunk) plus one per chunk of
//                     the local window (the own chunk causal): gathers the chunk's
//                     K/V rows (coalesced), softmax inside the chunk, o_c and its
//                     score (window chunks: their exact LSE, so that together they
//                     weigh as one softmax over the window); decode_combine fuses
//                     them with the softmax over the scores.
// (aitrends.kr article, "Methodology" and "Main results": sparse KV access gives
// near-constant decode cost; hotpaper.ai abstract: chunk outputs fused by the
// retrieval scores.)
#include <algorithm>

#include "hils_common.h"
#include "keylists.h"
#include "kernels.h"
#include <atomic>
#include <type_traits>

namespace hils {

constexpr int DS_CHUNKS = 1024;  // chunks scored per decode_scan workgroup
constexpr int DS_MAX_SPLIT = 64;  // scan workgroups per (b, h): N/S <= 65536
constexpr int DS_KEEP = 64;      // candidate slots per workgroup (K <= 32 fills 32 of them)
#ifndef DSM_UNR
#define DSM_UNR 2                // chunk passes per register buffer of the mirror scan
#endif

struct DecodeWs {
  size_t cand, sel_i, sel_s, nsel, part, sig, mcnt, ment, total;
};
// a survivor of the mirror scan: chunk, lower and upper bound of its exact score
struct MirrorEnt {
  int32_t c;
  float lo, up;
};
static size_t al2(size_t x) { return (x + 255) / 256 * 256; }
static int nsplit_of(const Geom& g) { return (g.C() + DS_CHUNKS - 1) / DS_CHUNKS; }
static DecodeWs decode_ws(const Geom& g, bool mirror = false) {
  DecodeWs w;
  const size_t bh = (size_t)g.B * g.Hq;
  size_t off = 0;
  w.cand = off;
  off += al2(bh * std::max(1, nsplit_of(g)) * DS_KEEP * 8);
  w.sel_i = off;
  off += al2(bh * g.K * 4);
  w.sel_s = off;
  off += al2(bh * g.K * 4);
  w.nsel = off;
  off += al2(bh * 4);
  w.part = off;
  off += al2(bh * (g.K + g.nw) * g.d * 4);
  w.sig = off;
  off += al2(bh * (g.K + g.nw) * 4);
  w.mcnt = w.ment = off;
  if (mirror) {   // the mirror scan's survivor lists: a count and up to DS_CHUNKS entries per split
    off += al2(bh * std::max(1, nsplit_of(g)) * 4);
    w.ment = off;
    off += al2(bh * std::max(1, nsplit_of(g)) * (size_t)DS_CHUNKS * sizeof(MirrorEnt));
  }
  w.total = off;
  return w;
}
size_t decode_workspace_bytes(const Geom& g, bool mirror) { return decode_ws(g, mirror).total; }

// 64-bit selection keys (make_key: larger = better, ties to the lower chunk; 0 = none)
// exchanged with lane j ^ X of the same 32-lane half
template <int X>
HILS_DEV uint64_t dxl(uint64_t v) {
  const int j = threadIdx.x & 31;
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  if constexpr (X == 16) {
    lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)lo, 0x401F);
    hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)hi, 0x401F);
  } else if constexpr (X == 31) {
    lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)lo, 0x7C1F);
    hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)hi, 0x7C1F);
  } else {
    lo = (uint32_t)__shfl_xor((int)lo, X);
    hi = (uint32_t)__shfl_xor((int)hi, X);
  }
  (void)j;
  return ((uint64_t)hi << 32) | lo;
}
template <int X>
HILS_DEV void dcx(uint64_t& k, bool keep_larger) {
  const uint64_t p = dxl<X>(k);
  k = ((p > k) == keep_larger) ? p : k;
}
// bitonic sort of one key per lane, best first, within each 32-lane half
HILS_DEV void dsort32(uint64_t& k) {
  const int j = threadIdx.x & 31;
#define HILS_STAGE(K_, X_) dcx<X_>(k, ((j & X_) == 0) == (((j & K_) == 0) || K_ == 32));
  HILS_STAGE(2, 1)
  HILS_STAGE(4, 2) HILS_STAGE(4, 1)
  HILS_STAGE(8, 4) HILS_STAGE(8, 2) HILS_STAGE(8, 1)
  HILS_STAGE(16, 8) HILS_STAGE(16, 4) HILS_STAGE(16, 2) HILS_STAGE(16, 1)
  HILS_STAGE(32, 16) HILS_STAGE(32, 8) HILS_STAGE(32, 4) HILS_STAGE(32, 2) HILS_STAGE(32, 1)
#undef HILS_STAGE
}
// merge the sorted (best-first) list nk into the sorted list lk of each half; keep 32
HILS_DEV void dmerge_sorted(uint64_t& lk, uint64_t nk) {
  const int j = threadIdx.x & 31;
  const uint64_t r = dxl<31>(nk);
  lk = r > lk ? r : lk;
  dcx<16>(lk, (j & 16) == 0);
  dcx<8>(lk, (j & 8) == 0);
  dcx<4>(lk, (j & 4) == 0);
  dcx<2>(lk, (j & 2) == 0);
  dcx<1>(lk, (j & 1) == 0);
}
// merge unsorted keys nk into the sorted list lk of each half; keep 32
HILS_DEV void dmerge(uint64_t& lk, uint64_t nk) {
  dsort32(nk);
  dmerge_sorted(lk, nk);
}

// The best 32 of the 1024 keys in LDS, sorted, in half 0 of wave 0 (256 threads; every
// thread calls it): each half-wave sorts 4 x 32 keys, the halves of a wave and then the
// four waves are merged.
HILS_DEV uint64_t best32_of_1024(const uint64_t* keys, uint64_t (*wl)[64]) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, j = lane & 31;
  {
    const int base = w * 256 + (lane >> 5) * 128 + j;
    uint64_t lk = keys[base];
    dsort32(lk);
    dmerge(lk, keys[base + 32]);
    dmerge(lk, keys[base + 64]);
    dmerge(lk, keys[base + 96]);
    dmerge_sorted(lk, __shfl(lk, j + 32));
    if (lane < 32) wl[w][lane] = lk;
  }
  __syncthreads();
  uint64_t lk = wl[(lane >> 5) * 2][j];   // halves merge waves 0+1 and 2+3, then each other
  dmerge_sorted(lk, wl[(lane >> 5) * 2 + 1][j]);
  dmerge_sorted(lk, __shfl(lk, j + 32));
  __syncthreads();   // wl may be reused
  return lk;
}

// The best 64 of the 1024 keys in LDS, as a sorted 64-list (hi, lo) in half 0 of wave 0
// (every thread of the block calls it; the first four waves do the work): each half-wave
// sorts 4 x 32 keys into a 64-list, the halves of a wave and then the four waves are merged.
HILS_DEV void best64_of_1024(const uint64_t* keys, uint64_t (*wl)[64], uint64_t& hi, uint64_t& lo) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, j = lane & 31;
  hi = lo = 0ull;
  if (w < 4) {
    const int base = w * 256 + (lane >> 5) * 128 + j;
    hi = keys[base];
    lo = keys[base + 32];
    uint64_t nk = keys[base + 64];
    kl::sort(hi, j);
    kl::sort(lo, j);
    kl::split(hi, lo, j);
    kl::sort(nk, j);
    kl::insert64(hi, lo, nk, j);
    nk = keys[base + 96];
    kl::sort(nk, j);
    kl::insert64(hi, lo, nk, j);
    kl::merge64(hi, lo, __shfl(hi, j + 32), __shfl(lo, j + 32), j);
    if (lane < 32) {
      wl[w][lane] = hi;
      wl[w][32 + lane] = lo;
    }
  }
  __syncthreads();
  if (w < 4) {
    const int a = (lane >> 5) * 2;   // wave 0: halves merge waves 0+1 and 2+3, then each other
    hi = wl[a][j];
    lo = wl[a][32 + j];
    kl::merge64(hi, lo, wl[a + 1][j], wl[a + 1][32 + j], j);
    kl::merge64(hi, lo, __shfl(hi, j + 32), __shfl(lo, j + 32), j);
  }
  __syncthreads();   // wl may be reused
}

// q^ = q + U (D q) for one head into LDS (fp32).  256 threads.
template <typename IO, int D>
HILS_DEV void qhat_to_lds(const IO* __restrict__ qv, const IO* __restrict__ Dw, const IO* __restrict__ Uw, int h, int r,
                          float* qs, float* ts) {
  const int t = threadIdx.x;
  if (t < D) qs[t] = io_traits<IO>::load(qv, t);
  __syncthreads();
  if (r > 0) {
    if (t < r) {
      float a = 0.f;
      for (int e = 0; e < D; ++e) a = fmaf(io_traits<IO>::load(Dw, ((int64_t)h * r + t) * D + e), qs[e], a);
      ts[t] = a;
    }
    __syncthreads();
    float add = 0.f;
    if (t < D)
      for (int a = 0; a < r; ++a) add = fmaf(io_traits<IO>::load(Uw, ((int64_t)h * D + t) * r + a), ts[a], add);
    __syncthreads();
    if (t < D) qs[t] += add;
    __syncthreads();
  }
}

// KB (32 < K <= 64): each workgroup keeps its best 64 as a sorted 64-list (keylists.h)
template <typename IO, int D, bool KB>
__global__ void __launch_bounds__(256) decode_scan(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                   const IO* __restrict__ Uw, const float* __restrict__ kc,
                                                   const float* __restrict__ bc, const int32_t* __restrict__ seq_lens,
                                                   uint64_t* __restrict__ cand, int Hq, int Hl, int C, int r,
                                                   int nsplit, int nw) {
  __shared__ __align__(16) float qs[D];
  __shared__ float ts[32];
  __shared__ uint64_t keys[DS_CHUNKS];
  __shared__ uint64_t wl[4][64];
  const int sp = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;
  const int b = bh / Hq, h = bh % Hq;
  const int L = seq_lens[b];
  const int P = candidate_chunks(L - 1, C, nw);
  const int c_beg = sp * DS_CHUNKS, c_end = min(P, c_beg + DS_CHUNKS);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  // TPC threads per chunk, each holding 16 of the D head dims as 4 float4 spread so
  // that the TPC lanes of a chunk read 128 contiguous bytes per load
  constexpr int TPC = D / 16;
  constexpr int CPP = 256 / TPC;    // chunks per pass
  constexpr int UNR = 2;            // passes per register buffer
  constexpr int STEP = CPP * UNR;
  const int sub = t % TPC, grp = t / TPC;
  const float tau = 1.0f / sqrtf((float)D);
  const int64_t lrow = (int64_t)b * Hl + h / (Hq / Hl);   // the query head's landmark head
  const float* kb = kc + lrow * C * D;
  const float* bb = bc + lrow * C;
  // the landmark keys are streamed once (non-temporal loads); chunks beyond c_end load
  // chunk c_end - 1 (in bounds) and are dropped; two register buffers alternate so that
  // the next STEP chunks are in flight while the current ones are scored
  f32x4_t ka[UNR][4], kb2[UNR][4];
  float ba[UNR], bb2[UNR];
  auto load = [&](int c0, f32x4_t(&kv)[UNR][4], float(&bv)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = min(c0 + u * CPP + grp, c_end - 1);
      const f32x4_t* row = reinterpret_cast<const f32x4_t*>(kb + (int64_t)c * D);
#pragma unroll
      for (int j = 0; j < 4; ++j) kv[u][j] = __builtin_nontemporal_load(row + sub + TPC * j);
      bv[u] = bb[c];
    }
  };
  // the first buffer's loads go out before q^ is prepared (they do not depend on it)
  if (c_beg < c_end) load(c_beg, ka, ba);
  qhat_to_lds<IO, D>(q + (int64_t)bh * D, Dw, Uw, h, r, qs, ts);
  f32x4_t qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qv[j] = *reinterpret_cast<const f32x4_t*>(&qs[4 * (sub + TPC * j)]);
  auto score = [&](int c0, const f32x4_t(&kv)[UNR][4], const float(&bv)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = fmaf(qv[j].x, kv[u][j].x, s);
        s = fmaf(qv[j].y, kv[u][j].y, s);
        s = fmaf(qv[j].z, kv[u][j].z, s);
        s = fmaf(qv[j].w, kv[u][j].w, s);
      }
#pragma unroll
      for (int o = TPC / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      const int c = c0 + u * CPP + grp;
      if (sub == 0) keys[c - c_beg] = c < c_end ? make_key(fmaf(s, tau, bv[u]), c) : 0ull;
    }
  };
  // every load is issued whether or not its chunks are live (they clamp in bounds): with a
  // fixed number of loads in flight the compiler waits for exactly the buffer it uses next
  static_assert(DS_CHUNKS % (2 * STEP) == 0, "");
  constexpr int NIT = DS_CHUNKS / (2 * STEP);
  if (c_beg < c_end) {   // uniform
    for (int it = 0; it < NIT - 1; ++it) {
      const int c0 = c_beg + it * 2 * STEP;
      load(c0 + STEP, kb2, bb2);
      score(c0, ka, ba);
      load(c0 + 2 * STEP, ka, ba);
      score(c0 + STEP, kb2, bb2);
    }
    const int c0 = c_beg + (NIT - 1) * 2 * STEP;
    load(c0 + STEP, kb2, bb2);
    score(c0, ka, ba);
    score(c0 + STEP, kb2, bb2);
  } else {
    for (int x = threadIdx.x; x < DS_CHUNKS; x += 256) keys[x] = 0ull;
  }
  __syncthreads();
  // best 32 (KB: 64) of this workgroup's chunks: each half-wave sorts 4 x 32 keys, the
  // halves and then the four waves are merged
  uint64_t* out = cand + ((int64_t)bh * nsplit + sp) * DS_KEEP;
  const int j = lane & 31;
  if constexpr (!KB) {
    const uint64_t lk = best32_of_1024(keys, wl);
    if (lane < 32 && w == 0) out[lane] = lk;
  } else {
    uint64_t hi, lo;
    best64_of_1024(keys, wl, hi, lo);
    if (lane < 32 && w == 0) {
      out[lane] = hi;
      out[32 + lane] = lo;
    }
  }
}

// The caller's copy of a (b, h)'s selection: the chunk ids of the first min(K, n) ranks of
// the sorted 64-list (hi, lo) of half 0 (ranks 0..31, 32..63) in ascending order, -1 after
// them.  Called by all 64 lanes of one wave; half 0 writes.
HILS_DEV void write_sel_ascending(uint64_t hi, uint64_t lo, int K, int n, int lane, int32_t* __restrict__ sel) {
  const int j = lane & 31, m = min(K, n);
  // float keys in [1, 2) whose bits hold 0xffff - chunk (chunk < 65536): larger for a lower
  // chunk; 0 for no chunk, which sorts last
  auto fkey = [](uint64_t k) { return __uint_as_float(0x3f800000u | ((0xffffu - (uint32_t)key_chunk(k)) << 7)); };
  auto chunk = [](float f) { return f != 0.f ? (int32_t)(0xffffu - ((__float_as_uint(f) >> 7) & 0xffffu)) : -1; };
  float a = j < m && hi ? fkey(hi) : 0.f;
  float b = 32 + j < m && lo ? fkey(lo) : 0.f;
  float pinf = INFINITY, ninf = -INFINITY;
  asm volatile("" : "+v"(pinf));
  asm volatile("" : "+v"(ninf));
  kl::sortf(a, j, pinf, ninf);
  if (m > 32) {
    kl::sortf(b, j, pinf, ninf);
    kl::splitf(a, b, j, pinf, ninf);
  }
  if (lane < 32) {
    if (j < K) sel[j] = chunk(a);
    if (32 + j < K) sel[32 + j] = chunk(b);
  }
}

// exact top-K of one (b, h) from the sorted candidate lists of its splits (cb: the first
// list), rank order, ties to the lowest id; n = min(K, candidate chunks).  Every thread of
// the block calls it (it has a block-wide barrier); the first four waves do the work:
// half-wave x of wave w takes lists 2w + x, 2w + x + 8, 2w + x + 16, ..., the halves of each
// wave merge, then wave 0 merges the four wave lists and writes ranks < K to out_i / out_s
// (chunk ids, -1 past n), and sel_user when given (the same ids in ascending order).
template <bool KB>
HILS_DEV void merge_splits(const uint64_t* __restrict__ cb, int nsplit, int K, int n, uint64_t (*wl)[64],
                           int32_t* out_i, float* out_s, int32_t* __restrict__ sel_user) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int j = lane & 31;
  const int li = 2 * w + (lane >> 5);
  // the best 32 (KB: 64) of all splits, sorted, in half 0 of wave 0 (half 1 ends up with a
  // list merged with itself); key of rank `lane`: hi of lane j < 32, lo of lane j of half 0
  // for ranks 32 + j
  uint64_t hi = 0, lo = 0;
  auto ld = [&](int l, int off) { return l < nsplit ? cb[l * DS_KEEP + off + j] : 0ull; };  // empty lists: zero keys
  if (w < 4) {
    // the same number of lists in every half-wave (empty ones are zero keys)
    if constexpr (!KB) {
      hi = ld(li, 0);
      for (int l0 = 8; l0 < nsplit; l0 += 8) dmerge_sorted(hi, ld(li + l0, 0));
      dmerge_sorted(hi, __shfl(hi, j + 32));
      if (lane < 32) wl[w][lane] = hi;
    } else {
      hi = ld(li, 0);
      lo = ld(li, 32);
      for (int l0 = 8; l0 < nsplit; l0 += 8) kl::merge64(hi, lo, ld(li + l0, 0), ld(li + l0, 32), j);
      kl::merge64(hi, lo, __shfl(hi, j + 32), __shfl(lo, j + 32), j);
      if (lane < 32) {
        wl[w][lane] = hi;
        wl[w][32 + lane] = lo;
      }
    }
  }
  __syncthreads();
  if (w != 0) return;
  if constexpr (!KB) {
    hi = wl[(lane >> 5) * 2][j];
    dmerge_sorted(hi, wl[(lane >> 5) * 2 + 1][j]);
    dmerge_sorted(hi, __shfl(hi, j + 32));
  } else {
    const int a = (lane >> 5) * 2;
    hi = wl[a][j];
    lo = wl[a][32 + j];
    kl::merge64(hi, lo, wl[a + 1][j], wl[a + 1][32 + j], j);
    kl::merge64(hi, lo, __shfl(hi, j + 32), __shfl(lo, j + 32), j);
  }
  const uint64_t lo0 = __shfl(lo, j);   // half 0's ranks 32 + j
  const uint64_t lk = lane < 32 ? hi : lo0;
  if (lane < K) {
    const bool ok = lane < n && lk != 0;
    out_i[lane] = ok ? key_chunk(lk) : -1;
    out_s[lane] = ok ? key_score(lk) : -INFINITY;
  }
  if (sel_user) write_sel_ascending(hi, lo0, K, n, lane, sel_user);
}

template <bool KB>
__global__ void __launch_bounds__(256) decode_merge(const uint64_t* __restrict__ cand,
                                                    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_i,
                                                    float* __restrict__ sel_s, int32_t* __restrict__ nsel_out,
                                                    int32_t* __restrict__ sel_user, int Hq, int C, int K, int nsplit,
                                                    int nw) {
  __shared__ uint64_t wl[4][64];
  const int bh = blockIdx.x;
  const int n = min(K, candidate_chunks(seq_lens[bh / Hq] - 1, C, nw));
  merge_splits<KB>(cand + (int64_t)bh * nsplit * DS_KEEP, nsplit, K, n, wl, sel_i + (int64_t)bh * K,
                   sel_s + (int64_t)bh * K, sel_user ? sel_user + (int64_t)bh * K : nullptr);
  if (threadIdx.x == 0) nsel_out[bh] = n;
}

// Per-head selection over the mirror scan's survivor lists (1024 threads; every thread of
// the block calls it).  Every split's list holds its chunks with U >= its own threshold,
// which include its n chunks with the largest L; so the n-th largest L over all lists is
// at most the n-th largest L of the head, hence at most its n-th best exact score (taken
// over the first 1024 entries only when the lists hold more: a subset gives a smaller, still
// valid threshold).  Every chunk of the exact top n has U >= theta; those entries are
// rescored exactly from kc/bc in decode_scan's arrangement and arithmetic (same lanes, same
// order of sums, so decode_scan's bits), in batches of 1024 entries, and the best 64 exact
// keys are kept.  Writes ranks < K (chunk ids, -1 past n, and their scores).
struct MirrorSelSmem {
  float qs[128];
  float ts[32];
  int cnt[DS_MAX_SPLIT], off[DS_MAX_SPLIT + 1], tot;
  float thw[16];
  int wcnt[16];
  int hist[256];
  int sel_b, sel_above;
  __align__(16) float eL[DS_CHUNKS];
  float eU[DS_CHUNKS];
  int eC[DS_CHUNKS], surv[DS_CHUNKS];
  uint64_t keys[DS_CHUNKS];
  uint64_t wl[4][64];
  uint64_t run[64];
};

template <typename IO, int D>
HILS_DEV void mirror_select(const IO* __restrict__ qv, const IO* __restrict__ Dw, const IO* __restrict__ Uw, int h,
                            int r, const float* __restrict__ kb, const float* __restrict__ bb,
                            const int32_t* __restrict__ cnts, const MirrorEnt* __restrict__ ents, int nsplit, int K,
                            int n, MirrorSelSmem& sm, int32_t* out_i, float* out_s, int32_t* __restrict__ sel_user) {
  constexpr int NT = 1024;
  static_assert(NT == DS_CHUNKS, "one entry per thread in a batch");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, j = lane & 31;
  // the counts and the first 64 entries of the first 16 lists are loaded together, before
  // the counts are known (thread t: list t / 64, entry t % 64; lists hold up to 1024 entries)
  const int32_t cnt_t = t < nsplit ? cnts[t] : 0;
  const MirrorEnt pre = t / 64 < nsplit ? ents[(int64_t)(t / 64) * DS_CHUNKS + (t % 64)] : MirrorEnt{0, 0.f, 0.f};
  qhat_to_lds<IO, D>(qv, Dw, Uw, h, r, sm.qs, sm.ts);   // block-wide barriers inside
  if (t < nsplit) sm.cnt[t] = cnt_t;
  if (t < 64) sm.run[t] = 0ull;
  __syncthreads();
  if (t == 0) {
    int o = 0;
    for (int s2 = 0; s2 < nsplit; ++s2) {
      sm.off[s2] = o;
      o += sm.cnt[s2];
    }
    sm.off[nsplit] = o;
    sm.tot = o;
  }
  __syncthreads();
  const int tot = sm.tot;
  auto entry = [&](int x) {   // entry x of the lists laid end to end
    int s2 = 0;
    while (x >= sm.off[s2 + 1]) ++s2;
    return ents[(int64_t)s2 * DS_CHUNKS + (x - sm.off[s2])];
  };
  // theta over the first batch: the preloaded entries go to their place in it; the
  // (rare) entries past 64 of a list are loaded now
  const int m1 = min(tot, DS_CHUNKS);
  sm.eL[t] = -INFINITY;
  __syncthreads();
  {
    const int l = t / 64, i = t % 64;
    if (l < nsplit && i < sm.cnt[l]) {
      const int x = sm.off[l] + i;
      if (x < m1) {
        sm.eL[x] = pre.lo;
        sm.eU[x] = pre.up;
        sm.eC[x] = pre.c;
      }
    }
    for (int x = t; x < m1; x += 1024) {
      int s2 = 0;
      while (x >= sm.off[s2 + 1]) ++s2;
      const int i2 = x - sm.off[s2];
      if (i2 >= 64 || s2 >= NT / 64) {   // not preloaded
        const MirrorEnt e = ents[(int64_t)s2 * DS_CHUNKS + i2];
        sm.eL[x] = e.lo;
        sm.eU[x] = e.up;
        sm.eC[x] = e.c;
      }
    }
  }
  __syncthreads();
  // theta: a radix select of the n-th largest L over the first batch on order_f32(L),
  // 8 bits at a time for the top 16: the smallest value with the 16 bits found has at
  // least n entries at or above it, so it is at most the n-th largest L
  float theta = -INFINITY;
  if (n > 0) {   // uniform
    const uint32_t key = t < m1 ? order_f32(sm.eL[t]) : 0u;
    uint32_t found = 0u;
    int above = 0;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = 24 - 8 * pass;
      if (t < 256) sm.hist[t] = 0;
      __syncthreads();
      if (t < m1 && (pass == 0 || (key >> 24) == (found >> 24))) atomicAdd(&sm.hist[(key >> shift) & 255u], 1);
      __syncthreads();
      if (w == 0) {   // the largest bucket whose count from the top reaches n
        int c4 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) c4 += sm.hist[4 * lane + i];
        int suf = c4;   // sum over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_down(suf, o);
          suf += lane + o < 64 ? v : 0;
        }
        // within the lane's 4 buckets, from the top
        int run = suf - c4 + above, bk = -1;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          const int hv = sm.hist[4 * lane + i];
          if (bk < 0 && run + hv >= n) bk = 4 * lane + i;
          if (bk < 0) run += hv;
        }
        // the highest lane that found one holds the answer
        const uint64_t bal = __ballot(bk >= 0);
        const int src = bal ? 63 - __builtin_clzll(bal) : 0;
        // no bucket (fewer than n entries, which the lists rule out): bucket 0, theta tiny
        const int bsel = bal ? __shfl(bk, src) : 0, asel = bal ? __shfl(run, src) : 0;
        if (lane == 0) {
          sm.sel_b = bsel;
          sm.sel_above = asel;
        }
      }
      __syncthreads();
      found |= (uint32_t)sm.sel_b << shift;
      above = sm.sel_above;
      __syncthreads();   // hist and sel_* are rewritten next pass
    }
    theta = unorder_f32(found);
  }
  constexpr int TPC = D / 16;       // decode_scan's arrangement
  constexpr int CPP = NT / TPC;
  const int sub = t % TPC, grp = t / TPC;
  f32x4_t qe[4];
#pragma unroll
  for (int y = 0; y < 4; ++y) qe[y] = *reinterpret_cast<const f32x4_t*>(&sm.qs[4 * (sub + TPC * y)]);
  const float tau = 1.0f / sqrtf((float)D);
  for (int bs = 0; bs < tot; bs += DS_CHUNKS) {   // uniform
    const int mb = min(DS_CHUNKS, tot - bs);
    if (bs > 0) {
      __syncthreads();   // the previous batch's reads of eU / eC are done
      if (t < mb) {
        const MirrorEnt e = entry(bs + t);
        sm.eU[t] = e.up;
        sm.eC[t] = e.c;
      }
      __syncthreads();
    }
    const bool sv = t < mb && sm.eU[t] >= theta;
    const uint64_t bal = __ballot(sv);
    if (lane == 0) sm.wcnt[w] = __popcll(bal);
    sm.keys[t] = 0ull;
    __syncthreads();
    int before = 0, ns = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      before += v < w ? sm.wcnt[v] : 0;
      ns += sm.wcnt[v];
    }
    if (sv) sm.surv[before + __popcll(bal & ((1ull << lane) - 1ull))] = sm.eC[t];
    __syncthreads();
    for (int p0 = 0; p0 < ns; p0 += CPP) {
      const int x = p0 + grp;
      const int c = sm.surv[min(x, ns - 1)];
      const f32x4_t* row = reinterpret_cast<const f32x4_t*>(kb + (int64_t)c * D);
      f32x4_t kv[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) kv[y] = row[sub + TPC * y];
      const float bv = bb[c];
      float s = 0.f;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        s = fmaf(qe[y].x, kv[y].x, s);
        s = fmaf(qe[y].y, kv[y].y, s);
        s = fmaf(qe[y].z, kv[y].z, s);
        s = fmaf(qe[y].w, kv[y].w, s);
      }
#pragma unroll
      for (int o = TPC / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (sub == 0 && x < ns) sm.keys[x] = make_key(fmaf(s, tau, bv), c);
    }
    __syncthreads();
    if (ns <= 64) {   // one sorted 64-list, merged into the running best (wave 0)
      if (w == 0) {
        uint64_t hi = j < ns ? sm.keys[j] : 0ull, lo = 32 + j < ns ? sm.keys[32 + j] : 0ull;
        kl::sort(hi, j);
        kl::sort(lo, j);
        kl::split(hi, lo, j);
        uint64_t rh = sm.run[j], rl = sm.run[32 + j];
        kl::merge64(rh, rl, hi, lo, j);
        if (lane < 32) {
          sm.run[lane] = rh;
          sm.run[32 + lane] = rl;
        }
      }
    } else {
      uint64_t hi, lo;
      best64_of_1024(sm.keys, sm.wl, hi, lo);
      if (w == 0) {
        uint64_t rh = sm.run[j], rl = sm.run[32 + j];
        kl::merge64(rh, rl, hi, lo, j);
        if (lane < 32) {
          sm.run[lane] = rh;
          sm.run[32 + lane] = rl;
        }
      }
    }
    __syncthreads();
  }
  if (w == 0) {
    if (lane < K) {
      const uint64_t lk = sm.run[lane];
      const bool ok = lane < n && lk != 0;
      out_i[lane] = ok ? key_chunk(lk) : -1;
      out_s[lane] = ok ? key_score(lk) : -INFINITY;
    }
    if (sel_user) write_sel_ascending(sm.run[j], sm.run[32 + j], K, n, lane, sel_user);
  }
}

// mirror_select as a kernel, one workgroup per (b, h), for the steps that do not fuse it
template <typename IO, int D>
__global__ void __launch_bounds__(1024) decode_merge_m(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                       const IO* __restrict__ Uw, const float* __restrict__ kc,
                                                       const float* __restrict__ bc, const int32_t* __restrict__ mcnt,
                                                       const MirrorEnt* __restrict__ ment,
                                                       const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_i,
                                                       float* __restrict__ sel_s, int32_t* __restrict__ nsel_out,
                                                       int32_t* __restrict__ sel_user, int Hq, int Hl, int C, int K,
                                                       int r, int nsplit, int nw) {
  __shared__ MirrorSelSmem sm;
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq;
  const int n = min(K, candidate_chunks(seq_lens[b] - 1, C, nw));
  const int64_t lrow = (int64_t)b * Hl + h / (Hq / Hl);
  mirror_select<IO, D>(q + (int64_t)bh * D, Dw, Uw, h, r, kc + lrow * C * D, bc + lrow * C,
                       mcnt + (int64_t)bh * nsplit, ment + (int64_t)bh * nsplit * DS_CHUNKS, nsplit, K, n, sm,
                       sel_i + (int64_t)bh * K, sel_s + (int64_t)bh * K, sel_user ? sel_user + (int64_t)bh * K : nullptr);
  if (threadIdx.x == 0) nsel_out[bh] = n;
}

// eight consecutive elements of a row, kept raw until used
template <typename IO>
struct raw8;
template <>
struct raw8<bf16_t> {
  u32x4_t u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ float operator[](int m) const {
    return __uint_as_float((m & 1) ? (u[m >> 1] & 0xffff0000u) : (u[m >> 1] << 16));
  }
};
template <>
struct raw8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4_t*>(p);
    b = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
  __device__ __forceinline__ float operator[](int m) const { return m < 4 ? a[m] : b[m - 4]; }
};

// slot s < nsel: selected chunk sel_i[s]; slot K + t: chunk own - t of the window
// (t < nw; slots before chunk 0 do nothing).  Writes the
// normalised chunk output (fp32) and the chunk's fusion score.  The V rows a thread
// needs are loaded together with the K rows, before the logits.
template <typename IO, int D>
__global__ void __launch_bounds__(256) decode_attend(const IO* __restrict__ q, const IO* __restrict__ kcache,
                                                     const IO* __restrict__ vcache, const int32_t* __restrict__ seq_lens,
                                                     const int32_t* __restrict__ sel_i, const float* __restrict__ sel_s,
                                                     const int32_t* __restrict__ nsel, float* __restrict__ part,
                                                     float* __restrict__ sig, int Hq, int Hkv, int N, int K, int nw,
                                                     KvPages pg) {
  constexpr int KJ = D / 32;        // logits: 4 threads per key, KJ runs of 8 dims each
  constexpr int TPR = D / 8;        // values: threads per row (8 dims each)
  constexpr int NG = 256 / TPR;     // key groups
  constexpr int KPG = 64 / NG;      // keys per group
  __shared__ float z[64];
  __shared__ float ml[2];
  __shared__ float red[NG][D];
  const int NSL = K + nw;  // slots: K selected chunks, then the window's chunks, own chunk first
  const int slot = blockIdx.x % NSL, bh = blockIdx.x / NSL;
  const int b = bh / Hq, h = bh % Hq, kvh = h / (Hq / Hkv);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int L = seq_lens[b];
  int c, nk;
  if (slot >= K) {
    c = (L - 1) / 64 - (slot - K);
    if (c < 0) return;  // the window reaches back past chunk 0
    nk = slot == K ? L - c * 64 : 64;
  } else {
    if (slot >= nsel[bh]) return;
    c = sel_i[(int64_t)bh * K + slot];
    if (c < 0) return;   // never for a selection the merge wrote; no access before the cache
    nk = 64;
  }
  const int64_t row0 = pg.chunk_row(b, kvh, Hkv, N, c);
  // keys past nk (own chunk only) read row nk - 1, in bounds, and get weight 0
  const int key = t >> 2, qd = t & 3;
  const int e8 = (t % TPR) * 8, kg = t / TPR;
  raw8<IO> kr[KJ], qr[KJ], vr[KPG];
  {
    const IO* krow = kcache + (row0 + min(key, nk - 1)) * D;
    const IO* qrow = q + (int64_t)bh * D;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      kr[j].load(krow + 8 * (qd + 4 * j));
      qr[j].load(qrow + 8 * (qd + 4 * j));
    }
#pragma unroll
    for (int u = 0; u < KPG; ++u) vr[u].load(vcache + (row0 + min(kg * KPG + u, nk - 1)) * D + e8);
  }
  const float tau = 1.0f / sqrtf((float)D);
  {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < KJ; ++j)
#pragma unroll
      for (int m = 0; m < 8; ++m) s = fmaf(qr[j][m], kr[j][m], s);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (qd == 0) z[key] = key < nk ? s * tau : -INFINITY;
  }
  __syncthreads();
  if (w == 0) {
    const float zz = z[lane];
    const float m = wave_max(zz);
    const float p = zz == -INFINITY ? 0.f : __expf(zz - m);
    const float l = wave_sum(p);
    z[lane] = p;
    if (lane == 0) {
      ml[0] = m;
      ml[1] = l;
    }
  }
  __syncthreads();
  {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      const float pj = z[kg * KPG + u];
#pragma unroll
      for (int m = 0; m < 8; ++m) a[m] = fmaf(pj, vr[u][m], a[m]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) red[kg][e8 + m] = a[m];
  }
  __syncthreads();
  if (t < D) {
    float o = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) o += red[g2][t];
    part[((int64_t)bh * NSL + slot) * D + t] = o / ml[1];
  }
  if (t == 0) sig[(int64_t)bh * NSL + slot] = slot >= K ? ml[0] + logf(ml[1]) : sel_s[(int64_t)bh * K + slot];
}

// o = sum over the live slots of softmax(sig)_s part_s, one workgroup per (b, h): the n
// selected chunks and the window's chunks from the own one back to chunk 0 (at most nw).
// Lane s of every wave holds slot s's weight (MAXS = 128: slot 64 + s's too); the live
// slot rows are all loaded at once.
// The top-K merge, chunk attention and fusion of one (b, h) in one workgroup of four groups
// of 256 threads (bf16 I/O).  First the selection: the first four waves merge the splits'
// candidate lists (merge_splits, as decode_merge), or, after the mirror scan, the block runs
// mirror_select on its survivor lists.  Slots are then decode_attend's; group g takes
// slots g, g + 4, ...
// Per slot a group computes what decode_attend computes (the chunk's softmax output o_c
// and its score: the selection score, or the window chunk's exact log-sum-exp) and folds
// it into a running fusion (m, z, acc) with an online softmax; the next slot's K and V
// rows are loaded while the current one is computed.  At the end the four groups' running
// fusions are merged.  It gives decode_combine's result up to the order of the fp32 sums.
template <int D, bool KB, bool MIR>
__global__ void __launch_bounds__(1024) decode_attend_fused(const bf16_t* __restrict__ q,
                                                            const bf16_t* __restrict__ kcache,
                                                            const bf16_t* __restrict__ vcache,
                                                            const int32_t* __restrict__ seq_lens,
                                                            const uint64_t* __restrict__ cand,
                                                            int32_t* __restrict__ sel_user, bf16_t* __restrict__ out,
                                                            int Hq, int Hkv, int N, int C, int K, int nsplit, int nw,
                                                            KvPages pg, const bf16_t* __restrict__ Dw,
                                                            const bf16_t* __restrict__ Uw, const float* __restrict__ kc,
                                                            const float* __restrict__ bc,
                                                            const int32_t* __restrict__ mcnt,
                                                            const MirrorEnt* __restrict__ ment, int Hl, int r) {
  constexpr int KJ = D / 32;        // logits: 4 threads per key, KJ runs of 8 dims each
  constexpr int TPR = D / 8;        // values: threads per row (8 dims each)
  constexpr int NG = 256 / TPR;     // key groups
  constexpr int KPG = 64 / NG;      // keys per group
  constexpr int MAXSL = 96;         // K + nw <= 64 + 32
  __shared__ float z[4][64];
  __shared__ float ml[4][2];
  __shared__ float red[4][NG][D];
  __shared__ int s_c[MAXSL], s_nk[MAXSL];
  __shared__ int64_t s_row[MAXSL];   // first K/V row of the slot's chunk (row 0 when none)
  __shared__ float s_sc[MAXSL];
  __shared__ float f_m[4], f_z[4];
  __shared__ float f_acc[4][D];
  __shared__ __align__(16) bf16_t qsh[D];   // the query (read per slot, not held in registers)
  __shared__ uint64_t wl[4][64];
  __shared__ int32_t m_i[64];
  __shared__ float m_s[64];
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq, kvh = h / (Hq / Hkv);
  const int t = threadIdx.x, g = t >> 8, tg = t & 255, lane = t & 63;
  const int L = seq_lens[b];
  const int NSL = K + nw;
  const int nsel = min(K, candidate_chunks(L - 1, C, nw));
  if (t < D / 8) *reinterpret_cast<u32x4_t*>(&qsh[8 * t]) = *reinterpret_cast<const u32x4_t*>(q + (int64_t)bh * D + 8 * t);
  if constexpr (MIR) {   // the selection from the mirror scan's survivor lists
    __shared__ MirrorSelSmem msm;
    const int64_t lrow = (int64_t)b * Hl + h / (Hq / Hl);
    mirror_select<bf16_t, D>(q + (int64_t)bh * D, Dw, Uw, h, r, kc + lrow * C * D, bc + lrow * C,
                             mcnt + (int64_t)bh * nsplit, ment + (int64_t)bh * nsplit * DS_CHUNKS, nsplit, K, nsel, msm,
                             m_i, m_s, sel_user ? sel_user + (int64_t)bh * K : nullptr);
  } else {
    merge_splits<KB>(cand + (int64_t)bh * nsplit * DS_KEEP, nsplit, K, nsel, wl, m_i, m_s,
                     sel_user ? sel_user + (int64_t)bh * K : nullptr);
  }
  __syncthreads();
  if (t < NSL) {   // slot table: chunk (-1: nothing), keys, score (selected slots)
    int c = -1, nk = 64;
    float sc = 0.f;
    if (t >= K) {
      c = (L - 1) / 64 - (t - K);
      if (t == K) nk = L - c * 64;
      if (c < 0) c = -1;
    } else if (t < nsel) {
      c = m_i[t];
      sc = m_s[t];
      if (c < 0) c = -1;
    }
    s_c[t] = c;
    s_nk[t] = c >= 0 ? nk : 1;
    s_sc[t] = sc;
    s_row[t] = pg.chunk_row(b, kvh, Hkv, N, max(c, 0));
  }
  const int key = tg >> 2, qd = tg & 3;
  const int e8 = (tg % TPR) * 8, kg = tg / TPR;
  __syncthreads();
  const int nit = (NSL + 3) / 4;
  // K and V rows of slot s into a register buffer; slots with no chunk load row 0 of the
  // (b, kv head) (in bounds) and are skipped
  auto load = [&](int s, raw8<bf16_t>(&kr)[KJ], raw8<bf16_t>(&vr)[KPG]) {
    const int sl = min(s, NSL - 1);   // slots past the table load a real slot's rows (in bounds)
    const int nk = s_nk[sl];
    const int64_t row0 = s_row[sl];
    const bf16_t* krow = kcache + (row0 + min(key, nk - 1)) * D;
#pragma unroll
    for (int j = 0; j < KJ; ++j) kr[j].load(krow + 8 * (qd + 4 * j));
#pragma unroll
    for (int u = 0; u < KPG; ++u) vr[u].load(vcache + (row0 + min(kg * KPG + u, nk - 1)) * D + e8);
  };
  const float tau = 1.0f / sqrtf((float)D);
  float run_m = -INFINITY, run_z = 0.f, acc = 0.f;   // the group's running fusion (acc: dim tg)
  raw8<bf16_t> ka[KJ], va[KPG], kb2[KJ], vb2[KPG];
  auto step = [&](int s, const raw8<bf16_t>(&kr)[KJ], const raw8<bf16_t>(&vr)[KPG]) {
    const int c = s < NSL ? s_c[s] : -1;   // uniform in the group
    const int nk = s_nk[min(s, NSL - 1)];
    {
      float sv = 0.f;
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        raw8<bf16_t> qr;
        qr.load(&qsh[8 * (qd + 4 * j)]);
#pragma unroll
        for (int m = 0; m < 8; ++m) sv = fmaf(qr[m], kr[j][m], sv);
      }
      sv += __shfl_xor(sv, 1);
      sv += __shfl_xor(sv, 2);
      if (qd == 0) z[g][key] = key < nk ? sv * tau : -INFINITY;
    }
    __syncthreads();
    if ((tg >> 6) == 0) {
      const float zz = z[g][lane];
      const float m = wave_max(zz);
      const float p = zz == -INFINITY ? 0.f : __expf(zz - m);
      const float l = wave_sum(p);
      z[g][lane] = p;
      if (lane == 0) {
        ml[g][0] = m;
        ml[g][1] = l;
      }
    }
    __syncthreads();
    {
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < KPG; ++u) {
        const float pj = z[g][kg * KPG + u];
#pragma unroll
        for (int m = 0; m < 8; ++m) a[m] = fmaf(pj, vr[u][m], a[m]);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) red[g][kg][e8 + m] = a[m];
    }
    __syncthreads();
    if (c >= 0 && tg < D) {
      float o = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) o += red[g][g2][tg];
      const float l = ml[g][1];
      const float sig = s >= K ? ml[g][0] + logf(l) : s_sc[s];
      const float mn = fmaxf(run_m, sig);
      const float a1 = __expf(run_m - mn), a2 = __expf(sig - mn);
      run_z = fmaf(run_z, a1, a2);
      acc = fmaf(acc, a1, (o / l) * a2);
      run_m = mn;
    }
  };
  // double buffer over the group's slots (every group runs nit iterations: the barriers
  // inside step are workgroup-wide)
  load(g, ka, va);
  int it = 0;
  for (; it + 2 < nit; it += 2) {
    load(4 * (it + 1) + g, kb2, vb2);
    step(4 * it + g, ka, va);
    load(4 * (it + 2) + g, ka, va);
    step(4 * (it + 1) + g, kb2, vb2);
  }
  if (it + 1 < nit) {   // two iterations left
    load(4 * (it + 1) + g, kb2, vb2);
    step(4 * it + g, ka, va);
    step(4 * (it + 1) + g, kb2, vb2);
  } else {              // one left
    step(4 * it + g, ka, va);
  }
  if (tg < D) {
    f_acc[g][tg] = acc;
    if (tg == 0) {
      f_m[g] = run_m;
      f_z[g] = run_z;
    }
  }
  __syncthreads();
  if (t < D) {
    const float M = fmaxf(fmaxf(f_m[0], f_m[1]), fmaxf(f_m[2], f_m[3]));
    float zs = 0.f, o = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < 4; ++g2) {
      const float w = f_m[g2] == -INFINITY ? 0.f : __expf(f_m[g2] - M);
      zs = fmaf(f_z[g2], w, zs);
      o = fmaf(f_acc[g2][t], w, o);
    }
    io_traits<bf16_t>::store(out, (int64_t)bh * D + t, o / zs);
  }
}

template <typename IO, int D, int MAXS>
__global__ void __launch_bounds__(256) decode_combine(const float* __restrict__ part, const float* __restrict__ sig,
                                                      const int32_t* __restrict__ nsel,
                                                      const int32_t* __restrict__ seq_lens, IO* __restrict__ out,
                                                      int Hq, int K, int nw) {
  constexpr int G = 256 / D;               // slot groups
  constexpr int MAXJ = (MAXS + G - 1) / G;   // K + nw <= MAXS slots
  __shared__ float red[G][D];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int n = nsel[bh];
  const int NSL = K + nw;
  const int nwl = min(nw, (seq_lens[bh / Hq] - 1) / 64 + 1);  // window chunks that exist
  const float* sg = sig + (int64_t)bh * NSL;
  const float* pp = part + (int64_t)bh * NSL * D;
  const int e = t % D, g = t / D;
  auto live_slot = [&](int s2) { return s2 < n || (s2 >= K && s2 < K + nwl); };
  float pv[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int s2 = g + j * G;
    pv[j] = live_slot(s2) ? pp[(int64_t)s2 * D + e] : 0.f;
  }
  const bool live = live_slot(lane), live2 = MAXS > 64 && live_slot(64 + lane);
  const float v = live ? sg[lane] : -INFINITY, v2 = live2 ? sg[64 + lane] : -INFINITY;
  const float M = wave_max(fmaxf(v, v2));
  const float wt = live ? expf(v - M) : 0.f, wt2 = live2 ? expf(v2 - M) : 0.f;
  const float Z = wave_sum(wt + wt2);
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int s2 = g + j * G;
    a = fmaf(s2 < 64 ? __shfl(wt, s2) : __shfl(wt2, min(s2 - 64, 63)), pv[j], a);
  }
  red[g][e] = a;
  __syncthreads();
  if (t < D) {
    float o = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2) o += red[g2][t];
    io_traits<IO>::store(out, (int64_t)bh * D + t, o / Z);
  }
}

// ---------------------------------------------------------------- landmark mirror
// An 8-bit mirror of the landmark cache for the decode scan, in two planes: per row
// (b, l, c) the signed codes u_e = rint(k'_e * (127 / m)) in [-127, 127], m = max_e |k'_e|
// (d bytes, so a row is one or two whole cache lines), then per row the pair
// (b'_c, s_c = m / 127) as fp32 [B*Hlmk*C, 2].  |k'_e - s_c u_e| <= s_c (1/2 + 2^-16): the
// rounding to an integer, plus the fp32 roundings of 127 / m and of the product.
template <int D>
__global__ void __launch_bounds__(256) mirror_build(const float* __restrict__ kc, const float* __restrict__ bc,
                                                    uint8_t* __restrict__ kcm, int C, int c_begin, int n,
                                                    int64_t rows, int64_t all_rows) {
  constexpr int TPR = D / 8;        // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;    // rows per workgroup pass
  const int t = threadIdx.x, sub = t % TPR;
  for (int64_t base = (int64_t)blockIdx.x * RPB; base < rows; base += (int64_t)gridDim.x * RPB) {
    const int64_t it = base + t / TPR;   // item: (b, l) * n + chunk offset
    const bool ok = it < rows;
    const int64_t r = ok ? (it / n) * C + c_begin + it % n : 0;   // row of kc / the mirror
    float x[8];
    if (ok) {
      const float4 a = *reinterpret_cast<const float4*>(kc + r * D + 8 * sub);
      const float4 b = *reinterpret_cast<const float4*>(kc + r * D + 8 * sub + 4);
      x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) mx = fmaxf(mx, fabsf(x[m]));
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (ok) {
      const float inv = mx > 0.f ? 127.0f / mx : 0.f;
      uint32_t wd[2] = {0u, 0u};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int code = (int)rintf(x[m] * inv);   // |x * inv| <= 127 (1 + 2^-23)
        wd[m >> 2] |= ((uint32_t)code & 0xffu) << (8 * (m & 3));
      }
      *reinterpret_cast<u32x2_t*>(kcm + r * D + 8 * sub) = u32x2_t{wd[0], wd[1]};
      if (sub == 0)
        reinterpret_cast<u32x2_t*>(kcm + all_rows * D)[r] = u32x2_t{__float_as_uint(bc[r]), __float_as_uint(mx / 127.0f)};
    }
  }
}

// The decode scan over the mirror.  Per chunk, from its codes, a lower and an upper bound of
// the exact score, L <= s <= U with s = fmaf(q^ . k', tau, b') as decode_scan computes it
// in fp32.  Within the workgroup's chunks, theta = the n-th largest of a subset of the L
// (n = min(K, chunks)) is at most the n-th largest L there; the chunks with U >= theta (the
// survivors) therefore include the workgroup's n chunks of largest L and every chunk of its
// exact best n.  They go to the split's list (chunk, L, U) for mirror_select.
template <typename IO, int D, bool KB, int UNR>
__global__ void __launch_bounds__(256) decode_scan_m(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                     const IO* __restrict__ Uw, const uint8_t* __restrict__ kcm,
                                                     const int32_t* __restrict__ seq_lens, int32_t* __restrict__ mcnt,
                                                     MirrorEnt* __restrict__ ment, int Hq, int Hl, int C, int K, int r,
                                                     int nsplit, int nw, int64_t mrows) {
  constexpr int TPM = D / 16;       // mirror: threads per chunk, 16 codes (one 16-byte load) each
  constexpr int CPM = 256 / TPM;    // mirror: chunks per pass
  constexpr int STEP = CPM * UNR;
  __shared__ __align__(16) float qs[D];
  __shared__ float ts[32];
  __shared__ float mq_s, l1_s;
  // theta comes from the T largest lower bounds of each chunk lane (NCL lanes, each
  // bounding every NCL-th chunk): the n-th largest of a subset is at most the n-th largest
  // of all, and with T = 2..4 it loses almost nothing (the survivors grow by about 2%)
  constexpr int NCL = 256 / TPM;
  constexpr int T = NCL == 32 ? (KB ? 4 : 3) : (KB ? 3 : 2);
  constexpr int NV = NCL * T;
  static_assert(NV <= 256 && NV % 4 == 0, "");
  __shared__ __align__(16) float lb_s[NV];   // each chunk lane's T largest lower bounds
  __shared__ float thw[4];
  __shared__ float lbs[DS_CHUNKS], ubs[DS_CHUNKS];   // lower and upper bounds
  __shared__ int16_t surv[DS_CHUNKS];    // survivors (offsets in the workgroup's range)
  __shared__ int wcnt[4];
  const int sp = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;
  const int b = bh / Hq, h = bh % Hq;
  const int L = seq_lens[b];
  const int P = candidate_chunks(L - 1, C, nw);
  const int c_beg = sp * DS_CHUNKS, c_end = min(P, c_beg + DS_CHUNKS);
  const int nloc = max(0, c_end - c_beg), n = min(K, nloc);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t* cnt_out = mcnt + (int64_t)bh * nsplit + sp;
  MirrorEnt* ent_out = ment + ((int64_t)bh * nsplit + sp) * DS_CHUNKS;
  if (n == 0) {   // no chunk here (uniform): an empty list
    if (t == 0) *cnt_out = 0;
    return;
  }
  const int msub = t % TPM, mgrp = t / TPM;
  const int64_t lrow = (int64_t)b * Hl + h / (Hq / Hl);
  const uint8_t* mb = kcm + lrow * C * D;   // this head's code rows
  const u32x2_t* mt = reinterpret_cast<const u32x2_t*>(kcm + mrows * D) + lrow * C;   // (b', s)
  u32x4_t ka[UNR], kb2[UNR];
  u32x2_t ta[UNR], tb[UNR];
  auto load = [&](int c0, u32x4_t(&kv)[UNR], u32x2_t(&tv)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = min(c0 + u * CPM + mgrp, c_end - 1);
      // the TPM lanes of a chunk read its whole row (64 or 128 bytes) in one load
      kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(mb + (int64_t)c * D + 16 * msub));
      // every lane loads the pair (the lanes of a chunk share it): a load under a lane mask
      // would make the compiler wait for all loads in flight
      tv[u] = __builtin_nontemporal_load(mt + c);
    }
  };
  // the first buffer's loads go out before q^ is prepared (they do not depend on it)
  load(c_beg, ka, ta);
  qhat_to_lds<IO, D>(q + (int64_t)bh * D, Dw, Uw, h, r, qs, ts);
  if (w == 0) {   // an upper bound of sum_e |q^_e|, and max_e |q^_e|
    float ab = 0.f, mq = 0.f;
    for (int e = lane; e < D; e += 64) {
      ab += fabsf(qs[e]);
      mq = fmaxf(mq, fabsf(qs[e]));
    }
    ab = wave_sum(ab);
    mq = wave_max(mq);
    if (lane == 0) {
      l1_s = ab * (1.0f + 1.0f / 4096.0f);
      mq_s = mq;
    }
  }
  __syncthreads();
  // q^ in two 8-bit parts: x_e = q^_e * fl(127 / max|q^|), hi_e = rint(x_e),
  // lo_e = rint((x_e - hi_e) * 254), so q^_e = s_q (hi_e + lo_e / 254) within
  // s_q (0.5 + 2^-17) / 254 + s_q 127 2^-21 < 0.0021 s_q, s_q = fl(max|q^| / 127).
  // Lane msub holds dims 16 msub + 4 i + y as byte y of word i.
  const float mq = mq_s;
  const float invq = mq > 0.f ? 127.0f / mq : 0.f, sq = mq / 127.0f;
  int qhi[4], qlo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h4 = 0u, l4 = 0u;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const float x = qs[16 * msub + 4 * i + y] * invq;
      const float hf = rintf(x);
      const int lo = (int)rintf((x - hf) * 254.0f);
      h4 |= ((uint32_t)(int)hf & 0xffu) << (8 * y);
      l4 |= ((uint32_t)lo & 0xffu) << (8 * y);
    }
    qhi[i] = (int)h4;
    qlo[i] = (int)l4;
  }
  const float tau = 1.0f / sqrtf((float)D);
  // Per chunk, with s its scale and u its codes: the mirror's dot product is
  // s s_q (sum hi_e u_e + (sum lo_e u_e) / 254) (integer sums, exact), and
  //   |q^ . k' - that| <= s (1/2 + 2^-16) ||q^||_1 + 0.0021 s_q s sum_e |u_e|
  //                    <= s (||q^||_1 (1/2 + 2^-16) + 0.27 D s_q).
  // The fp32 steps (the lanes' sums, the products with s and s_q, and the exact path's own
  // dot product, at most about 127 D 2^-24 s ||q^||_1) take far less than the 2^-5 margin
  // on the first term.  The roundings of the last fma (s tau + b') on both sides are covered
  // by 2^-20 (|s| + |b'|), values below the normal range by a tiny absolute term.
  const float dfac = tau * (l1_s * (0.5f + 1.0f / 32.0f) + 0.27f * (float)D * sq);
  const float dabs = 0x1p-110f * (l1_s + 1.0f);
  float top[T];   // this chunk lane's largest lower bounds, descending
#pragma unroll
  for (int k = 0; k < T; ++k) top[k] = -INFINITY;
  auto bound = [&](int c0, const u32x4_t(&kv)[UNR], const u32x2_t(&tv)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int wd[4] = {(int)kv[u].x, (int)kv[u].y, (int)kv[u].z, (int)kv[u].w};
      int ih = 0, il = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ih = __builtin_amdgcn_sdot4(qhi[i], wd[i], ih, false);
        il = __builtin_amdgcn_sdot4(qlo[i], wd[i], il, false);
      }
      float acc = fmaf((float)il, 1.0f / 254.0f, (float)ih);
#pragma unroll
      for (int o = TPM / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
      const int c = c0 + u * CPM + mgrp;
      if (msub == 0) {
        const float bv = __uint_as_float(tv[u].x), sc = __uint_as_float(tv[u].y);
        const float sh = fmaf((sc * sq) * acc, tau, bv);
        const float dl = fmaf(dfac, sc, fmaf(0x1p-20f, fabsf(sh) + fabsf(bv), dabs));
        const bool live = c < c_end;
        const float lv = live ? sh - dl : -INFINITY;
        lbs[c - c_beg] = lv;
        ubs[c - c_beg] = live ? sh + dl : -INFINITY;
#pragma unroll
        for (int k = T - 1; k >= 1; --k) top[k] = fmaxf(top[k], fminf(top[k - 1], lv));
        top[0] = fmaxf(top[0], lv);
      }
    }
  };
  // Two register buffers alternate.  Every load is issued whether or not its chunks are
  // live (they clamp to chunk c_end - 1, so they stay in bounds): with a fixed number of
  // loads in flight the compiler waits for exactly the buffer it is about to use.
  static_assert(DS_CHUNKS % (2 * STEP) == 0, "");
  constexpr int NIT = DS_CHUNKS / (2 * STEP);
  for (int it = 0; it < NIT - 1; ++it) {
    const int c0 = c_beg + it * 2 * STEP;
    load(c0 + STEP, kb2, tb);
    bound(c0, ka, ta);
    load(c0 + 2 * STEP, ka, ta);
    bound(c0 + STEP, kb2, tb);
  }
  {
    const int c0 = c_beg + (NIT - 1) * 2 * STEP;
    load(c0 + STEP, kb2, tb);
    bound(c0, ka, ta);
    bound(c0 + STEP, kb2, tb);
  }
  if (msub == 0)
#pragma unroll
    for (int k = 0; k < T; ++k) lb_s[mgrp * T + k] = top[k];
  __syncthreads();
  // theta: the largest of those lower bounds that at least n of them reach
  {
    float cand = -INFINITY;
    if (t < NV) {
      const float v = lb_s[t];
      int cnt = 0;
#pragma unroll 8
      for (int x = 0; x < NV; x += 4) {
        const f32x4_t y = *reinterpret_cast<const f32x4_t*>(&lb_s[x]);
        cnt += (int)(y.x >= v) + (int)(y.y >= v) + (int)(y.z >= v) + (int)(y.w >= v);
      }
      cand = cnt >= n ? v : -INFINITY;
    }
    cand = wave_max(cand);
    if (lane == 0) thw[w] = cand;
  }
  __syncthreads();
  const float theta = fmaxf(fmaxf(thw[0], thw[1]), fmaxf(thw[2], thw[3]));
  // survivors U >= theta, in chunk order
  int ns = 0;
#pragma unroll
  for (int i = 0; i < DS_CHUNKS / 256; ++i) {
    const int x = i * 256 + t;
    const bool sv = ubs[x] >= theta;
    const uint64_t bal = __ballot(sv);
    if (lane == 0) wcnt[w] = __popcll(bal);
    __syncthreads();
    int before = ns, total = ns;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      before += v < w ? wcnt[v] : 0;
      total += wcnt[v];
    }
    if (sv) surv[before + __popcll(bal & ((1ull << lane) - 1ull))] = (int16_t)x;
    ns = total;
    __syncthreads();   // wcnt is rewritten next round
  }
  // the survivors go to this split's list; the per-head selection (mirror_select) takes
  // the threshold over all splits' lists and rescores what reaches it
  for (int x = t; x < ns; x += 256) {
    const int o = surv[x];
    ent_out[x] = MirrorEnt{c_beg + o, lbs[o], ubs[o]};
  }
  if (t == 0) *cnt_out = ns;
}

template <int D>
static hipError_t launch_mirror_d(const float* kc, const float* bc, uint8_t* kcm, int BL, int C, int c_begin, int n,
                                  hipStream_t st) {
  const int64_t rows = (int64_t)BL * n;
  const int64_t rpb = 256 / (D / 8);
  const unsigned gs = (unsigned)std::min<int64_t>((rows + rpb - 1) / rpb, 16384);
  hipLaunchKernelGGL((mirror_build<D>), dim3(gs), dim3(256), 0, st, kc, bc, kcm, C, c_begin, n, rows,
                     (int64_t)BL * C);
  return hipGetLastError();
}

hipError_t launch_mirror(const Geom& g, const float* kc, const float* bc, uint8_t* kcm, int c_begin, int c_end,
                         hipStream_t st) {
  const int n = c_end - c_begin;
  if (n <= 0) return hipSuccess;
  return g.d == 64 ? launch_mirror_d<64>(kc, bc, kcm, g.B * g.Hl, g.C(), c_begin, n, st)
                   : launch_mirror_d<128>(kc, bc, kcm, g.B * g.Hl, g.C(), c_begin, n, st);
}

// compute units of the current device (cached per device)
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1 << 30;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1 << 30;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename IO, int D>
static hipError_t launch_decode_t(const Geom& g, const void* q, const void* kcache, const void* vcache,
                                  const int32_t* seq_lens, const float* kc, const float* bc, const uint8_t* kcm,
                                  const void* Dw, const void* Uw, int32_t* sel_user, void* o, char* ws, hipStream_t st,
                                  hipEvent_t* ev, KvPages pg) {
  const DecodeWs w = decode_ws(g, kcm != nullptr);
  uint64_t* cand = (uint64_t*)(ws + w.cand);
  int32_t* sel_i = (int32_t*)(ws + w.sel_i);
  float* sel_s = (float*)(ws + w.sel_s);
  int32_t* nsel = (int32_t*)(ws + w.nsel);
  float* part = (float*)(ws + w.part);
  float* sig = (float*)(ws + w.sig);
  int32_t* mcnt = (int32_t*)(ws + w.mcnt);
  MirrorEnt* ment = (MirrorEnt*)(ws + w.ment);
  const int C = g.C(), BH = g.B * g.Hq;
  const int nsplit = std::max(1, nsplit_of(g));  // one (empty) split still writes the selection
  if (nsplit > DS_MAX_SPLIT) return hipErrorInvalidValue;  // N/S > 16384, rejected by the ABI first
  if (ev) (void)hipEventRecord(ev[0], st);
  const bool kb = g.K > 32;   // keep 64 candidates per split
  bool fused = false;   // one workgroup per (b, h) fills the chip: merge, attention and fusion in one kernel
  if constexpr (std::is_same<IO, bf16_t>::value) fused = BH >= device_cus();
  if (kcm) {   // the scan over the 8-bit mirror: each split's survivors of its bounds
    if (kb)
      hipLaunchKernelGGL((decode_scan_m<IO, D, true, DSM_UNR>), dim3(BH * nsplit), dim3(256), 0, st, (const IO*)q,
                         (const IO*)Dw, (const IO*)Uw, kcm, seq_lens, mcnt, ment, g.Hq, g.Hl, C, g.K, g.r, nsplit,
                         g.nw, (int64_t)g.B * g.Hl * C);
    else
      hipLaunchKernelGGL((decode_scan_m<IO, D, false, DSM_UNR>), dim3(BH * nsplit), dim3(256), 0, st, (const IO*)q,
                         (const IO*)Dw, (const IO*)Uw, kcm, seq_lens, mcnt, ment, g.Hq, g.Hl, C, g.K, g.r, nsplit,
                         g.nw, (int64_t)g.B * g.Hl * C);
  } else if (kb) {
    hipLaunchKernelGGL((decode_scan<IO, D, true>), dim3(BH * nsplit), dim3(256), 0, st, (const IO*)q, (const IO*)Dw,
                       (const IO*)Uw, kc, bc, seq_lens, cand, g.Hq, g.Hl, C, g.r, nsplit, g.nw);
  } else {
    hipLaunchKernelGGL((decode_scan<IO, D, false>), dim3(BH * nsplit), dim3(256), 0, st, (const IO*)q,
                       (const IO*)Dw, (const IO*)Uw, kc, bc, seq_lens, cand, g.Hq, g.Hl, C, g.r, nsplit, g.nw);
  }
  if (ev) (void)hipEventRecord(ev[1], st);
  if (fused) {
    if (ev) (void)hipEventRecord(ev[2], st);   // the merge runs inside the fused kernel
    if constexpr (std::is_same<IO, bf16_t>::value) {
      const bf16_t *qb = (const bf16_t*)q, *kb16 = (const bf16_t*)kcache, *vb16 = (const bf16_t*)vcache;
      const bf16_t *Db = (const bf16_t*)Dw, *Ub = (const bf16_t*)Uw;
      if (kcm)
        hipLaunchKernelGGL((decode_attend_fused<D, false, true>), dim3(BH), dim3(1024), 0, st, qb, kb16, vb16, seq_lens,
                           (const uint64_t*)cand, sel_user, (bf16_t*)o, g.Hq, g.Hkv, g.N, C, g.K, nsplit, g.nw, pg, Db,
                           Ub, kc, bc, (const int32_t*)mcnt, (const MirrorEnt*)ment, g.Hl, g.r);
      else if (kb)
        hipLaunchKernelGGL((decode_attend_fused<D, true, false>), dim3(BH), dim3(1024), 0, st, qb, kb16, vb16, seq_lens,
                           (const uint64_t*)cand, sel_user, (bf16_t*)o, g.Hq, g.Hkv, g.N, C, g.K, nsplit, g.nw, pg, Db,
                           Ub, kc, bc, (const int32_t*)mcnt, (const MirrorEnt*)ment, g.Hl, g.r);
      else
        hipLaunchKernelGGL((decode_attend_fused<D, false, false>), dim3(BH), dim3(1024), 0, st, qb, kb16, vb16,
                           seq_lens, (const uint64_t*)cand, sel_user, (bf16_t*)o, g.Hq, g.Hkv, g.N, C, g.K, nsplit,
                           g.nw, pg, Db, Ub, kc, bc, (const int32_t*)mcnt, (const MirrorEnt*)ment, g.Hl, g.r);
    }
  } else {
    if (kcm)
      hipLaunchKernelGGL((decode_merge_m<IO, D>), dim3(BH), dim3(1024), 0, st, (const IO*)q, (const IO*)Dw,
                         (const IO*)Uw, kc, bc, (const int32_t*)mcnt, (const MirrorEnt*)ment, seq_lens, sel_i, sel_s,
                         nsel, sel_user, g.Hq, g.Hl, C, g.K, g.r, nsplit, g.nw);
    else if (kb)
      hipLaunchKernelGGL(decode_merge<true>, dim3(BH), dim3(256), 0, st, (const uint64_t*)cand, seq_lens, sel_i,
                         sel_s, nsel, sel_user, g.Hq, C, g.K, nsplit, g.nw);
    else
      hipLaunchKernelGGL(decode_merge<false>, dim3(BH), dim3(256), 0, st, (const uint64_t*)cand, seq_lens, sel_i,
                         sel_s, nsel, sel_user, g.Hq, C, g.K, nsplit, g.nw);
    if (ev) (void)hipEventRecord(ev[2], st);
    hipLaunchKernelGGL((decode_attend<IO, D>), dim3(BH * (g.K + g.nw)), dim3(256), 0, st, (const IO*)q,
                       (const IO*)kcache, (const IO*)vcache, seq_lens, sel_i, sel_s, nsel, part, sig, g.Hq, g.Hkv, g.N,
                       g.K, g.nw, pg);
    if (g.K + g.nw > 64)
      hipLaunchKernelGGL((decode_combine<IO, D, 128>), dim3(BH), dim3(256), 0, st, (const float*)part,
                         (const float*)sig, (const int32_t*)nsel, seq_lens, (IO*)o, g.Hq, g.K, g.nw);
    else
      hipLaunchKernelGGL((decode_combine<IO, D, 64>), dim3(BH), dim3(256), 0, st, (const float*)part,
                         (const float*)sig, (const int32_t*)nsel, seq_lens, (IO*)o, g.Hq, g.K, g.nw);
  }
  if (ev) (void)hipEventRecord(ev[3], st);
  return hipGetLastError();
}

hipError_t launch_decode(const Geom& g, const void* q, const void* kcache, const void* vcache, const int32_t* seq_lens,
                         const float* kc, const float* bc, const uint8_t* kcm, const void* Dw, const void* Uw,
                         int32_t* sel_idx_out, void* o, void* ws, size_t ws_bytes, hipStream_t st, hipEvent_t* ev,
                         KvPages pg) {
  if (ws_bytes < decode_workspace_bytes(g, kcm != nullptr)) return hipErrorInvalidValue;
  char* w = (char*)ws;
  if (g.io == 0)
    return g.d == 64
               ? launch_decode_t<float, 64>(g, q, kcache, vcache, seq_lens, kc, bc, kcm, Dw, Uw, sel_idx_out, o, w, st, ev, pg)
               : launch_decode_t<float, 128>(g, q, kcache, vcache, seq_lens, kc, bc, kcm, Dw, Uw, sel_idx_out, o, w, st, ev, pg);
  return g.d == 64
             ? launch_decode_t<bf16_t, 64>(g, q, kcache, vcache, seq_lens, kc, bc, kcm, Dw, Uw, sel_idx_out, o, w, st, ev, pg)
             : launch_decode_t<bf16_t, 128>(g, q, kcache, vcache, seq_lens, kc, bc, kcm, Dw, Uw, sel_idx_out, o, w, st, ev, pg);
}

}  // namespace hils

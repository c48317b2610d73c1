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
#include "kernels.h"

namespace hils {

constexpr int DS_CHUNKS = 1024;  // chunks scored per decode_scan workgroup
constexpr int DS_MAX_SPLIT = 16;  // scan workgroups per (b, h): N/S <= 16384
constexpr int DS_KEEP = 32;      // candidates kept per workgroup (>= K)

struct DecodeWs {
  size_t cand, sel_i, sel_s, nsel, part, sig, total;
};
static size_t al2(size_t x) { return (x + 255) / 256 * 256; }
static int nsplit_of(const Geom& g) { return (g.C() + DS_CHUNKS - 1) / DS_CHUNKS; }
static DecodeWs decode_ws(const Geom& g) {
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
  w.total = off;
  return w;
}
size_t decode_workspace_bytes(const Geom& g) { return decode_ws(g).total; }

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

template <typename IO, int D>
__global__ void __launch_bounds__(256) decode_scan(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                   const IO* __restrict__ Uw, const float* __restrict__ kc,
                                                   const float* __restrict__ bc, const int32_t* __restrict__ seq_lens,
                                                   uint64_t* __restrict__ cand, int Hq, int C, int r, int nsplit,
                                                   int nw) {
  __shared__ __align__(16) float qs[D];
  __shared__ float ts[32];
  __shared__ uint64_t keys[DS_CHUNKS];
  __shared__ uint64_t wl[4][32];
  const int sp = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;
  const int b = bh / Hq, h = bh % Hq;
  const int L = seq_lens[b];
  const int P = candidate_chunks(L - 1, C, nw);
  const int c_beg = sp * DS_CHUNKS, c_end = min(P, c_beg + DS_CHUNKS);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  qhat_to_lds<IO, D>(q + (int64_t)bh * D, Dw, Uw, h, r, qs, ts);
  // TPC threads per chunk, each holding 16 of the D head dims as 4 float4 spread so
  // that the TPC lanes of a chunk read 128 contiguous bytes per load
  constexpr int TPC = D / 16;
  constexpr int CPP = 256 / TPC;    // chunks per pass
  constexpr int UNR = 2;            // passes per register buffer
  constexpr int STEP = CPP * UNR;
  const int sub = t % TPC, grp = t / TPC;
  f32x4_t qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qv[j] = *reinterpret_cast<const f32x4_t*>(&qs[4 * (sub + TPC * j)]);
  const float tau = 1.0f / sqrtf((float)D);
  const float* kb = kc + (int64_t)bh * C * D;
  const float* bb = bc + (int64_t)bh * C;
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
  static_assert(DS_CHUNKS % (2 * STEP) == 0, "");
  if (c_beg < c_end) load(c_beg, ka, ba);
  for (int c0 = c_beg; c0 < c_beg + DS_CHUNKS; c0 += 2 * STEP) {
    if (c0 + STEP < c_end) load(c0 + STEP, kb2, bb2);
    score(c0, ka, ba);
    if (c0 + 2 * STEP < c_end) load(c0 + 2 * STEP, ka, ba);
    score(c0 + STEP, kb2, bb2);
  }
  __syncthreads();
  // best 32 of this workgroup's chunks: each half-wave sorts 4 x 32 keys, the halves
  // and then the four waves are merged
  {
    const int base = w * 256 + (lane >> 5) * 128 + (lane & 31);
    uint64_t lk = keys[base];
    dsort32(lk);
    dmerge(lk, keys[base + 32]);
    dmerge(lk, keys[base + 64]);
    dmerge(lk, keys[base + 96]);
    const uint64_t other = __shfl(lk, (lane & 31) + 32);
    dmerge_sorted(lk, other);
    if (lane < 32) wl[w][lane] = lk;
  }
  __syncthreads();
  if (w == 0) {  // halves merge waves 0+1 and 2+3, then each other
    uint64_t lk = wl[(lane >> 5) * 2][lane & 31];
    dmerge_sorted(lk, wl[(lane >> 5) * 2 + 1][lane & 31]);
    const uint64_t other = __shfl(lk, (lane & 31) + 32);
    dmerge_sorted(lk, other);
    if (lane < 32) cand[((int64_t)bh * nsplit + sp) * DS_KEEP + lane] = lk;
  }
}

// exact top-K of one (b, h) from the sorted candidate lists of its splits, rank order.
// Half-wave x of wave w takes lists 2w + x and 2w + x + 8, the halves of each wave
// merge, then wave 0 merges the four wave lists.
__global__ void __launch_bounds__(256) decode_merge(const uint64_t* __restrict__ cand,
                                                    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_i,
                                                    float* __restrict__ sel_s, int32_t* __restrict__ nsel_out,
                                                    int32_t* __restrict__ sel_user, int Hq, int C, int K, int nsplit,
                                                    int nw) {
  static_assert(DS_MAX_SPLIT == 16, "two lists per half-wave");
  __shared__ uint64_t wl[4][32];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int li = 2 * w + (lane >> 5);
  const uint64_t* cb = cand + (int64_t)bh * nsplit * DS_KEEP + (lane & 31);
  uint64_t lk = li < nsplit ? cb[li * DS_KEEP] : 0ull;        // empty lists are all-zero keys
  const uint64_t l2 = li + 8 < nsplit ? cb[(li + 8) * DS_KEEP] : 0ull;
  dmerge_sorted(lk, l2);
  dmerge_sorted(lk, __shfl(lk, (lane & 31) + 32));
  if (lane < 32) wl[w][lane] = lk;
  __syncthreads();
  if (w != 0) return;
  lk = wl[(lane >> 5) * 2][lane & 31];
  dmerge_sorted(lk, wl[(lane >> 5) * 2 + 1][lane & 31]);
  dmerge_sorted(lk, __shfl(lk, (lane & 31) + 32));
  const int L = seq_lens[bh / Hq];
  const int n = min(K, candidate_chunks(L - 1, C, nw));
  if (lane < K) {
    const bool ok = lane < n && lk != 0;
    const int32_t ci = ok ? key_chunk(lk) : -1;
    sel_i[(int64_t)bh * K + lane] = ci;
    sel_s[(int64_t)bh * K + lane] = ok ? key_score(lk) : -INFINITY;
    if (sel_user) sel_user[(int64_t)bh * K + lane] = ci;
  }
  if (lane == 0) nsel_out[bh] = n;
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
// Lane s of every wave holds slot s's weight; the live slot rows are all loaded at once.
template <typename IO, int D>
__global__ void __launch_bounds__(256) decode_combine(const float* __restrict__ part, const float* __restrict__ sig,
                                                      const int32_t* __restrict__ nsel,
                                                      const int32_t* __restrict__ seq_lens, IO* __restrict__ out,
                                                      int Hq, int K, int nw) {
  constexpr int G = 256 / D;               // slot groups
  constexpr int MAXJ = (64 + G - 1) / G;   // K + nw <= 64 slots
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
  const bool live = live_slot(lane);
  const float v = live ? sg[lane] : -INFINITY;
  const float M = wave_max(v);
  const float wt = live ? expf(v - M) : 0.f;
  const float Z = wave_sum(wt);
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) a = fmaf(__shfl(wt, min(g + j * G, 63)), pv[j], a);
  red[g][e] = a;
  __syncthreads();
  if (t < D) {
    float o = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2) o += red[g2][t];
    io_traits<IO>::store(out, (int64_t)bh * D + t, o / Z);
  }
}

template <typename IO, int D>
static hipError_t launch_decode_t(const Geom& g, const void* q, const void* kcache, const void* vcache,
                                  const int32_t* seq_lens, const float* kc, const float* bc, const void* Dw,
                                  const void* Uw, int32_t* sel_user, void* o, char* ws, hipStream_t st,
                                  hipEvent_t* ev, KvPages pg) {
  const DecodeWs w = decode_ws(g);
  uint64_t* cand = (uint64_t*)(ws + w.cand);
  int32_t* sel_i = (int32_t*)(ws + w.sel_i);
  float* sel_s = (float*)(ws + w.sel_s);
  int32_t* nsel = (int32_t*)(ws + w.nsel);
  float* part = (float*)(ws + w.part);
  float* sig = (float*)(ws + w.sig);
  const int C = g.C(), BH = g.B * g.Hq;
  const int nsplit = std::max(1, nsplit_of(g));  // one (empty) split still writes the selection
  if (nsplit > DS_MAX_SPLIT) return hipErrorInvalidValue;  // N/S > 16384, rejected by the ABI first
  if (ev) (void)hipEventRecord(ev[0], st);
  hipLaunchKernelGGL((decode_scan<IO, D>), dim3(BH * nsplit), dim3(256), 0, st, (const IO*)q, (const IO*)Dw,
                     (const IO*)Uw, kc, bc, seq_lens, cand, g.Hq, C, g.r, nsplit, g.nw);
  if (ev) (void)hipEventRecord(ev[1], st);
  hipLaunchKernelGGL(decode_merge, dim3(BH), dim3(256), 0, st, (const uint64_t*)cand, seq_lens, sel_i, sel_s, nsel,
                     sel_user, g.Hq, C, g.K, nsplit, g.nw);
  if (ev) (void)hipEventRecord(ev[2], st);
  hipLaunchKernelGGL((decode_attend<IO, D>), dim3(BH * (g.K + g.nw)), dim3(256), 0, st, (const IO*)q,
                     (const IO*)kcache, (const IO*)vcache, seq_lens, sel_i, sel_s, nsel, part, sig, g.Hq, g.Hkv, g.N,
                     g.K, g.nw, pg);
  hipLaunchKernelGGL((decode_combine<IO, D>), dim3(BH), dim3(256), 0, st, (const float*)part, (const float*)sig,
                     (const int32_t*)nsel, seq_lens, (IO*)o, g.Hq, g.K, g.nw);
  if (ev) (void)hipEventRecord(ev[3], st);
  return hipGetLastError();
}

hipError_t launch_decode(const Geom& g, const void* q, const void* kcache, const void* vcache, const int32_t* seq_lens,
                         const float* kc, const float* bc, const void* Dw, const void* Uw, int32_t* sel_idx_out,
                         void* o, void* ws, size_t ws_bytes, hipStream_t st, hipEvent_t* ev, KvPages pg) {
  if (ws_bytes < decode_workspace_bytes(g)) return hipErrorInvalidValue;
  char* w = (char*)ws;
  if (g.io == 0)
    return g.d == 64
               ? launch_decode_t<float, 64>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev, pg)
               : launch_decode_t<float, 128>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev, pg);
  return g.d == 64
             ? launch_decode_t<bf16_t, 64>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev, pg)
             : launch_decode_t<bf16_t, 128>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev, pg);
}

}  // namespace hils

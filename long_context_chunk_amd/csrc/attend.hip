// Intra-chunk attention and fusion for prefill, given each query's selection.
//
//   o_ic   = sum_{j in c} softmax_j(q_i . k_j / sqrt(d)) v_j       for each selected chunk c
//   o_own  = the same over the own chunk, keys cS .. i (causal); LSE_own its log-sum-exp
//   o_i    = sum_c w_c o_ic + w_own o_own,  w = softmax over {s_ic} U {LSE_own}
// (hotpaper.ai abstract: each query attends each retrieved chunk independently
// and the outputs are fused by the chunk retrieval scores; aitrends.kr
// "Methodology" calculation flow; ai-papers.net Fig. 1.)
//
// Chunk-major execution.  The pages' kernel packs M adjacent queries x G heads and
// loads the union of their chunks; on near-independent selections that union is
// dozens of times larger than K and most MFMA work is masked out.  Here every
// (query row, selected chunk) pair is bucketed by (batch, KV head, chunk); each
// workgroup loads one chunk's K/V tile into LDS once and runs full 32-row MFMA
// tiles of gathered query rows against it.  Per pair it writes the normalised
// chunk output o_ic (fp16 for bf16 I/O, fp32 for fp32 I/O) to a slot of its row;
// a per-query-chunk pass then computes the own chunk on the MFMA and fuses.
//
//   bucket_count  : LDS-privatised histogram of the selections per bucket
//   bucket_scan   : exclusive scans -> bucket offsets and tile offsets
//   bucket_scatter: pair ids (= linear index into sel_idx) grouped by bucket
//   chunk_attend  : gathered-row MFMA attention per (bucket, 128-row tile)
//   fuse_own      : own-chunk MFMA attention + softmax fusion -> o
#include <algorithm>

#include "hils_common.h"
#include "kernels.h"

namespace hils {

constexpr int AT_ROWS = 128;        // gathered rows per chunk_attend workgroup (4 waves x 32)
constexpr int HIST_SLICE = 1 << 18; // selection entries per bucket_count / bucket_scatter workgroup
constexpr int MAX_C = 16384;        // largest chunk count the LDS histograms hold

struct AttendWs {
  size_t counts, cursor, boff, toff, pairs, partial, total;
};

static size_t al(size_t x) { return (x + 255) / 256 * 256; }

static AttendWs attend_ws(const Geom& g) {
  AttendWs w;
  const size_t nbk = (size_t)g.B * g.Hkv * g.C();
  const size_t ent = (size_t)g.B * g.Hq * g.N * g.K;
  size_t off = 0;
  w.counts = off;
  off += al(nbk * 4);
  w.cursor = off;
  off += al(nbk * 4);
  w.boff = off;
  off += al((nbk + 1) * 4);
  w.toff = off;
  off += al((nbk + 1) * 4);
  w.pairs = off;
  off += al(ent * 4);
  w.partial = off;
  off += al(ent * g.d * (g.io == 0 ? 4 : 2));
  w.total = off;
  return w;
}

size_t attend_workspace_bytes(const Geom& g) { return attend_ws(g).total; }

// ------------------------------------------------------------------ bucketing
__global__ void __launch_bounds__(256) zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// Selection entries of one (b, kv head) group are contiguous in sel_idx:
// heads kvh*G .. kvh*G+G-1 of batch b, all rows, all K slots.
__global__ void __launch_bounds__(256) bucket_count(const int32_t* __restrict__ sel, uint32_t* __restrict__ counts,
                                                    int64_t group_len, int slices_per_group, int C) {
  __shared__ uint32_t hist[MAX_C];
  const int grp = blockIdx.x / slices_per_group, sl = blockIdx.x % slices_per_group;
  for (int i = threadIdx.x; i < C; i += 256) hist[i] = 0;
  __syncthreads();
  const int64_t beg = (int64_t)sl * HIST_SLICE, end = min(group_len, beg + HIST_SLICE);
  const int32_t* s = sel + (int64_t)grp * group_len;
  for (int64_t i = beg + threadIdx.x; i < end; i += 256) {
    const int c = s[i];
    if (c >= 0) atomicAdd(&hist[c], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += 256)
    if (hist[i]) atomicAdd(&counts[(int64_t)grp * C + i], hist[i]);
}

// Single workgroup: boff = exclusive scan of counts, toff = exclusive scan of
// ceil(count / AT_ROWS).  Both get a final total entry.
__global__ void __launch_bounds__(1024) bucket_scan(const uint32_t* __restrict__ counts, uint32_t* __restrict__ boff,
                                                    uint32_t* __restrict__ toff, int nbk) {
  __shared__ uint32_t sa[1024], sb[1024];
  const int t = threadIdx.x;
  const int per = (nbk + 1023) / 1024;
  const int beg = min(nbk, t * per), end = min(nbk, beg + per);
  uint32_t a = 0, b = 0;
  for (int i = beg; i < end; ++i) {
    a += counts[i];
    b += (counts[i] + AT_ROWS - 1) / AT_ROWS;
  }
  sa[t] = a;
  sb[t] = b;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const uint32_t xa = t >= o ? sa[t - o] : 0, xb = t >= o ? sb[t - o] : 0;
    __syncthreads();
    sa[t] += xa;
    sb[t] += xb;
    __syncthreads();
  }
  uint32_t ra = sa[t] - a, rb = sb[t] - b;  // exclusive prefix of this thread's range
  for (int i = beg; i < end; ++i) {
    boff[i] = ra;
    toff[i] = rb;
    ra += counts[i];
    rb += (counts[i] + AT_ROWS - 1) / AT_ROWS;
  }
  if (t == 1023) {
    boff[nbk] = sa[t];
    toff[nbk] = sb[t];
  }
}

__global__ void __launch_bounds__(256) bucket_scatter(const int32_t* __restrict__ sel, const uint32_t* __restrict__ boff,
                                                      uint32_t* __restrict__ cursor, uint32_t* __restrict__ pairs,
                                                      int64_t group_len, int slices_per_group, int C) {
  __shared__ uint32_t hist[MAX_C];
  __shared__ uint32_t base[MAX_C];
  const int grp = blockIdx.x / slices_per_group, sl = blockIdx.x % slices_per_group;
  for (int i = threadIdx.x; i < C; i += 256) hist[i] = 0;
  __syncthreads();
  const int64_t beg = (int64_t)sl * HIST_SLICE, end = min(group_len, beg + HIST_SLICE);
  const int32_t* s = sel + (int64_t)grp * group_len;
  for (int64_t i = beg + threadIdx.x; i < end; i += 256) {
    const int c = s[i];
    if (c >= 0) atomicAdd(&hist[c], 1u);
  }
  __syncthreads();
  // reserve this slice's range inside every bucket it touches
  for (int i = threadIdx.x; i < C; i += 256) {
    const uint32_t h = hist[i];
    const int64_t bk = (int64_t)grp * C + i;
    base[i] = h ? boff[bk] + atomicAdd(&cursor[bk], h) : 0;
    hist[i] = 0;
  }
  __syncthreads();
  const int64_t e0 = (int64_t)grp * group_len;
  for (int64_t i = beg + threadIdx.x; i < end; i += 256) {
    const int c = s[i];
    if (c >= 0) {
      const uint32_t rank = atomicAdd(&hist[c], 1u);
      pairs[base[c] + rank] = (uint32_t)(e0 + i);
    }
  }
}

// ------------------------------------------------------ K/V chunk tile in LDS
// K planes [key][d] (row stride D + 4) feed the A operand of S^T = K Q^T;
// V^T planes [d][key] (row stride 68) feed the A operand of O^T = V^T P^T.
// Keys at or beyond `nvalid` are stored as zeros.  NT bf16 terms per value.
template <typename IO, int D, int NT>
struct KVTile {
  static constexpr int LDK = D + 4;
  static constexpr int LDV = 64 + 4;
  uint16_t k[NT][64 * LDK];
  uint16_t vt[NT][D * LDV];
};

template <typename IO, int D, int NT>
HILS_DEV void stage_kv(KVTile<IO, D, NT>& tile, const IO* __restrict__ k, const IO* __restrict__ v, int64_t row0,
                       int nvalid) {
  constexpr int LDK = KVTile<IO, D, NT>::LDK, LDV = KVTile<IO, D, NT>::LDV;
  for (int i = threadIdx.x * 4; i < 64 * D; i += 256 * 4) {
    const int key = i / D, e = i % D;
    float kx[4], vx[4];
    const bool ok = key < nvalid;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kx[u] = ok ? io_traits<IO>::load(k, (row0 + key) * D + e + u) : 0.f;
      vx[u] = ok ? io_traits<IO>::load(v, (row0 + key) * D + e + u) : 0.f;
    }
    uint16_t ks[4][NT], vs[4][NT];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      split_bf16<NT>(kx[u], ks[u]);
      split_bf16<NT>(vx[u], vs[u]);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      u32x2_t pk;
      pk.x = (uint32_t)ks[0][j] | ((uint32_t)ks[1][j] << 16);
      pk.y = (uint32_t)ks[2][j] | ((uint32_t)ks[3][j] << 16);
      *reinterpret_cast<u32x2_t*>(&tile.k[j][key * LDK + e]) = pk;
#pragma unroll
      for (int u = 0; u < 4; ++u) tile.vt[j][(e + u) * LDV + key] = vs[u][j];
    }
  }
}

HILS_DEV bf16x8_t lds_kop(const uint16_t* rowp, int ks, int hf) {
  const uint16_t* p = rowp + 16 * ks + 4 * hf;
  return pack8(*reinterpret_cast<const u32x2_t*>(p), *reinterpret_cast<const u32x2_t*>(p + 8));
}

// One wave: 32 query rows (B operands qb, NT terms) against the staged chunk.
// Returns, per lane (row n = lane & 31, half hf), the O^T accumulators (unnormalised)
// and the row's softmax max m and sum l over the keys allowed by `key_lim`
// (key j is used iff j < key_lim; per row).
template <typename IO, int D, int NT>
HILS_DEV void wave_chunk_attention(const KVTile<IO, D, NT>& tile, const bf16x8_t (&qb)[NT][D / 16], int key_lim,
                                   f32x16_t (&o)[D / 32], float& m_out, float& l_out) {
  constexpr int NKS = D / 16;
  constexpr int LDK = KVTile<IO, D, NT>::LDK, LDV = KVTile<IO, D, NT>::LDV;
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float tau = 1.0f / sqrtf((float)D);
  f32x16_t s[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    s[tt] = zero16();
    const int key = 32 * tt + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8_t a = lds_kop(&tile.k[j][key * LDK], ks, hf);
#pragma unroll
        for (int i = 0; i < NT; ++i)
          if (i + j < NT) s[tt] = mfma32(a, qb[i][ks], s[tt]);
      }
  }
  float m = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 32 * tt + acc_row(rr, hf);
      const float z = key < key_lim ? s[tt][rr] * tau : -INFINITY;
      s[tt][rr] = z;
      m = fmaxf(m, z);
    }
  m = fmaxf(m, __shfl_xor(m, 32));
  float l = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float p = (m == -INFINITY) ? 0.f : expf(s[tt][rr] - m);
      s[tt][rr] = p;
      l += p;
    }
  l += __shfl_xor(l, 32);
  // P^T as B operand: k-step ks2 (keys 16*ks2 ..), element mm = register 8*(ks2&1)+mm of tile ks2>>1
  bf16x8_t pb[NT][4];
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
    uint16_t t[NT][8];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      uint16_t sp[NT];
      split_bf16<NT>(s[ks2 >> 1][8 * (ks2 & 1) + mm], sp);
#pragma unroll
      for (int j = 0; j < NT; ++j) t[j][mm] = sp[j];
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) pb[j][ks2] = pack8(t[j]);
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    o[dt] = zero16();
    const int e = 32 * dt + (lane & 31);
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8_t a = lds_kop(&tile.vt[j][e * LDV], ks2, hf);
#pragma unroll
        for (int i = 0; i < NT; ++i)
          if (i + j < NT) o[dt] = mfma32(a, pb[i][ks2], o[dt]);
      }
  }
  m_out = m;
  l_out = l;
}

// Loads query row `qrow_off` (element offset of the row) as NT-term B operands.
template <typename IO, int D, int NT>
HILS_DEV void load_q_operand(const IO* __restrict__ q, int64_t qrow_off, bool ok, bf16x8_t (&qb)[NT][D / 16]) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint16_t t[NT][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float x = ok ? io_traits<IO>::load(q, qrow_off + kperm(ks, hf, m)) : 0.f;
      uint16_t s[NT];
      split_bf16<NT>(x, s);
#pragma unroll
      for (int j = 0; j < NT; ++j) t[j][m] = s[j];
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) qb[j][ks] = pack8(t[j]);
  }
}

template <typename IO>
struct partial_t {
  using type = uint16_t;  // fp16 bits
  static constexpr int bytes = 2;
};
template <>
struct partial_t<float> {
  using type = float;
  static constexpr int bytes = 4;
};

// ------------------------------------------------------------- chunk_attend
template <typename IO, int D>
__global__ void __launch_bounds__(256) chunk_attend(const IO* __restrict__ q, const IO* __restrict__ k,
                                                    const IO* __restrict__ v, const uint32_t* __restrict__ pairs,
                                                    const uint32_t* __restrict__ boff, const uint32_t* __restrict__ toff,
                                                    void* __restrict__ partial_v, int Hkv, int N, int C, int K,
                                                    int nbk, int grid_items) {
  constexpr int NT = io_traits<IO>::terms;
  using PT = typename partial_t<IO>::type;
  __shared__ KVTile<IO, D, NT> tile;
  const int tix = remap_xcd(blockIdx.x, grid_items);
  const uint32_t ntiles = toff[nbk];
  if (tix >= grid_items || (uint32_t)tix >= ntiles) return;
  // bucket = last index with toff[bk] <= tix
  int lo = 0, hi = nbk - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (toff[mid] <= (uint32_t)tix) lo = mid;
    else hi = mid - 1;
  }
  const int bk = lo;
  const uint32_t count = boff[bk + 1] - boff[bk];
  const uint32_t first = ((uint32_t)tix - toff[bk]) * AT_ROWS;
  const int c = bk % C, kvh = (bk / C) % Hkv, b = bk / (C * Hkv);
  const int64_t row0 = ((int64_t)b * Hkv + kvh) * N + (int64_t)c * 64;
  stage_kv<IO, D, NT>(tile, k, v, row0, 64);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hf = lane >> 5;
  const uint32_t p = first + 32 * w + (lane & 31);
  const bool ok = p < count;
  const uint32_t e_pair = ok ? pairs[boff[bk] + p] : 0;
  const int64_t qrow = e_pair / (uint32_t)K;  // (b*Hq + h)*N + i
  bf16x8_t qb[NT][D / 16];
  load_q_operand<IO, D, NT>(q, qrow * D, ok, qb);
  __syncthreads();
  f32x16_t o[D / 32];
  float m, l;
  wave_chunk_attention<IO, D, NT>(tile, qb, 64, o, m, l);
  if (ok) {
    const float inv = 1.0f / l;
    PT* dst = reinterpret_cast<PT*>(partial_v) + (int64_t)e_pair * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int e = 32 * dt + 8 * g4 + 4 * hf;
        if constexpr (sizeof(PT) == 2) {
          u32x2_t pk;
          pk.x = (uint32_t)f32_to_f16(o[dt][4 * g4 + 0] * inv) | ((uint32_t)f32_to_f16(o[dt][4 * g4 + 1] * inv) << 16);
          pk.y = (uint32_t)f32_to_f16(o[dt][4 * g4 + 2] * inv) | ((uint32_t)f32_to_f16(o[dt][4 * g4 + 3] * inv) << 16);
          *reinterpret_cast<u32x2_t*>(dst + e) = pk;
        } else {
          *reinterpret_cast<float4*>(dst + e) = make_float4(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv,
                                                            o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv);
        }
      }
  }
}

// ---------------------------------------------------------------- fuse_own
// One workgroup per (b, h, query chunk qc): rows qc*64 .. qc*64+63.
template <typename IO, int D>
__global__ void __launch_bounds__(256) fuse_own(const IO* __restrict__ q, const IO* __restrict__ k,
                                                const IO* __restrict__ v, const int32_t* __restrict__ sel_idx,
                                                const float* __restrict__ sel_score, const void* __restrict__ partial_v,
                                                IO* __restrict__ o, int Hq, int Hkv, int N, int K, int NQC) {
  constexpr int NT = io_traits<IO>::terms;
  using PT = typename partial_t<IO>::type;
  __shared__ KVTile<IO, D, NT> tile;
  __shared__ float own[64][D + 1];
  __shared__ float lse[64];
  const int qc = blockIdx.x % NQC, bh = blockIdx.x / NQC;
  const int h = bh % Hq, b = bh / Hq;
  const int kvh = h / (Hq / Hkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hf = lane >> 5;
  const int key0 = qc * 64;
  const int nkeys = min(64, N - key0);
  stage_kv<IO, D, NT>(tile, k, v, ((int64_t)b * Hkv + kvh) * N + key0, nkeys);
  __syncthreads();
  if (w < 2) {  // own chunk on the MFMA: wave w takes rows 32w .. 32w+31 of the chunk
    const int rl = 32 * w + (lane & 31);
    const int i = key0 + rl;
    const bool ok = i < N;
    bf16x8_t qb[NT][D / 16];
    load_q_operand<IO, D, NT>(q, ((int64_t)bh * N + (ok ? i : 0)) * D, ok, qb);
    f32x16_t oa[D / 32];
    float m, l;
    wave_chunk_attention<IO, D, NT>(tile, qb, rl + 1, oa, m, l);  // causal: keys 0..rl
    const float inv = 1.0f / l;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) own[rl][32 * dt + acc_row(rr, hf)] = oa[dt][rr] * inv;
    if (hf == 0) lse[rl] = m + logf(l);
  }
  __syncthreads();
  // fusion: wave w handles rows w, w+4, ...; lane owns head dims lane, lane+64
  for (int rl = w; rl < 64; rl += 4) {
    const int i = key0 + rl;
    if (i >= N) break;
    const int64_t row = (int64_t)bh * N + i;
    const float sc = lane < K ? sel_score[row * K + lane] : -INFINITY;
    const int ci = lane < K ? sel_idx[row * K + lane] : -1;
    const float lo = lse[rl];
    const float M = fmaxf(wave_max(ci >= 0 ? sc : -INFINITY), lo);
    const float wt = ci >= 0 ? expf(sc - M) : 0.f;
    const float wo = expf(lo - M);
    const float Z = wave_sum(wt) + wo;
    const int nsel = __popcll(__ballot(ci >= 0));
    float acc0 = wo * own[rl][lane];
    float acc1 = (D > 64) ? wo * own[rl][lane + 64] : 0.f;
    const PT* src = reinterpret_cast<const PT*>(partial_v) + row * K * D;
    for (int t = 0; t < nsel; ++t) {
      const float wtt = __shfl(wt, t);
      const PT* ps = src + (int64_t)t * D;
      if constexpr (sizeof(PT) == 2) {
        acc0 = fmaf(wtt, f16_to_f32(ps[lane]), acc0);
        if (D > 64) acc1 = fmaf(wtt, f16_to_f32(ps[lane + 64]), acc1);
      } else {
        acc0 = fmaf(wtt, ps[lane], acc0);
        if (D > 64) acc1 = fmaf(wtt, ps[lane + 64], acc1);
      }
    }
    const float inv = 1.0f / Z;
    io_traits<IO>::store(o, row * D + lane, acc0 * inv);
    if (D > 64) io_traits<IO>::store(o, row * D + lane + 64, acc1 * inv);
  }
}

// ------------------------------------------------------------------ launcher
template <typename IO, int D>
static hipError_t launch_attend_t(const Geom& g, const void* q, const void* k, const void* v, const int32_t* sel,
                                  const float* scr, void* o, char* ws, hipStream_t st, hipEvent_t* ev) {
  const AttendWs w = attend_ws(g);
  uint32_t* counts = (uint32_t*)(ws + w.counts);
  uint32_t* cursor = (uint32_t*)(ws + w.cursor);
  uint32_t* boff = (uint32_t*)(ws + w.boff);
  uint32_t* toff = (uint32_t*)(ws + w.toff);
  uint32_t* pairs = (uint32_t*)(ws + w.pairs);
  void* partial = ws + w.partial;
  const int C = g.C();
  const int nbk = g.B * g.Hkv * C;
  // zero counts and cursors (contiguous) with a kernel: no memset nodes in captured streams
  const int64_t nz = (int64_t)(w.boff - w.counts) / 4;
  hipLaunchKernelGGL(zero_u32, dim3((unsigned)std::min<int64_t>((nz + 255) / 256, 4096)), dim3(256), 0, st, counts, nz);
  if (nbk > 0) {
    const int64_t group_len = (int64_t)g.G() * g.N * g.K;
    const int spg = (int)((group_len + HIST_SLICE - 1) / HIST_SLICE);
    const int ngrp = g.B * g.Hkv;
    hipLaunchKernelGGL(bucket_count, dim3(ngrp * spg), dim3(256), 0, st, sel, counts, group_len, spg, C);
    hipLaunchKernelGGL(bucket_scan, dim3(1), dim3(1024), 0, st, counts, boff, toff, nbk);
    hipLaunchKernelGGL(bucket_scatter, dim3(ngrp * spg), dim3(256), 0, st, sel, boff, cursor, pairs, group_len, spg, C);
    if (ev) hipEventRecord(ev[0], st);
    // tiles <= total pairs / AT_ROWS + number of buckets (host bound, exact count read on the device)
    // rows of query chunk p (64 of them, fewer in the tail) select min(K, p, C) chunks each
    int64_t pairs_total = 0;
    for (int p = 0; p * 64 < g.N; ++p) pairs_total += (int64_t)std::min(64, g.N - p * 64) * std::min(g.K, std::min(C, p));
    pairs_total *= (int64_t)g.B * g.Hq;
    const int64_t tiles = (pairs_total + AT_ROWS - 1) / AT_ROWS + nbk;
    const int grid_items = (int)tiles;
    const int grid = ((grid_items + 7) / 8) * 8;
    if (pairs_total > 0)
      hipLaunchKernelGGL((chunk_attend<IO, D>), dim3(grid), dim3(256), 0, st, (const IO*)q, (const IO*)k, (const IO*)v,
                         pairs, boff, toff, partial, g.Hkv, g.N, C, g.K, nbk, grid_items);
    if (ev) hipEventRecord(ev[1], st);
  } else if (ev) {
    hipEventRecord(ev[0], st);
    hipEventRecord(ev[1], st);
  }
  const int NQC = (g.N + 63) / 64;
  hipLaunchKernelGGL((fuse_own<IO, D>), dim3(g.B * g.Hq * NQC), dim3(256), 0, st, (const IO*)q, (const IO*)k,
                     (const IO*)v, sel, scr, (const void*)partial, (IO*)o, g.Hq, g.Hkv, g.N, g.K, NQC);
  if (ev) hipEventRecord(ev[2], st);
  return hipGetLastError();
}

hipError_t launch_prefill_attend(const Geom& g, const void* q, const void* k, const void* v, const int32_t* sel_idx,
                                 const float* sel_score, void* o, void* ws, size_t ws_bytes, hipStream_t st,
                                 hipEvent_t* ev) {
  if (ws_bytes < attend_workspace_bytes(g)) return hipErrorInvalidValue;
  if (g.C() > MAX_C) return hipErrorNotSupported;
  char* w = (char*)ws;
  if (g.io == 0)
    return g.d == 64 ? launch_attend_t<float, 64>(g, q, k, v, sel_idx, sel_score, o, w, st, ev)
                     : launch_attend_t<float, 128>(g, q, k, v, sel_idx, sel_score, o, w, st, ev);
  return g.d == 64 ? launch_attend_t<bf16_t, 64>(g, q, k, v, sel_idx, sel_score, o, w, st, ev)
                   : launch_attend_t<bf16_t, 128>(g, q, k, v, sel_idx, sel_score, o, w, st, ev);
}

}  // namespace hils

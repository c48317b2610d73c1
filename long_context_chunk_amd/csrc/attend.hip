// Intra-chunk attention and fusion for prefill, given each query's selection.
//
//   o_ic   = sum_{j in c} softmax_j(q_i . k_j / sqrt(d)) v_j       for each selected chunk c
//   o_own  = the same over the own chunk, keys cS .. i (causal); LSE_own its log-sum-exp.
//            With a local window of nw chunks: one softmax over chunks c - nw + 1 .. c
//            (keys up to i), and the selections come from the chunks before them.
//   o_i    = sum_c w_c o_ic + w_own o_own,  w = softmax over {s_ic} U {LSE_own}
// (hotpaper.ai abstract: each query attends each retrieved chunk independently
// and the outputs are fused by the chunk retrieval scores; aitrends.kr
// "Methodology" calculation flow; ai-papers.net Fig. 1.)
//
// Chunk-major execution.  The pages' kernel packs M adjacent queries x G heads and
// loads the union of their chunks; on near-independent selections that union is
// dozens of times larger than K and most MFMA work is masked out.  Here every
// (query row, selected chunk) pair is bucketed by (batch, query head, chunk); each
// workgroup loads one chunk's K/V tile into LDS once and runs full 32-row MFMA
// tiles of gathered query rows against it.  Per pair it writes the normalised
// chunk output o_ic (fp16 for bf16 I/O, fp32 for fp32 I/O) to a slot of its row
// (K + 1 slots per row); a per-query-chunk pass writes the own chunk's output to
// the last slot, and a streaming pass fuses the slots.
//
//   bucket_count  : LDS-privatised histogram of the selections per bucket
//   bucket_scan   : exclusive scans -> bucket offsets and tile offsets
//   bucket_part1/2: two-digit counting sort of the pair ids (= linear index into
//                   sel_idx) by bucket: first into ranges of 64 chunks, then into
//                   chunks, each pass sorting tiles in LDS and writing whole runs
//   chunk_attend  : gathered-row MFMA attention per (bucket, 128-row tile)
//   own_attend    : causal own-chunk MFMA attention -> slot K and LSE_own
//   window_attend : the same over a local window of several chunks (online softmax)
//   fuse          : softmax over {s_ic} U {LSE_own}, weighted sum of the slots -> o
#include <algorithm>

#include "attn_tile.h"
#include "hils_common.h"
#include "kernels.h"

namespace hils {

constexpr int AT_ROWS = 128;        // gathered rows per chunk_attend tile (4 waves x 32)
constexpr int AT_TILES = 8;         // tiles per chunk_attend work item (one K/V staging)
constexpr int ITEM_ROWS = AT_ROWS * AT_TILES;
static_assert(ITEM_ROWS == BUCKET_ITEM_ROWS, "one work-item size for every user of the bucketing");
constexpr int HIST_SLICE = 1 << 17; // largest slice of selection entries per bucket_count / bucket_part1 workgroup
constexpr int P2_SPLIT = 4;         // fewest workgroups sharing one 64-chunk range in bucket_part2
constexpr int BK_FILL = 512;        // workgroups the bucketing passes aim for (two per CU)
constexpr int BK_TILE = 8192;       // entries sorted in LDS at a time by bucket_part1/2
constexpr int BK_PER = BK_TILE / 256;
constexpr int FINE_BITS = 6;        // chunks per first-pass range: 64
constexpr int LOCAL_BITS = 26;      // in-group pair index bits of the first-pass keys
constexpr int MAX_C = 16384;        // largest chunk count the LDS histograms hold

struct AttendWs {
  size_t counts, cursor, boff, toff, pairs, imap, partial, lse, sink, total;
};

static size_t al(size_t x) { return (x + 255) / 256 * 256; }

static AttendWs attend_ws(const Geom& g) {
  AttendWs w;
  const size_t nbk = (size_t)g.B * g.Hq * g.C();
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
  w.imap = off;
  off += al((size_t)bucket_items_bound(g) * 4);
  // per row K + 1 output slots: the selected chunks' in selection order, then the own chunk
  const size_t rows = (size_t)g.B * g.Hq * g.N;
  w.partial = off;
  off += al(rows * (g.K + 1) * g.d * (g.io == 0 ? 4 : 2));
  w.lse = off;
  off += al(rows * 4);
  w.sink = off;  // target of the stores of padding rows (never read)
  off += al(4096);
  w.total = off;
  return w;
}

size_t attend_workspace_bytes(const Geom& g) { return attend_ws(g).total; }

// ------------------------------------------------------------------ bucketing
__global__ void __launch_bounds__(256) zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// Buckets are (b, h, chunk), numbered head-major; the selection entries of one
// (b, h) group (all rows, all K slots) are contiguous in sel_idx.
__global__ void __launch_bounds__(256) bucket_count(const int32_t* __restrict__ sel, uint32_t* __restrict__ counts,
                                                    int64_t group_len, int64_t slice, int slices_per_group, int C) {
  __shared__ uint32_t hist[MAX_C];
  const int grp = blockIdx.x / slices_per_group, sl = blockIdx.x % slices_per_group;
  for (int i = threadIdx.x; i < C; i += 256) hist[i] = 0;
  __syncthreads();
  const int64_t beg = (int64_t)sl * slice, end = min(group_len, beg + slice);
  const int32_t* s = sel + (int64_t)grp * group_len;
  for (int64_t t0 = beg; t0 < end; t0 += BK_TILE) {
    int32_t c[BK_PER];  // every load of the tile in flight at once
#pragma unroll
    for (int u = 0; u < BK_PER; ++u) {
      const int64_t i = t0 + threadIdx.x + 256 * u;
      c[u] = i < end ? s[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < BK_PER; ++u)
      if ((unsigned)c[u] < (unsigned)C) atomicAdd(&hist[c[u]], 1u);  // -1 (padding) and bad ids skipped
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += 256)
    if (hist[i]) atomicAdd(&counts[(int64_t)grp * C + i], hist[i]);
}

// Single workgroup: boff = exclusive scan of counts, toff = exclusive scan of
// ceil(count / ITEM_ROWS) (work items).  Both get a final total entry; counts is
// left zeroed for reuse as per-bucket cursors.
__global__ void __launch_bounds__(1024) bucket_scan(uint32_t* __restrict__ counts, uint32_t* __restrict__ boff,
                                                    uint32_t* __restrict__ toff, int nbk) {
  __shared__ uint32_t sa[1024], sb[1024];
  const int t = threadIdx.x;
  const int per = (nbk + 1023) / 1024;
  const int beg = min(nbk, t * per), end = min(nbk, beg + per);
  uint32_t a = 0, b = 0;
  for (int i = beg; i < end; ++i) {
    a += counts[i];
    b += (counts[i] + ITEM_ROWS - 1) / ITEM_ROWS;
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
    const uint32_t ci = counts[i];
    boff[i] = ra;
    toff[i] = rb;
    ra += ci;
    rb += (ci + ITEM_ROWS - 1) / ITEM_ROWS;
    counts[i] = 0;  // from here on: the second sorting pass's cursor of bucket i
  }
  if (t == 1023) {
    boff[nbk] = sa[t];
    toff[nbk] = sb[t];
  }
}

// The same scan for many buckets, in three steps over blocks of 1024 buckets: block
// totals (parked in the first entry of the block's boff / toff range), their exclusive
// scan by one workgroup (which also writes the grand totals), then each block's own scan
// from its offset.  Each block reads only its own parked totals before overwriting them.
constexpr int SCAN_BLOCK = 1024;

__global__ void __launch_bounds__(256) bucket_block_sums(const uint32_t* __restrict__ counts,
                                                         uint32_t* __restrict__ boff, uint32_t* __restrict__ toff,
                                                         int nbk) {
  __shared__ uint32_t wsum[8];
  const int i0 = blockIdx.x * SCAN_BLOCK, t = threadIdx.x;
  uint32_t a = 0, b = 0;
  for (int i = i0 + t; i < min(nbk, i0 + SCAN_BLOCK); i += 256) {
    const uint32_t ci = counts[i];
    a += ci;
    b += (ci + ITEM_ROWS - 1) / ITEM_ROWS;
  }
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  if ((t & 63) == 0) {
    wsum[t >> 6] = a;
    wsum[4 + (t >> 6)] = b;
  }
  __syncthreads();
  if (t == 0) {
    boff[i0] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    toff[i0] = wsum[4] + wsum[5] + wsum[6] + wsum[7];
  }
}

__global__ void __launch_bounds__(1024) bucket_block_scan(uint32_t* __restrict__ boff, uint32_t* __restrict__ toff,
                                                          int nbk, int nblk) {
  __shared__ uint32_t sa[1024], sb[1024];
  const int t = threadIdx.x;
  const int per = (nblk + 1023) / 1024;
  const int beg = min(nblk, t * per), end = min(nblk, beg + per);
  uint32_t a = 0, b = 0;
  for (int j = beg; j < end; ++j) {
    a += boff[j * SCAN_BLOCK];
    b += toff[j * SCAN_BLOCK];
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
  uint32_t ra = sa[t] - a, rb = sb[t] - b;
  for (int j = beg; j < end; ++j) {
    const uint32_t xa = boff[j * SCAN_BLOCK], xb = toff[j * SCAN_BLOCK];
    boff[j * SCAN_BLOCK] = ra;
    toff[j * SCAN_BLOCK] = rb;
    ra += xa;
    rb += xb;
  }
  if (t == 1023) {
    boff[nbk] = sa[t];
    toff[nbk] = sb[t];
  }
}

__global__ void __launch_bounds__(256) bucket_block_fill(uint32_t* __restrict__ counts, uint32_t* __restrict__ boff,
                                                         uint32_t* __restrict__ toff, int nbk) {
  __shared__ uint32_t wsum[8];
  const int i0 = blockIdx.x * SCAN_BLOCK, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint32_t a0 = boff[i0], b0 = toff[i0];  // the block's offsets (parked by the scan)
  // four consecutive buckets per thread
  uint32_t c[4], it[4], a = 0, b = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int i = i0 + 4 * t + m;
    c[m] = i < nbk ? counts[i] : 0u;
    it[m] = (c[m] + ITEM_ROWS - 1) / ITEM_ROWS;
    a += c[m];
    b += it[m];
  }
  // exclusive scan of (a, b) over the 256 threads
  uint32_t xa = a, xb = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ya = __shfl_up(xa, o), yb = __shfl_up(xb, o);
    if (lane >= o) {
      xa += ya;
      xb += yb;
    }
  }
  if (lane == 63) {
    wsum[w] = xa;
    wsum[4 + w] = xb;
  }
  __syncthreads();  // every thread has read boff[i0] / toff[i0] above
  uint32_t ra = a0 + xa - a, rb = b0 + xb - b;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < w) {
      ra += wsum[j];
      rb += wsum[4 + j];
    }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int i = i0 + 4 * t + m;
    if (i < nbk) {
      boff[i] = ra;
      toff[i] = rb;
      counts[i] = 0;  // from here on: the second sorting pass's cursor of bucket i
    }
    ra += c[m];
    rb += it[m];
  }
}

// Work item -> bucket: each bucket writes its own items' entries, so the work kernels
// find their bucket with one load instead of a search over toff.
__global__ void __launch_bounds__(256) bucket_item_map(const uint32_t* __restrict__ toff, uint32_t* __restrict__ imap,
                                                       int nbk) {
  const int bk = blockIdx.x * 256 + threadIdx.x;
  if (bk >= nbk) return;
  const uint32_t t0 = toff[bk], t1 = toff[bk + 1];
  for (uint32_t t = t0; t < t1; ++t) imap[t] = (uint32_t)bk;
}

// exclusive scan of v over the 256 threads of the workgroup; returns the total
HILS_DEV uint32_t block_exscan256(uint32_t v, uint32_t& excl, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    before += j < w ? wsum[j] : 0u;
    total += wsum[j];
  }
  excl = before + x - v;
  return total;
}

// First pass: the entries of one slice of a (b, h) group, LDS tile by LDS tile, are
// sorted by 64-chunk range and each range's run is appended (one atomic reservation per
// tile and range) to that range's region of the bucket-ordered array, which is the
// concatenation of its chunks' buckets (offsets from boff).  Keys: (chunk & 63) << 26 |
// in-group entry index.
__global__ void __launch_bounds__(256) bucket_part1(const int32_t* __restrict__ sel, const uint32_t* __restrict__ boff,
                                                    uint32_t* __restrict__ rcur, uint32_t* __restrict__ tmp,
                                                    int64_t group_len, int64_t slice, int slices_per_group, int C,
                                                    int nrg) {
  __shared__ uint32_t skey[BK_TILE];
  __shared__ uint8_t srg[BK_TILE];
  __shared__ uint32_t hist[256], loff[256], gpos[256], wsum[4];
  const int grp = blockIdx.x / slices_per_group, sl = blockIdx.x % slices_per_group;
  const int t = threadIdx.x;
  const int64_t beg = (int64_t)sl * slice, end = min(group_len, beg + slice);
  const int32_t* s = sel + (int64_t)grp * group_len;
  // a tile's entries, loaded during the previous tile's scatter and writes (indices past
  // the slice read its last entry, in bounds, and are dropped)
  int32_t nx[BK_PER];
  auto fetch = [&](int64_t t0n) {
#pragma unroll
    for (int u = 0; u < BK_PER; ++u) nx[u] = s[min(t0n + t + 256 * u, end - 1)];
  };
  if (beg < end) fetch(beg);
  for (int64_t t0 = beg; t0 < end; t0 += BK_TILE) {
    hist[t] = 0;
    int32_t c[BK_PER];
    uint32_t rk[BK_PER];
#pragma unroll
    for (int u = 0; u < BK_PER; ++u) {
      const int64_t i = t0 + t + 256 * u;
      c[u] = i < end && (unsigned)nx[u] < (unsigned)C ? nx[u] : -1;  // the same entries bucket_count counted
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < BK_PER; ++u)
      if (c[u] >= 0) rk[u] = atomicAdd(&hist[c[u] >> FINE_BITS], 1u);
    __syncthreads();
    const uint32_t h = hist[t];  // t < nrg <= 256; hist[t] = 0 beyond
    uint32_t ex;
    block_exscan256(h, ex, wsum);
    loff[t] = ex;
    if (t < nrg && h) {
      const int64_t bk0 = (int64_t)grp * C + ((int64_t)t << FINE_BITS);
      gpos[t] = boff[bk0] + atomicAdd(&rcur[(int64_t)grp * nrg + t], h);
    }
    __syncthreads();
    if (t0 + BK_TILE < end) fetch(t0 + BK_TILE);  // after this tile's global reads, before its writes
#pragma unroll
    for (int u = 0; u < BK_PER; ++u)
      if (c[u] >= 0) {
        const int r = c[u] >> FINE_BITS;
        const uint32_t pos = loff[r] + rk[u];
        skey[pos] = ((uint32_t)(c[u] & ((1 << FINE_BITS) - 1)) << LOCAL_BITS) | (uint32_t)(t0 + t + 256 * u);
        srg[pos] = (uint8_t)r;
      }
    __syncthreads();
    const uint32_t n = loff[255] + hist[255];
    for (uint32_t i = t; i < n; i += 256) {
      const int r = srg[i];
      tmp[gpos[r] + (i - loff[r])] = skey[i];
    }
    __syncthreads();
  }
}

// Second pass: `split` workgroups per (group, 64-chunk range) sort the range's region by
// chunk, LDS tile by LDS tile (tiles dealt round-robin), reserving each chunk's run with
// one atomic per (tile, chunk) on that bucket's cursor.
__global__ void __launch_bounds__(256) bucket_part2(const uint32_t* __restrict__ tmp, const uint32_t* __restrict__ boff,
                                                    uint32_t* __restrict__ fcur, uint32_t* __restrict__ pairs,
                                                    int64_t group_len, int C, int nrg, int split) {
  constexpr int NF = 1 << FINE_BITS;
  __shared__ uint32_t skey[BK_TILE];
  __shared__ uint8_t sfb[BK_TILE];
  __shared__ uint32_t hist[NF], loff[NF], gpos[NF];
  const int sp = blockIdx.x % split, gr = blockIdx.x / split;
  const int grp = gr / nrg, rg = gr % nrg;
  const int t = threadIdx.x, lane = t & 63;
  const int c0 = rg << FINE_BITS;
  const int nf = min(NF, C - c0);
  const int64_t bk0 = (int64_t)grp * C + c0;
  const uint32_t R0 = boff[bk0], R1 = boff[bk0 + nf];
  const uint32_t ebase = (uint32_t)(grp * group_len);
  const uint32_t stride = (uint32_t)split * BK_TILE;
  // a tile's keys, loaded during the previous tile's scatter and writes (indices past the
  // range read its last key, in bounds, and are dropped)
  uint32_t nx[BK_PER];
  auto fetch = [&](uint32_t t0n) {
#pragma unroll
    for (int u = 0; u < BK_PER; ++u) nx[u] = tmp[min(t0n + t + 256 * u, R1 - 1)];
  };
  // 64-bit tile starts: R1 may lie within one stride of 2^32
  if ((uint64_t)R0 + (uint64_t)sp * BK_TILE < R1) fetch(R0 + (uint32_t)sp * BK_TILE);
  for (uint64_t t0l = (uint64_t)R0 + (uint64_t)sp * BK_TILE; t0l < R1; t0l += stride) {
    const uint32_t t0 = (uint32_t)t0l;
    if (t < NF) hist[t] = 0;
    uint32_t key[BK_PER], rk[BK_PER];
#pragma unroll
    for (int u = 0; u < BK_PER; ++u) key[u] = t0l + t + 256 * u < R1 ? nx[u] : 0xffffffffu;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < BK_PER; ++u)
      if (key[u] != 0xffffffffu) rk[u] = atomicAdd(&hist[key[u] >> LOCAL_BITS], 1u);
    __syncthreads();
    if (t < 64) {  // one wave scans the NF = 64 chunk counts and reserves their runs
      const uint32_t h = hist[lane];
      uint32_t x = h;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      loff[lane] = x - h;
      if (lane < nf && h) gpos[lane] = boff[bk0 + lane] + atomicAdd(&fcur[bk0 + lane], h);
    }
    __syncthreads();
    if (t0l + stride < R1) fetch(t0 + stride);  // after this tile's global reads, before its writes
#pragma unroll
    for (int u = 0; u < BK_PER; ++u)
      if (key[u] != 0xffffffffu) {
        const int f = key[u] >> LOCAL_BITS;
        const uint32_t pos = loff[f] + rk[u];
        skey[pos] = key[u] & ((1u << LOCAL_BITS) - 1);
        sfb[pos] = (uint8_t)f;
      }
    __syncthreads();
    const uint32_t n = min((uint32_t)BK_TILE, R1 - t0);
    for (uint32_t i = t; i < n; i += 256) {
      const int f = sfb[i];
      pairs[gpos[f] + (i - loff[f])] = ebase + skey[i];
    }
    __syncthreads();
  }
}


template <typename IO>
struct partial_t {
  using type = uint16_t;  // fp16 bits
};
template <>
struct partial_t<float> {
  using type = float;
};

// ------------------------------------------------------------- chunk_attend
// One work item = up to AT_TILES tiles of 128 gathered rows of one bucket (b, h, c):
// the chunk's K/V tile is staged into LDS once; then each wave runs its own pipeline
// over its 32 rows of every tile (no further barriers): the query rows of the next
// tile are loaded into registers (16 bytes per lane, whole rows) while the current
// tile is on the MFMA, and the normalised outputs leave through the wave's LDS rows
// as whole-row 16-byte stores.  Work items run in bucket order, head-major, so the
// rows gathered at any time come from one head and stay cache-resident.
template <typename IO, int D>
__global__ void __launch_bounds__(256, 2) chunk_attend(const IO* __restrict__ q, const IO* __restrict__ k,
                                                       const IO* __restrict__ v, const uint32_t* __restrict__ pairs,
                                                       const uint32_t* __restrict__ boff,
                                                       const uint32_t* __restrict__ toff,
                                                       const uint32_t* __restrict__ imap, void* __restrict__ partial_v,
                                                       char* __restrict__ sink, int Hq, int Hkv, int N, int C, int K,
                                                       int nbk) {
  constexpr int NT = io_traits<IO>::terms;
  constexpr bool STAGE = NT == 1;
  constexpr int LDQ = D + 8;   // bf16 row stride of the staged rows (16-byte aligned rows)
  constexpr int SEGS = D / 8;  // 16-byte segments per bf16 row
  constexpr int RPL = 64 / SEGS;  // rows covered by one wave-wide 16-byte load
  constexpr int NLD = 32 / RPL;   // loads per lane for the wave's 32 rows
  __shared__ KVTile<IO, D, NT> tile;
  __shared__ __align__(16) uint16_t qs[STAGE ? AT_ROWS * LDQ : 8];
  __shared__ uint32_t ipid[ITEM_ROWS];  // the item's output slots (in-head, K + 1 per row) ...
  __shared__ uint32_t irow[ITEM_ROWS];  // ... and their in-head query rows
  const int item = blockIdx.x;
  if ((uint32_t)item >= toff[nbk]) return;
  const int bk = (int)imap[item];
  const uint32_t count = boff[bk + 1] - boff[bk];
  const uint32_t first = ((uint32_t)item - toff[bk]) * ITEM_ROWS;
  const uint32_t nrows = min((uint32_t)ITEM_ROWS, count - first);
  const uint32_t* pp = pairs + boff[bk] + first;
  const int c = bk % C, h = (bk / C) % Hq, b = bk / (C * Hq);
  const int kvh = h / (Hq / Hkv);
  const int64_t row0 = ((int64_t)b * Hkv + kvh) * N + (int64_t)c * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5;
  // every row of a bucket belongs to head bh: 32-bit offsets from the head's bases
  const int64_t bh = bk / C;
  const IO* __restrict__ q_head = q + bh * N * D;
  using PT = typename partial_t<IO>::type;
  PT* __restrict__ part_head = reinterpret_cast<PT*>(partial_v) + bh * N * (K + 1) * D;
  const uint32_t e_head = (uint32_t)(bh * N * K);
  // each wave records the pair ids and query rows of its own 32 rows of every tile, so
  // its gathers need no barrier and the first one overlaps the K/V staging below
#pragma unroll
  for (int j = 0; j < AT_TILES; j += 2) {
    const int r = (j + (lane >> 5)) * AT_ROWS + 32 * w + (lane & 31);
    const bool ok = (uint32_t)r < nrows;
    const uint32_t el = ok ? pp[r] - e_head : 0u;  // in-head pair index i*K + slot
    const uint32_t i = el / (uint32_t)K;
    ipid[r] = ok ? el + i : 0xffffffffu;  // slot of row i, K + 1 slots per row
    irow[r] = i;
  }
  __builtin_amdgcn_wave_barrier();
  const int ntile = (int)((nrows + AT_ROWS - 1) / AT_ROWS);
  const int rl = 32 * w + (lane & 31);
  if constexpr (STAGE) {
    uint16_t* myq = &qs[32 * w * LDQ];   // this wave's 32 staged rows
    const int lr = lane / SEGS, sg = lane % SEGS;
    char* pbase = reinterpret_cast<char*>(part_head) + 16 * sg;
    char* sinkp = sink + 16 * sg;
    // query rows of tiles j and j+1 in flight in two named register buffers, one per
    // tile parity.  Tiles past the item load query row 0 and padding rows store to the
    // sink: every load and store is issued unconditionally, so the wait counts stay exact
    // and the loads land straight in the buffer they are consumed from.
    u32x4_t qa[NLD], qb2[NLD];
    auto gather = [&](int j, u32x4_t(&buf)[NLD]) {
      const uint32_t keep = j < ntile ? 0xffffffffu : 0u;  // uniform
      const int jr = min(j, AT_TILES - 1);
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const uint32_t ir = irow[jr * AT_ROWS + 32 * w + RPL * u + lr] & keep;
        buf[u] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(q_head) +
                                                   (ir * (uint32_t)(D * sizeof(IO)) + 16u * sg));
      }
    };
    // tile j: its rows (in buf) to the wave's LDS rows, the prefetch of tile j + 2 into
    // buf, then the MFMA attention and whole-row fp16 stores through the same LDS rows
    auto step = [&](int j, u32x4_t(&buf)[NLD]) {
#pragma unroll
      for (int u = 0; u < NLD; ++u) *reinterpret_cast<u32x4_t*>(&myq[(RPL * u + lr) * LDQ + 8 * sg]) = buf[u];
      __builtin_amdgcn_wave_barrier();
      gather(j + 2, buf);
      if (j < ntile) {
        bf16x8_t qb[1][D / 16];
        lds_q_operand<D>(&myq[(lane & 31) * LDQ], qb);
        f32x16_t o[D / 32];
        float m, l;
        wave_chunk_attention<IO, D, NT, false>(tile, *reinterpret_cast<bf16x8_t(*)[NT][D / 16]>(&qb), 64, o, m, l);
        const float inv = __builtin_amdgcn_rcpf(l);  // l >= 1 (the max logit's term)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int e = 32 * dt + 8 * g4 + 4 * hf;
            u32x2_t pk;
            pk.x = pack_f16x2(o[dt][4 * g4 + 0] * inv, o[dt][4 * g4 + 1] * inv);
            pk.y = pack_f16x2(o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv);
            *reinterpret_cast<u32x2_t*>(&myq[(lane & 31) * LDQ + e]) = pk;
          }
        __builtin_amdgcn_wave_barrier();
        uint32_t slot[NLD];
        u32x4_t val[NLD];
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
          slot[u] = ipid[j * AT_ROWS + 32 * w + RPL * u + lr];
          val[u] = *reinterpret_cast<const u32x4_t*>(&myq[(RPL * u + lr) * LDQ + 8 * sg]);
        }
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
          char* dst = slot[u] != 0xffffffffu ? pbase + (uint64_t)slot[u] * (D * sizeof(PT)) : sinkp;
          __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4_t*>(dst));
        }
      }
      __builtin_amdgcn_wave_barrier();
    };
    gather(0, qa);
    gather(1, qb2);
    stage_kv<IO, D, NT>(tile, k, v, row0, 64, tid, 256);
    __syncthreads();
    for (int j = 0; j < ntile; j += 2) {
      step(j, qa);
      step(j + 1, qb2);
    }
  } else {
    stage_kv<IO, D, NT>(tile, k, v, row0, 64, tid, 256);
    __syncthreads();
    for (int j = 0; j < ntile; ++j) {
      const int r = j * AT_ROWS + rl;
      const uint32_t slot = ipid[r];
      const bool ok = slot != 0xffffffffu;
      bf16x8_t qb[NT][D / 16];
      load_q_operand<IO, D, NT>(q_head, (int64_t)irow[r] * D, ok, qb);
      f32x16_t o[D / 32];
      float m, l;
      wave_chunk_attention<IO, D, NT, false>(tile, qb, 64, o, m, l);
      const float inv = 1.0f / l;
      if (ok) {
        PT* dst = part_head + (int64_t)slot * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int e = 32 * dt + 8 * g4 + 4 * hf;
            *reinterpret_cast<float4*>(dst + e) =
                make_float4(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv, o[dt][4 * g4 + 2] * inv,
                            o[dt][4 * g4 + 3] * inv);
          }
      }
    }
  }
}

// ---------------------------------------------------------------- own_attend
// One workgroup per (b, KV head, query chunk qc) and group of up to OWN_HEADS of its
// query heads, two waves per head: rows qc*64 .. qc*64+63 of each head attend their own
// chunk causally on the MFMA, against one staging of the chunk's K/V; the normalised
// output goes to output slot K of the row and its log-sum-exp to lse[row].
constexpr int OWN_HEADS = 4;

template <typename IO, int D>
__global__ void __launch_bounds__(128 * OWN_HEADS) own_attend(const IO* __restrict__ q, const IO* __restrict__ k,
                                                              const IO* __restrict__ v, void* __restrict__ partial_v,
                                                              float* __restrict__ lse, int Hq, int Hkv, int N, int K,
                                                              int NQC, int hpw) {
  constexpr int NT = io_traits<IO>::terms;
  using PT = typename partial_t<IO>::type;
  __shared__ KVTile<IO, D, NT> tile;
  const int G = Hq / Hkv;
  const int ngb = (G + hpw - 1) / hpw;
  const int gb = blockIdx.x % ngb, rest = blockIdx.x / ngb;
  const int qc = rest % NQC, bkv = rest / NQC;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5;
  const int gi = gb * hpw + (w >> 1);  // this wave pair's query head in the group
  const bool head_ok = gi < G;
  const int h = kvh * G + min(gi, G - 1);
  const int bh = b * Hq + h;
  const int key0 = qc * 64;
  const int nkeys = min(64, N - key0);
  stage_kv<IO, D, NT>(tile, k, v, ((int64_t)b * Hkv + kvh) * N + key0, nkeys, tid, blockDim.x);
  const int rl = 32 * (w & 1) + (lane & 31);
  const int i = key0 + rl;
  const bool ok = i < N && head_ok;
  bf16x8_t qb[NT][D / 16];
  load_q_operand<IO, D, NT>(q, ((int64_t)bh * N + (ok ? i : 0)) * D, ok, qb);
  __syncthreads();
  f32x16_t oa[D / 32];
  float m, l;
  wave_chunk_attention<IO, D, NT, true>(tile, qb, rl + 1, oa, m, l);  // causal: keys 0..rl
  if (!ok) return;
  const int64_t row = (int64_t)bh * N + i;
  const float inv = 1.0f / l;
  PT* dst = reinterpret_cast<PT*>(partial_v) + (row * (K + 1) + K) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int e = 32 * dt + 8 * g4 + 4 * hf;
      if constexpr (sizeof(PT) == 2) {
        u32x2_t pk;
        pk.x = pack_f16x2(oa[dt][4 * g4 + 0] * inv, oa[dt][4 * g4 + 1] * inv);
        pk.y = pack_f16x2(oa[dt][4 * g4 + 2] * inv, oa[dt][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(dst + e) = pk;
      } else {
        *reinterpret_cast<float4*>(dst + e) = make_float4(oa[dt][4 * g4] * inv, oa[dt][4 * g4 + 1] * inv,
                                                          oa[dt][4 * g4 + 2] * inv, oa[dt][4 * g4 + 3] * inv);
      }
    }
  if (hf == 0) lse[row] = m + logf(l);
}

// ------------------------------------------------------------- window_attend
// The own chunk widened to a local window of nw > 1 chunks.  One workgroup of 256
// threads per (b, KV head, query chunk qc) and pair of its query heads, two waves per
// head (the waves of a head past the group's last only help staging): rows qc*64 ..
// qc*64+63 of each head attend chunks max(0, qc - nw + 1) .. qc, the own chunk qc
// causally, with one online softmax on the MFMA.  Each chunk's K/V is staged once for
// both heads, and the next chunk's global loads are issued before the current one is
// computed; two workgroups per CU overlap one's staging with the other's MFMA work.
// Output slot K and lse[row] as in own_attend.
constexpr int WIN_HEADS = 2;
constexpr int WIN_THREADS = 128 * WIN_HEADS;

template <typename IO, int D>
__global__ void __launch_bounds__(WIN_THREADS, 2) window_attend(const IO* __restrict__ q, const IO* __restrict__ k,
                                                             const IO* __restrict__ v, void* __restrict__ partial_v,
                                                             float* __restrict__ lse, int Hq, int Hkv, int N, int K,
                                                             int NQC, int nw) {
  constexpr int NT = io_traits<IO>::terms;
  using PT = typename partial_t<IO>::type;
  __shared__ KVTile<IO, D, NT> tile;
  const int G = Hq / Hkv;
  const int ngb = (G + WIN_HEADS - 1) / WIN_HEADS;
  const int gb = blockIdx.x % ngb, rest = blockIdx.x / ngb;
  const int qc = rest % NQC, bkv = rest / NQC;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5;
  const int gi = gb * WIN_HEADS + (w >> 1);  // this wave pair's query head in the group
  const bool head_ok = gi < G;
  const int h = kvh * G + min(gi, G - 1);
  const int bh = b * Hq + h;
  const int64_t kv0 = ((int64_t)b * Hkv + kvh) * N;
  const int rl = 32 * (w & 1) + (lane & 31);
  const int i = qc * 64 + rl;
  const bool ok = i < N && head_ok;
  bf16x8_t qb[NT][D / 16];
  load_q_operand<IO, D, NT>(q, ((int64_t)bh * N + (ok ? i : 0)) * D, ok, qb);
  const int c0 = max(0, qc - nw + 1);
  KVPrefetch<IO, D, NT, WIN_THREADS> pf;
  pf.load(k, v, kv0 + (int64_t)c0 * 64, min(64, N - c0 * 64), tid);
  f32x16_t oa[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oa[dt] = zero16();
  float m = -INFINITY, l = 0.f;
  for (int c = c0; c <= qc; ++c) {
    if (c > c0) __syncthreads();  // every wave is done with the previous chunk
    pf.store(tile, min(64, N - c * 64), tid);
    __syncthreads();
    if (c < qc) pf.load(k, v, kv0 + (int64_t)(c + 1) * 64, min(64, N - (c + 1) * 64), tid);
    if (head_ok)  // the own chunk causally (keys 0..rl), earlier chunks whole
      wave_chunk_online<IO, D, NT, true>(tile, qb, c == qc ? rl + 1 : 64, oa, m, l);
  }
  if (!ok) return;
  const int64_t row = (int64_t)bh * N + i;
  const float inv = 1.0f / l;
  PT* dst = reinterpret_cast<PT*>(partial_v) + (row * (K + 1) + K) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int e = 32 * dt + 8 * g4 + 4 * hf;
      if constexpr (sizeof(PT) == 2) {
        u32x2_t pk;
        pk.x = pack_f16x2(oa[dt][4 * g4 + 0] * inv, oa[dt][4 * g4 + 1] * inv);
        pk.y = pack_f16x2(oa[dt][4 * g4 + 2] * inv, oa[dt][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(dst + e) = pk;
      } else {
        *reinterpret_cast<float4*>(dst + e) = make_float4(oa[dt][4 * g4] * inv, oa[dt][4 * g4 + 1] * inv,
                                                          oa[dt][4 * g4 + 2] * inv, oa[dt][4 * g4 + 3] * inv);
      }
    }
  if (hf == 0) lse[row] = m * (1.0f / sqrtf((float)D)) + logf(l);
}

// ---------------------------------------------------------------------- fuse
// o_i = sum over the row's chunk outputs (selected chunks, then its own chunk or local
// window) weighted by the softmax of their scores (the selected chunks' s_ic, the own
// entry's LSE).  The number of selected chunks is min(K, candidate chunks), known
// without reading the selection, so every load of a row is issued at
// once; each wave works on two rows at a time.  16-byte loads of whole output rows.
// rows per wave: few, so that the workgroups in flight stream a compact address range
// (16 rows per wave ran 12% slower at 256K: more pages in use at once)
constexpr int FZ_ROWS = 4;

// KMAX: the largest K served (32, or 64 for 32 < K <= 64: scores for slots 64.. in a
// second register per lane)
template <typename IO, int D, int KMAX>
__global__ void __launch_bounds__(256) fuse(const float* __restrict__ sel_score, const float* __restrict__ lse,
                                            const void* __restrict__ partial_v, IO* __restrict__ o, int N, int C,
                                            int K, int64_t rows, int nw) {
  using PT = typename partial_t<IO>::type;
  constexpr int EPL = 16 / sizeof(PT);   // partial elements per 16-byte load
  constexpr int LPS = D / EPL;           // lanes per output row
  constexpr int SPL = 64 / LPS;          // output rows per wave-wide load
  constexpr int NSEG = (KMAX + 1 + SPL - 1) / SPL;  // loads per lane for up to KMAX + 1 slots
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int slot = lane / LPS, dpos = (lane % LPS) * EPL;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + w) * FZ_ROWS;
  const PT* part = reinterpret_cast<const PT*>(partial_v);
  // bf16 outputs of the wave's rows, written at the end as one contiguous burst: small
  // writes scattered through the read stream cost far more than their bytes
  __shared__ __align__(16) IO ostage[4][sizeof(IO) == 2 ? FZ_ROWS * D : 8];
  // two rows per buffer, two buffers: the loads of the next two rows are in flight while
  // the current two are reduced
  struct Rows {
    u32x4_t raw[2][NSEG];
    float sc[2], sc2[2];   // the score of slot lane, and of slot 64 + lane (KMAX = 64)
    int nsel[2];
    bool live[2];
  };
  auto issue = [&](int u, Rows& R) {
#pragma unroll
    for (int v2 = 0; v2 < 2; ++v2) {
      const int64_t row = row0 + u + v2;
      R.live[v2] = u < FZ_ROWS && row < rows;
      const int i = R.live[v2] ? (int)(row % N) : 0;
      const int ns = min(K, candidate_chunks(i, C, nw));
      R.nsel[v2] = ns;
      R.sc[v2] = R.sc2[v2] = -INFINITY;
      if (R.live[v2]) {
        if (lane < ns) R.sc[v2] = sel_score[row * K + lane];
        else if (lane == ns) R.sc[v2] = lse[row];
        if constexpr (KMAX > 32) {
          if (64 + lane < ns) R.sc2[v2] = sel_score[row * K + 64 + lane];
          else if (64 + lane == ns) R.sc2[v2] = lse[row];
        }
      }
#pragma unroll
      for (int sg = 0; sg < NSEG; ++sg) {
        const int t = sg * SPL + slot;           // logical slot: 0..ns-1 selected, ns = own
        const int phys = t < ns ? t : K;
        R.raw[v2][sg] = (R.live[v2] && t <= ns)
                            ? __builtin_nontemporal_load(
                                  reinterpret_cast<const u32x4_t*>(part + (row * (K + 1) + phys) * D + dpos))
                            : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto finish = [&](int u, const Rows& R) {
#pragma unroll
    for (int v2 = 0; v2 < 2; ++v2) {
      if (!R.live[v2]) continue;
      const int64_t row = row0 + u + v2;
      const float M = wave_max(KMAX > 32 ? fmaxf(R.sc[v2], R.sc2[v2]) : R.sc[v2]);
      const float wt = R.sc[v2] == -INFINITY ? 0.f : __expf(R.sc[v2] - M);
      const float wt2 = KMAX > 32 && R.sc2[v2] != -INFINITY ? __expf(R.sc2[v2] - M) : 0.f;
      const float inv = 1.0f / wave_sum(wt + wt2);
      float acc[EPL];
#pragma unroll
      for (int x = 0; x < EPL; ++x) acc[x] = 0.f;
#pragma unroll
      for (int sg = 0; sg < NSEG; ++sg) {
        const int t = sg * SPL + slot;
        const float wtt = (KMAX > 32 && t >= 64 ? __shfl(wt2, t - 64) : __shfl(wt, t < 64 ? t : 0)) *
                          (t <= R.nsel[v2] ? 1.f : 0.f);
        const u32x4_t rw = R.raw[v2][sg];
        if constexpr (sizeof(PT) == 2) {
          const uint32_t wd[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            acc[2 * x] = fmaf(wtt, f16_to_f32((uint16_t)(wd[x] & 0xffffu)), acc[2 * x]);
            acc[2 * x + 1] = fmaf(wtt, f16_to_f32((uint16_t)(wd[x] >> 16)), acc[2 * x + 1]);
          }
        } else {
          acc[0] = fmaf(wtt, __uint_as_float(rw.x), acc[0]);
          acc[1] = fmaf(wtt, __uint_as_float(rw.y), acc[1]);
          acc[2] = fmaf(wtt, __uint_as_float(rw.z), acc[2]);
          acc[3] = fmaf(wtt, __uint_as_float(rw.w), acc[3]);
        }
      }
      // sum the slot groups (lanes with the same dpos)
#pragma unroll
      for (int st = LPS; st < 64; st <<= 1)
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc[x] += __shfl_xor(acc[x], st);
      if (lane < LPS) {
        if constexpr (sizeof(IO) == 2) {
          u32x4_t pk;
          pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
          pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
          pk.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
          pk.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
          *reinterpret_cast<u32x4_t*>(&ostage[w][(u + v2) * D + dpos]) = pk;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(o) + row * D + dpos) =
              make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        }
      }
    }
  };
  static_assert(FZ_ROWS % 4 == 0, "");
  Rows ra, rb;
  issue(0, ra);
  for (int u = 0; u < FZ_ROWS; u += 4) {
    issue(u + 2, rb);
    finish(u, ra);
    issue(u + 4, ra);  // past the wave's rows: nothing is loaded
    finish(u + 2, rb);
  }
  if constexpr (sizeof(IO) == 2) {
    __builtin_amdgcn_wave_barrier();
    const int nr = (int)min((int64_t)FZ_ROWS, rows - row0);  // rows of this wave that exist
    constexpr int SEG16 = FZ_ROWS * D * (int)sizeof(IO) / 16;
    for (int x = lane; x < SEG16; x += 64) {
      if (x * 16 < nr * D * (int)sizeof(IO))
        __builtin_nontemporal_store(reinterpret_cast<const u32x4_t*>(&ostage[w][0])[x],
                                    reinterpret_cast<u32x4_t*>(o + row0 * D) + x);
    }
  }
}

// ------------------------------------------------------- shared bucketing launch
void launch_bucket_pairs(const Geom& g, const int32_t* sel, BucketBufs bb, hipStream_t st) {
  const int C = g.C();
  const int nbk = g.B * g.Hq * C;
  // zero counts and cursors (contiguous) with a kernel: no memset nodes in captured streams
  const int64_t nz = (int64_t)(bb.boff - bb.counts);
  if (nz > 0)
    hipLaunchKernelGGL(zero_u32, dim3((unsigned)std::min<int64_t>((nz + 255) / 256, 4096)), dim3(256), 0, st,
                       bb.counts, nz);
  if (nbk == 0) return;
  const int64_t group_len = (int64_t)g.N * g.K;
  const int ngrp = g.B * g.Hq;
  // slices of whole LDS tiles, at most HIST_SLICE entries, small enough that the passes
  // over them fill the chip when the groups are few (short sequences)
  const int64_t want = (BK_FILL + ngrp - 1) / ngrp;
  const int64_t slice =
      std::min<int64_t>(HIST_SLICE, std::max<int64_t>(BK_TILE, ((group_len + want - 1) / want + BK_TILE - 1) / BK_TILE * BK_TILE));
  const int spg = (int)((group_len + slice - 1) / slice);
  hipLaunchKernelGGL(bucket_count, dim3(ngrp * spg), dim3(256), 0, st, sel, bb.counts, group_len, slice, spg, C);
  if (nbk <= 16 * 1024) {  // one workgroup scans up to 16K buckets quickly
    hipLaunchKernelGGL(bucket_scan, dim3(1), dim3(1024), 0, st, bb.counts, bb.boff, bb.toff, nbk);
  } else {
    const int nblk = (nbk + SCAN_BLOCK - 1) / SCAN_BLOCK;
    hipLaunchKernelGGL(bucket_block_sums, dim3(nblk), dim3(256), 0, st, (const uint32_t*)bb.counts, bb.boff, bb.toff,
                       nbk);
    hipLaunchKernelGGL(bucket_block_scan, dim3(1), dim3(1024), 0, st, bb.boff, bb.toff, nbk, nblk);
    hipLaunchKernelGGL(bucket_block_fill, dim3(nblk), dim3(256), 0, st, bb.counts, bb.boff, bb.toff, nbk);
  }
  hipLaunchKernelGGL(bucket_item_map, dim3((nbk + 255) / 256), dim3(256), 0, st, (const uint32_t*)bb.toff, bb.imap,
                     nbk);
  const int nrg = (C + (1 << FINE_BITS) - 1) >> FINE_BITS;
  hipLaunchKernelGGL(bucket_part1, dim3(ngrp * spg), dim3(256), 0, st, sel, bb.boff, bb.cursor, bb.tmp, group_len,
                     slice, spg, C, nrg);
  const int split = std::min(64, std::max(P2_SPLIT, (BK_FILL + ngrp * nrg - 1) / (ngrp * nrg)));
  hipLaunchKernelGGL(bucket_part2, dim3(ngrp * nrg * split), dim3(256), 0, st, (const uint32_t*)bb.tmp, bb.boff,
                     bb.counts, bb.pairs, group_len, C, nrg, split);
}

int64_t bucket_items_bound(const Geom& g) {
  // rows of query chunk p (64 of them, fewer in the tail) select min(K, p - nw + 1, C) chunks each
  const int C = g.C();
  int64_t pairs_total = 0;
  for (int p = 0; p * 64 < g.N; ++p)
    pairs_total += (int64_t)std::min(64, g.N - p * 64) * std::min(g.K, std::min(C, std::max(0, p - g.nw + 1)));
  pairs_total *= (int64_t)g.B * g.Hq;
  if (pairs_total == 0) return 0;
  // work items <= total pairs / ITEM_ROWS + number of buckets (the exact count is read on the device)
  return std::min<int64_t>((pairs_total + ITEM_ROWS - 1) / ITEM_ROWS + (int64_t)g.B * g.Hq * C, 0x7fffffff);
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
  uint32_t* imap = (uint32_t*)(ws + w.imap);
  void* partial = ws + w.partial;
  const int C = g.C();
  const int nbk = g.B * g.Hq * C;
  if (nbk > 0) {
    // the first pass's output lives in the (not yet written) partial-output region
    launch_bucket_pairs(g, sel, BucketBufs{counts, cursor, boff, toff, pairs, (uint32_t*)partial, imap}, st);
    if (ev) hipEventRecord(ev[0], st);
    const int64_t items = bucket_items_bound(g);
    if (items > 0)
      hipLaunchKernelGGL((chunk_attend<IO, D>), dim3((unsigned)items), dim3(256), 0, st, (const IO*)q, (const IO*)k,
                         (const IO*)v, pairs, boff, toff, imap, partial, ws + w.sink, g.Hq, g.Hkv, g.N, C, g.K,
                         nbk);
    if (ev) hipEventRecord(ev[1], st);
  } else if (ev) {
    hipEventRecord(ev[0], st);
    hipEventRecord(ev[1], st);
  }
  const int NQC = (g.N + 63) / 64;
  float* lse = (float*)(ws + w.lse);
  if (g.nw > 1) {
    const int ngb = (g.G() + WIN_HEADS - 1) / WIN_HEADS;
    hipLaunchKernelGGL((window_attend<IO, D>), dim3(g.B * g.Hkv * NQC * ngb), dim3(WIN_THREADS), 0, st,
                       (const IO*)q, (const IO*)k, (const IO*)v, partial, lse, g.Hq, g.Hkv, g.N, g.K, NQC, g.nw);
  } else {
    const int hpw = std::min(g.G(), OWN_HEADS);
    const int ngb = (g.G() + hpw - 1) / hpw;
    hipLaunchKernelGGL((own_attend<IO, D>), dim3(g.B * g.Hkv * NQC * ngb), dim3(128 * hpw), 0, st, (const IO*)q,
                       (const IO*)k, (const IO*)v, partial, lse, g.Hq, g.Hkv, g.N, g.K, NQC, hpw);
  }
  if (ev) hipEventRecord(ev[2], st);
  const int64_t rows = (int64_t)g.B * g.Hq * g.N;
  const int64_t nwg = (rows + 4 * FZ_ROWS - 1) / (4 * FZ_ROWS);
  if (g.K > 32)
    hipLaunchKernelGGL((fuse<IO, D, 64>), dim3((unsigned)nwg), dim3(256), 0, st, scr, (const float*)lse,
                       (const void*)partial, (IO*)o, g.N, C, g.K, rows, g.nw);
  else if (g.K > 16)
    hipLaunchKernelGGL((fuse<IO, D, 32>), dim3((unsigned)nwg), dim3(256), 0, st, scr, (const float*)lse,
                       (const void*)partial, (IO*)o, g.N, C, g.K, rows, g.nw);
  else
    hipLaunchKernelGGL((fuse<IO, D, 16>), dim3((unsigned)nwg), dim3(256), 0, st, scr, (const float*)lse,
                       (const void*)partial, (IO*)o, g.N, C, g.K, rows, g.nw);
  if (ev) hipEventRecord(ev[3], st);
  return hipGetLastError();
}

hipError_t launch_prefill_attend(const Geom& g, const void* q, const void* k, const void* v, const int32_t* sel_idx,
                                 const float* sel_score, void* o, void* ws, size_t ws_bytes, hipStream_t st,
                                 hipEvent_t* ev) {
  if (ws_bytes < attend_workspace_bytes(g)) return hipErrorInvalidValue;
  if (g.C() > MAX_C) return hipErrorNotSupported;
  // first-pass keys hold an in-group entry index (N*K < 2^26 whenever N/S <= 16384, K <= 32)
  if ((int64_t)g.N * g.K >= (int64_t)1 << LOCAL_BITS) return hipErrorNotSupported;
  static_assert(MAX_C <= 256 << FINE_BITS, "first-pass ranges fit one 256-thread scan");
  char* w = (char*)ws;
  if (g.io == 0)
    return g.d == 64 ? launch_attend_t<float, 64>(g, q, k, v, sel_idx, sel_score, o, w, st, ev)
                     : launch_attend_t<float, 128>(g, q, k, v, sel_idx, sel_score, o, w, st, ev);
  return g.d == 64 ? launch_attend_t<bf16_t, 64>(g, q, k, v, sel_idx, sel_score, o, w, st, ev)
                   : launch_attend_t<bf16_t, 128>(g, q, k, v, sel_idx, sel_score, o, w, st, ev);
}

}  // namespace hils

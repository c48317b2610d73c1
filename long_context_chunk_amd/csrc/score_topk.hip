// Chunk scoring and top-K for a block of queries.
//
//   s_ic = q^_i . k'_c / sqrt(d) + b'_c   for every candidate chunk c < floor(p_i/S) - (nw - 1)
//                                        (the complete chunks before the local window of nw chunks)
// where query i of batch b sits at position p_i = pos0[b] + i (prefill: pos0 = 0, the
// block is the whole sequence) and k' comes from its landmark head h / (Hq / Hl).
//   q^_i = q_i + U_h (D_h q_i)             (Q-Cal; q^ = q without it)
// keep the K best (ties -> lower chunk id).  (aitrends.kr article,
// "Methodology": the score formula, the calculation flow and the Q-Cal module.)
//
// Q-Cal is applied on the key side: q^_i . k'_c = q_i . k~_hc with
//   k~_hc = k'_c + D_h^T (U_h^T k'_c),
// one fp32 row per (batch, query head, chunk) made once per call by prep_kprime.  The
// queries then enter as given: a bf16 query is one exact bf16 term, so the selection
// pass needs two products per score (q . k~_hi + q . k~_lo) instead of three, and
// neither pass computes q^.
//
// Two passes over the past chunks, both on v_mfma_f32_32x32x16_bf16, one workgroup per
// 128 consecutive queries of one (batch, head) (32 per wave), with k' tiles staged
// through LDS and shared by the four waves:
//
//   1. score_threshold (queries = M, chunks = N: accumulator register r of a lane holds
//      one chunk's score for one row; the 32 lanes of a half-wave cover 32 chunks of
//      that row): one bf16 product per score, bf16(q) . bf16(k~_c/sqrt(d)), with b'_c
//      and an error allowance e_i |k'_c| folded into one extra MFMA k-step, so every
//      value is at most the fp32-accurate score of pass 2.  Each lane keeps the two
//      largest values of its column of chunks; the K-th largest of these 64 values of
//      distinct chunks is a threshold theta_i that the row's K-th best score can not
//      be below.
//   2. score_topk_kernel (chunks = M, queries = N: each lane owns one row's scores):
//      the scores to ~2^-17 relative (tau k~ split into bf16 hi + lo terms, q too
//      when it is not exactly bf16; b' through an extra k-step), tested against the
//      row's threshold, which starts at theta_i, so only about K candidates per row
//      are kept.  Each lane appends its row's candidates to its own half of the row's
//      LDS list; a full list is sorted by bitonic networks (DPP and swizzle lane
//      exchanges), cut to the best K and the threshold raised.
//   k' is rewritten once per call into bf16 term rows whose 16-element k-blocks are
//   stored in MFMA operand order, so staging is a copy and an operand is one 16-byte
//   LDS read.
#include <algorithm>
#include <type_traits>

#include "hils_common.h"
#include "keylists.h"
#include "kernels.h"

namespace hils {

constexpr int ST_ROWS = 128;   // queries per workgroup
constexpr int ST_TILE = 64;    // chunks per LDS tile
constexpr int KP_PAD = 64;     // k' rows per head are padded to a multiple of this (zero rows)

static __host__ __device__ inline int kp_rows(int C) { return (C + KP_PAD - 1) / KP_PAD * KP_PAD; }

template <int CTRL>
HILS_DEV int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false);
}
// value of lane j ^ X, within each 32-lane half (j = lane & 31)
template <int X>
HILS_DEV int xlane(int v, int j) {
  if constexpr (X == 1) {
    return dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (X == 2) {
    return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (X == 4 || X == 8) {
    const int up = dpp<0x100 + X>(v);  // row_shl: lane i <- lane i + X
    const int dn = dpp<0x110 + X>(v);  // row_shr: lane i <- lane i - X
    return (j & X) ? dn : up;
  } else if constexpr (X == 16) {
    return __builtin_amdgcn_ds_swizzle(v, 0x401F);  // xor 16 within 32 lanes
  } else {
    static_assert(X == 31, "");
    return __builtin_amdgcn_ds_swizzle(v, 0x7C1F);  // reverse within 32 lanes
  }
}

// value of lane j ^ X (within each 32-lane half) of a 64-bit key
template <int X>
HILS_DEV uint64_t xlane64(uint64_t v, int j) {
  const uint32_t lo = (uint32_t)xlane<X>((int)(uint32_t)v, j);
  const uint32_t hi = (uint32_t)xlane<X>((int)(uint32_t)(v >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}

// compare-exchange of 64-bit selection keys (make_key: larger = better, ties to the lower
// chunk; 0 = empty) with lane j ^ X: keep the larger of the pair if kb, else the smaller
template <int X>
HILS_DEV void cxk(uint64_t& k, int j, bool kb) {
  const uint64_t p = xlane64<X>(k, j);
  k = ((p > k) == kb) ? p : k;
}

// bitonic sort of one key per lane, best first, within each 32-lane half
HILS_DEV void sort32k(uint64_t& k, int j) {
#define HILS_STAGE(K_, X_) cxk<X_>(k, j, ((j & X_) == 0) == (((j & K_) == 0) || K_ == 32));
  HILS_STAGE(2, 1)
  HILS_STAGE(4, 2) HILS_STAGE(4, 1)
  HILS_STAGE(8, 4) HILS_STAGE(8, 2) HILS_STAGE(8, 1)
  HILS_STAGE(16, 8) HILS_STAGE(16, 4) HILS_STAGE(16, 2) HILS_STAGE(16, 1)
  HILS_STAGE(32, 16) HILS_STAGE(32, 8) HILS_STAGE(32, 4) HILS_STAGE(32, 2) HILS_STAGE(32, 1)
#undef HILS_STAGE
}

// merge the unsorted keys nk into the sorted list lk of each half; keep the best K
HILS_DEV void merge_intok(uint64_t& lk, uint64_t nk, int j, int K) {
  sort32k(nk, j);
  const uint64_t r = xlane64<31>(nk, j);  // lane j: the (31-j)-th best new key
  lk = r > lk ? r : lk;
  // the 32 kept keys form a bitonic sequence: half-cleaners sort it best-first
  cxk<16>(lk, j, (j & 16) == 0);
  cxk<8>(lk, j, (j & 8) == 0);
  cxk<4>(lk, j, (j & 4) == 0);
  cxk<2>(lk, j, (j & 2) == 0);
  cxk<1>(lk, j, (j & 1) == 0);
  if (j >= K) lk = 0;
}

HILS_DEV float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// value of lane j ^ X within each 32-lane half: DPP quad permutations for X < 4, one
// ds_swizzle (xor mode) otherwise
template <int X>
HILS_DEV float xl1(float v) {
  if constexpr (X == 1 || X == 2) {
    return __int_as_float(dpp<X == 1 ? 0xB1 : 0x4E>(__float_as_int(v)));
  } else {
    static_assert(X == 4 || X == 8 || X == 16 || X == 31, "");
    constexpr int OFS = X == 31 ? 0x7C1F : (0x1F | (X << 10));  // X == 31: reverse the half
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), OFS));
  }
}

// One compare-exchange stage with lane j ^ X on R independent registers: med3(s, p, +inf)
// keeps the larger, med3(s, p, -inf) the smaller; the bound is chosen per lane.
template <int X, int R>
HILS_DEV void cx_stage(float (&s)[R], float bnd) {
  float p[R];
#pragma unroll
  for (int i = 0; i < R; ++i) p[i] = xl1<X>(s[i]);
#pragma unroll
  for (int i = 0; i < R; ++i) s[i] = __builtin_amdgcn_fmed3f(s[i], p[i], bnd);
}

// Descending bitonic sort within each 32-lane half, R registers at once.  pinf / ninf
// are +-inf hidden from the compiler, so the med3s stay med3s.
template <int R>
HILS_DEV void sort32f_r(float (&s)[R], int j, float pinf, float ninf) {
#define HILS_STAGE(K_, X_) cx_stage<X_, R>(s, (((j & X_) == 0) == (((j & K_) == 0) || K_ == 32)) ? pinf : ninf);
  HILS_STAGE(2, 1)
  HILS_STAGE(4, 2) HILS_STAGE(4, 1)
  HILS_STAGE(8, 4) HILS_STAGE(8, 2) HILS_STAGE(8, 1)
  HILS_STAGE(16, 8) HILS_STAGE(16, 4) HILS_STAGE(16, 2) HILS_STAGE(16, 1)
  HILS_STAGE(32, 16) HILS_STAGE(32, 8) HILS_STAGE(32, 4) HILS_STAGE(32, 2) HILS_STAGE(32, 1)
#undef HILS_STAGE
}

// For R registers at once: the K-th largest (K <= 64) of the 64 values {a, b} of each
// 32-lane half, left in lane (K - 1) & 31 of the half.  a is overwritten with the half's
// 32 largest (K <= 32) or 32 smallest (K > 32), sorted best first: with a and b sorted,
// lane j's larger (smaller) of a_j and b_(31-j) forms the top (bottom) half of the 64 as
// a bitonic sequence.
template <int R>
HILS_DEV void kth_of_pairs_r(float (&a)[R], float (&b)[R], int j, int K, float pinf, float ninf) {
  sort32f_r<R>(a, j, pinf, ninf);
  sort32f_r<R>(b, j, pinf, ninf);
  const float side = K > 32 ? ninf : pinf;
#pragma unroll
  for (int i = 0; i < R; ++i) a[i] = __builtin_amdgcn_fmed3f(a[i], xl1<31>(b[i]), side);
  cx_stage<16, R>(a, (j & 16) == 0 ? pinf : ninf);
  cx_stage<8, R>(a, (j & 8) == 0 ? pinf : ninf);
  cx_stage<4, R>(a, (j & 4) == 0 ? pinf : ninf);
  cx_stage<2, R>(a, (j & 2) == 0 ? pinf : ninf);
  cx_stage<1, R>(a, (j & 1) == 0 ? pinf : ninf);
}

// 64-bit key of lane j ^ X within each 32-lane half (X as in xl1)
template <int X>
HILS_DEV uint64_t xl64(uint64_t v) {
  const uint32_t lo = __float_as_uint(xl1<X>(__uint_as_float((uint32_t)v)));
  const uint32_t hi = __float_as_uint(xl1<X>(__uint_as_float((uint32_t)(v >> 32))));
  return ((uint64_t)hi << 32) | lo;
}
// compare-exchange of R independent 64-bit keys with lane j ^ X: keep the larger if kb
template <int X, int R>
HILS_DEV void cxk_r(uint64_t (&k)[R], bool kb) {
  uint64_t p[R];
#pragma unroll
  for (int i = 0; i < R; ++i) p[i] = xl64<X>(k[i]);
#pragma unroll
  for (int i = 0; i < R; ++i) k[i] = ((p[i] > k[i]) == kb) ? p[i] : k[i];
}
// best-first bitonic sort within each 32-lane half, R registers at once
template <int R>
HILS_DEV void sort32k_r(uint64_t (&k)[R], int j) {
#define HILS_STAGE(K_, X_) cxk_r<X_, R>(k, ((j & X_) == 0) == (((j & K_) == 0) || K_ == 32));
  HILS_STAGE(2, 1)
  HILS_STAGE(4, 2) HILS_STAGE(4, 1)
  HILS_STAGE(8, 4) HILS_STAGE(8, 2) HILS_STAGE(8, 1)
  HILS_STAGE(16, 8) HILS_STAGE(16, 4) HILS_STAGE(16, 2) HILS_STAGE(16, 1)
  HILS_STAGE(32, 16) HILS_STAGE(32, 8) HILS_STAGE(32, 4) HILS_STAGE(32, 2) HILS_STAGE(32, 1)
#undef HILS_STAGE
}

// bf16 bits of the smallest bf16 >= x (x >= 0), clamped to the largest finite bf16
HILS_DEV uint16_t bf16_up(float x) {
  if (!(x < 3.38e38f)) return 0x7f7f;
  uint16_t b = f32_to_bf16(x);
  if (bf16_to_f32(b) < x) ++b;
  return b;
}

// This lane's query row (zero when !row_ok), delivered one MFMA k-step at a time in the
// A-operand layout: sink(ks, v) gets v[m] = q[kperm(ks, hf, m)].  Q-Cal never touches
// the queries: it is folded into the chunk rows (prep_kprime).
template <typename IO, int D, typename Sink>
HILS_DEV void q_rows(const IO* __restrict__ q, int64_t qrow, bool row_ok, int lane, Sink&& sink) {
  constexpr int NKS = D / 16;
  const int hf = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    float a4[4], b4[4];
    if (row_ok) {
      io_traits<IO>::load4(q, qrow + kperm(ks, hf, 0), a4);
      io_traits<IO>::load4(q, qrow + kperm(ks, hf, 4), b4);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) a4[m] = b4[m] = 0.f;
    }
    float v[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v[m] = a4[m];
      v[4 + m] = b4[m];
    }
    sink(ks, v);
  }
}

// ------------------------------------------------------------- threshold pass
// Error allowance of the one-product scores bf(q) . bf(tau k~): with u = 2^-8 (bf16
// rounding), |bf(x) bf(y) - x y| <= (2u + u^2) |x y|, and <= u |x y| when x is exactly a
// bf16 value (a bf16 query), so over the head dimension the product error is at most
// (2u + u^2) |q| |tau k~|, or u |q| |tau k~| (Cauchy-Schwarz).  TH_REL exceeds these by
// enough to cover pass 2's own ~2^-16 relative error and fp32 accumulation, and TH_ABS
// covers the two-term split of b'.
template <typename IO>
constexpr float th_rel() { return io_traits<IO>::terms == 1 ? 0.0042f : 0.008f; }
constexpr float TH_ABS = 1.0f / 4096.0f;   // bf16 0x3980
constexpr int TH_EXT = 16;                  // elements of the extension k-step

// Hl: heads of the chunk rows t1 (the landmark heads, or the query heads under Q-Cal).
template <typename IO, int D>
__global__ void __launch_bounds__(256, 3) score_threshold(const IO* __restrict__ q, const uint16_t* __restrict__ t1,
                                                          float* __restrict__ theta, const int32_t* __restrict__ pos0,
                                                          int H, int Hl, int N, int C, int K, int NB, int items,
                                                          int nw) {
  constexpr int NKS = D / 16;
  constexpr int DE = D + TH_EXT;      // bf16 elements of a chunk row
  constexpr int LDT = DE + 8;         // LDS row stride (16-byte pad: conflict-free 16-byte reads)
  constexpr int SEGS = DE / 8;
  constexpr int NSEG = ST_TILE * SEGS;
  constexpr int PL = (NSEG + 255) / 256;
  constexpr int TILE_BYTES = 2 * ST_TILE * LDT * 2;
  __shared__ __align__(16) unsigned char smem[TILE_BYTES];
  uint16_t(*kt)[ST_TILE * LDT] = reinterpret_cast<uint16_t(*)[ST_TILE * LDT]>(smem);

  const int item = remap_xcd(blockIdx.x, items);
  if (item >= items) return;
  const int bh = item / NB;
  const int rb = NB - 1 - (item % NB);  // heavier (later) row blocks first
  const int hh = bh % H, bb = bh / H;
  const int p0 = pos0 ? pos0[bb] : 0;   // position of the block's query 0 (N = queries here)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int r0 = rb * ST_ROWS;
  const int row = r0 + 32 * w + n;
  const bool row_ok = row < N;
  const int last = min(r0 + ST_ROWS, N) - 1;
  const int Pmax = candidate_chunks(p0 + last, C, nw);
  const int Pmin = candidate_chunks(p0 + r0, C, nw);
  const int64_t qrow = ((int64_t)bh * N + (row_ok ? row : 0)) * D;

  // A operands: bf16(q), then the extension step [1, 1, -1, -e_i] against the
  // chunk's [b'_hi, b'_lo, TH_ABS, |tau k~_c| rounded up], e_i = TH_REL |q_i| rounded up
  bf16x8_t qa[NKS + 1];
  float ss = 0.f;
  q_rows<IO, D>(q, qrow, row_ok, lane, [&](int ks, const float(&v)[8]) {
    float x[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      x[m] = v[m];
      ss = fmaf(x[m], x[m], ss);
    }
    u32x4_t t[1];
    split8<1>(x, t);
    qa[ks] = __builtin_bit_cast(bf16x8_t, t[0]);
  });
  ss += __shfl_xor(ss, 32);
  {
    uint16_t t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (hf == 0) {
      t[0] = t[1] = 0x3f80;
      t[2] = 0xbf80;
      t[3] = (uint16_t)(bf16_up(th_rel<IO>() * sqrtf(ss)) | 0x8000u);
    }
    qa[NKS] = pack8(t);
  }

  // the landmark head's rows, padded to a multiple of KP_PAD zero rows: a tile never reads
  // past them.  A tile's rows are contiguous: thread t moves 16-byte segments t + 256 u
  // (the final partial group repeats the last segment; its duplicate store writes the
  // same bytes), at offsets that are the same for every tile.
  const uint16_t* src = t1 + ((int64_t)bb * Hl + hh / (H / Hl)) * kp_rows(C) * DE;
  int goff[PL], soff[PL];
#pragma unroll
  for (int u = 0; u < PL; ++u) {
    const int it = min(tid + 256 * u, NSEG - 1);
    goff[u] = 8 * it;
    soff[u] = (it / SEGS) * LDT + 8 * (it % SEGS);
  }
  u32x4_t pf[PL];
  auto load_tile = [&](int t) {
    const uint16_t* tp = src + (int64_t)t * ST_TILE * DE;
#pragma unroll
    for (int u = 0; u < PL; ++u) pf[u] = *reinterpret_cast<const u32x4_t*>(tp + goff[u]);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PL; ++u) *reinterpret_cast<u32x4_t*>(&kt[buf][soff[u]]) = pf[u];
  };

  // each lane: the two largest values of its column of chunks, for 2 rows per register.
  // +inf goes through an empty asm so that med3(m1, v, +inf) stays one v_med3_f32
  // instead of becoming an IEEE max with operand canonicalisation.
  float pinf = INFINITY;
  asm volatile("" : "+v"(pinf));
  float m1[16], m2[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) m1[rr] = m2[rr] = -INFINITY;
  const int ntiles = (Pmax + ST_TILE - 1) / ST_TILE;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  // One tile: the two 32-chunk halves' MFMA chains interleaved (independent
  // accumulators), so each hides the other's latency and the updates of the first half
  // overlap the second.  MASKED tiles reach chunks >= Pmin, which are not candidates of
  // every row (the chunks of a last tile past Pmax, later chunks or zero padding rows,
  // are masked out with them).  Masked and unmasked tiles run in separate loops: one loop
  // with both kinds makes the compiler copy the running top-two at every iteration.
  auto tile_step = [&](int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);
    f32x16_t acc[2] = {zero16(), zero16()};
#pragma unroll
    for (int ks = 0; ks <= NKS; ++ks)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(&kt[buf][(32 * tt + n) * LDT + 16 * ks + 8 * hf]);
        acc[tt] = mfma32(qa[ks], bk, acc[tt]);
      }
    // top two per lane (m1 >= m2): m2 = median(m1, m2, v), m1 = median(m1, v, +inf)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int c = t * ST_TILE + 32 * tt + n;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float v = acc[tt][rr];
        if constexpr (MASKED) {
          const int rw = r0 + 32 * w + acc_row(rr, hf);
          const int prow = rw < N ? candidate_chunks(p0 + rw, C, nw) : 0;
          v = c >= prow ? -INFINITY : v;
        }
        m2[rr] = __builtin_amdgcn_fmed3f(m1[rr], m2[rr], v);
        m1[rr] = __builtin_amdgcn_fmed3f(m1[rr], v, pinf);
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  };
  const int t_open = min(ntiles, Pmin / ST_TILE);  // tiles whose chunks are all below Pmin
  int t = 0;
  for (; t < t_open; ++t) tile_step(t, std::false_type{});
  for (; t < ntiles; ++t) tile_step(t, std::true_type{});
  // theta per row: all 16 register rows (two rows each, one per half) at once
  float ninf = -INFINITY;
  asm volatile("" : "+v"(ninf));
  kth_of_pairs_r<16>(m1, m2, n, K, pinf, ninf);
  const int kl = (K - 1) & 31;   // lane of the K-th within the half
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int rw = r0 + 32 * w + acc_row(rr, hf);
    const float t0 = readlane_f(m1[rr], kl), t1 = readlane_f(m1[rr], 32 + kl);
    const float th = hf ? t1 : t0;
    if (n == 0 && rw < N) theta[(int64_t)bh * N + rw] = th;
  }
}


// ------------------------------------------------------------- selection pass
// S^T = k~ q^T on the MFMA: k~ rows (chunks) are the A operand, the queries the B
// operand, so accumulator register r of lane l holds the score of chunk
// acc_row(r, l >> 5) of the 32-chunk tile for query row l & 31.  Each lane therefore
// owns one row's scores (half of each tile's chunks) and appends its passing candidates
// to its own half of the row's list in LDS.  Only lanes whose score passes the row's
// threshold execute an append (about 2% of the scores pass), and the appends of tile ct
// are interleaved one for one with the MFMAs of tile ct + 1.  A half list that overflows
// takes further candidates in a spill slot (lost for now); the row is then compacted to
// its best K, its threshold raised to the K-th of them, and the lost ones appended again.
// tau is folded into the k' planes and b' (three exact bf16 terms) enters through an
// extra k-step against a constant [1, 1, 1, 0 ...] query operand.
constexpr int SEL_CT = 32;     // chunks per column tile (single LDS buffer)
constexpr int SEL_HALF = 32;   // candidate slots per half-row list (plus one spill slot)
constexpr int P2_EXT = 16;     // extension elements after plane 0: [b'_hi, b'_mid, b'_lo, 0 ...]

// KB (K > 32): half lists of SEL_HALF_KB slots and 64-entry sorted lists (two keys per
// lane of a half-wave, keylists.h) for compaction and output; the LDS this takes leaves
// one workgroup per CU.
constexpr int SEL_HALF_KB = 48;

// LM, the list mode: 0 for K <= 16 (half lists of SEL_HALF_SMALL slots: with the smaller
// lists, three workgroups fit a CU where the score operands leave the registers for it),
// 1 for K <= 32, 2 for K > 32 (KB).
constexpr int SEL_HALF_SMALL = 16;
template <int LM, int NQ, int NK>
constexpr int sel_wgs() { return LM == 2 ? 1 : (LM == 0 && NQ * NK <= 2) ? 3 : 2; }

template <typename IO, int D, int NQ, int NK, int LM>
__global__ void __launch_bounds__(256, (sel_wgs<LM, NQ, NK>())) score_topk_kernel(const IO* __restrict__ q,
                                                           const uint16_t* __restrict__ p2,
                                                           const float* __restrict__ theta,
                                                           int32_t* __restrict__ sel_idx,
                                                           float* __restrict__ sel_score,
                                                           const int32_t* __restrict__ pos0, int H, int Hl, int N,
                                                           int C, int K, int NB, int items, int nw) {
  constexpr int NKS = D / 16;
  constexpr int DE2 = NK * D + P2_EXT;  // elements of a chunk row: plane 0, extension, planes 1..
  constexpr int LDR = DE2 + 8;          // LDS row stride (16-byte pad)
  constexpr int SEGS = DE2 / 8;
  constexpr int NSEG = SEL_CT * SEGS;
  constexpr int PL = (NSEG + 255) / 256;
  constexpr bool KB = LM == 2;
  constexpr int SH = KB ? SEL_HALF_KB : LM == 0 ? SEL_HALF_SMALL : SEL_HALF;   // slots per half list
  constexpr int HSTR = SH + 1;          // half-list stride: SH slots + a spill slot
  constexpr int LIST = 2 * HSTR;        // slots per row
  constexpr int NPROD = NQ > NK ? NQ : NK;
  constexpr int NMF = [] {              // MFMAs per tile: the products i + j < NPROD, then b'
    int c = 0;
    for (int i = 0; i < NQ; ++i)
      for (int j = 0; j < NK; ++j) c += i + j < NPROD ? 1 : 0;
    return c * NKS + 1;
  }();
  // candidate lists: scores (fp32) then chunks (uint16) of slot s at byte 4 s and
  // CI_OFS + 2 s: one address register serves both writes
  constexpr int CI_OFS = ST_ROWS * LIST * 4;
  __shared__ __align__(16) uint16_t kt[SEL_CT * LDR];
  __shared__ __align__(16) unsigned char lists[ST_ROWS * LIST * 6];
  float* cs = reinterpret_cast<float*>(lists);
  uint16_t* ci = reinterpret_cast<uint16_t*>(lists + CI_OFS);

  const int item = remap_xcd(blockIdx.x, items);
  if (item >= items) return;
  const int bh = item / NB;
  const int rb = NB - 1 - (item % NB);  // heavier (later) row blocks first
  const int hh = bh % H, bb = bh / H;
  const int p0 = pos0 ? pos0[bb] : 0;   // position of the block's query 0 (N = queries here)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int r0 = rb * ST_ROWS;
  const int row = r0 + 32 * w + n;       // this lane's query row
  const bool row_ok = row < N;
  const int last = min(r0 + ST_ROWS, N) - 1;
  const int Pmax = candidate_chunks(p0 + last, C, nw);
  const int Pmin = candidate_chunks(p0 + r0, C, nw);
  const int prow = row_ok ? candidate_chunks(p0 + row, C, nw) : 0;   // candidate chunks of this lane's row
  const int64_t qrow = ((int64_t)bh * N + (row_ok ? row : 0)) * D;

  // ---- the query's B operands: q split into NQ bf16 terms, plus the constant extension
  bf16x8_t qb[NQ][NKS];
  q_rows<IO, D>(q, qrow, row_ok, lane, [&](int ks, const float(&v)[8]) {
    float x[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) x[m] = v[m];
    u32x4_t t[NQ];
    split8<NQ>(x, t);
#pragma unroll
    for (int j = 0; j < NQ; ++j) qb[j][ks] = __builtin_bit_cast(bf16x8_t, t[j]);
  });
  bf16x8_t qext;
  {
    uint16_t t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (hf == 0) t[0] = t[1] = t[2] = 0x3f80;
    qext = pack8(t);
  }

  // ---- per-lane state: the row's threshold (theta, raised when its list is compacted)
  // and the fill of this half's list; rows beyond N take +inf and never collect anything
  float th = row_ok ? theta[(int64_t)bh * N + row] : INFINITY;
  const int lrow = 32 * w + n;           // row within the workgroup
  const int lbase = lrow * LIST + hf * HSTR;
  const uint32_t cap4 = 4u * (lbase + SH);   // byte offset of the spill slot's score
  int fill = 0;
  const int kh = (K + 1) >> 1;           // a compacted row keeps its best kh in half 0, the rest in half 1

  // The candidates of row rw (of this wave) as a sorted list of selection keys, best
  // first: K <= 32: x, lane j of the half = rank j (the best 32); KB: the 64-list (x, y),
  // ranks 0..31 and 32..63.  Half list 0 holds slots 0.., half list 1 the rest.
  auto row_list = [&](int rw, uint64_t& x, uint64_t& y) {
    const int f0 = min(__shfl(fill, rw), SH), f1 = min(__shfl(fill, 32 + rw), SH);
    const int base = (32 * w + rw) * LIST;
    auto key = [&](int s2) { return make_key(cs[base + s2], ci[base + s2]); };
    if constexpr (!KB) {
      x = n < f0 ? key(n) : 0ull;
      y = n < f1 ? key(HSTR + n) : 0ull;
      sort32k(x, n);
      merge_intok(x, y, n, 32);
      y = 0;
    } else {
      // 96 slots as three 32-key registers: list 0 [0, 32), list 0 [32, 48) + list 1
      // [0, 16), list 1 [16, 48)
      static_assert(SH == 48, "");
      x = n < f0 ? key(n) : 0ull;
      y = n < 16 ? (32 + n < f0 ? key(32 + n) : 0ull) : (n - 16 < f1 ? key(HSTR + n - 16) : 0ull);
      uint64_t z = 16 + n < f1 ? key(HSTR + 16 + n) : 0ull;
      kl::sort(x, n);
      kl::sort(y, n);
      kl::sort(z, n);
      kl::split(x, y, n);
      kl::insert64(x, y, z, n);
    }
  };
  // Compact rows ra (lanes 0..31) and rb2 (lanes 32..63) of this wave: keep the best K,
  // the best kh back in half list 0 and the rest in half list 1.  nvalid: the number
  // kept; kkey: the K-th best key (0 if fewer than K), both per half.
  auto settle2 = [&](int ra, int rb2, int& nvalid, uint64_t& kkey) {
    const int rw = hf ? rb2 : ra;
    const int base = (32 * w + rw) * LIST;
    uint64_t x, y;
    row_list(rw, x, y);
    if (n >= K) x = 0;
    if (n + 32 >= K) y = 0;
    const uint64_t vx = __ballot(x != 0), vy = __ballot(y != 0);
    nvalid = __popc(hf ? (uint32_t)(vx >> 32) : (uint32_t)vx) + __popc(hf ? (uint32_t)(vy >> 32) : (uint32_t)vy);
    auto put = [&](int rank, uint64_t kk) {
      if (rank < K) {
        const int slot = rank < kh ? rank : HSTR + rank - kh;
        cs[base + slot] = key_score(kk);
        ci[base + slot] = (uint16_t)key_chunk(kk);
      }
    };
    put(n, x);
    if constexpr (KB) put(32 + n, y);
    kkey = kl::rank_key(x, y, K - 1, lane);
  };

  // the tile's rows are contiguous: thread t moves 16-byte segments t + 256 u; the global
  // and LDS offsets are the same for every tile (the final partial group repeats the last
  // segment, whose duplicate store writes the same bytes)
  int goff[PL], soff[PL];
#pragma unroll
  for (int u = 0; u < PL; ++u) {
    const int it = min(tid + 256 * u, NSEG - 1);
    goff[u] = 8 * it;
    soff[u] = (it / SEGS) * LDR + 8 * (it % SEGS);
  }
  // k' rows of the landmark head, padded to a multiple of KP_PAD zero rows: a tile never
  // reads past them
  const uint16_t* src = p2 + ((int64_t)bb * Hl + hh / (H / Hl)) * kp_rows(C) * DE2;
  u32x4_t pf[PL];
  auto load_tile = [&](int ct) {
    const uint16_t* t = src + (int64_t)ct * SEL_CT * DE2;
#pragma unroll
    for (int u = 0; u < PL; ++u) pf[u] = *reinterpret_cast<const u32x4_t*>(t + goff[u]);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < PL; ++u) *reinterpret_cast<u32x4_t*>(&kt[soff[u]]) = pf[u];
  };

  // The MFMAs of a tile's scores (chunk n of the tile is the A operand row): per k-step
  // the products (i, j) with i + j < NPROD, then b'.  after(m) runs after MFMA number m;
  // the A operands of the next k-step are read from LDS one k-step ahead.
  constexpr int PF = 1;   // k-steps of A operands read ahead
  auto tile_mfma = [&](f32x16_t& a_, auto&& after) {
    const uint16_t* krow = &kt[n * LDR];
    auto opA = [&](int ks, int j) {
      return *reinterpret_cast<const bf16x8_t*>(krow + j * D + (j ? P2_EXT : 0) + 16 * ks + 8 * hf);
    };
    bf16x8_t A[PF + 1][NK];
#pragma unroll
    for (int k0 = 0; k0 < PF && k0 < NKS; ++k0)
#pragma unroll
      for (int j = 0; j < NK; ++j) A[k0][j] = opA(k0, j);
    const bf16x8_t ae = *reinterpret_cast<const bf16x8_t*>(krow + D + 8 * hf);
    int m = 0;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + PF < NKS)
#pragma unroll
        for (int j = 0; j < NK; ++j) A[(ks + PF) % (PF + 1)][j] = opA(ks + PF, j);
#pragma unroll
      for (int j = 0; j < NK; ++j)
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          if (i + j >= NPROD) continue;
          a_ = mfma32(A[ks % (PF + 1)][j], qb[i][ks], a_);
          after(m++);
        }
    }
    a_ = mfma32(ae, qext, a_);  // + b'
    after(m);
  };
  auto tile_scores = [&]() {
    f32x16_t a_ = zero16();
    tile_mfma(a_, [](int) {});
    return a_;
  };

  // Software pipeline: while tile ct's scores are tested and appended, the MFMAs of
  // tile ct + 1 (already staged in LDS) run; tile ct + 2 is in flight from memory.
  // (A second LDS buffer, saving one barrier per tile, measured no faster: it leaves
  // room for fewer candidate slots.)
  const int nct = (Pmax + SEL_CT - 1) / SEL_CT;
  if (nct > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();
  f32x16_t acc = tile_scores();
  if (nct > 1) load_tile(1);
  __syncthreads();  // every wave has read tile 0
  if (nct > 1) store_tile();
  // No load may reach the loop still in flight on any path (the threshold's load does
  // where nct < 2): the compiler would then wait for all loads at the first use of th in
  // every iteration, the k' tile two ahead included, and expose its full latency.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int ct = 0; ct < nct; ++ct) {
    const bool more2 = ct + 2 < nct;
    if (more2) load_tile(ct + 2);
    // register rr holds chunk cb + 8 (rr >> 2) + (rr & 3)
    const int cb = ct * SEL_CT + 4 * hf;
    const int fill0 = fill;
    const float th0 = th;
    const int lim = prow - cb;   // this row's chunks in the tile: offsets < lim
    // append of register rr: only the lanes whose score passes run it.  MASKED tiles
    // reach chunks >= Pmin, which are not past chunks of every row, and test the row's
    // limit; the two kinds run as separate code.
    f32x16_t an = zero16();
    auto run = [&](auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      auto append = [&](int rr) {
        const bool inside = !MASKED || 8 * (rr >> 2) + (rr & 3) < lim;
        if (acc[rr] >= th && inside) {   // NaN never passes
          const uint32_t a4 = min(4u * (lbase + fill), cap4);
          *reinterpret_cast<float*>(lists + a4) = acc[rr];
          *reinterpret_cast<uint16_t*>(lists + CI_OFS + (a4 >> 1)) = (uint16_t)(cb + 8 * (rr >> 2) + (rr & 3));
          ++fill;
        }
      };
      tile_mfma(an, [&](int m) {
        if (m < 16) append(m);
        if (m == NMF - 1)
          for (int rr = NMF; rr < 16; ++rr) append(rr);   // fewer MFMAs than registers
      });
    };
    if ((ct + 1) * SEL_CT > Pmin)
      run(std::true_type{});
    else
      run(std::false_type{});
    if (__ballot(fill > SH)) {
      // Rare: some half lists overflowed; the passes of this tile at slot index >= SH
      // went to the spill slot and are lost for now.  Compact the rows of the
      // overflowed lanes (each half then holds at most 16), drop the lost ones that no
      // longer pass the raised thresholds, append the rest while there is room, and
      // repeat for lanes that filled up again.
      uint32_t lost = 0;
      {
        int running = fill0;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          if (acc[rr] >= th0 && 8 * (rr >> 2) + (rr & 3) < lim) {
            if (running >= SH) lost |= 1u << rr;
            ++running;
          }
        }
      }
      uint64_t ovf = __ballot(fill > SH);
      while (ovf) {
        uint32_t rows_big = (uint32_t)ovf | (uint32_t)(ovf >> 32);
        while (rows_big) {
          const int ra = __builtin_ctz(rows_big);
          rows_big &= rows_big - 1;
          int rb2 = ra;
          const bool two = rows_big != 0;
          if (two) {
            rb2 = __builtin_ctz(rows_big);
            rows_big &= rows_big - 1;
          }
          uint64_t kk;
          int nv;
          settle2(ra, rb2, nv, kk);
          // new fills and thresholds of the two rows (half 0 of the wave did row ra, half 1 row rb2)
          const int nva = __shfl(nv, 0), nvb = __shfl(nv, 32);
          const uint64_t kka = __shfl(kk, 0), kkb = __shfl(kk, 32);
          const float ka = kka ? key_score(kka) : -INFINITY, kb = kkb ? key_score(kkb) : -INFINITY;
          if (n == ra) {
            fill = hf ? max(0, nva - kh) : min(nva, kh);
            th = fmaxf(th, ka);
          }
          if (two && n == rb2) {
            fill = hf ? max(0, nvb - kh) : min(nvb, kh);
            th = fmaxf(th, kb);
          }
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          if ((lost >> rr) & 1u) {
            const float sv = acc[rr];
            if (!(sv >= th)) {
              lost &= ~(1u << rr);
            } else if (fill < SH) {
              cs[lbase + fill] = sv;
              ci[lbase + fill] = (uint16_t)(cb + 8 * (rr >> 2) + (rr & 3));
              ++fill;
              lost &= ~(1u << rr);
            }
          }
        }
        if (lost) fill = SH + 1;   // still lost ones: the half is full, compact again
        ovf = __ballot(lost != 0);
      }
    }
    __syncthreads();  // every wave is done with tile ct + 1 in LDS
    if (more2) store_tile();
    __syncthreads();
    acc = an;
  }

  // ---- final selection and output in ascending chunk id order.  K <= 32: eight row pairs
  // (p, p + 16) at a time, the two half lists of a row sorted as keys and merged to the best
  // 32, the best K sorted again by chunk id; lane j of each half writes slot j.  KB: one row
  // pair at a time as 64-lists.
  if constexpr (!KB) {
    constexpr int FR = NQ * NK > 4 ? 4 : 8;  // fewer at once where the score operands take more registers
    float pinf = INFINITY, ninf = -INFINITY;  // hidden from the compiler: the sort's med3s stay med3s
    asm volatile("" : "+v"(pinf));
    asm volatile("" : "+v"(ninf));
#pragma unroll 1
    for (int p0r = 0; p0r < 16; p0r += FR) {
      uint64_t x[FR], y[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int rw = hf ? p0r + i + 16 : p0r + i;
        const int f0 = min(__shfl(fill, rw), SH), f1 = min(__shfl(fill, 32 + rw), SH);
        const int base = (32 * w + rw) * LIST;
        x[i] = n < f0 ? make_key(cs[base + n], ci[base + n]) : 0ull;
        y[i] = n < f1 ? make_key(cs[base + HSTR + n], ci[base + HSTR + n]) : 0ull;
      }
      sort32k_r<FR>(x, n);
      sort32k_r<FR>(y, n);
#pragma unroll
      for (int i = 0; i < FR; ++i) {  // the 32 best of both lists, a bitonic sequence
        const uint64_t rk = xl64<31>(y[i]);
        x[i] = rk > x[i] ? rk : x[i];
      }
      if (K < 32) {  // the ranks matter only when fewer than 32 are kept
        cxk_r<16, FR>(x, (n & 16) == 0);
        cxk_r<8, FR>(x, (n & 8) == 0);
        cxk_r<4, FR>(x, (n & 4) == 0);
        cxk_r<2, FR>(x, (n & 2) == 0);
        cxk_r<1, FR>(x, (n & 1) == 0);
      }
      // the kept keys in ascending chunk order: float keys in [1, 2) whose bits hold
      // (0x3fff - chunk, lane), larger for a lower chunk (chunk < 16384), 0 for none;
      // after a descending sort lane j takes the score from the lane its key names
      float fk[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i)
        fk[i] = x[i] != 0 && n < K
                    ? __uint_as_float(0x3f800000u | ((0x3fffu - (uint32_t)key_chunk(x[i])) << 5) | (uint32_t)n)
                    : 0.f;
      sort32f_r<FR>(fk, n, pinf, ninf);
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const uint32_t fb = __float_as_uint(fk[i]);
        const float sc = __shfl(key_score(x[i]), (lane & 32) | (int)(fb & 31u));
        const int rw = r0 + 32 * w + (hf ? p0r + i + 16 : p0r + i);
        if (rw < N && n < K) {
          const int64_t o = ((int64_t)bh * N + rw) * K + n;
          const bool ok = fb != 0;
          sel_idx[o] = ok ? (int)(0x3fffu - ((fb >> 5) & 0x3fffu)) : -1;
          sel_score[o] = ok ? sc : -INFINITY;
        }
      }
    }
  } else {
#pragma unroll 1
    for (int p = 0; p < 16; ++p) {
      uint64_t x, y;
      row_list(hf ? p + 16 : p, x, y);
      kl::ids_ascending(x, y, K, n);
      const int rw = r0 + 32 * w + (hf ? p + 16 : p);
      auto out = [&](int rank, uint64_t kk) {
        if (rw < N && rank < K) {
          const int64_t o = ((int64_t)bh * N + rw) * K + rank;
          sel_idx[o] = kk ? key_chunk(kk) : -1;
          sel_score[o] = kk ? key_score(kk) : -INFINITY;
        }
      };
      out(n, x);
      out(32 + n, y);
    }
  }
}

// ---------------------------------------------------------------- k' preparation
// k' (fp32) -> chunk rows k~ for both passes: k~ = k' without Q-Cal, one row per
// (batch, landmark head, chunk); with Q-Cal (r > 0) k~_hc = k'_c + D_h^T (U_h^T k'_c) in
// fp32, one row per (batch, query head, chunk), so that q^ . k' = q . k~.  Written as
// (a) the selection pass's rows: tau*k~ split into NK bf16 term planes with the extension
// [b'_hi, b'_mid, b'_lo, 0 ...] after plane 0, and (b) the threshold pass's rows:
// bf16(tau*k~) followed by [b'_hi, b'_lo, TH_ABS, |tau*k~_c| rounded up, 0 ...].  Both
// hold each 16-element k-block in MFMA operand order: position 16 ks + 8 h + m holds
// element kperm(ks, h, m).  Each (batch, row head) gets kp_rows(C) rows, those past C
// zero.  Hp: heads of the output rows (Hl, or Hq under Q-Cal).
constexpr int QC_MAXR = 32;   // largest Q-Cal rank

template <typename IO, int D, int NK>
__global__ void __launch_bounds__(256) prep_kprime(const float* __restrict__ kc, const float* __restrict__ bc,
                                                   const IO* __restrict__ Dw, const IO* __restrict__ Uw,
                                                   uint16_t* __restrict__ p2, uint16_t* __restrict__ t1,
                                                   int64_t rows, int C, int Cp, int Hp, int Hl, int r) {
  constexpr int SPR = D / 8;        // 16-byte segments (threads) per chunk row
  constexpr int RPB = 256 / SPR;    // chunk rows per workgroup pass (one row head: RPB divides Cp)
  constexpr int APT = QC_MAXR / SPR;   // entries of w per thread
  constexpr int DE = D + TH_EXT;
  constexpr int DE2 = NK * D + P2_EXT;
  // Q-Cal staging: U_h as [e][a] and D_h as [a][e] (fp32, zero past rank r), the pass's
  // k' rows and their w = U_h^T k'
  __shared__ __align__(16) float Us[D * QC_MAXR];
  __shared__ __align__(16) float Ds[QC_MAXR * D];
  __shared__ __align__(16) float Ks[RPB * (D + 4)];
  __shared__ __align__(16) float Ws[RPB * QC_MAXR];
  const float tau = 1.0f / sqrtf((float)D);
  const int tid = threadIdx.x;
  const int sg = tid % SPR, ks = sg >> 1, h = sg & 1, lr = tid / SPR;
  // each workgroup takes a contiguous range of passes, so the row head rarely changes
  const int64_t npass = (rows + RPB - 1) / RPB;
  const int64_t ppw = (npass + gridDim.x - 1) / gridDim.x;
  const int64_t pbeg = (int64_t)blockIdx.x * ppw, pend = min(npass, pbeg + ppw);
  int staged = -1;
  for (int64_t pass = pbeg; pass < pend; ++pass) {
    const int64_t rw = pass * RPB + lr;    // output row: (b, row head) * Cp + chunk
    const bool ok = rw < rows;
    const int c = (int)(rw % Cp);
    const bool real = ok && c < C;         // rows c >= C are zero padding
    const int64_t bhp = rw / Cp;           // (b, row head)
    const int hp = (int)(bhp % Hp);
    const int64_t sr = (bhp / Hp * Hl + hp / (Hp / Hl)) * C + c;   // source row of kc / bc
    float x[8];
    if (real) {
      const float4 a = *reinterpret_cast<const float4*>(kc + sr * D + kperm(ks, h, 0));
      const float4 b = *reinterpret_cast<const float4*>(kc + sr * D + kperm(ks, h, 4));
      x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = 0.f;
    }
    if (r > 0) {
      // k~ = k' + D_h^T w with w = U_h^T k'.  The pass's rows share one row head (every
      // thread agrees on hp0, so the branches and barriers are uniform).
      const int hp0 = (int)((pass * RPB / Cp) % Hp);
      if (hp0 != staged) {
        __syncthreads();
        for (int i = tid; i < D * QC_MAXR; i += 256) {
          const int e = i / QC_MAXR, a = i % QC_MAXR;   // Us[e][a] = U_h[e][a]
          Us[i] = a < r ? io_traits<IO>::load(Uw, ((int64_t)hp0 * D + e) * r + a) : 0.f;
          const int a2 = i / D, e2 = i % D;             // Ds[a][e] = D_h[a][e]
          Ds[i] = a2 < r ? io_traits<IO>::load(Dw, ((int64_t)hp0 * r + a2) * D + e2) : 0.f;
        }
        staged = hp0;
      }
      {
        float* kr = Ks + lr * (D + 4);
        *reinterpret_cast<float4*>(kr + kperm(ks, h, 0)) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(kr + kperm(ks, h, 4)) = make_float4(x[4], x[5], x[6], x[7]);
      }
      __syncthreads();
      {
        // w[lr][a] for a = APT sg + j
        float wv[APT];
#pragma unroll
        for (int j = 0; j < APT; ++j) wv[j] = 0.f;
        const float* kr = Ks + lr * (D + 4);
        for (int e = 0; e < D; e += 4) {
          const float4 kv = *reinterpret_cast<const float4*>(kr + e);
          const float ke[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < APT; ++j) wv[j] = fmaf(Us[(e + i) * QC_MAXR + APT * sg + j], ke[i], wv[j]);
        }
#pragma unroll
        for (int j = 0; j < APT; ++j) Ws[lr * QC_MAXR + APT * sg + j] = wv[j];
      }
      __syncthreads();
      float kt[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) kt[m] = x[m];
      for (int a = 0; a < r; ++a) {
        const float wa = Ws[lr * QC_MAXR + a];
        const float4 d0 = *reinterpret_cast<const float4*>(Ds + a * D + kperm(ks, h, 0));
        const float4 d1 = *reinterpret_cast<const float4*>(Ds + a * D + kperm(ks, h, 4));
        kt[0] = fmaf(d0.x, wa, kt[0]);
        kt[1] = fmaf(d0.y, wa, kt[1]);
        kt[2] = fmaf(d0.z, wa, kt[2]);
        kt[3] = fmaf(d0.w, wa, kt[3]);
        kt[4] = fmaf(d1.x, wa, kt[4]);
        kt[5] = fmaf(d1.y, wa, kt[5]);
        kt[6] = fmaf(d1.z, wa, kt[6]);
        kt[7] = fmaf(d1.w, wa, kt[7]);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = real ? kt[m] : 0.f;
    }
    float s2 = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) s2 = fmaf(x[m], x[m], s2);
#pragma unroll
    for (int o = 1; o < SPR; o <<= 1) s2 += __shfl_xor(s2, o);
    float xs[8], xh[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      xs[m] = tau * x[m];
      xh[m] = tau * x[m];
    }
    u32x4_t tm[NK], hi[1];
    split8<NK>(xs, tm);
    split8<1>(xh, hi);
    if (ok) {
      uint16_t* o2 = p2 + rw * DE2;
#pragma unroll
      for (int j = 0; j < NK; ++j) *reinterpret_cast<u32x4_t*>(o2 + j * D + (j ? P2_EXT : 0) + 8 * sg) = tm[j];
      uint16_t* o1 = t1 + rw * DE;
      *reinterpret_cast<u32x4_t*>(o1 + 8 * sg) = hi[0];
      if (sg < 2) {
        uint16_t e[8] = {0, 0, 0, 0, 0, 0, 0, 0}, f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (sg == 0) {
          const float bv = real ? bc[sr] : 0.f;
          uint16_t sp3[3], sp2[2];
          split_bf16<3>(bv, sp3);
          split_bf16<2>(bv, sp2);
          e[0] = sp2[0];
          e[1] = sp2[1];
          e[2] = f32_to_bf16(TH_ABS);  // 2^-12, exact in bf16 (0x3980)
          e[3] = bf16_up(tau * sqrtf(s2));
          f[0] = sp3[0];
          f[1] = sp3[1];
          f[2] = sp3[2];
        }
        *reinterpret_cast<bf16x8_t*>(o1 + D + 8 * sg) = pack8(e);
        *reinterpret_cast<bf16x8_t*>(o2 + D + 8 * sg) = pack8(f);
      }
    }
  }
}

static size_t al3(size_t x) { return (x + 255) / 256 * 256; }
static int nk_of(const Geom& g) { return g.io == 0 ? 3 : 2; }
// heads of the chunk rows: the landmark heads, or the query heads when Q-Cal folds into them
static int row_heads(const Geom& g) { return g.r > 0 ? g.Hq : g.Hl; }

struct ScoreWs {
  size_t planes, t1, theta, total;
};
static ScoreWs score_ws(const Geom& g) {
  const size_t rows = (size_t)g.B * row_heads(g) * kp_rows(g.C());   // chunk rows per (b, row head): padded
  ScoreWs w;
  size_t off = 0;
  w.planes = off;
  off += al3(rows * ((size_t)nk_of(g) * g.d + P2_EXT) * 2);
  w.t1 = off;
  off += al3(rows * (g.d + TH_EXT) * 2);
  w.theta = off;
  off += al3((size_t)g.B * g.Hq * g.N * 4);   // one per query, for up to N queries
  w.total = off;
  return w;
}

size_t score_workspace_bytes(const Geom& g) { return score_ws(g).total; }

template <typename IO, int D, int NQ, int NK>
static void launch_st(const Geom& g, int Nq, const int32_t* pos0, const void* q, const uint16_t* planes,
                      const uint16_t* t1, float* theta, int32_t* si, float* ss, hipStream_t st, hipEvent_t* ev) {
  const int NB = (Nq + ST_ROWS - 1) / ST_ROWS;
  const int items = g.B * g.Hq * NB;
  const int grid = ((items + 7) / 8) * 8;
  const int Hp = row_heads(g);
  if (items > 0) {
    hipLaunchKernelGGL((score_threshold<IO, D>), dim3(grid), dim3(256), 0, st, (const IO*)q, t1, theta, pos0, g.Hq,
                       Hp, Nq, g.C(), g.K, NB, items, g.nw);
  }
  if (ev) hipEventRecord(ev[0], st);
  if (items > 0) {
    if (g.K > 32)
      hipLaunchKernelGGL((score_topk_kernel<IO, D, NQ, NK, 2>), dim3(grid), dim3(256), 0, st, (const IO*)q, planes,
                         (const float*)theta, si, ss, pos0, g.Hq, Hp, Nq, g.C(), g.K, NB, items, g.nw);
    else if (g.K > 16)
      hipLaunchKernelGGL((score_topk_kernel<IO, D, NQ, NK, 1>), dim3(grid), dim3(256), 0, st, (const IO*)q, planes,
                         (const float*)theta, si, ss, pos0, g.Hq, Hp, Nq, g.C(), g.K, NB, items, g.nw);
    else
      hipLaunchKernelGGL((score_topk_kernel<IO, D, NQ, NK, 0>), dim3(grid), dim3(256), 0, st, (const IO*)q, planes,
                         (const float*)theta, si, ss, pos0, g.Hq, Hp, Nq, g.C(), g.K, NB, items, g.nw);
  }
}

template <typename IO, int D>
static void launch_prep(const Geom& g, const float* kc, const float* bc, const void* Dw, const void* Uw,
                        uint16_t* planes, uint16_t* t1, hipStream_t st) {
  const int Cp = kp_rows(g.C());
  const int Hp = row_heads(g);
  const int64_t rows = (int64_t)g.B * Hp * Cp;
  const int64_t rpb = 256 / (D / 8);
  const unsigned gs = (unsigned)std::min<int64_t>((rows + rpb - 1) / rpb, 2048);
  constexpr int NK = io_traits<IO>::terms == 3 ? 3 : 2;   // nk_of(g)
  hipLaunchKernelGGL((prep_kprime<IO, D, NK>), dim3(gs), dim3(256), 0, st, kc, bc, (const IO*)Dw, (const IO*)Uw,
                     planes, t1, rows, g.C(), Cp, Hp, g.Hl, g.r);
}

// q enters the products as NQ exact bf16 terms (one for bf16, three for fp32); the chunk
// rows as NK terms (hi + lo for bf16 I/O, three for fp32)
template <typename IO, int D>
static void launch_all(const Geom& g, int Nq, const int32_t* pos0, const void* q, const void* Dw, const void* Uw,
                       const float* kc, const float* bc, uint16_t* planes, uint16_t* t1, float* theta, int32_t* si,
                       float* ss, hipStream_t st, hipEvent_t* ev) {
  constexpr bool F32 = io_traits<IO>::terms == 3;
  if (g.C() > 0) launch_prep<IO, D>(g, kc, bc, Dw, Uw, planes, t1, st);
  launch_st<IO, D, F32 ? 3 : 1, F32 ? 3 : 2>(g, Nq, pos0, q, planes, t1, theta, si, ss, st, ev);
}

hipError_t launch_score_topk(const Geom& g, int Nq, const int32_t* pos0, const void* q, const void* Dw, const void* Uw,
                             const float* kc, const float* bc, int32_t* sel_idx, float* sel_score, void* ws,
                             size_t ws_bytes, hipStream_t st, hipEvent_t* ev) {
  if (ws_bytes < score_workspace_bytes(g) || Nq > g.N) return hipErrorInvalidValue;
  const ScoreWs w = score_ws(g);
  uint16_t* planes = (uint16_t*)((char*)ws + w.planes);
  uint16_t* t1 = (uint16_t*)((char*)ws + w.t1);
  float* theta = (float*)((char*)ws + w.theta);
  if (g.io == 0) {
    if (g.d == 64)
      launch_all<float, 64>(g, Nq, pos0, q, Dw, Uw, kc, bc, planes, t1, theta, sel_idx, sel_score, st, ev);
    else
      launch_all<float, 128>(g, Nq, pos0, q, Dw, Uw, kc, bc, planes, t1, theta, sel_idx, sel_score, st, ev);
  } else {
    if (g.d == 64)
      launch_all<bf16_t, 64>(g, Nq, pos0, q, Dw, Uw, kc, bc, planes, t1, theta, sel_idx, sel_score, st, ev);
    else
      launch_all<bf16_t, 128>(g, Nq, pos0, q, Dw, Uw, kc, bc, planes, t1, theta, sel_idx, sel_score, st, ev);
  }
  if (ev) hipEventRecord(ev[1], st);
  return hipGetLastError();
}

}  // namespace hils

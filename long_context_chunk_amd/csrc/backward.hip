// Backward pass of the prefill forward: gradients of the output with respect to q, k, v,
// the landmark queries and the Q-Cal projections, with the selection held fixed (top-K is
// piecewise constant).  End-to-end retrieval learning: the training signal reaches the
// landmark queries and the query calibration through the chunk scores (hotpaper.ai
// abstract and "Key contributions"; aitrends.kr "Key contributions").
//
// Per query row i with output gradient g = dO_i, forward output o_i and fusion
// weights w_e = exp(sigma_e - Lambda_i), Lambda_i = log sum_e exp(sigma_e):
//   selected chunk c (score s_ic = tau q^.k'_c + b'_c, chunk softmax P over its keys):
//     dP'_j = g.v_j,  e_c = sum_j P_j dP'_j (= g.o_ic),  dsigma_c = w_c (e_c - g.o_i),
//     dS_j = P_j w_c (dP'_j - e_c)     (gradient of the logit tau q.k_j)
//   window (score = its exact LSE, softmax P over the window's keys):
//     dS_j = P_j w_w (dP'_j - g.o_i)   (the LSE's own gradient folded in)
//   dq += tau sum_j dS_j k_j,  dk_j += tau dS_j q,  dv_j += P_j w g;
//   scores: dq^ += tau dsigma_c k'_c,  dk'_c += tau dsigma_c q^,  db'_c += dsigma_c;
//   Q-Cal: dq += dq^ + D^T (U^T dq^),  dU += dq^ (D q)^T,  dD += (U^T dq^) q^T;
//   compression: da_j = dk'.k_j - db' (log a_j + 1), dz_j = a_j (da_j - sum a da),
//     dL_c = tau sum_j dz_j k_j,  dk_j += a_j dk'_c + tau dz_j L_c.
//
// Kernels, in launch order (bf16 I/O, fp32 accumulation in the workspace):
//   bwd_kdq       (Q-Cal) per chunk: the score direction k'_c + D^T (U^T k'_c)
//   bwd_window    per (b, KV head, query chunk, pair of heads): the window's LSE, the
//                 row's fusion normaliser Lambda_i and g.o_i, then the window's
//                 gradients on the MFMA (dq stored, dk/dv added atomically)
//   bucketing     the forward's (b, head, chunk) bucketing of the selection pairs
//   bwd_pairs     per bucket work item, eight waves: the chunk's K/V staged once, 16
//                 gathered rows per wave: S, dP' on the MFMA, dsigma and the pair's dq
//                 (with its score term) as a bf16 partial, then dk/dv over the tile's 128
//                 rows on the MFMA from transposed LDS tiles; the chunk's sum dsigma q, db'
//   bwd_dq_sum    per row: the window's dq plus the pairs' partials, rounded to the output
//   bwd_qcal_g    (Q-Cal) per head: G = tau sum_c k'_c (sum dsigma q)_c^T, then
//                 dU = G D^T, dD = U^T G (bwd_qcal_weights)
//   bwd_compress  per (b, KV head, chunk): the landmark compression's backward
//   bwd_convert   dk, dv accumulators to the output dtype
#include <algorithm>

#include "attn_tile.h"
#include "hils_common.h"
#include "kernels.h"

namespace hils {

namespace {

constexpr int BW_ROWS = 128;  // rows per tile: 4 waves x 32
constexpr int LDP = 64 + 8;   // bf16 row stride of the [row][key] P and dS tiles

struct BwdWs {
  size_t dq, dk, dv, dkc, dbc, G, lam, dd, dsig, dqp, kdq, counts, cursor, boff, toff, pairs, tmp, imap, total;
};
size_t alb(size_t x) { return (x + 255) / 256 * 256; }
BwdWs bwd_ws(const Geom& g) {
  BwdWs w;
  const size_t rows = (size_t)g.B * g.Hq * g.N, kvrows = (size_t)g.B * g.Hkv * g.N;
  const size_t nbk = (size_t)g.B * g.Hq * g.C();
  const size_t ent = rows * g.K, r = (size_t)g.r;
  size_t off = 0;
  auto take = [&](size_t& f, size_t bytes) {
    f = off;
    off += alb(bytes);
  };
  take(w.dq, rows * g.d * 4);
  take(w.dk, kvrows * g.d * 4);  // dk .. dU are zeroed together: keep them contiguous
  take(w.dv, kvrows * g.d * 4);
  take(w.dkc, nbk * g.d * 4);  // per query head: a shared landmark head sums its query heads' terms
  take(w.dbc, nbk * 4);
  take(w.G, r > 0 ? (size_t)g.Hq * g.d * g.d * 4 : 0);  // G = tau sum_c k'_c S_c^T per head (S_c = sum dsigma q)
  take(w.lam, rows * 4);
  take(w.dd, rows * 4);
  take(w.dsig, ent * 4);
  take(w.dqp, ent * g.d * 2);  // per (row, slot) dq of the selected chunk's attention (bf16)
  take(w.kdq, r > 0 ? nbk * g.d * 4 : 0);  // k'_c + D_h^T U_h^T k'_c per (query head, chunk) (Q-Cal)
  take(w.counts, nbk * 4);  // counts and cursor contiguous (zeroed together)
  take(w.cursor, nbk * 4);
  take(w.boff, (nbk + 1) * 4);
  take(w.toff, (nbk + 1) * 4);
  take(w.pairs, ent * 4);
  take(w.tmp, ent * 4);
  take(w.imap, (size_t)bucket_items_bound(g) * 4);
  w.total = off;
  return w;
}

HILS_DEV float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ void __launch_bounds__(256) bwd_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// --------------------------------------------------------- shared tile gradients
// LDS of one gradient tile: the chunk's K/V, and for the tile's 128 rows their q and
// g (bf16, [row][dim]) and P*w and dS (bf16, [row][key]) for the dk/dv products.
template <int D>
struct GradLds {
  static constexpr int LDR = D + 8;
  KVTile<bf16_t, D, 1, 8> kv;  // V is read by whole rows only (dP' = g V^T)
  uint16_t qt[BW_ROWS * LDR];
  uint16_t gt[BW_ROWS * LDR];
  uint16_t pt[BW_ROWS * LDP];
  uint16_t st[BW_ROWS * LDP];
};

// S^T = K Q^T style product of the staged chunk (plane = K or V, row stride LD) with a
// wave's 32 rows given as B operands: x[tt][rr] = row n . key (32 tt + acc_row(rr, hf)).
template <int D, int LD>
HILS_DEV void keys_dot_rows(const uint16_t* plane, const bf16x8_t (&rb)[D / 16], f32x16_t (&x)[2]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    x[tt] = zero16();
    const int key = 32 * tt + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) x[tt] = mfma32(lds_op16(&plane[key * LD + 16 * ks + 8 * hf]), rb[ks], x[tt]);
  }
}

// The key-indexed registers x (layout of keys_dot_rows) as B operands over the keys.
HILS_DEV void keys_to_b(const f32x16_t (&x)[2], bf16x8_t (&b)[4]) {
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
    float pv[8];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) pv[mm] = x[ks2 >> 1][8 * (ks2 & 1) + mm];
    u32x4_t t[1];
    split8<1>(pv, t);
    b[ks2] = __builtin_bit_cast(bf16x8_t, t[0]);
  }
}

// Writes a wave's key-indexed registers (bf16) to its 32 rows of a [row][key] tile.
HILS_DEV void keys_to_lds(const f32x16_t (&x)[2], uint16_t* tile, int row) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2_t pk;
      pk.x = pack_bf16x2(x[tt][4 * g4], x[tt][4 * g4 + 1]);
      pk.y = pack_bf16x2(x[tt][4 * g4 + 2], x[tt][4 * g4 + 3]);
      *reinterpret_cast<u32x2_t*>(&tile[row * LDP + 32 * tt + 8 * g4 + 4 * hf]) = pk;
    }
}

// A wave's 32 rows of B operands (D/16 x 8 dims per lane) to its rows of a [row][dim] tile.
template <int D>
HILS_DEV void rows_to_lds(const bf16x8_t (&rb)[D / 16], uint16_t* tile, int row) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    *reinterpret_cast<bf16x8_t*>(&tile[row * GradLds<D>::LDR + 16 * ks + 8 * hf]) = rb[ks];
}

// dq^T += K^T dS^T for the wave's rows: dq[dt][rr] = dim (32 dt + acc_row(rr, hf)) of row n.
template <int D>
HILS_DEV void dq_from_ds(const KVTile<bf16_t, D, 1, 8>& kv, const f32x16_t (&ds)[2], f32x16_t (&dq)[D / 32]) {
  constexpr int LDK = KVTile<bf16_t, D, 1, 8>::LDK;
  const int lane = threadIdx.x & 63;
  bf16x8_t db[4];
  keys_to_b(ds, db);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) dq[dt] = mfma32(vt_operand<LDK>(kv.k[0], dt, ks2, lane), db[ks2], dq[dt]);
}

// dv = sum_rows (P w)^T g and dk = tau sum_rows dS^T q over the tile's 128 rows (all four
// waves' rows, from the LDS tiles), added to the fp32 accumulators of the chunk's keys
// (row kvrow0 + key).  Each wave takes a quarter of the (kind, key tile, dim tile) blocks.
template <int D>
HILS_DEV void dkdv_from_tiles(const GradLds<D>& L, float* __restrict__ dk, float* __restrict__ dv, int64_t kvrow0,
                              int nkeys, float tau) {
  constexpr int NDT = D / 32, NBLK = 2 * 2 * NDT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hf = lane >> 5;
  for (int blk = w; blk < NBLK; blk += 4) {
    const bool isk = blk >= 2 * NDT;
    const int kt = (blk % (2 * NDT)) / NDT, dt = blk % NDT;
    const uint16_t* a_tile = isk ? L.st : L.pt;
    const uint16_t* b_tile = isk ? L.qt : L.gt;
    f32x16_t acc = zero16();
#pragma unroll
    for (int ks2 = 0; ks2 < BW_ROWS / 16; ++ks2)
      acc = mfma32(vt_operand<LDP>(a_tile, kt, ks2, lane), vt_operand<GradLds<D>::LDR>(b_tile, dt, ks2, lane), acc);
    float* dst = isk ? dk : dv;
    const float sc = isk ? tau : 1.0f;
    const int e = 32 * dt + (lane & 31);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 32 * kt + acc_row(rr, hf);
      if (key < nkeys) atomicAdd(&dst[(kvrow0 + key) * D + e], acc[rr] * sc);
    }
  }
}

// ------------------------------------------------------------------ bwd_window
// One workgroup per (b, KV head, query chunk qc, pair of its query heads), two waves per
// head (rows qc*64 .. qc*64+63).  Pass 1: the window's LSE by an online max/sum over
// its chunks.  Row statistics: Lambda_i over the selected scores and the window's LSE,
// g.o_i from the forward output.  Pass 2, per window chunk: P = exp(tau s - LSE),
// dS = P w (dP' - g.o), dq on the MFMA (kept in registers, stored at the end: this
// kernel writes every row's dq first), dk/dv over the 128 rows, added atomically.
template <int D>
__global__ void __launch_bounds__(256) bwd_window(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                  const bf16_t* __restrict__ v, const bf16_t* __restrict__ o,
                                                  const bf16_t* __restrict__ dO, const float* __restrict__ sel_score,
                                                  float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                                                  float* __restrict__ lam, float* __restrict__ dd, int Hq, int Hkv,
                                                  int N, int C, int K, int NQC, int nw) {
  __shared__ GradLds<D> L;
  const int G = Hq / Hkv;
  const int ngb = (G + 1) / 2;
  const int gb = blockIdx.x % ngb, rest = blockIdx.x / ngb;
  const int qc = rest % NQC, bkv = rest / NQC;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5;
  const int gi = gb * 2 + (w >> 1);
  const bool head_ok = gi < G;
  const int h = kvh * G + min(gi, G - 1);
  const int64_t bh = (int64_t)b * Hq + h;
  const int64_t kv0 = ((int64_t)b * Hkv + kvh) * N;
  const int rl = 32 * (w & 1) + (lane & 31);
  const int i = qc * 64 + rl;
  const bool ok = i < N && head_ok;
  const int64_t row = bh * N + (ok ? i : 0);
  const float tau = 1.0f / sqrtf((float)D);
  const float cl = tau * 1.44269504088896340736f;
  // the row's q, g and o as MFMA operands (16 bytes per k-step), read unconditionally:
  // a row past N or of a missing head reads row 0 of the head and gets zero weight below
  bf16x8_t qb[1][D / 16], gb8[D / 16], ob[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int64_t off = row * D + 16 * ks + 8 * hf;
    qb[0][ks] = *reinterpret_cast<const bf16x8_t*>(q + off);
    gb8[ks] = *reinterpret_cast<const bf16x8_t*>(dO + off);
    ob[ks] = *reinterpret_cast<const bf16x8_t*>(o + off);
  }
  // g.o_i (each lane half holds 8 of every 16 dims)
  float go = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4_t gw = __builtin_bit_cast(u32x4_t, gb8[ks]), ow = __builtin_bit_cast(u32x4_t, ob[ks]);
    const uint32_t g4[4] = {gw.x, gw.y, gw.z, gw.w}, o4[4] = {ow.x, ow.y, ow.z, ow.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      go = fmaf(__uint_as_float(g4[m] << 16), __uint_as_float(o4[m] << 16), go);
      go = fmaf(__uint_as_float(g4[m] & 0xffff0000u), __uint_as_float(o4[m] & 0xffff0000u), go);
    }
  }
  go += __shfl_xor(go, 32);
  const int c0 = max(0, qc - nw + 1);
  // pass 1: the window's max logit and sum
  float m = -INFINITY, l = 0.f;
  for (int c = c0; c <= qc; ++c) {
    if (c > c0) __syncthreads();
    stage_kv<bf16_t, D, 1>(L.kv, k, v, kv0 + (int64_t)c * 64, min(64, N - c * 64), tid, 256);
    __syncthreads();
    f32x16_t s[2];
    keys_dot_rows<D, KVTile<bf16_t, D, 1, 8>::LDK>(L.kv.k[0], qb[0], s);
    const int lim = c == qc ? rl + 1 : 64;
    float mt = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        if (32 * tt + acc_row(rr, hf) >= lim) s[tt][rr] = -INFINITY;
        mt = fmaxf(mt, s[tt][rr]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    float lt = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) lt += __builtin_amdgcn_exp2f(fmaf(s[tt][rr], cl, -mn * cl));
    lt += __shfl_xor(lt, 32);
    l = fmaf(l, __builtin_amdgcn_exp2f((m - mn) * cl), lt);
    m = mn;
  }
  const float lse = m * tau + logf(l);
  // the fusion normaliser over the selected scores and the window's LSE
  const int ns = min(K, candidate_chunks(i, C, nw));
  float smax = lse;
  for (int x = 0; x < ns; ++x) smax = fmaxf(smax, ok ? sel_score[row * K + x] : -INFINITY);
  float z = __expf(lse - smax);
  for (int x = 0; x < ns; ++x) z += ok ? __expf(sel_score[row * K + x] - smax) : 0.f;
  const float Lam = smax + logf(z);
  const float ww = ok ? __expf(lse - Lam) : 0.f;
  if (ok && hf == 0) {
    lam[row] = Lam;
    dd[row] = go;
  }
  // the rows' q and g as [row][dim] tiles for the dk / dv products (constant over the window)
  const int trow = 32 * w + (lane & 31);
  rows_to_lds<D>(qb[0], L.qt, trow);
  {
    bf16x8_t gs[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) gs[ks] = ww == 0.f ? bf16x8_t{} : gb8[ks];
    rows_to_lds<D>(gs, L.gt, trow);  // rows with no weight contribute nothing
  }
  f32x16_t dqa[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqa[dt] = zero16();
  const float lse2 = lse * 1.44269504088896340736f;
  for (int c = c0; c <= qc; ++c) {
    const int nkeys = min(64, N - c * 64);
    if (c0 != qc) {  // a one-chunk window reuses the tile pass 1 left staged
      __syncthreads();  // every wave is done with the previous chunk's tiles
      stage_kv<bf16_t, D, 1>(L.kv, k, v, kv0 + (int64_t)c * 64, nkeys, tid, 256);
      __syncthreads();
    }
    f32x16_t s[2], dp[2];
    keys_dot_rows<D, KVTile<bf16_t, D, 1, 8>::LDK>(L.kv.k[0], qb[0], s);
    keys_dot_rows<D, KVTile<bf16_t, D, 1, 8>::LDV>(L.kv.v[0], gb8, dp);
    const int lim = c == qc ? rl + 1 : 64;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float p = 32 * tt + acc_row(rr, hf) < lim ? __builtin_amdgcn_exp2f(fmaf(s[tt][rr], cl, -lse2)) * ww : 0.f;
        s[tt][rr] = p;                         // P w
        dp[tt][rr] = p * (dp[tt][rr] - go);    // dS
      }
    keys_to_lds(s, L.pt, trow);
    keys_to_lds(dp, L.st, trow);
    dq_from_ds<D>(L.kv, dp, dqa);
    __syncthreads();
    dkdv_from_tiles<D>(L, dk, dv, kv0 + (int64_t)c * 64, nkeys, tau);
  }
  if (!ok) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int e = 32 * dt + 8 * g4 + 4 * hf;
      *reinterpret_cast<float4*>(&dq[row * D + e]) =
          make_float4(dqa[dt][4 * g4] * tau, dqa[dt][4 * g4 + 1] * tau, dqa[dt][4 * g4 + 2] * tau,
                      dqa[dt][4 * g4 + 3] * tau);
    }
}

// ------------------------------------------------------------------- bwd_pairs
// One work item = up to BUCKET_ITEM_ROWS gathered rows of one bucket (b, h, c), in
// tiles of 128 rows, eight waves: two waves share each SIMD, so one hides the other's
// latencies.  Per row (16 per wave, on 16x16x32 MFMAs): S and dP' against the staged
// chunk, the chunk softmax P, e = sum_j P_j dP'_j, w = exp(s_ic - Lambda_i),
// dsigma = w (e - g.o_i) (stored per pair), dS = P w (dP' - e) and the pair's dq (stored
// as a bf16 partial).  Then, over the tile's 128 rows (32x32x16 MFMAs from transposed
// LDS tiles), dk/dv summed in registers over the item's tiles before one atomic flush,
// and the item's sum dsigma q (q^ = (I + U D) q is linear in q) and db'_c = sum dsigma,
// added atomically.
//
// The q and g rows of a wave's 16 rows are gathered as whole rows (16 bytes per lane)
// into registers one tile ahead and written to the wave's rows of the LDS tiles, from
// which both the row operands of S and dP' and the transposed operands of the dk/dv
// products are read.  sum dsigma q runs on the MFMA beside dk: dsigma (split into two
// bf16 terms) sits in columns 64 and 65 of the P w tile's rows (its padding), and a
// 32-column operand read there meets the q tile; only output columns 0 and 1 are used
// (an MFMA output column depends on its own operand column only).
// LDS of the pair kernel: as GradLds, but the q and g rows have a stride of D + 32 (so
// the transposing reads of 4 consecutive rows hit disjoint banks) and their 16-byte
// segments are swizzled by row (segment s of row r at s ^ pseg(r)), so that 16 lanes
// reading one segment of 16 consecutive rows hit disjoint banks too.
template <int D>
struct PairLds {
  static constexpr int LDR = D + 32;
  KVTile<bf16_t, D, 1, 8> kv;
  uint16_t qt[BW_ROWS * LDR];
  uint16_t gt[BW_ROWS * LDR];
  uint16_t pt[BW_ROWS * LDP];
  uint16_t st[BW_ROWS * LDP];  // follows pt: the 32-column read at column 64 of pt's last rows stays inside
};
HILS_DEV constexpr int pseg(int r) { return (r >> 2) & 3; }

// vt_operand on a swizzled q / g tile
template <int LD>
HILS_DEV bf16x8_t vt_operand_sw(const uint16_t* plane, int dt, int ks2, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int e = 32 * dt + 16 * (g & 1) + 4 * (j & 3);
  const int key = 16 * ks2 + 4 * (g >> 1) + (j >> 2);
  auto at = [&](int r) { return plane + r * LD + (((e >> 3) ^ pseg(r)) << 3) + (e & 7); };
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)at(key));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)at(key + 8));
  u32x4_t u;
  u.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  u.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  u.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  u.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

constexpr int BP_WAVES = 8;
constexpr int BP_THREADS = 64 * BP_WAVES;
constexpr int BP_RW = BW_ROWS / BP_WAVES;  // rows per wave in the row products
static_assert(BP_RW == 16, "the row products are 16x16x32 MFMAs");

// K^T as the A operand of dq^T = K^T dS^T (16x16x32): lane l gets head dim 16 dt + (l & 15)
// and keys 32 kk + 4 (l >> 4) + 0..3, then 32 kk + 16 + 4 (l >> 4) + 0..3 -- the keys
// that lane's dS registers hold -- by two transposing reads of the [key][dim] tile.
template <int LDK>
HILS_DEV bf16x8_t kt16_operand(const uint16_t* kplane, int dt, int kk, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int e = 16 * dt + 4 * (j & 3);
  const int k0 = 32 * kk + 4 * g + (j >> 2);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kplane + k0 * LDK + e));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(kplane + (k0 + 16) * LDK + e));
  u32x4_t u;
  u.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  u.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  u.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  u.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

template <int D>
__global__ void __launch_bounds__(BP_THREADS) bwd_pairs(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                        const bf16_t* __restrict__ v, const bf16_t* __restrict__ dO,
                                                        const float* __restrict__ sel_score,
                                                        const float* __restrict__ lam, const float* __restrict__ dd,
                                                        const uint32_t* __restrict__ pairs,
                                                        const uint32_t* __restrict__ boff,
                                                        const uint32_t* __restrict__ toff,
                                                        const uint32_t* __restrict__ imap,
                                                        const float* __restrict__ kdq, float* __restrict__ dsig,
                                                        uint16_t* __restrict__ dqp, float* __restrict__ dk,
                                                        float* __restrict__ dv, float* __restrict__ dkc,
                                                        float* __restrict__ dbc, int Hq, int Hkv, int N, int C, int K,
                                                        int nbk, int Hd) {
  constexpr int LDR = PairLds<D>::LDR;
  constexpr int LDK = KVTile<bf16_t, D, 1, 8>::LDK, LDV = KVTile<bf16_t, D, 1, 8>::LDV;
  constexpr int SEGS = D / 8;       // 16-byte segments of a bf16 row
  constexpr int RPL = 64 / SEGS;    // rows covered by one wave-wide 16-byte load
  constexpr int NLD = BP_RW / RPL;  // loads per lane for the wave's 16 rows
  constexpr int NDT = D / 32;       // 32-dim tiles of the dk / dv blocks
  constexpr int NB = 4 * NDT / BP_WAVES;  // dk / dv blocks per wave
  static_assert(NB >= 1 && NB * BP_WAVES == 4 * NDT, "whole dk / dv blocks per wave");
  static_assert(LDP >= 66, "dsigma terms live in columns 64 and 65 of the P w rows");
  __shared__ PairLds<D> L;
  __shared__ uint32_t ipid[BUCKET_ITEM_ROWS];  // in-head pair index (row * K + slot); 0 past the item
  __shared__ __align__(16) float kdq_s[D];     // the chunk's score direction (I + D^T U^T) k'_c
  const int item = blockIdx.x;
  if ((uint32_t)item >= toff[nbk]) return;
  const int bk = (int)imap[item];
  const uint32_t count = boff[bk + 1] - boff[bk];
  const uint32_t first = ((uint32_t)item - toff[bk]) * BUCKET_ITEM_ROWS;
  const uint32_t nrows = min((uint32_t)BUCKET_ITEM_ROWS, count - first);
  const uint32_t* pp = pairs + boff[bk] + first;
  const int c = bk % C;
  const int64_t bhq = bk / C;  // b * Hq + h
  const int h = (int)(bhq % Hq), b = (int)(bhq / Hq);
  const int kvh = h / (Hq / Hkv);
  const int64_t kvrow0 = ((int64_t)b * Hkv + kvh) * N + (int64_t)c * 64;
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g4 = lane >> 4;
  const float tau = 1.0f / sqrtf((float)D);
  const float cl = tau * 1.44269504088896340736f;
  const int trow = BP_RW * w + j16;  // this lane's row of the tile in the row products
  // every row of a bucket belongs to head bhq: 32-bit offsets from the head's bases
  const char* q_head = reinterpret_cast<const char*>(q + bhq * N * D);
  const char* g_head = reinterpret_cast<const char*>(dO + bhq * N * D);
  const uint32_t e_head = (uint32_t)(bhq * N * K);
  // in-head row = index / K as (index * (floor(2^32 / K) + 1)) >> 32: exact for
  // index < 2^26 and K <= 64 (the multiplier's excess adds less than 2^-6 <= 1/K to
  // index / K, whose fraction is at most 1 - 1/K)
  const uint64_t kmul = 0x100000000ull / (uint32_t)K + 1u;
  auto row_of = [&](uint32_t x) { return (uint32_t)(((uint64_t)x * kmul) >> 32); };
  for (int x = tid; x < BUCKET_ITEM_ROWS; x += BP_THREADS) ipid[x] = (uint32_t)x < nrows ? pp[x] - e_head : 0u;
  // the chunk's score direction: kdq holds Hd heads, one per query head (Q-Cal) or the
  // landmark heads (k' itself)
  if (tid < D) kdq_s[tid] = kdq[(((bhq / Hq) * Hd + h / (Hq / Hd)) * C + c) * D + tid];
  const int ntile = (int)((nrows + BW_ROWS - 1) / BW_ROWS);
  __syncthreads();  // ipid

  // a tile's inputs: the wave's 16 rows of q and g as raw 16-byte row segments, and
  // this lane's row's pair id, score, Lambda and g.o
  const int lr = lane / SEGS, sg = lane % SEGS;
  u32x4_t gq[NLD], gg[NLD];
  uint32_t n_pid;
  float n_sc, n_lam, n_go;
  auto fetch = [&](int j) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const uint32_t off = row_of(ipid[j * BW_ROWS + BP_RW * w + RPL * u + lr]) * (uint32_t)(D * 2) + 16u * sg;
      gq[u] = *reinterpret_cast<const u32x4_t*>(q_head + off);
      gg[u] = *reinterpret_cast<const u32x4_t*>(g_head + off);
    }
    const uint32_t el = ipid[j * BW_ROWS + trow];
    const bool ok = (uint32_t)(j * BW_ROWS + trow) < nrows;
    n_pid = ok ? e_head + el : 0xffffffffu;
    const int64_t row = bhq * N + row_of(el);
    n_sc = ok ? sel_score[n_pid] : 0.f;
    n_lam = lam[row];
    n_go = dd[row];
  };
  if (ntile > 0) fetch(0);
  stage_kv<bf16_t, D, 1>(L.kv, k, v, kvrow0, 64, tid, BP_THREADS);
  f32x16_t dkv[NB];  // this wave's dk / dv blocks, summed over the item's tiles
#pragma unroll
  for (int ib = 0; ib < NB; ++ib) dkv[ib] = zero16();
  f32x16_t kq = zero16();  // sum dsigma q for dim tile kq_dt (waves with kq_wave)
  // two blocks per wave: the dk waves 4..7, each on a dim tile of its own blocks;
  // otherwise the last NDT waves
  const bool kq_wave = NB == 2 ? w >= 4 : w >= BP_WAVES - NDT;
  const int kq_dt = NB == 2 ? 2 * (w & 1) + ((w >> 1) & 1) : w - (BP_WAVES - NDT);
  float bacc = 0.f;  // sum dsigma over this lane's rows
  for (int j = 0; j < ntile; ++j) {
    __syncthreads();  // K/V staged (first tile); the previous tile's LDS tiles consumed
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int r = BP_RW * w + RPL * u + lr;
      *reinterpret_cast<u32x4_t*>(&L.qt[r * LDR + 8 * (sg ^ pseg(r))]) = gq[u];
      *reinterpret_cast<u32x4_t*>(&L.gt[r * LDR + 8 * (sg ^ pseg(r))]) = gg[u];
    }
    const uint32_t pid = n_pid;
    const bool ok = pid != 0xffffffffu;
    const float sc = n_sc, Lam = n_lam, go = n_go;
    if (j + 1 < ntile) fetch(j + 1);  // the next tile's rows load during this whole tile
    __builtin_amdgcn_wave_barrier();  // the wave's rows are in LDS
    // S^T and dP'^T in four 16-key tiles: register i of tile t holds key 16 t + 4 g4 + i
    // of row trow
    f32x4_t s[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = dp[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int so = 8 * ((4 * ks + g4) ^ pseg(trow));
      const bf16x8_t bq = lds_op16(&L.qt[trow * LDR + so]);
      const bf16x8_t bg = lds_op16(&L.gt[trow * LDR + so]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s[t] = mfma16(lds_op16(&L.kv.k[0][(16 * t + j16) * LDK + 32 * ks + 8 * g4]), bq, s[t]);
        dp[t] = mfma16(lds_op16(&L.kv.v[0][(16 * t + j16) * LDV + 32 * ks + 8 * g4]), bg, dp[t]);
      }
    }
    // the row's softmax over its 64 keys: 16 in each of the lanes j16 + 16 g4
    float mt = s[0][0];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[t][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    float lt = 0.f, e = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[t][i] = __builtin_amdgcn_exp2f((s[t][i] - mt) * cl);
        lt += s[t][i];
        e = fmaf(s[t][i], dp[t][i], e);
      }
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    e += __shfl_xor(e, 16);
    e += __shfl_xor(e, 32);
    const float inv = __builtin_amdgcn_rcpf(lt);  // lt >= 1 (the largest logit's term)
    e *= inv;
    const float wc = ok ? __expf(sc - Lam) : 0.f;
    const float dsg = wc * (e - go);
    const float pw = inv * wc;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = s[t][i] * pw;
        s[t][i] = p;                      // P w
        dp[t][i] = p * (dp[t][i] - e);    // dS
      }
    // P w and dS rows (bf16) for the dk/dv products; dsigma's two terms in columns 64, 65
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      *reinterpret_cast<u32x2_t*>(&L.pt[trow * LDP + 16 * t + 4 * g4]) =
          u32x2_t{pack_bf16x2(s[t][0], s[t][1]), pack_bf16x2(s[t][2], s[t][3])};
      *reinterpret_cast<u32x2_t*>(&L.st[trow * LDP + 16 * t + 4 * g4]) =
          u32x2_t{pack_bf16x2(dp[t][0], dp[t][1]), pack_bf16x2(dp[t][2], dp[t][3])};
    }
    if (g4 == 0) {
      const uint16_t s_hi = f32_to_bf16(dsg);
      const uint16_t s_lo = f32_to_bf16(dsg - bf16_to_f32(s_hi));
      *reinterpret_cast<uint32_t*>(&L.pt[trow * LDP + 64]) = (uint32_t)s_hi | ((uint32_t)s_lo << 16);
      bacc += dsg;
      if (ok) dsig[pid] = dsg;
    }
    // the pair's dq: dq^T = K^T dS^T, 16 dims at a time (register i of tile dt holds dim
    // 16 dt + 4 g4 + i of row trow), plus the score term dsigma (I + D^T U^T) k'_c, times
    // tau, stored as a bf16 partial (bwd_dq_sum adds a row's)
    bf16x8_t db[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4_t u;
      u.x = pack_bf16x2(dp[2 * kk][0], dp[2 * kk][1]);
      u.y = pack_bf16x2(dp[2 * kk][2], dp[2 * kk][3]);
      u.z = pack_bf16x2(dp[2 * kk + 1][0], dp[2 * kk + 1][1]);
      u.w = pack_bf16x2(dp[2 * kk + 1][2], dp[2 * kk + 1][3]);
      db[kk] = __builtin_bit_cast(bf16x8_t, u);
    }
    uint16_t* dst = dqp + (int64_t)(ok ? pid : 0u) * D + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) a = mfma16(kt16_operand<LDK>(L.kv.k[0], dt, kk, lane), db[kk], a);
      if (ok) {
        const f32x4_t kd = *reinterpret_cast<const f32x4_t*>(&kdq_s[16 * dt + 4 * g4]);
        *reinterpret_cast<u32x2_t*>(dst + 16 * dt) =
            u32x2_t{pack_bf16x2(tau * fmaf(dsg, kd[0], a[0]), tau * fmaf(dsg, kd[1], a[1])),
                    pack_bf16x2(tau * fmaf(dsg, kd[2], a[2]), tau * fmaf(dsg, kd[3], a[3]))};
      }
    }
    __syncthreads();  // all eight waves' rows of the P w, dS, q and g tiles are written
    // dk / dv blocks over the tile's 128 rows, and sum dsigma q for one 32-dim tile.  With
    // two blocks per wave (D = 128) a wave owns one kind and key tile and two dim tiles, so
    // their P w / dS operand is read once, and the dk waves' sum dsigma q reuses one of
    // their q operands.
    if constexpr (NB == 2) {
      const bool isk = w >= 4;
      const int kt = (w >> 1) & 1, dt0 = 2 * (w & 1);
      const uint16_t* at = isk ? L.st : L.pt;
      const uint16_t* bt = isk ? L.qt : L.gt;
#pragma unroll 2
      for (int ks2 = 0; ks2 < BW_ROWS / 16; ++ks2) {
        const bf16x8_t a = vt_operand<LDP>(at, kt, ks2, lane);
        const bf16x8_t b0 = vt_operand_sw<LDR>(bt, dt0, ks2, lane);
        const bf16x8_t b1 = vt_operand_sw<LDR>(bt, dt0 + 1, ks2, lane);
        dkv[0] = mfma32(a, b0, dkv[0]);
        dkv[1] = mfma32(a, b1, dkv[1]);
        if (isk) kq = mfma32(kt ? b1 : b0, vt_operand<LDP>(L.pt, 2, ks2, lane), kq);
      }
    } else {
#pragma unroll 2
      for (int ks2 = 0; ks2 < BW_ROWS / 16; ++ks2) {
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) {
          const int blk = w + BP_WAVES * ib;
          const bool isk = blk >= 2 * NDT;
          const int kt = (blk % (2 * NDT)) / NDT, dt = blk % NDT;
          dkv[ib] = mfma32(vt_operand<LDP>(isk ? L.st : L.pt, kt, ks2, lane),
                           vt_operand_sw<LDR>(isk ? L.qt : L.gt, dt, ks2, lane), dkv[ib]);
        }
        if (kq_wave)
          kq = mfma32(vt_operand_sw<LDR>(L.qt, kq_dt, ks2, lane), vt_operand<LDP>(L.pt, 2, ks2, lane), kq);
      }
    }
  }
  // flush: register rr of block (kt, dt) holds key 32 kt + acc_row(rr, hf), dim 32 dt + (lane & 31)
#pragma unroll
  for (int ib = 0; ib < NB; ++ib) {
    const int blk = w + BP_WAVES * ib;
    const bool isk = NB == 2 ? w >= 4 : blk >= 2 * NDT;
    const int kt = NB == 2 ? (w >> 1) & 1 : (blk % (2 * NDT)) / NDT;
    const int dt = NB == 2 ? 2 * (w & 1) + ib : blk % NDT;
    float* dst = isk ? dk : dv;
    const float scl = isk ? tau : 1.0f;
    const int e = 32 * dt + (lane & 31);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      atomicAdd(&dst[(kvrow0 + 32 * kt + acc_row(rr, hf)) * D + e], dkv[ib][rr] * scl);
  }
  const int64_t ci = bhq * C + c;  // the chunk sums are kept per query head
  if (kq_wave) {
    // column 0 (lanes 0, 32) holds the high terms' sums, column 1 (lanes 1, 33) the low
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float lo2 = __shfl_down(kq[rr], 1);
      if ((lane & 31) == 0) atomicAdd(&dkc[ci * D + 32 * kq_dt + acc_row(rr, hf)], kq[rr] + lo2);
    }
  }
  bacc = wave_sum_f(bacc);  // lanes g4 != 0 hold 0
  if (lane == 0) atomicAdd(&dbc[ci], bacc);
}

// ------------------------------------------------------------------ bwd_dq_sum
// Per row (one wave): the output dq (bf16) = the window's dq (fp32) + the selected chunks'
// dq partials (bf16; each already holds the pair's score term tau dsigma (I + D^T U^T)
// k'_c).  The row's number of selections comes from one ballot.  A slot row is read by
// D/8 lanes with 16-byte loads, 64/(D/8) slots per wave-wide load, every load of the row
// at once; the lanes' sums over their slots are then added across the slot groups.  This
// is the last step of dq, so the sum is rounded straight into the output.
template <int D, int KMAX>
__global__ void __launch_bounds__(256) bwd_dq_sum(const int32_t* __restrict__ sel, const uint16_t* __restrict__ dqp,
                                                  const float* __restrict__ dq, bf16_t* __restrict__ out, int K,
                                                  int64_t rows) {
  constexpr int LPS = D / 8;                        // lanes per slot row (8 dims each)
  constexpr int SPL = 64 / LPS;                     // slot rows per wave-wide load
  constexpr int NSEG = (KMAX + SPL - 1) / SPL;      // loads per lane
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sl = lane / LPS, dp = (lane % LPS) * 8;
  for (int64_t row = (int64_t)blockIdx.x * 4 + w; row < rows; row += (int64_t)gridDim.x * 4) {
    const int32_t sv = lane < K ? sel[row * K + lane] : -1;
    const int n = __popcll(__ballot(sv >= 0));  // valid selections come first
    const uint16_t* pr = dqp + row * K * D + dp;
    // slots t = SPL g + sl; those past n read slot 0 (in bounds) and are dropped
    u32x4_t pv[NSEG];
#pragma unroll
    for (int g = 0; g < NSEG; ++g) {
      const int t = SPL * g + sl;
      pv[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pr + (int64_t)(t < n ? t : 0) * D));
    }
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = 0.f;
#pragma unroll
    for (int g = 0; g < NSEG; ++g) {
      if (SPL * g + sl < n) {
        const uint32_t wd[4] = {pv[g].x, pv[g].y, pv[g].z, pv[g].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[2 * m] += __uint_as_float(wd[m] << 16);
          acc[2 * m + 1] += __uint_as_float(wd[m] & 0xffff0000u);
        }
      }
    }
#pragma unroll
    for (int o = LPS; o < 64; o <<= 1)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] += __shfl_xor(acc[m], o);
    if (lane < LPS) {
      const float4 d0 = *reinterpret_cast<const float4*>(dq + row * D + dp);
      const float4 d1 = *reinterpret_cast<const float4*>(dq + row * D + dp + 4);
      u32x4_t pk;
      pk.x = pack_bf16x2(d0.x + acc[0], d0.y + acc[1]);
      pk.y = pack_bf16x2(d0.z + acc[2], d0.w + acc[3]);
      pk.z = pack_bf16x2(d1.x + acc[4], d1.y + acc[5]);
      pk.w = pack_bf16x2(d1.z + acc[6], d1.w + acc[7]);
      *reinterpret_cast<u32x4_t*>(out + row * D + dp) = pk;
    }
  }
}

// -------------------------------------------------------------------- Q-Cal
// The scores' query gradient dq^_i = tau sum_x dsigma_ix k'_(c_x) enters dq through
// (I + D^T U^T), and the weight gradients through G_h = sum_i dq^_i q_i^T.  Both are
// linear in the per-chunk quantities, so neither needs dq^ per row:
//   dq_i gets tau dsigma_ic (k'_c + D^T U^T k'_c) with each selected pair (bwd_pairs adds
//     it to the pair's partial; bwd_kdq forms k'_c + D^T (U^T k'_c) per chunk), and
//   G_h = tau sum_(b,c) k'_(b,h,c) S_(b,h,c)^T with S_c = sum over the chunk's pairs of
//     dsigma q, the sums bwd_pairs leaves for the compression backward (bwd_qcal_g).
// dU = G D^T and dD = U^T G follow per head (bwd_qcal_weights).
constexpr int KDQ_CHUNKS = 8;  // chunks per bwd_kdq workgroup

template <int D>
__global__ void __launch_bounds__(256) bwd_kdq(const float* __restrict__ kc, const bf16_t* __restrict__ Dw,
                                               const bf16_t* __restrict__ Uw, float* __restrict__ kdq, int Hq,
                                               int Hl, int C, int r) {
  __shared__ float kr[D], t[32];
  const int nblk = (C + KDQ_CHUNKS - 1) / KDQ_CHUNKS;
  const int64_t bh = blockIdx.x / nblk;  // b * Hq + h
  const int h = (int)(bh % Hq);
  const int64_t lb = bh / Hq * Hl + h / (Hq / Hl);  // b * Hl + the landmark head of h
  const int c0 = (int)(blockIdx.x % nblk) * KDQ_CHUNKS;
  const int tid = threadIdx.x;
  for (int c = c0; c < min(C, c0 + KDQ_CHUNKS); ++c) {
    const int64_t row = (bh * C + c) * D;
    __syncthreads();  // the previous chunk's kr / t consumed
    if (tid < D) kr[tid] = kc[(lb * C + c) * D + tid];
    __syncthreads();
    if (tid < r) {  // t = U_h^T k'_c
      float acc = 0.f;
      for (int e = 0; e < D; ++e) acc = fmaf(bf16_to_f32(Uw[((int64_t)h * D + e) * r + tid].bits), kr[e], acc);
      t[tid] = acc;
    }
    __syncthreads();
    if (tid < D) {  // k'_c + D_h^T t
      float acc = kr[tid];
      for (int a = 0; a < r; ++a) acc = fmaf(bf16_to_f32(Dw[((int64_t)h * r + a) * D + tid].bits), t[a], acc);
      kdq[row + tid] = acc;
    }
  }
}

// G_h[a][e] = tau sum over (b, c) of k'[b,h,c][a] S[b,h,c][e]; one workgroup per head and
// 16 rows a, one thread per (e, group of rows).
template <int D>
__global__ void __launch_bounds__(256) bwd_qcal_g(const float* __restrict__ kc, const float* __restrict__ S,
                                                  float* __restrict__ G, int B, int Hq, int Hl, int C) {
  constexpr int ARB = 16;               // rows a per workgroup
  constexpr int TPE = 256 / D;          // threads per column e
  constexpr int APT = ARB / TPE;        // rows per thread
  const int h = blockIdx.x / (D / ARB), a0 = (blockIdx.x % (D / ARB)) * ARB;
  const int e = threadIdx.x % D, ag = threadIdx.x / D;
  float acc[APT];
#pragma unroll
  for (int m = 0; m < APT; ++m) acc[m] = 0.f;
  for (int b = 0; b < B; ++b) {
    const int64_t base = ((int64_t)b * Hq + h) * C * D;                   // S: per query head
    const int64_t kbase = ((int64_t)b * Hl + h / (Hq / Hl)) * C * D;     // k': its landmark head
    for (int c = 0; c < C; ++c) {
      const float sv = S[base + (int64_t)c * D + e];
      const float* kr = kc + kbase + (int64_t)c * D + a0 + ag * APT;
#pragma unroll
      for (int m = 0; m < APT; ++m) acc[m] = fmaf(kr[m], sv, acc[m]);
    }
  }
  const float tau = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int m = 0; m < APT; ++m) G[((int64_t)h * D + a0 + ag * APT + m) * D + e] = tau * acc[m];
}

// dU_h = G_h D_h^T and dD_h = U_h^T G_h (bf16 out), one workgroup per head.
template <int D>
__global__ void __launch_bounds__(256) bwd_qcal_weights(const float* __restrict__ G, const bf16_t* __restrict__ Dw,
                                                        const bf16_t* __restrict__ Uw, bf16_t* __restrict__ dD,
                                                        bf16_t* __restrict__ dU, int r) {
  const int h = blockIdx.x;
  const float* Gh = G + (int64_t)h * D * D;
  for (int x = threadIdx.x; x < D * r; x += 256) {
    const int e = x / r, a = x % r;  // dU [e][a] = sum_f G[e][f] D[a][f]
    float acc = 0.f;
    for (int f = 0; f < D; ++f) acc = fmaf(Gh[e * D + f], bf16_to_f32(Dw[((int64_t)h * r + a) * D + f].bits), acc);
    dU[((int64_t)h * D + e) * r + a].bits = f32_to_bf16(acc);
  }
  for (int x = threadIdx.x; x < r * D; x += 256) {
    const int a = x / D, f = x % D;  // dD [a][f] = sum_e U[e][a] G[e][f]
    float acc = 0.f;
    for (int e = 0; e < D; ++e) acc = fmaf(bf16_to_f32(Uw[((int64_t)h * D + e) * r + a].bits), Gh[e * D + f], acc);
    dD[((int64_t)h * r + a) * D + f].bits = f32_to_bf16(acc);
  }
}

// ---------------------------------------------------------------- bwd_compress
// One workgroup per (b, KV head, chunk), looping over the landmark heads of the KV head:
// recompute the compression weights a, then dz, the landmark query's gradient (written
// out) and the keys' gradient, summed in LDS and added to the keys' accumulator (each
// chunk's keys belong to this workgroup alone).
template <int D>
__global__ void __launch_bounds__(256) bwd_compress(const bf16_t* __restrict__ k, const bf16_t* __restrict__ lmk,
                                                    const float* __restrict__ dkc, const float* __restrict__ dbc,
                                                    const bf16_t* __restrict__ Dw, const bf16_t* __restrict__ Uw,
                                                    float* __restrict__ dk, bf16_t* __restrict__ dlmk, int Hq, int Hl,
                                                    int Hkv, int N, int C, int r) {
  __shared__ float ks[64][D + 1];
  __shared__ float acc[64][D + 1];
  __shared__ float Ls[D], gk[D], gs[D], tr[32];
  __shared__ float zs[64], as[64], das[64];
  const int c = blockIdx.x % C, bkv = blockIdx.x / C;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t kb = ((int64_t)b * Hkv + kvh) * N + (int64_t)c * 64;
  const float tau = 1.0f / sqrtf((float)D);
  for (int x = tid * 8; x < 64 * D; x += 256 * 8) {  // 16-byte loads: the chunk's rows are consecutive
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(k + kb * D + x);
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      ks[x / D][x % D + 2 * m] = __uint_as_float(wd[m] << 16);
      ks[x / D][x % D + 2 * m + 1] = __uint_as_float(wd[m] & 0xffff0000u);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[x / D][x % D + m] = 0.f;
  }
  const int lpk = Hl / Hkv, gq = Hq / Hl;
  for (int li = 0; li < lpk; ++li) {
    const int l = kvh * lpk + li;
    const int64_t ci = ((int64_t)b * Hl + l) * C + c;
    __syncthreads();
    for (int e = tid; e < D; e += 256) {
      Ls[e] = bf16_to_f32(lmk[ci * D + e].bits);
      gs[e] = 0.f;
    }
    // dk'_c = sum over the query heads h of landmark head l of tau (I + U_h D_h) S_hc, with
    // S_hc the sum over head h's pairs with chunk c of dsigma q (the scores use
    // q^ = q + U_h (D_h q)); db'_c = the sum of those pairs' dsigma
    float gb = 0.f;
    for (int hi = 0; hi < gq; ++hi) {
      const int hq = l * gq + hi;
      const int64_t qi = ((int64_t)b * Hq + hq) * C + c;
      __syncthreads();  // the previous head's gk consumed
      for (int e = tid; e < D; e += 256) gk[e] = dkc[qi * D + e];
      gb += dbc[qi];
      __syncthreads();
      if (r > 0) {
        {  // t = D_h gk: eight threads per rank index a, each over D / 8 dims
          const int a = tid >> 3, part = tid & 7;
          float t = 0.f;
          if (a < r)
            for (int e = part; e < D; e += 8) t = fmaf(bf16_to_f32(Dw[((int64_t)hq * r + a) * D + e].bits), gk[e], t);
          t += __shfl_xor(t, 1);
          t += __shfl_xor(t, 2);
          t += __shfl_xor(t, 4);
          if (a < r && part == 0) tr[a] = t;
        }
        __syncthreads();
        {  // gk += U_h t: 256 / D threads per dim, each over a share of the rank
          constexpr int TPE = 256 / D;
          const int e = tid / TPE, part = tid % TPE;
          float acc2 = 0.f;
          for (int a2 = part; a2 < r; a2 += TPE) acc2 = fmaf(bf16_to_f32(Uw[((int64_t)hq * D + e) * r + a2].bits), tr[a2], acc2);
          for (int o = 1; o < TPE; o <<= 1) acc2 += __shfl_xor(acc2, o);
          __syncthreads();  // every thread has read gk (in t) before it is rewritten
          if (part == 0) gk[e] = (gk[e] + acc2) * tau;
        }
      } else {
        for (int e = tid; e < D; e += 256) gk[e] *= tau;
      }
      __syncthreads();
      for (int e = tid; e < D; e += 256) gs[e] += gk[e];
    }
    __syncthreads();
    // z_j and dk'.k_j, four threads per key
    {
      const int j = tid >> 2, part = tid & 3;
      float zz = 0.f, gg = 0.f;
      for (int e = part; e < D; e += 4) {
        zz = fmaf(Ls[e], ks[j][e], zz);
        gg = fmaf(gs[e], ks[j][e], gg);
      }
      zz += __shfl_xor(zz, 1);
      zz += __shfl_xor(zz, 2);
      gg += __shfl_xor(gg, 1);
      gg += __shfl_xor(gg, 2);
      if (part == 0) {
        zs[j] = zz * tau;
        das[j] = gg;
      }
    }
    __syncthreads();
    if (w == 0) {
      const float zz = zs[lane];
      float mx = zz;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float ex = __expf(zz - mx);
      const float a = ex / wave_sum_f(ex);
      const float da = das[lane] - (a > 0.f ? gb * (logf(a) + 1.0f) : 0.f);
      const float sda = wave_sum_f(a * da);
      as[lane] = a;
      das[lane] = a * (da - sda);  // dz_j
    }
    __syncthreads();
    for (int e = tid; e < D; e += 256) {
      float s = 0.f;
      for (int j = 0; j < 64; ++j) s = fmaf(das[j], ks[j][e], s);
      dlmk[ci * D + e].bits = f32_to_bf16(s * tau);
    }
    for (int x = tid; x < 64 * D; x += 256) {
      const int j = x / D, e = x % D;
      acc[j][e] += as[j] * gs[e] + tau * das[j] * Ls[e];
    }
  }
  __syncthreads();
  for (int x = tid * 4; x < 64 * D; x += 256 * 4) {
    float4 d4 = *reinterpret_cast<const float4*>(dk + kb * D + x);
    d4.x += acc[x / D][x % D];
    d4.y += acc[x / D][x % D + 1];
    d4.z += acc[x / D][x % D + 2];
    d4.w += acc[x / D][x % D + 3];
    *reinterpret_cast<float4*>(dk + kb * D + x) = d4;
  }
}

__global__ void __launch_bounds__(256) bwd_convert(const float* __restrict__ src, bf16_t* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i].bits = f32_to_bf16(src[i]);
}

unsigned grid_for(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536)); }

template <int D>
hipError_t launch_bwd_d(const Geom& g, const BwdArgs& a, char* ws, hipStream_t st) {
  const BwdWs w = bwd_ws(g);
  float* dq = (float*)(ws + w.dq);
  float* dk = (float*)(ws + w.dk);
  float* dv = (float*)(ws + w.dv);
  float* dkc = (float*)(ws + w.dkc);
  float* dbc = (float*)(ws + w.dbc);
  float* G = (float*)(ws + w.G);
  float* lam = (float*)(ws + w.lam);
  float* dd = (float*)(ws + w.dd);
  float* dsig = (float*)(ws + w.dsig);
  const int C = g.C();
  const int64_t rows = (int64_t)g.B * g.Hq * g.N;
  const bf16_t *q = (const bf16_t*)a.q, *k = (const bf16_t*)a.k, *v = (const bf16_t*)a.v;
  const bf16_t *Dw = (const bf16_t*)a.D, *Uw = (const bf16_t*)a.U;
  // the accumulators dk .. dU are contiguous
  const int64_t nz = (int64_t)(w.lam - w.dk) / 4;
  hipLaunchKernelGGL(bwd_zero, dim3(grid_for(nz)), dim3(256), 0, st, dk, nz);
  // the chunks' score directions: k' itself, or k' + D^T U^T k' under Q-Cal
  const float* kdq = a.kc;
  if (g.r > 0 && C > 0) {
    kdq = (const float*)(ws + w.kdq);
    hipLaunchKernelGGL((bwd_kdq<D>), dim3(g.B * g.Hq * ((C + KDQ_CHUNKS - 1) / KDQ_CHUNKS)), dim3(256), 0, st, a.kc,
                       Dw, Uw, (float*)(ws + w.kdq), g.Hq, g.Hl, C, g.r);
  }
  const int NQC = (g.N + 63) / 64;
  const int ngb = (g.G() + 1) / 2;
  hipLaunchKernelGGL((bwd_window<D>), dim3(g.B * g.Hkv * NQC * ngb), dim3(256), 0, st, q, k, v, (const bf16_t*)a.o,
                     (const bf16_t*)a.dO, a.sel_score, dq, dk, dv, lam, dd, g.Hq, g.Hkv, g.N, C, g.K, NQC, g.nw);
  const int nbk = g.B * g.Hq * C;
  const int64_t items = bucket_items_bound(g);
  if (nbk > 0 && items > 0) {
    uint32_t* boff = (uint32_t*)(ws + w.boff);
    uint32_t* toff = (uint32_t*)(ws + w.toff);
    uint32_t* pairs = (uint32_t*)(ws + w.pairs);
    launch_bucket_pairs(g, a.sel_idx,
                        BucketBufs{(uint32_t*)(ws + w.counts), (uint32_t*)(ws + w.cursor), boff, toff, pairs,
                                   (uint32_t*)(ws + w.tmp), (uint32_t*)(ws + w.imap)},
                        st);
    hipLaunchKernelGGL((bwd_pairs<D>), dim3((unsigned)items), dim3(BP_THREADS), 0, st, q, k, v, (const bf16_t*)a.dO,
                       a.sel_score, (const float*)lam, (const float*)dd, (const uint32_t*)pairs,
                       (const uint32_t*)boff, (const uint32_t*)toff, (const uint32_t*)(ws + w.imap), kdq, dsig,
                       (uint16_t*)(ws + w.dqp), dk, dv, dkc, dbc,
                       g.Hq, g.Hkv, g.N, C, g.K, nbk, g.r > 0 ? g.Hq : g.Hl);
  }
  {
    const dim3 grid((unsigned)std::min<int64_t>((rows + 3) / 4, 1 << 20));
    const uint16_t* dqp = (const uint16_t*)(ws + w.dqp);
    if (g.K <= 8)
      hipLaunchKernelGGL((bwd_dq_sum<D, 8>), grid, dim3(256), 0, st, a.sel_idx, dqp, (const float*)dq,
                         (bf16_t*)a.dq, g.K, rows);
    else if (g.K <= 16)
      hipLaunchKernelGGL((bwd_dq_sum<D, 16>), grid, dim3(256), 0, st, a.sel_idx, dqp, (const float*)dq,
                         (bf16_t*)a.dq, g.K, rows);
    else if (g.K <= 32)
      hipLaunchKernelGGL((bwd_dq_sum<D, 32>), grid, dim3(256), 0, st, a.sel_idx, dqp, (const float*)dq,
                         (bf16_t*)a.dq, g.K, rows);
    else
      hipLaunchKernelGGL((bwd_dq_sum<D, 64>), grid, dim3(256), 0, st, a.sel_idx, dqp, (const float*)dq,
                         (bf16_t*)a.dq, g.K, rows);
  }
  if (g.r > 0) {
    hipLaunchKernelGGL((bwd_qcal_g<D>), dim3(g.Hq * (D / 16)), dim3(256), 0, st, a.kc, (const float*)dkc, G, g.B,
                       g.Hq, g.Hl, C);
    hipLaunchKernelGGL((bwd_qcal_weights<D>), dim3(g.Hq), dim3(256), 0, st, (const float*)G, Dw, Uw, (bf16_t*)a.dD,
                       (bf16_t*)a.dU, g.r);
  }
  if (C > 0)
    hipLaunchKernelGGL((bwd_compress<D>), dim3(g.B * g.Hkv * C), dim3(256), 0, st, k, (const bf16_t*)a.lmk,
                       (const float*)dkc, (const float*)dbc, Dw, Uw, dk, (bf16_t*)a.dlmk, g.Hq, g.Hl, g.Hkv, g.N, C,
                       g.r);
  const int64_t kvn = (int64_t)g.B * g.Hkv * g.N * D;
  hipLaunchKernelGGL(bwd_convert, dim3(grid_for(kvn)), dim3(256), 0, st, (const float*)dk, (bf16_t*)a.dk, kvn);
  hipLaunchKernelGGL(bwd_convert, dim3(grid_for(kvn)), dim3(256), 0, st, (const float*)dv, (bf16_t*)a.dv, kvn);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(const Geom& g) { return bwd_ws(g).total; }

hipError_t launch_backward(const Geom& g, const BwdArgs& a, void* ws, size_t ws_bytes, hipStream_t st) {
  if (ws_bytes < backward_workspace_bytes(g)) return hipErrorInvalidValue;
  if (g.io != 1) return hipErrorNotSupported;
  return g.d == 64 ? launch_bwd_d<64>(g, a, (char*)ws, st) : launch_bwd_d<128>(g, a, (char*)ws, st);
}

}  // namespace hils

// Chunk scoring and streaming top-K for prefill queries.
//
//   s_ic = q^_i . k'_c / sqrt(d) + b'_c   for every complete past chunk c < floor(i/S)
//   q^_i = q_i + U_h (D_h q_i)             (Q-Cal; q^ = q without it)
// keep the K best (ties -> lower chunk id).  (aitrends.kr article,
// "Methodology": the score formula, the calculation flow and the Q-Cal module.)
//
// Design (gfx950):
//   * One workgroup = 128 consecutive queries of one (batch, head); wave w owns 32
//     of them as the M dimension of v_mfma_f32_32x32x16_bf16 and the chunks are the
//     N dimension, so accumulator register r of a lane holds one chunk's score for
//     a query row, and the 32 lanes of each half-wave cover 32 chunks of one row.
//   * k' tiles of 64 chunks are staged through LDS (double-buffered, the next tile
//     prefetched into registers while the current one is on the MFMA) and shared
//     by the four waves.  k' (fp32) is split into bf16 terms (hi + lo, or three
//     terms for fp32 I/O) and q^ likewise, so the bf16 MFMA reproduces the fp32
//     dot product to ~2^-17 relative: index parity needs score errors far below
//     1e-4, which a single bf16 rounding of k' does not give.
//   * Q-Cal runs on the same MFMA (T = D q, then U T), chained through the
//     accumulator layout without any cross-lane movement.
//   * Chunk order: each block scans its past chunks in descending order of b'
//     (the query-independent part of the score), from a per-head sort, so that
//     the running K-th best rises early and few later chunks still qualify.
//     k' is split into bf16 planes once per call, so staging a tile is a copy.
//   * Top-K: every row keeps its exact running top K sorted across the 32 lanes
//     of its half-wave (lane j = j-th best) in registers, plus an unsorted
//     32-slot candidate buffer.  New scores are tested against the row's K-th
//     best with one compare; passing ones are appended to the buffer with one
//     lane permute; a full buffer is bitonic-sorted and merged into the list
//     (DPP and swizzle lane exchanges, no LDS traffic).
#include <algorithm>

#include "hils_common.h"
#include "kernels.h"

namespace hils {

constexpr int ST_ROWS = 128;   // queries per workgroup
constexpr int ST_TILE = 64;    // chunks per LDS tile
constexpr int ST_BUF = 31;     // candidate buffer slots per row (slot 31 is a sink)

HILS_DEV bool better(float s1, int c1, float s2, int c2) { return s1 > s2 || (s1 == s2 && c1 < c2); }

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

// compare-exchange with lane j ^ X; keep the better of the pair if kb, else the worse
template <int X>
HILS_DEV void cx(float& s, int& c, int j, bool kb) {
  const float ps = __int_as_float(xlane<X>(__float_as_int(s), j));
  const int pc = xlane<X>(c, j);
  const bool take = kb ? better(ps, pc, s, c) : better(s, c, ps, pc);
  s = take ? ps : s;
  c = take ? pc : c;
}

// bitonic sort of one (score, chunk) per lane, best first, within each 32-lane half
HILS_DEV void sort32(float& s, int& c, int j) {
#define HILS_STAGE(K_, X_) cx<X_>(s, c, j, ((j & X_) == 0) == (((j & K_) == 0) || K_ == 32));
  HILS_STAGE(2, 1)
  HILS_STAGE(4, 2) HILS_STAGE(4, 1)
  HILS_STAGE(8, 4) HILS_STAGE(8, 2) HILS_STAGE(8, 1)
  HILS_STAGE(16, 8) HILS_STAGE(16, 4) HILS_STAGE(16, 2) HILS_STAGE(16, 1)
  HILS_STAGE(32, 16) HILS_STAGE(32, 8) HILS_STAGE(32, 4) HILS_STAGE(32, 2) HILS_STAGE(32, 1)
#undef HILS_STAGE
}

// merge the unsorted (ns, nc) into the sorted list (ls, li) of each half; keep the best K
HILS_DEV void merge_into(float& ls, int& li, float ns, int nc, int j, int K) {
  sort32(ns, nc, j);
  const float rs = __int_as_float(xlane<31>(__float_as_int(ns), j));  // lane j: the (31-j)-th best new one
  const int rc = xlane<31>(nc, j);
  if (better(rs, rc, ls, li)) {
    ls = rs;
    li = rc;
  }
  // the 32 kept entries form a bitonic sequence: half-cleaners sort it best-first
  cx<16>(ls, li, j, (j & 16) == 0);
  cx<8>(ls, li, j, (j & 8) == 0);
  cx<4>(ls, li, j, (j & 4) == 0);
  cx<2>(ls, li, j, (j & 2) == 0);
  cx<1>(ls, li, j, (j & 1) == 0);
  if (j >= K) {
    ls = -INFINITY;
    li = 0x7fffffff;
  }
}

HILS_DEV float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// the K-th best (score, chunk) of each half's list, broadcast to its lanes
HILS_DEV void kth(float ls, int li, int hf, int K, float& ts, int& ti) {
  const float t0 = readlane_f(ls, K - 1), t1 = readlane_f(ls, 32 + K - 1);
  const int i0 = __builtin_amdgcn_readlane(li, K - 1), i1 = __builtin_amdgcn_readlane(li, 32 + K - 1);
  ts = hf ? t1 : t0;
  ti = hf ? i1 : i0;
}

// append this lane's candidate (if `pass`) to its half's buffer; mk = ballot(pass);
// f0 / f1: filled slots of the two halves (wave-uniform)
HILS_DEV void append(float& bs, int& bi, int& f0, int& f1, float s, int c, bool pass, uint64_t mk, int j, int hf) {
  const uint32_t lo = (uint32_t)mk, hi = (uint32_t)(mk >> 32);
  const int m0 = __popc(lo), m1 = __popc(hi);
  const int fl = hf ? f1 : f0, mown = hf ? m1 : m0;
  const int rank = hf ? (int)__builtin_amdgcn_mbcnt_hi(hi, 0u) : (int)__builtin_amdgcn_mbcnt_lo(lo, 0u);
  const int dst = 32 * hf + (pass ? fl + rank : ST_BUF);
  const int rs = __builtin_amdgcn_ds_permute(dst * 4, __float_as_int(s));
  const int rc = __builtin_amdgcn_ds_permute(dst * 4, c);
  const bool neu = j >= fl && j < fl + mown;
  bs = neu ? __int_as_float(rs) : bs;
  bi = neu ? rc : bi;
  f0 += m0;
  f1 += m1;
}

// merge the buffer into the list and empty it; refresh the K-th best
HILS_DEV void flush(float& ls, int& li, float& bs, int& bi, int& f0, int& f1, float& ts, int& ti, int j, int hf,
                    int K) {
  const bool v = j < (hf ? f1 : f0);
  merge_into(ls, li, v ? bs : -INFINITY, v ? bi : 0x7fffffff, j, K);
  f0 = f1 = 0;
  kth(ls, li, hf, K, ts, ti);
}

template <typename IO, int D, int NQ, int NK, bool QCAL>
__global__ void __launch_bounds__(256, 2) score_topk_kernel(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                             const IO* __restrict__ Uw,
                                                             const uint16_t* __restrict__ planes,
                                                             const float* __restrict__ bc,
                                                             const int32_t* __restrict__ order,
                                                             int32_t* __restrict__ sel_idx,
                                                             float* __restrict__ sel_score, int H, int N, int C, int K,
                                                             int r, int NB, int items) {
  constexpr int LDK = D + 4;            // padded bf16 row stride of the k' tile planes
  constexpr int NKS = D / 16;           // MFMA k-steps over the head dimension
  constexpr int NIO = io_traits<IO>::terms;
  constexpr int SEGS = D / 8;           // 16-byte segments of a plane row
  constexpr int PH = ST_TILE / 2 * NK * SEGS / 256;  // 16-byte prefetch loads per thread per half tile
  __shared__ uint16_t kt[NK][ST_TILE * LDK];   // the current tile; its two halves are refilled in turn
  __shared__ float bt[ST_TILE];
  __shared__ int ct[ST_TILE];
  __shared__ int wsum[4];
  __shared__ float lsl[4][16][64];              // per-row sorted lists (see below)
  __shared__ int lil[4][16][64];
  extern __shared__ uint16_t lst[];    // this block's past chunks in scan order (C entries)

  const int item = remap_xcd(blockIdx.x, items);
  if (item >= items) return;
  const int bh = item / NB;
  const int rb = NB - 1 - (item % NB);  // heavier (later) row blocks first
  const int hh = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int r0 = rb * ST_ROWS;
  const int row = r0 + 32 * w + n;       // this lane's row as an MFMA A-operand supplier
  const bool row_ok = row < N;
  const int last = min(r0 + ST_ROWS, N) - 1;
  const int Pmax = min(C, last / 64);
  const float tau = 1.0f / sqrtf((float)D);
  const int64_t qrow = ((int64_t)bh * N + (row_ok ? row : 0)) * D;

  // ---- the query's A operands (k-permuted head-dim slices), split into bf16 terms
  bf16x8_t qb[NQ][NKS];
  {
    float qf[NKS][8];
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
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        qf[ks][m] = a4[m];
        qf[ks][4 + m] = b4[m];
      }
    }
    if constexpr (!QCAL) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint16_t t[NQ][8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint16_t sp[NQ];
          split_bf16<NQ>(qf[ks][m], sp);
#pragma unroll
          for (int j = 0; j < NQ; ++j) t[j][m] = sp[j];
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) qb[j][ks] = pack8(t[j]);
      }
    } else {
      // raw q terms (exact: NIO bf16 terms carry an io value exactly), as B operands
      bf16x8_t qr[NIO][NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint16_t t[NIO][8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint16_t sp[NIO];
          split_bf16<NIO>(qf[ks][m], sp);
#pragma unroll
          for (int j = 0; j < NIO; ++j) t[j][m] = sp[j];
        }
#pragma unroll
        for (int j = 0; j < NIO; ++j) qr[j][ks] = pack8(t[j]);
      }
      // T^T[a][row] = sum_e D[a][e] q[row][e]   (a < r; rows a >= r are zero)
      f32x16_t T = zero16();
      const int a_row = lane & 31;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint16_t dt[NIO][8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float x = a_row < r ? io_traits<IO>::load(Dw, ((int64_t)hh * r + a_row) * D + kperm(ks, hf, m)) : 0.f;
          uint16_t sp[NIO];
          split_bf16<NIO>(x, sp);
#pragma unroll
          for (int j = 0; j < NIO; ++j) dt[j][m] = sp[j];
        }
#pragma unroll
        for (int i = 0; i < NIO; ++i)
#pragma unroll
          for (int j = 0; j < NIO; ++j)
            if (i + j < NIO) T = mfma32(pack8(dt[i]), qr[j][ks], T);
      }
      // T as the B operand of U T: accumulator register 8*ks2 + m -> k-step ks2, element m
      constexpr int NT = NIO == 1 ? 2 : 3;
      bf16x8_t tb[NT][2];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        uint16_t t[NT][8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint16_t sp[NT];
          split_bf16<NT>(T[8 * ks2 + m], sp);
#pragma unroll
          for (int j = 0; j < NT; ++j) t[j][m] = sp[j];
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) tb[j][ks2] = pack8(t[j]);
      }
      constexpr int NP = NIO > NT ? NIO : NT;
#pragma unroll
      for (int dt2 = 0; dt2 < D / 32; ++dt2) {
        f32x16_t Q = zero16();
        const int e = 32 * dt2 + (lane & 31);
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          uint16_t ut[NIO][8];
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int a = kperm(ks2, hf, m);
            const float x = a < r ? io_traits<IO>::load(Uw, ((int64_t)hh * D + e) * r + a) : 0.f;
            uint16_t sp[NIO];
            split_bf16<NIO>(x, sp);
#pragma unroll
            for (int j = 0; j < NIO; ++j) ut[j][m] = sp[j];
          }
#pragma unroll
          for (int i = 0; i < NIO; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
              if (i + j < NP) Q = mfma32(pack8(ut[i]), tb[j][ks2], Q);
        }
        // register rr of this tile is head dim 32*dt2 + acc_row(rr, hf) = k-step 2*dt2 + rr/8, element rr%8
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int ks = 2 * dt2 + half;
          uint16_t t[NQ][8];
          float a4[4], b4[4];  // reload the raw q slice (cheaper than keeping it live)
          if (row_ok) {
            io_traits<IO>::load4(q, qrow + kperm(ks, hf, 0), a4);
            io_traits<IO>::load4(q, qrow + kperm(ks, hf, 4), b4);
          } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) a4[m] = b4[m] = 0.f;
          }
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const float qh = (m < 4 ? a4[m] : b4[m - 4]) + Q[8 * half + m];
            uint16_t sp[NQ];
            split_bf16<NQ>(qh, sp);
#pragma unroll
            for (int j = 0; j < NQ; ++j) t[j][m] = sp[j];
          }
#pragma unroll
          for (int j = 0; j < NQ; ++j) qb[j][ks] = pack8(t[j]);
        }
      }
    }
  }

  // ---- scan order: past chunks c < Pmin (valid for every row of the block) by descending
  // b', then the chunks Pmin .. Pmax-1 that only the later rows of the block see.
  const int Pmin = min(C, r0 / 64);
  {
    const int32_t* ord = order + (int64_t)bh * C;
    int base = 0;
    for (int i0 = 0; i0 < C; i0 += 256) {
      const int i = i0 + tid;
      const int c = i < C ? ord[i] : C;
      const bool v = c < Pmin;
      const uint64_t bm = __ballot(v);
      const int pre = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
      if (lane == 0) wsum[w] = __popcll(bm);
      __syncthreads();
      int off = base;
      for (int x = 0; x < w; ++x) off += wsum[x];
      if (v) lst[off + pre] = (uint16_t)c;
      base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
      __syncthreads();
    }
    for (int x = tid; x < Pmax - Pmin; x += 256) lst[Pmin + x] = (uint16_t)(Pmin + x);
    __syncthreads();
  }

  // ---- per-row top-K state: register rr holds rows acc_row(rr, 0) (lanes 0..31) and
  // acc_row(rr, 1) (lanes 32..63) of this wave.  Lane j of a half holds buffer slot j
  // (bs, bi) of its row in registers; the row's sorted list (lane j = j-th best) lives
  // in LDS (lsl, lil) and is only touched when a buffer is merged.  ts = K-th best score.
  float bs[16], ts[16];
  int bi[16], ff[16];  // ff: wave-uniform buffer fills, lanes 0..31 in bits 0..7, lanes 32..63 in bits 8..15
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    bs[rr] = ts[rr] = -INFINITY;
    bi[rr] = 0x7fffffff;
    ff[rr] = 0;
    lsl[w][rr][lane] = -INFINITY;
    lil[w][rr][lane] = 0x7fffffff;
  }

  const int64_t PL = (int64_t)(items / NB) * C * D;    // elements per plane: B*H*C*D
  const float* bcb = bc + (int64_t)bh * C;
  const int ntiles = (Pmax + ST_TILE - 1) / ST_TILE;
  // The next tile is prefetched in two halves of 32 chunks: loads issued before each
  // 32-chunk MFMA column tile, written to the other LDS buffer after it.
  u32x4_t pf[PH];
  int pcid = 0;
  float pb = 0.f;
  auto prefetch = [&](int t, int part) {
#pragma unroll
    for (int u = 0; u < PH; ++u) {
      const int it = tid + 256 * u;
      const int e = 32 * part + it / (NK * SEGS);
      const int rem = it % (NK * SEGS);
      const int pl = rem / SEGS, sg = rem % SEGS;
      const int idx = t * ST_TILE + e;
      const int cid = idx < Pmax ? (int)lst[idx] : -1;
      pf[u] = cid >= 0 ? *reinterpret_cast<const u32x4_t*>(planes + pl * PL + ((int64_t)bh * C + cid) * D + 8 * sg)
                       : u32x4_t{0u, 0u, 0u, 0u};
    }
    if (tid < 32) {
      const int idx = t * ST_TILE + 32 * part + tid;
      pcid = idx < Pmax ? (int)lst[idx] : 0x7fffffff;
      pb = idx < Pmax ? bcb[pcid] : 0.f;
    }
  };
  // merge row-register rr's buffer into its LDS list; refresh ts
  auto flush_rr = [&](int rr, float& b_s, int& b_i, int& bff, float& t_s, int& t_i) {
    float ls = lsl[w][rr][lane];
    int li = lil[w][rr][lane];
    int bf0 = bff & 0xff, bf1 = bff >> 8;
    flush(ls, li, b_s, b_i, bf0, bf1, t_s, t_i, n, hf, K);
    bff = 0;
    lsl[w][rr][lane] = ls;
    lil[w][rr][lane] = li;
  };
  auto commit = [&](int part) {
#pragma unroll
    for (int u = 0; u < PH; ++u) {
      const int it = tid + 256 * u;
      const int e = 32 * part + it / (NK * SEGS);
      const int rem = it % (NK * SEGS);
      const int pl = rem / SEGS, sg = rem % SEGS;
      uint16_t* dstp = &kt[pl][e * LDK + 8 * sg];
      *reinterpret_cast<u32x2_t*>(dstp) = u32x2_t{pf[u].x, pf[u].y};
      *reinterpret_cast<u32x2_t*>(dstp + 4) = u32x2_t{pf[u].z, pf[u].w};
    }
    if (tid < 32) {
      ct[32 * part + tid] = pcid;
      bt[32 * part + tid] = pb;
    }
  };

  if (ntiles > 0) {
    prefetch(0, 0);
    commit(0);
    prefetch(0, 1);
    commit(1);
  }
  __syncthreads();
  // Half tile tt of the next tile is loaded into registers before the MFMA of half tt and
  // written over half tt after a barrier; half tt is only read by column tile tt.
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    const bool masked = (t + 1) * ST_TILE > Pmin;  // entries beyond Pmin are not valid for every row
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (more) prefetch(t + 1, tt);
      f32x16_t acc = zero16();
      const int ch = 32 * tt + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          const uint16_t* kr = &kt[j][ch * LDK + 16 * ks + 4 * hf];
          const bf16x8_t bk = pack8(*reinterpret_cast<const u32x2_t*>(kr), *reinterpret_cast<const u32x2_t*>(kr + 8));
#pragma unroll
          for (int i = 0; i < NQ; ++i)
            if (i + j < (NQ > NK ? NQ : NK)) acc = mfma32(qb[i][ks], bk, acc);
        }
      }
      const int c = ct[ch];
      const float bprime = bt[ch];
      // filter against each row's K-th best; append the survivors; overflowing
      // buffers are handled after the pass (one copy of the merge code)
      auto score_of = [&](float a, int rr) {
        float s = fmaf(a, tau, bprime);
        if (masked) {
          const int rw = r0 + 32 * w + acc_row(rr, hf);
          const int prow = rw < N ? min(C, rw / 64) : 0;
          if (c >= prow) s = __builtin_nanf("");
        }
        return s;
      };
      uint32_t ovf = 0;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float s = score_of(acc[rr], rr);
        bool pass = s > ts[rr];  // NaN never passes
        if (__ballot(s == ts[rr])) {
          const int ti = lil[w][rr][32 * hf + K - 1];
          pass = pass || (s == ts[rr] && c < ti);
        }
        const uint64_t mk = __ballot(pass);
        if (mk) {
          int a0 = ff[rr] & 0xff, a1 = ff[rr] >> 8;
          if (a0 + __popc((uint32_t)mk) > ST_BUF || a1 + __popc((uint32_t)(mk >> 32)) > ST_BUF) {
            ovf |= 1u << rr;
          } else {
            append(bs[rr], bi[rr], a0, a1, s, c, pass, mk, n, hf);
            ff[rr] = a0 | (a1 << 8);
          }
        }
      }
      while (ovf) {
        const int rr = __builtin_ctz(ovf);
        ovf &= ovf - 1;
        float wb, wt, wa;
        int wj, wf;
        switch (rr) {
#define HILS_PICK(R) \
  case R:            \
    wb = bs[R];      \
    wj = bi[R];      \
    wf = ff[R];      \
    wt = ts[R];      \
    wa = acc[R];     \
    break;
          HILS_PICK(0) HILS_PICK(1) HILS_PICK(2) HILS_PICK(3) HILS_PICK(4) HILS_PICK(5) HILS_PICK(6) HILS_PICK(7)
          HILS_PICK(8) HILS_PICK(9) HILS_PICK(10) HILS_PICK(11) HILS_PICK(12) HILS_PICK(13) HILS_PICK(14)
          HILS_PICK(15)
#undef HILS_PICK
          default:
            wb = wt = wa = 0.f;
            wj = wf = 0;
        }
        const float ws = score_of(wa, rr);
        int wti;
        flush_rr(rr, wb, wj, wf, wt, wti);
        const bool pass = better(ws, c, wt, wti);
        const uint64_t mk = __ballot(pass);
        int m0 = __popc((uint32_t)mk), m1 = __popc((uint32_t)(mk >> 32));
        if ((m0 > m1 ? m0 : m1) > ST_BUF) {  // more than a buffer of new candidates: merge them directly
          float ls = lsl[w][rr][lane];
          int li = lil[w][rr][lane];
          merge_into(ls, li, pass ? ws : -INFINITY, pass ? c : 0x7fffffff, n, K);
          kth(ls, li, hf, K, wt, wti);
          lsl[w][rr][lane] = ls;
          lil[w][rr][lane] = li;
        } else if (mk) {
          int a0 = 0, a1 = 0;
          append(wb, wj, a0, a1, ws, c, pass, mk, n, hf);
          wf = a0 | (a1 << 8);
        }
        switch (rr) {
#define HILS_PUT(R) \
  case R:           \
    bs[R] = wb;     \
    bi[R] = wj;     \
    ff[R] = wf;     \
    ts[R] = wt;     \
    break;
          HILS_PUT(0) HILS_PUT(1) HILS_PUT(2) HILS_PUT(3) HILS_PUT(4) HILS_PUT(5) HILS_PUT(6) HILS_PUT(7)
          HILS_PUT(8) HILS_PUT(9) HILS_PUT(10) HILS_PUT(11) HILS_PUT(12) HILS_PUT(13) HILS_PUT(14) HILS_PUT(15)
#undef HILS_PUT
          default:
            break;
        }
      }
      __syncthreads();  // every wave is done with half tt of this tile
      if (more) commit(tt);
    }
  }

  // ---- final merges and output: lane j of each half writes slot j of its row
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    if (ff[rr] != 0) {
      int tdummy;
      flush_rr(rr, bs[rr], bi[rr], ff[rr], ts[rr], tdummy);
    }
    const int rw = r0 + 32 * w + acc_row(rr, hf);
    if (rw < N && n < K) {
      const int64_t o = ((int64_t)bh * N + rw) * K + n;
      const int li = lil[w][rr][lane];
      const bool ok = li != 0x7fffffff;
      sel_idx[o] = ok ? li : -1;
      sel_score[o] = ok ? lsl[w][rr][lane] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------- helpers kernels
// k' (fp32) -> NK bf16 planes: plane j holds term j of every element (same layout as k')
template <int NK>
__global__ void __launch_bounds__(256) split_kprime(const float* __restrict__ kc, uint16_t* __restrict__ planes,
                                                    int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (int64_t)gridDim.x * 256 * 4) {
    const float4 v = *reinterpret_cast<const float4*>(kc + i);
    uint16_t s0[NK], s1[NK], s2[NK], s3[NK];
    split_bf16<NK>(v.x, s0);
    split_bf16<NK>(v.y, s1);
    split_bf16<NK>(v.z, s2);
    split_bf16<NK>(v.w, s3);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      u32x2_t pk;
      pk.x = (uint32_t)s0[j] | ((uint32_t)s1[j] << 16);
      pk.y = (uint32_t)s2[j] | ((uint32_t)s3[j] << 16);
      *reinterpret_cast<u32x2_t*>(planes + j * n + i) = pk;
    }
  }
}

// per (b, h): chunk ids ordered by descending b' (ties: lower id first); bitonic sort in LDS
__global__ void __launch_bounds__(1024) sort_bprime(const float* __restrict__ bc, int32_t* __restrict__ order, int C,
                                                    int Cp2) {
  extern __shared__ uint64_t keys[];
  const int bh = blockIdx.x, t = threadIdx.x;
  for (int i = t; i < Cp2; i += 1024) keys[i] = i < C ? make_key(bc[(int64_t)bh * C + i], i) : 0ull;
  __syncthreads();
  for (int k = 2; k <= Cp2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < Cp2; i += 1024) {
        const int l = i ^ jj;
        if (l > i) {
          const uint64_t a = keys[i], b = keys[l];
          const bool desc = (i & k) == 0;
          if (desc ? a < b : a > b) {
            keys[i] = b;
            keys[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < C; i += 1024) order[(int64_t)bh * C + i] = key_chunk(keys[i]);
}

static size_t al3(size_t x) { return (x + 255) / 256 * 256; }
static int nk_of(const Geom& g) { return g.io == 0 ? 3 : 2; }

size_t score_workspace_bytes(const Geom& g) {
  const size_t n = (size_t)g.B * g.Hq * g.C() * g.d;
  return al3((size_t)nk_of(g) * n * 2) + al3((size_t)g.B * g.Hq * g.C() * 4);
}

template <typename IO, int D, int NQ, int NK, bool QCAL>
static void launch_st(const Geom& g, const void* q, const void* Dw, const void* Uw, const uint16_t* planes,
                      const float* bc, const int32_t* order, int32_t* si, float* ss, hipStream_t st) {
  const int NB = (g.N + ST_ROWS - 1) / ST_ROWS;
  const int items = g.B * g.Hq * NB;
  const int grid = ((items + 7) / 8) * 8;
  const size_t dyn = ((size_t)g.C() * 2 + 15) / 16 * 16 + 16;
  auto kern = score_topk_kernel<IO, D, NQ, NK, QCAL>;
  hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), dyn, st, (const IO*)q, (const IO*)Dw, (const IO*)Uw, planes, bc,
                     order, si, ss, g.Hq, g.N, g.C(), g.K, g.r, NB, items);
}

template <typename IO, int D>
static void launch_st_d(const Geom& g, const void* q, const void* Dw, const void* Uw, const uint16_t* planes,
                        const float* bc, const int32_t* order, int32_t* si, float* ss, hipStream_t st) {
  constexpr bool F32 = io_traits<IO>::terms == 3;
  if (g.r > 0)
    launch_st<IO, D, F32 ? 3 : 2, F32 ? 3 : 2, true>(g, q, Dw, Uw, planes, bc, order, si, ss, st);
  else
    launch_st<IO, D, F32 ? 3 : 1, F32 ? 3 : 2, false>(g, q, Dw, Uw, planes, bc, order, si, ss, st);
}

hipError_t launch_score_topk(const Geom& g, const void* q, const void* Dw, const void* Uw, const float* kc,
                             const float* bc, int32_t* sel_idx, float* sel_score, void* ws, size_t ws_bytes,
                             hipStream_t st) {
  if (ws_bytes < score_workspace_bytes(g)) return hipErrorInvalidValue;
  const int C = g.C();
  const int64_t n = (int64_t)g.B * g.Hq * C * g.d;
  uint16_t* planes = (uint16_t*)ws;
  int32_t* order = (int32_t*)((char*)ws + al3((size_t)nk_of(g) * n * 2));
  if (C > 0) {
    const unsigned gs = (unsigned)std::min<int64_t>((n / 4 + 255) / 256, 8192);
    if (nk_of(g) == 3)
      hipLaunchKernelGGL(split_kprime<3>, dim3(gs), dim3(256), 0, st, kc, planes, n);
    else
      hipLaunchKernelGGL(split_kprime<2>, dim3(gs), dim3(256), 0, st, kc, planes, n);
    int Cp2 = 1;
    while (Cp2 < C) Cp2 <<= 1;
    const size_t dyn = (size_t)Cp2 * 8;
    hipFuncSetAttribute((const void*)sort_bprime, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    hipLaunchKernelGGL(sort_bprime, dim3(g.B * g.Hq), dim3(1024), dyn, st, bc, order, C, Cp2);
  }
  if (g.io == 0) {
    if (g.d == 64)
      launch_st_d<float, 64>(g, q, Dw, Uw, planes, bc, order, sel_idx, sel_score, st);
    else
      launch_st_d<float, 128>(g, q, Dw, Uw, planes, bc, order, sel_idx, sel_score, st);
  } else {
    if (g.d == 64)
      launch_st_d<bf16_t, 64>(g, q, Dw, Uw, planes, bc, order, sel_idx, sel_score, st);
    else
      launch_st_d<bf16_t, 128>(g, q, Dw, Uw, planes, bc, order, sel_idx, sel_score, st);
  }
  return hipGetLastError();
}

}  // namespace hils

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
//   * Top-K: every row keeps its exact running top K sorted across the 32 lanes
//     of its half-wave (lane j = j-th best) in registers.  New scores are tested
//     against the row's K-th best with one compare; the few that pass are inserted
//     with a ballot/shuffle step each, and when many pass at once (the first tiles)
//     they are bitonic-sorted and merged with the list in one go.
#include "hils_common.h"
#include "kernels.h"

namespace hils {

constexpr int ST_ROWS = 128;   // queries per workgroup
constexpr int ST_TILE = 64;    // chunks per LDS tile
constexpr int ST_BULK = 8;     // more candidates than this in a half-wave: sort-and-merge

HILS_DEV bool better(float s1, int c1, float s2, int c2) { return s1 > s2 || (s1 == s2 && c1 < c2); }

// Bitonic sort of one (score, chunk) per lane, best first, within each 32-lane half.
HILS_DEV void sort32_desc(float& s, int& c, int j) {
#pragma unroll
  for (int k = 2; k <= 32; k <<= 1) {
#pragma unroll
    for (int st = k >> 1; st >= 1; st >>= 1) {
      const float ps = __shfl_xor(s, st);
      const int pc = __shfl_xor(c, st);
      const bool desc = (j & k) == 0 || k == 32;
      const bool lower = (j & st) == 0;
      const bool take = (lower == desc) ? better(ps, pc, s, c) : better(s, c, ps, pc);
      if (take) {
        s = ps;
        c = pc;
      }
    }
  }
}

// Merge this half-wave's new candidates (ns, nc) into the sorted list (ls, li), keep the best K.
HILS_DEV void bulk_merge(float& ls, int& li, float ns, int nc, int j, int K) {
  sort32_desc(ns, nc, j);
  const float rs = __shfl_xor(ns, 31);  // reversed: lane j sees the (31-j)-th best new one
  const int rc = __shfl_xor(nc, 31);
  if (better(rs, rc, ls, li)) {
    ls = rs;
    li = rc;
  }
#pragma unroll
  for (int st = 16; st >= 1; st >>= 1) {  // the 32 kept values form a bitonic sequence
    const float ps = __shfl_xor(ls, st);
    const int pc = __shfl_xor(li, st);
    const bool lower = (j & st) == 0;
    const bool take = lower ? better(ps, pc, ls, li) : better(ls, li, ps, pc);
    if (take) {
      ls = ps;
      li = pc;
    }
  }
  if (j >= K) {
    ls = -INFINITY;
    li = 0x7fffffff;
  }
}

HILS_DEV float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
HILS_DEV int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
// lane i receives lane i-1 (DPP wave_shr:1); lane 0 keeps its own value
HILS_DEV float shr1_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x138, 0xf, 0xf, false));
}
HILS_DEV int shr1_i(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x138, 0xf, 0xf, false); }

// Update the two row lists of one accumulator register with this 32-chunk tile.
// s: this lane's score (NaN if the chunk is not a candidate of its row), c: its chunk id.
// ts: the row's K-th best score (-inf while the list is not full); the K-th best
// chunk id is only fetched when a new score ties with it exactly.
HILS_DEV void topk_update(float& ls, int& li, float& ts, float s, int c, int j, int hf, int K) {
  bool pass = s > ts;  // NaN never passes
  if (__ballot(s == ts)) {
    const int ti = __shfl(li, K - 1, 32);
    pass = pass || (s == ts && c < ti);
  }
  const uint64_t mk = __ballot(pass);
  if (mk == 0) return;
  const int n0 = __popc((uint32_t)mk), n1 = __popc((uint32_t)(mk >> 32));
  const int nmax = n0 > n1 ? n0 : n1;
  if (nmax > ST_BULK) {
    bulk_merge(ls, li, pass ? s : -INFINITY, pass ? c : 0x7fffffff, j, K);
  } else {
    // one candidate per half-wave per round: broadcast it (readlane), find its rank in
    // the sorted list (ballot), shift the worse entries up one lane (DPP) and insert
    uint32_t lo = (uint32_t)mk, hi = (uint32_t)(mk >> 32);
    for (int it = 0; it < nmax; ++it) {
      const int s0 = lo ? __builtin_ctz(lo) : 0;
      const int s1 = hi ? __builtin_ctz(hi) + 32 : 32;
      const float cs0 = readlane_f(s, s0), cs1 = readlane_f(s, s1);
      const int cc0 = readlane_i(c, s0), cc1 = readlane_i(c, s1);
      const bool act = hf ? (hi != 0) : (lo != 0);
      const float cs = hf ? cs1 : cs0;
      const int cc = hf ? cc1 : cc0;
      const bool bt = j < K && better(ls, li, cs, cc);
      const uint64_t bm = __ballot(bt);
      const int pos = __popc(hf ? (uint32_t)(bm >> 32) : (uint32_t)bm);
      const float us = shr1_f(ls);
      const int ui = shr1_i(li);
      if (act && j < K && j >= pos) {
        ls = (j == pos) ? cs : us;
        li = (j == pos) ? cc : ui;
      }
      lo &= lo - 1;
      hi &= hi - 1;
    }
  }
  const float t0 = readlane_f(ls, K - 1), t1 = readlane_f(ls, 32 + K - 1);
  ts = hf ? t1 : t0;
}

template <typename IO, int D, int NQ, int NK, bool QCAL>
__global__ void __launch_bounds__(256, 2) score_topk_kernel(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                             const IO* __restrict__ Uw, const float* __restrict__ kc,
                                                             const float* __restrict__ bc,
                                                             int32_t* __restrict__ sel_idx,
                                                             float* __restrict__ sel_score, int H, int N, int C, int K,
                                                             int r, int NB, int items) {
  constexpr int LDK = D + 4;            // padded bf16 row stride of the k' tile planes
  constexpr int NKS = D / 16;           // MFMA k-steps over the head dimension
  constexpr int NIO = io_traits<IO>::terms;
  constexpr int PF = ST_TILE * D / (256 * 4);  // float4 prefetch loads per thread per tile
  __shared__ uint16_t kt[2][NK][ST_TILE * LDK];
  __shared__ float bt[2][ST_TILE];

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

  // ---- per-row top-K lists: register rr holds rows acc_row(rr, 0) (lanes 0..31) and
  // acc_row(rr, 1) (lanes 32..63) of this wave; lane j of a half = the row's j-th best.
  float ls[16], ts[16];
  int li[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    ls[rr] = ts[rr] = -INFINITY;
    li[rr] = 0x7fffffff;
  }

  const float* kcb = kc + (int64_t)bh * C * D;
  const float* bcb = bc + (int64_t)bh * C;
  const int ntiles = (Pmax + ST_TILE - 1) / ST_TILE;
  // The next tile is prefetched in two halves: loads issued before each 32-chunk MFMA
  // column tile, converted and written to the other LDS buffer after it.
  constexpr int PH = PF / 2;
  float4 pf[PH];
  float pb = 0.f;
  auto prefetch = [&](int t, int part) {
    const int c0 = t * ST_TILE;
#pragma unroll
    for (int u = 0; u < PH; ++u) {
      const int i = (tid + 256 * (u + part * PH)) * 4;
      const int ch = i / D, e = i % D;
      pf[u] = (c0 + ch < Pmax) ? *reinterpret_cast<const float4*>(kcb + (int64_t)(c0 + ch) * D + e)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (part == 0 && tid < ST_TILE) pb = (c0 + tid < Pmax) ? bcb[c0 + tid] : 0.f;
  };
  auto commit = [&](int buf, int part) {
#pragma unroll
    for (int u = 0; u < PH; ++u) {
      const int i = (tid + 256 * (u + part * PH)) * 4;
      const int ch = i / D, e = i % D;
      uint16_t s0[NK], s1[NK], s2[NK], s3[NK];
      split_bf16<NK>(pf[u].x, s0);
      split_bf16<NK>(pf[u].y, s1);
      split_bf16<NK>(pf[u].z, s2);
      split_bf16<NK>(pf[u].w, s3);
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        u32x2_t pk;
        pk.x = (uint32_t)s0[j] | ((uint32_t)s1[j] << 16);
        pk.y = (uint32_t)s2[j] | ((uint32_t)s3[j] << 16);
        *reinterpret_cast<u32x2_t*>(&kt[buf][j][ch * LDK + e]) = pk;
      }
    }
    if (part == 0 && tid < ST_TILE) bt[buf][tid] = pb;
  };

  if (ntiles > 0) {
    prefetch(0, 0);
    commit(0, 0);
    prefetch(0, 1);
    commit(0, 1);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int c0 = t * ST_TILE;
    const bool more = t + 1 < ntiles;
    const bool masked = c0 + ST_TILE > min(C, (r0 + 32 * w) / 64);  // some row of this wave may stop inside
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (more) prefetch(t + 1, tt);
      f32x16_t acc = zero16();
      const int ch = 32 * tt + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          const uint16_t* kr = &kt[buf][j][ch * LDK + 16 * ks + 4 * hf];
          const bf16x8_t bk = pack8(*reinterpret_cast<const u32x2_t*>(kr), *reinterpret_cast<const u32x2_t*>(kr + 8));
#pragma unroll
          for (int i = 0; i < NQ; ++i)
            if (i + j < (NQ > NK ? NQ : NK)) acc = mfma32(qb[i][ks], bk, acc);
        }
      }
      const int c = c0 + ch;
      const float bprime = bt[buf][ch];
      // scores of the 16 registers and which of them have a candidate (wave-uniform bits)
      float sv[16];
      uint32_t need = 0;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float s = fmaf(acc[rr], tau, bprime);
        if (masked) {
          const int rw = r0 + 32 * w + acc_row(rr, hf);
          const int prow = rw < N ? min(C, rw / 64) : 0;
          if (c >= prow) s = __builtin_nanf("");
        }
        sv[rr] = s;
        if (__ballot(s >= ts[rr])) need |= 1u << rr;  // ties are resolved exactly in topk_update
      }
      // one copy of the update code; the register is picked by a uniform switch
      while (need) {
        const int rr = __builtin_ctz(need);
        need &= need - 1;
        float wl, wt, ws;
        int wi;
        switch (rr) {
#define HILS_PICK(R) \
  case R:            \
    wl = ls[R];      \
    wi = li[R];      \
    wt = ts[R];      \
    ws = sv[R];      \
    break;
          HILS_PICK(0) HILS_PICK(1) HILS_PICK(2) HILS_PICK(3) HILS_PICK(4) HILS_PICK(5) HILS_PICK(6) HILS_PICK(7)
          HILS_PICK(8) HILS_PICK(9) HILS_PICK(10) HILS_PICK(11) HILS_PICK(12) HILS_PICK(13) HILS_PICK(14)
          HILS_PICK(15)
#undef HILS_PICK
          default:
            wl = wt = ws = 0.f;
            wi = 0;
        }
        topk_update(wl, wi, wt, ws, c, n, hf, K);
        switch (rr) {
#define HILS_PUT(R) \
  case R:           \
    ls[R] = wl;     \
    li[R] = wi;     \
    ts[R] = wt;     \
    break;
          HILS_PUT(0) HILS_PUT(1) HILS_PUT(2) HILS_PUT(3) HILS_PUT(4) HILS_PUT(5) HILS_PUT(6) HILS_PUT(7)
          HILS_PUT(8) HILS_PUT(9) HILS_PUT(10) HILS_PUT(11) HILS_PUT(12) HILS_PUT(13) HILS_PUT(14) HILS_PUT(15)
#undef HILS_PUT
          default:
            break;
        }
      }
      if (more) commit(buf ^ 1, tt);
    }
    __syncthreads();
  }

  // ---- write the lists: lane j of each half writes slot j of its row
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int rw = r0 + 32 * w + acc_row(rr, hf);
    if (rw < N && n < K) {
      const int64_t o = ((int64_t)bh * N + rw) * K + n;
      const bool ok = li[rr] != 0x7fffffff;
      sel_idx[o] = ok ? li[rr] : -1;
      sel_score[o] = ok ? ls[rr] : -INFINITY;
    }
  }
}

template <typename IO, int D, int NQ, int NK, bool QCAL>
static void launch_st(const Geom& g, const void* q, const void* Dw, const void* Uw, const float* kc, const float* bc,
                      int32_t* si, float* ss, hipStream_t st) {
  const int NB = (g.N + ST_ROWS - 1) / ST_ROWS;
  const int items = g.B * g.Hq * NB;
  const int grid = ((items + 7) / 8) * 8;
  hipLaunchKernelGGL((score_topk_kernel<IO, D, NQ, NK, QCAL>), dim3(grid), dim3(256), 0, st, (const IO*)q,
                     (const IO*)Dw, (const IO*)Uw, kc, bc, si, ss, g.Hq, g.N, g.C(), g.K, g.r, NB, items);
}

template <typename IO, int D>
static void launch_st_d(const Geom& g, const void* q, const void* Dw, const void* Uw, const float* kc, const float* bc,
                        int32_t* si, float* ss, hipStream_t st) {
  constexpr bool F32 = io_traits<IO>::terms == 3;
  if (g.r > 0)
    launch_st<IO, D, F32 ? 3 : 2, F32 ? 3 : 2, true>(g, q, Dw, Uw, kc, bc, si, ss, st);
  else
    launch_st<IO, D, F32 ? 3 : 1, F32 ? 3 : 2, false>(g, q, Dw, Uw, kc, bc, si, ss, st);
}

hipError_t launch_score_topk(const Geom& g, const void* q, const void* Dw, const void* Uw, const float* kc,
                             const float* bc, int32_t* sel_idx, float* sel_score, hipStream_t st) {
  if (g.io == 0) {
    if (g.d == 64)
      launch_st_d<float, 64>(g, q, Dw, Uw, kc, bc, sel_idx, sel_score, st);
    else
      launch_st_d<float, 128>(g, q, Dw, Uw, kc, bc, sel_idx, sel_score, st);
  } else {
    if (g.d == 64)
      launch_st_d<bf16_t, 64>(g, q, Dw, Uw, kc, bc, sel_idx, sel_score, st);
    else
      launch_st_d<bf16_t, 128>(g, q, Dw, Uw, kc, bc, sel_idx, sel_score, st);
  }
  return hipGetLastError();
}

}  // namespace hils

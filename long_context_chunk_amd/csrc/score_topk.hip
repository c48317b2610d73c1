// Chunk scoring and streaming top-K for prefill queries.
//
//   s_ic = q^_i . k'_c / sqrt(d) + b'_c   for every complete past chunk c < floor(i/S)
//   q^_i = q_i + U_h (D_h q_i)             (Q-Cal; q^ = q without it)
// keep the K best (ties -> lower chunk id).  (aitrends.kr article,
// "Methodology": the score formula, the calculation flow and the Q-Cal module.)
//
// Design (gfx950):
//   * One workgroup = 128 consecutive queries of one (batch, head); wave w owns 32
//     of them as the N dimension of v_mfma_f32_32x32x16_bf16, the chunks are the
//     M dimension.  Each lane ends up with 16 scores of one query per MFMA.
//   * k' tiles of 64 chunks are staged through LDS once per workgroup and shared
//     by the four waves.  k' (fp32) is split into bf16 terms (hi + lo, or three
//     terms for fp32 I/O) and q^ likewise, so the bf16 MFMA reproduces the fp32
//     dot product to ~2^-17 relative: index parity needs score errors far below
//     1e-4, which a single bf16 rounding of k' does not give.
//   * Q-Cal runs on the same MFMA (T = D q, then U T), chained through the
//     accumulator layout without any cross-lane movement.
//   * Top-K: each lane keeps a min-heap of K (score, chunk) keys in LDS for its
//     half of the query's chunks; candidates are filtered against both halves'
//     current K-th best, queued per lane, and inserted in rounds (log K LDS steps
//     per insertion).  At the end each heap is heap-sorted and the two halves are
//     merged into the query's top K in rank order.
#include "hils_common.h"
#include "kernels.h"

namespace hils {

constexpr int ST_ROWS = 128;   // queries per workgroup
constexpr int ST_TILE = 64;    // chunks per LDS tile
constexpr int ST_KMAX = 32;    // largest supported K
constexpr int ST_QLEN = 16;    // candidate queue length per lane (one half tile)

template <typename IO, int D, int NQ, int NK, bool QCAL>
__global__ void __launch_bounds__(256) score_topk_kernel(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                          const IO* __restrict__ Uw, const float* __restrict__ kc,
                                                          const float* __restrict__ bc, int32_t* __restrict__ sel_idx,
                                                          float* __restrict__ sel_score, int H, int N, int C, int K,
                                                          int r, int NB, int items) {
  constexpr int LDK = D + 4;            // padded bf16 row stride of the k' tile planes
  constexpr int NKS = D / 16;           // MFMA k-steps over the head dimension
  constexpr int NIO = io_traits<IO>::terms;
  __shared__ uint16_t kt[NK][ST_TILE * LDK];
  __shared__ float bt[ST_TILE];
  __shared__ uint64_t heap[4][ST_KMAX][64];
  __shared__ uint64_t queue[4][ST_QLEN][64];

  const int item = remap_xcd(blockIdx.x, items);
  if (item >= items) return;
  const int bh = item / NB;
  const int rb = NB - 1 - (item % NB);  // heavier (later) row blocks first
  const int hh = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int r0 = rb * ST_ROWS;
  const int row = r0 + 32 * w + n;
  const bool row_ok = row < N;
  const int P_row = row_ok ? min(C, row / 64) : 0;
  const int last = min(r0 + ST_ROWS, N) - 1;
  const int Pmax = min(C, last / 64);
  const float tau = 1.0f / sqrtf((float)D);
  const int64_t qrow = ((int64_t)bh * N + (row_ok ? row : 0)) * D;

  // ---- the query's B operands (k-permuted head-dim slices), split into bf16 terms
  bf16x8_t qb[NQ][NKS];
  {
    float qf[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int m = 0; m < 8; ++m) qf[ks][m] = row_ok ? io_traits<IO>::load(q, qrow + kperm(ks, hf, m)) : 0.f;
    if constexpr (!QCAL) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint16_t t[NQ][8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint16_t s[NQ];
          split_bf16<NQ>(qf[ks][m], s);
#pragma unroll
          for (int j = 0; j < NQ; ++j) t[j][m] = s[j];
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) qb[j][ks] = pack8(t[j]);
      }
    } else {
      // raw q terms (exact: NIO bf16 terms carry an io value exactly)
      bf16x8_t qr[NIO][NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint16_t t[NIO][8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint16_t s[NIO];
          split_bf16<NIO>(qf[ks][m], s);
#pragma unroll
          for (int j = 0; j < NIO; ++j) t[j][m] = s[j];
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
          uint16_t s[NIO];
          split_bf16<NIO>(x, s);
#pragma unroll
          for (int j = 0; j < NIO; ++j) dt[j][m] = s[j];
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
          uint16_t s[NT];
          split_bf16<NT>(T[8 * ks2 + m], s);
#pragma unroll
          for (int j = 0; j < NT; ++j) t[j][m] = s[j];
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
            uint16_t s[NIO];
            split_bf16<NIO>(x, s);
#pragma unroll
            for (int j = 0; j < NIO; ++j) ut[j][m] = s[j];
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
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const float qh = qf[ks][m] + Q[8 * half + m];
            uint16_t s[NQ];
            split_bf16<NQ>(qh, s);
#pragma unroll
            for (int j = 0; j < NQ; ++j) t[j][m] = s[j];
          }
#pragma unroll
          for (int j = 0; j < NQ; ++j) qb[j][ks] = pack8(t[j]);
        }
      }
    }
  }

  // ---- streaming top-K state
  uint64_t* hp = &heap[w][0][lane];   // own heap entry j at hp[64 * j]
  uint64_t* qp = &queue[w][0][lane];
  int cnt = 0;                         // entries in the own heap
  uint64_t root = 0;                   // own K-th best (valid when cnt == K)

  const float* kcb = kc + (int64_t)bh * C * D;
  const float* bcb = bc + (int64_t)bh * C;
  const int ntiles = (Pmax + ST_TILE - 1) / ST_TILE;
  for (int t = 0; t < ntiles; ++t) {
    const int c0 = t * ST_TILE;
    __syncthreads();  // previous tile fully consumed
    // stage k' (fp32 -> NK bf16 planes) and b'
    for (int i = tid * 4; i < ST_TILE * D; i += 256 * 4) {
      const int ch = i / D, e = i % D;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + ch < Pmax) v = *reinterpret_cast<const float4*>(kcb + (int64_t)(c0 + ch) * D + e);
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
        *reinterpret_cast<u32x2_t*>(&kt[j][ch * LDK + e]) = pk;
      }
    }
    if (tid < ST_TILE) bt[tid] = (c0 + tid < Pmax) ? bcb[c0 + tid] : 0.f;
    __syncthreads();

#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x16_t acc = zero16();
      const int ch = 32 * tt + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          const uint16_t* kr = &kt[j][ch * LDK + 16 * ks + 4 * hf];
          const bf16x8_t a = pack8(*reinterpret_cast<const u32x2_t*>(kr), *reinterpret_cast<const u32x2_t*>(kr + 8));
#pragma unroll
          for (int i = 0; i < NQ; ++i)
            if (i + j < (NQ > NK ? NQ : NK)) acc = mfma32(a, qb[i][ks], acc);
        }
      }
      // filter this lane's 16 candidates against both halves' K-th best, queue them
      const uint32_t plo = __shfl_xor((uint32_t)root, 32), phi = __shfl_xor((uint32_t)(root >> 32), 32);
      const uint64_t proot = ((uint64_t)phi << 32) | plo;
      const bool pfull = __shfl_xor(cnt, 32) == K;
      int qn = 0;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int cl = 32 * tt + acc_row(rr, hf);
        const int c = c0 + cl;
        const float s = fmaf(acc[rr], tau, bt[cl]);
        const uint64_t x = make_key(s, c);
        const bool pass = (c < P_row) && (cnt < K || x > root) && (!pfull || x > proot);
        if (pass) {
          qp[64 * qn] = x;
          ++qn;
        }
      }
      const int qmax = wave_max_i(qn);
      for (int j = 0; j < qmax; ++j) {
        if (j < qn) {
          const uint64_t x = qp[64 * j];
          if (cnt < K) {  // fill: sift up
            int pos = cnt++;
            while (pos > 0) {
              const int par = (pos - 1) >> 1;
              const uint64_t pk = hp[64 * par];
              if (pk <= x) break;
              hp[64 * pos] = pk;
              pos = par;
            }
            hp[64 * pos] = x;
          } else if (x > root) {  // replace the K-th best: sift down
            int pos = 0;
            while (true) {
              int ch2 = 2 * pos + 1;
              if (ch2 >= K) break;
              uint64_t ck = hp[64 * ch2];
              if (ch2 + 1 < K) {
                const uint64_t c2 = hp[64 * (ch2 + 1)];
                if (c2 < ck) {
                  ck = c2;
                  ++ch2;
                }
              }
              if (ck >= x) break;
              hp[64 * pos] = ck;
              pos = ch2;
            }
            hp[64 * pos] = x;
          }
          root = (cnt == K) ? hp[0] : 0;
        }
      }
    }
  }

  // ---- heap-sort the own heap into rank order (best first)
  for (int end = cnt - 1; end > 0; --end) {
    const uint64_t top = hp[0];
    const uint64_t x = hp[64 * end];
    hp[64 * end] = top;
    int pos = 0;
    while (true) {
      int ch2 = 2 * pos + 1;
      if (ch2 >= end) break;
      uint64_t ck = hp[64 * ch2];
      if (ch2 + 1 < end) {
        const uint64_t c2 = hp[64 * (ch2 + 1)];
        if (c2 < ck) {
          ck = c2;
          ++ch2;
        }
      }
      if (ck >= x) break;
      hp[64 * pos] = ck;
      pos = ch2;
    }
    hp[64 * pos] = x;
  }
  const int pcnt = __shfl_xor(cnt, 32);
  __syncthreads();
  // ---- lane half 0 merges both halves into the query's top K
  if (hf == 0 && row_ok) {
    const uint64_t* pp = &heap[w][0][lane + 32];
    int ia = 0, ib = 0;
    int32_t* oi = sel_idx + ((int64_t)bh * N + row) * K;
    float* os = sel_score + ((int64_t)bh * N + row) * K;
    for (int t = 0; t < K; ++t) {
      const uint64_t xa = ia < cnt ? hp[64 * ia] : 0;
      const uint64_t xb = ib < pcnt ? pp[64 * ib] : 0;
      uint64_t x;
      if (xa >= xb) {
        x = xa;
        ++ia;
      } else {
        x = xb;
        ++ib;
      }
      oi[t] = x ? key_chunk(x) : -1;
      os[t] = x ? key_score(x) : -INFINITY;
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

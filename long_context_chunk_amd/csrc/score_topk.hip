// Chunk scoring and top-K for prefill queries.
//
//   s_ic = q^_i . k'_c / sqrt(d) + b'_c   for every candidate chunk c < floor(i/S) - (nw - 1)
//                                        (the complete chunks before the local window of nw chunks)
//   q^_i = q_i + U_h (D_h q_i)             (Q-Cal; q^ = q without it)
// keep the K best (ties -> lower chunk id).  (aitrends.kr article,
// "Methodology": the score formula, the calculation flow and the Q-Cal module.)
//
// Two passes over the past chunks, both on v_mfma_f32_32x32x16_bf16, one workgroup per
// 128 consecutive queries of one (batch, head) (32 per wave), with k' tiles staged
// through LDS and shared by the four waves:
//
//   1. score_threshold (queries = M, chunks = N: accumulator register r of a lane holds
//      one chunk's score for one row; the 32 lanes of a half-wave cover 32 chunks of
//      that row): one bf16 product per score, bf16(q^/sqrt(d)) . bf16(k'_c), with b'_c
//      and an error allowance e_i |k'_c| folded into one extra MFMA k-step, so every
//      value is at most the fp32-accurate score of pass 2.  Each lane keeps the two
//      largest values of its column of chunks; the K-th largest of these 64 values of
//      distinct chunks is a threshold theta_i that the row's K-th best score can not
//      be below.
//   2. score_topk_kernel (chunks = M, queries = N: each lane owns one row's scores):
//      the scores to ~2^-17 relative (tau k' split into bf16 hi + lo terms, q^ too
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
#include "kernels.h"

namespace hils {

constexpr int ST_ROWS = 128;   // queries per workgroup
constexpr int ST_TILE = 64;    // chunks per LDS tile

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

// For R registers at once: the K-th largest of the 64 values {a, b} of each 32-lane half,
// left in lane K - 1 of the half (a is overwritten with the half's 32 largest, sorted).
template <int R>
HILS_DEV void kth_of_pairs_r(float (&a)[R], float (&b)[R], int j, float pinf, float ninf) {
  sort32f_r<R>(a, j, pinf, ninf);
  sort32f_r<R>(b, j, pinf, ninf);
#pragma unroll
  for (int i = 0; i < R; ++i) a[i] = __builtin_amdgcn_fmed3f(a[i], xl1<31>(b[i]), pinf);  // the 32 largest, bitonic
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

// q^ = q + U_h (D_h q) of this lane's row (zero when !row_ok), delivered one MFMA
// k-step at a time in the A-operand layout: sink(ks, v) gets v[m] = q^[kperm(ks, hf, m)].
// Q-Cal runs on the MFMA (T = D q, then U T), chained through the accumulator layout.
template <typename IO, int D, bool QCAL, typename Sink>
HILS_DEV void qhat_rows(const IO* __restrict__ q, const IO* __restrict__ Dw, const IO* __restrict__ Uw, int hh, int r,
                        int64_t qrow, bool row_ok, int lane, Sink&& sink) {
  constexpr int NKS = D / 16;
  constexpr int NIO = io_traits<IO>::terms;
  const int hf = lane >> 5;
  auto load8 = [&](int ks, float(&v)[8]) {
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
      v[m] = a4[m];
      v[4 + m] = b4[m];
    }
  };
  if constexpr (!QCAL) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float v[8];
      load8(ks, v);
      sink(ks, v);
    }
  } else {
    // raw q terms (exact: NIO bf16 terms carry an io value exactly), as B operands
    bf16x8_t qr[NIO][NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float v[8];
      load8(ks, v);
      u32x4_t t[NIO];
      split8<NIO>(v, t);
#pragma unroll
      for (int j = 0; j < NIO; ++j) qr[j][ks] = __builtin_bit_cast(bf16x8_t, t[j]);
    }
    // T^T[a][row] = sum_e D[a][e] q[row][e]   (a < r; rows a >= r are zero)
    f32x16_t T = zero16();
    const int a_row = lane & 31;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4_t dt[NIO];
      float dv[8];
      {
        float a4[4], b4[4];
        const int64_t drow = ((int64_t)hh * r + min(a_row, r - 1)) * D;  // clamped: no divergent loads
        io_traits<IO>::load4(Dw, drow + kperm(ks, hf, 0), a4);
        io_traits<IO>::load4(Dw, drow + kperm(ks, hf, 4), b4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          dv[m] = a_row < r ? a4[m] : 0.f;
          dv[4 + m] = a_row < r ? b4[m] : 0.f;
        }
      }
      split8<NIO>(dv, dt);
#pragma unroll
      for (int i = 0; i < NIO; ++i)
#pragma unroll
        for (int j = 0; j < NIO; ++j)
          if (i + j < NIO) T = mfma32(__builtin_bit_cast(bf16x8_t, dt[i]), qr[j][ks], T);
    }
    // T as the B operand of U T: accumulator register 8*ks2 + m -> k-step ks2, element m
    constexpr int NT = NIO == 1 ? 2 : 3;
    bf16x8_t tb[NT][2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      float tv[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) tv[m] = T[8 * ks2 + m];
      u32x4_t t[NT];
      split8<NT>(tv, t);
#pragma unroll
      for (int j = 0; j < NT; ++j) tb[j][ks2] = __builtin_bit_cast(bf16x8_t, t[j]);
    }
    constexpr int NP = NIO > NT ? NIO : NT;
#pragma unroll
    for (int dt2 = 0; dt2 < D / 32; ++dt2) {
      f32x16_t Q = zero16();
      const int e = 32 * dt2 + (lane & 31);
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        float uv[8];
        const int64_t urow = ((int64_t)hh * D + e) * r;
        if ((r & 3) == 0) {  // 4-aligned rows: two vector loads
          float a4[4], b4[4];
          io_traits<IO>::load4(Uw, urow + min(kperm(ks2, hf, 0), r - 4), a4);
          io_traits<IO>::load4(Uw, urow + min(kperm(ks2, hf, 4), r - 4), b4);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            uv[m] = kperm(ks2, hf, m) < r ? a4[m] : 0.f;
            uv[4 + m] = kperm(ks2, hf, 4 + m) < r ? b4[m] : 0.f;
          }
        } else {
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int a = kperm(ks2, hf, m);
            const float x = io_traits<IO>::load(Uw, urow + min(a, r - 1));
            uv[m] = a < r ? x : 0.f;
          }
        }
        u32x4_t ut[NIO];
        split8<NIO>(uv, ut);
#pragma unroll
        for (int i = 0; i < NIO; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            if (i + j < NP) Q = mfma32(__builtin_bit_cast(bf16x8_t, ut[i]), tb[j][ks2], Q);
      }
      // register rr of this tile is head dim 32*dt2 + acc_row(rr, hf) = k-step 2*dt2 + rr/8, element rr%8
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ks = 2 * dt2 + half;
        float v[8];
        load8(ks, v);  // reload the raw q slice (cheaper than keeping it live)
#pragma unroll
        for (int m = 0; m < 8; ++m) v[m] += Q[8 * half + m];
        sink(ks, v);
      }
    }
  }
}

// ------------------------------------------------------------- threshold pass
// Error allowance of the one-product scores: with u = 2^-8 (bf16 rounding),
// |bf(x) bf(y) - x y| <= (2u + u^2) |x y|, so over the head dimension the product
// error is at most (2u + u^2) |tau q^| |k'| (Cauchy-Schwarz); TH_REL exceeds 2u + u^2
// by enough to cover pass 2's own ~2^-16 relative error and fp32 accumulation, and
// TH_ABS covers the two-term split of b'.
constexpr float TH_REL = 0.008f;
constexpr float TH_ABS = 1.0f / 4096.0f;   // bf16 0x3980
constexpr int TH_EXT = 16;                  // elements of the extension k-step

template <typename IO, int D, bool QCAL>
__global__ void __launch_bounds__(256, 2) score_threshold(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                          const IO* __restrict__ Uw, const uint16_t* __restrict__ t1,
                                                          float* __restrict__ theta, int H, int N, int C, int K, int r,
                                                          int NB, int items, int nw) {
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
  const int hh = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int r0 = rb * ST_ROWS;
  const int row = r0 + 32 * w + n;
  const bool row_ok = row < N;
  const int last = min(r0 + ST_ROWS, N) - 1;
  const int Pmax = candidate_chunks(last, C, nw);
  const int Pmin = candidate_chunks(r0, C, nw);
  const float tau = 1.0f / sqrtf((float)D);
  const int64_t qrow = ((int64_t)bh * N + (row_ok ? row : 0)) * D;

  // A operands: bf16(tau q^), then the extension step [1, 1, -1, -e_i] against the
  // chunk's [b'_hi, b'_lo, TH_ABS, |k'_c| rounded up], e_i = TH_REL |tau q^_i| rounded up
  bf16x8_t qa[NKS + 1];
  float ss = 0.f;
  qhat_rows<IO, D, QCAL>(q, Dw, Uw, hh, r, qrow, row_ok, lane, [&](int ks, const float(&v)[8]) {
    float x[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      x[m] = v[m] * tau;
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
      t[3] = (uint16_t)(bf16_up(TH_REL * sqrtf(ss)) | 0x8000u);
    }
    qa[NKS] = pack8(t);
  }

  const uint16_t* src = t1 + (int64_t)bh * C * DE;
  u32x4_t pf[PL];
  // chunks beyond Pmax load chunk Pmax-1 (finite; masked out below); the last partial
  // group of segments repeats the final segment: no divergent loads
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int it = min(tid + 256 * u, NSEG - 1);
      const int e = it / SEGS, sg = it % SEGS;
      const int c = min(t * ST_TILE + e, Pmax - 1);
      pf[u] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)c * DE + 8 * sg);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int it = min(tid + 256 * u, NSEG - 1);
      const int e = it / SEGS, sg = it % SEGS;
      *reinterpret_cast<u32x4_t*>(&kt[buf][e * LDT + 8 * sg]) = pf[u];
    }
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
  // every row (the half of a last tile past Pmax holds copies of chunk Pmax - 1 and is
  // masked out with them).  Masked and unmasked tiles run in separate loops: one loop
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
          const int prow = rw < N ? candidate_chunks(rw, C, nw) : 0;
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
  kth_of_pairs_r<16>(m1, m2, n, pinf, ninf);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int rw = r0 + 32 * w + acc_row(rr, hf);
    const float t0 = readlane_f(m1[rr], K - 1), t1 = readlane_f(m1[rr], 32 + K - 1);
    const float th = hf ? t1 : t0;
    if (n == 0 && rw < N) theta[(int64_t)bh * N + rw] = th;
  }
}


// ------------------------------------------------------------- selection pass
// S^T = k' q^T on the MFMA: k' rows (chunks) are the A operand, the queries the B
// operand, so accumulator register r of lane l holds the score of chunk
// acc_row(r, l >> 5) of the 32-chunk tile for query row l & 31.  Each lane therefore
// owns one row's scores and appends its passing candidates to its own half of the
// row's list (LDS) with a per-lane fill: no cross-lane bookkeeping per score.
// tau is folded into the k' planes and b' (three exact bf16 terms) enters through an
// extra k-step against a constant [1, 1, 1, 0 ...] query operand.
constexpr int SEL_CT = 32;     // chunks per column tile (single LDS buffer)
constexpr int SEL_HALF = 32;   // candidate slots per half-row list (plus one spill slot)
constexpr int P2_EXT = 16;     // extension elements after plane 0: [b'_hi, b'_mid, b'_lo, 0 ...]

template <typename IO, int D, int NQ, int NK, bool QCAL>
__global__ void __launch_bounds__(256, NQ * NK > 4 ? 1 : 2) score_topk_kernel(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                             const IO* __restrict__ Uw,
                                                             const uint16_t* __restrict__ p2,
                                                             const float* __restrict__ theta,
                                                             int32_t* __restrict__ sel_idx,
                                                             float* __restrict__ sel_score, int H, int N, int C, int K,
                                                             int r, int NB, int items, int nw) {
  constexpr int NKS = D / 16;
  constexpr int DE2 = NK * D + P2_EXT;  // elements of a chunk row: plane 0, extension, planes 1..
  constexpr int LDR = DE2 + 8;          // LDS row stride (16-byte pad)
  constexpr int SEGS = DE2 / 8;
  constexpr int NSEG = SEL_CT * SEGS;
  constexpr int PL = (NSEG + 255) / 256;
  constexpr int HSTR = SEL_HALF + 1;    // half-list stride: SEL_HALF slots + a spill slot
  constexpr int LIST = 2 * HSTR;        // slots per row
  __shared__ __align__(16) uint16_t kt[SEL_CT * LDR];
  __shared__ float cs[ST_ROWS * LIST + 256];      // candidate scores; the last 256 are per-lane sinks
  __shared__ uint16_t ci[ST_ROWS * LIST + 256];   // candidate chunks

  const int item = remap_xcd(blockIdx.x, items);
  if (item >= items) return;
  const int bh = item / NB;
  const int rb = NB - 1 - (item % NB);  // heavier (later) row blocks first
  const int hh = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int r0 = rb * ST_ROWS;
  const int row = r0 + 32 * w + n;       // this lane's query row
  const bool row_ok = row < N;
  const int last = min(r0 + ST_ROWS, N) - 1;
  const int Pmax = candidate_chunks(last, C, nw);
  const int Pmin = candidate_chunks(r0, C, nw);
  const int prow = row_ok ? candidate_chunks(row, C, nw) : 0;   // candidate chunks of this lane's row
  const int64_t qrow = ((int64_t)bh * N + (row_ok ? row : 0)) * D;

  // ---- the query's B operands: q^ split into NQ bf16 terms, plus the constant extension
  bf16x8_t qb[NQ][NKS];
  qhat_rows<IO, D, QCAL>(q, Dw, Uw, hh, r, qrow, row_ok, lane, [&](int ks, const float(&v)[8]) {
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
  // and this half's list position lf (absolute slot index, lbase + fill); rows beyond
  // N take +inf and never collect anything
  float th = row_ok ? theta[(int64_t)bh * N + row] : INFINITY;
  const int lrow = 32 * w + n;           // row within the workgroup
  const int lbase = lrow * LIST + hf * HSTR;
  const int lcap = lbase + SEL_HALF;     // the spill slot
  const int sink = ST_ROWS * LIST + tid;
  int lf = lbase;

  // Sort the lists of rows ra (lanes 0..31) and rb_ (lanes 32..63) of this wave as
  // selection keys (lane j holds slot j of each half list), keep the best K (lane j =
  // j-th best) and optionally write them back split over the two half lists.
  auto settle2 = [&](int ra, int rb2, bool write_back, uint64_t& lk, int& nvalid) {
    const int rw = hf ? rb2 : ra;
    const int myfill = lf - lbase;
    const int f0 = min(__shfl(myfill, rw), SEL_HALF), f1 = min(__shfl(myfill, 32 + rw), SEL_HALF);
    const int base = (32 * w + rw) * LIST;
    uint64_t x = 0, y = 0;
    if (n < f0) x = make_key(cs[base + n], ci[base + n]);
    if (n < f1) y = make_key(cs[base + HSTR + n], ci[base + HSTR + n]);
    sort32k(x, n);
    merge_intok(x, y, n, K);
    const uint64_t vm = __ballot(x != 0);
    nvalid = __popc(hf ? (uint32_t)(vm >> 32) : (uint32_t)vm);
    if (write_back && n < K) {  // best (K+1)/2 to half 0, the rest to half 1
      const int kh = (K + 1) >> 1;
      const int slot = n < kh ? n : HSTR + n - kh;
      cs[base + slot] = key_score(x);
      ci[base + slot] = (uint16_t)key_chunk(x);
    }
    lk = x;
  };

  const uint16_t* src = p2 + (int64_t)bh * C * DE2;
  u32x4_t pf[PL];
  // chunks beyond Pmax load chunk Pmax-1 (finite; masked out below) and the last
  // partial group of segments repeats the final segment: no divergent loads
  auto load_tile = [&](int ct) {
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int it = min(tid + 256 * u, NSEG - 1);
      const int e = it / SEGS, sg = it % SEGS;
      const int c = min(ct * SEL_CT + e, Pmax - 1);
      pf[u] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)c * DE2 + 8 * sg);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int it = min(tid + 256 * u, NSEG - 1);
      const int e = it / SEGS, sg = it % SEGS;
      *reinterpret_cast<u32x4_t*>(&kt[e * LDR + 8 * sg]) = pf[u];
    }
  };

  // the scores of the tile in LDS (chunk n of the tile is the A operand row)
  auto tile_scores = [&]() {
    f32x16_t a_ = zero16();
    const uint16_t* krow = &kt[n * LDR];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + j * D + (j ? P2_EXT : 0) + 16 * ks + 8 * hf);
#pragma unroll
        for (int i = 0; i < NQ; ++i)
          if (i + j < (NQ > NK ? NQ : NK)) a_ = mfma32(a, qb[i][ks], a_);
      }
    return mfma32(*reinterpret_cast<const bf16x8_t*>(krow + D + 8 * hf), qext, a_);  // + b'
  };

  // Software pipeline: while tile ct's scores are tested and appended, the MFMAs of
  // tile ct + 1 (already staged in LDS) run; tile ct + 2 is in flight from memory.
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
    f32x16_t acc_next;
    // candidates: s >= th goes to this lane's half list.  A full list takes further
    // candidates in its spill slot (lost for now); the row is compacted after the tile
    // and the lost ones are appended again against the raised threshold.
    const int cb = ct * SEL_CT + 4 * hf;
    const int lf_start = lf;
    const float th_old = th;
    auto score_at = [&](int rr, auto masked_tag) {
      float s = acc[rr];
      if constexpr (decltype(masked_tag)::value) {
        if (cb + 8 * (rr >> 2) + (rr & 3) >= prow) s = __builtin_nanf("");
      }
      return s;
    };
    auto append_all = [&](auto masked_tag) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float s = score_at(rr, masked_tag);
        const bool pass = s >= th;   // NaN never passes
        const int pos = pass ? min(lf, lcap) : sink;
        cs[pos] = s;
        ci[pos] = (uint16_t)(cb + 8 * (rr >> 2) + (rr & 3));
        lf += pass ? 1 : 0;
      }
    };
    auto reappend_lost = [&](auto masked_tag) {
      int running = lf_start;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float s = score_at(rr, masked_tag);
        const bool was = s >= th_old;
        running += was ? 1 : 0;
        if (was && running > lcap && s >= th) {  // at most 16 after a compaction to <= 16
          cs[lf] = s;
          ci[lf] = (uint16_t)(cb + 8 * (rr >> 2) + (rr & 3));
          ++lf;
        }
      }
    };
    // The MFMAs of tile ct + 1 (past the last tile they recompute the last one; never
    // used) and the appends of tile ct in one block, interleaved one MFMA per score, so
    // the matrix core works while the vector unit appends.
    auto scores_and_append = [&](auto masked_tag) {
      acc_next = tile_scores();
      append_all(masked_tag);
      if constexpr (NQ * NK <= 4)  // the fp32 path has too few registers left to interleave
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // the VALU of one append
        __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);   // its two LDS writes
      }
    };
    const bool masked = (ct + 1) * SEL_CT > Pmin;  // chunks >= Pmin are not past chunks of every row
    if (masked)
      scores_and_append(std::true_type{});
    else
      scores_and_append(std::false_type{});
    const uint64_t ovf = __ballot(lf > lcap);
    if (ovf) {  // rare: compact the rows with a full half list, then re-append what was lost
      uint32_t rows_big = (uint32_t)ovf | (uint32_t)(ovf >> 32);
      const int kh = (K + 1) >> 1;
      while (rows_big) {
        const int ra = __builtin_ctz(rows_big);
        rows_big &= rows_big - 1;
        int rb2 = ra;
        const bool two = rows_big != 0;
        if (two) {
          rb2 = __builtin_ctz(rows_big);
          rows_big &= rows_big - 1;
        }
        uint64_t lk;
        int nv;
        settle2(ra, rb2, true, lk, nv);
        // new fills and thresholds of the two rows (half 0 of the wave did row ra, half 1 row rb2)
        const int nva = __shfl(nv, 0), nvb = __shfl(nv, 32);
        const uint64_t kka = __shfl(lk, K - 1), kkb = __shfl(lk, 32 + K - 1);
        const float ka = kka ? key_score(kka) : -INFINITY, kb = kkb ? key_score(kkb) : -INFINITY;
        if (n == ra) {
          lf = lbase + (hf ? max(0, nva - kh) : min(nva, kh));
          th = fmaxf(th, ka);
        }
        if (two && n == rb2) {
          lf = lbase + (hf ? max(0, nvb - kh) : min(nvb, kh));
          th = fmaxf(th, kb);
        }
      }
      if (masked)
        reappend_lost(std::true_type{});
      else
        reappend_lost(std::false_type{});
    }
    __syncthreads();  // every wave is done with tile ct + 1 in LDS
    if (more2) store_tile();
    __syncthreads();
    acc = acc_next;
  }

  // ---- final selection and output: eight row pairs (p, p + 16) at a time, the two half
  // lists of a row sorted as keys and merged to the best K; lane j of each half writes slot j
  constexpr int FR = NQ * NK > 4 ? 4 : 8;  // fewer at once where the score operands take more registers
  const int myfill = lf - lbase;
#pragma unroll 1
  for (int p0 = 0; p0 < 16; p0 += FR) {
    uint64_t x[FR], y[FR];
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int rw = hf ? p0 + i + 16 : p0 + i;
      const int f0 = min(__shfl(myfill, rw), SEL_HALF), f1 = min(__shfl(myfill, 32 + rw), SEL_HALF);
      const int base = (32 * w + rw) * LIST;
      x[i] = n < f0 ? make_key(cs[base + n], ci[base + n]) : 0ull;
      y[i] = n < f1 ? make_key(cs[base + HSTR + n], ci[base + HSTR + n]) : 0ull;
    }
    sort32k_r<FR>(x, n);
    sort32k_r<FR>(y, n);
#pragma unroll
    for (int i = 0; i < FR; ++i) {  // the 32 best of both lists, a bitonic sequence
      const uint64_t r = xl64<31>(y[i]);
      x[i] = r > x[i] ? r : x[i];
    }
    cxk_r<16, FR>(x, (n & 16) == 0);
    cxk_r<8, FR>(x, (n & 8) == 0);
    cxk_r<4, FR>(x, (n & 4) == 0);
    cxk_r<2, FR>(x, (n & 2) == 0);
    cxk_r<1, FR>(x, (n & 1) == 0);
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int rw = r0 + 32 * w + (hf ? p0 + i + 16 : p0 + i);
      if (rw < N && n < K) {
        const int64_t o = ((int64_t)bh * N + rw) * K + n;
        const bool ok = x[i] != 0;
        sel_idx[o] = ok ? key_chunk(x[i]) : -1;
        sel_score[o] = ok ? key_score(x[i]) : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------- k' preparation
// k' (fp32) -> (a) the selection pass's rows: tau*k' split into NK bf16 term planes with
// the extension [b'_hi, b'_mid, b'_lo, 0 ...] after plane 0, and (b) the threshold pass's
// rows: bf16(k') followed by [b'_hi, b'_lo, TH_ABS, |k'_c| rounded up, 0 ...].  Both hold
// each 16-element k-block in MFMA operand order: position 16 ks + 8 h + m holds element
// kperm(ks, h, m).
template <int D, int NK>
__global__ void __launch_bounds__(256) prep_kprime(const float* __restrict__ kc, const float* __restrict__ bc,
                                                   uint16_t* __restrict__ p2, uint16_t* __restrict__ t1,
                                                   int64_t rows) {
  constexpr int SPR = D / 8;        // 16-byte segments (threads) per chunk row
  constexpr int RPB = 256 / SPR;    // chunk rows per workgroup pass
  constexpr int DE = D + TH_EXT;
  constexpr int DE2 = NK * D + P2_EXT;
  const float tau = 1.0f / sqrtf((float)D);
  const int tid = threadIdx.x;
  const int sg = tid % SPR, ks = sg >> 1, h = sg & 1;
  for (int64_t base = (int64_t)blockIdx.x * RPB; base < rows; base += (int64_t)gridDim.x * RPB) {
    const int64_t rw = base + tid / SPR;
    const bool ok = rw < rows;
    float x[8];
    if (ok) {
      const float4 a = *reinterpret_cast<const float4*>(kc + rw * D + kperm(ks, h, 0));
      const float4 b = *reinterpret_cast<const float4*>(kc + rw * D + kperm(ks, h, 4));
      x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = 0.f;
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
      xh[m] = x[m];
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
          const float bv = bc[rw];
          uint16_t sp3[3], sp2[2];
          split_bf16<3>(bv, sp3);
          split_bf16<2>(bv, sp2);
          e[0] = sp2[0];
          e[1] = sp2[1];
          e[2] = f32_to_bf16(TH_ABS);  // 2^-12, exact in bf16 (0x3980)
          e[3] = bf16_up(sqrtf(s2));
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

struct ScoreWs {
  size_t planes, t1, theta, total;
};
static ScoreWs score_ws(const Geom& g) {
  const size_t rows = (size_t)g.B * g.Hq * g.C();
  ScoreWs w;
  size_t off = 0;
  w.planes = off;
  off += al3(rows * ((size_t)nk_of(g) * g.d + P2_EXT) * 2);
  w.t1 = off;
  off += al3(rows * (g.d + TH_EXT) * 2);
  w.theta = off;
  off += al3((size_t)g.B * g.Hq * g.N * 4);
  w.total = off;
  return w;
}

size_t score_workspace_bytes(const Geom& g) { return score_ws(g).total; }

template <typename IO, int D, int NQ, int NK, bool QCAL>
static void launch_st(const Geom& g, const void* q, const void* Dw, const void* Uw, const uint16_t* planes,
                      const uint16_t* t1, float* theta, const float* bc, int32_t* si, float* ss, hipStream_t st,
                      hipEvent_t* ev) {
  const int NB = (g.N + ST_ROWS - 1) / ST_ROWS;
  const int items = g.B * g.Hq * NB;
  const int grid = ((items + 7) / 8) * 8;
  hipLaunchKernelGGL((score_threshold<IO, D, QCAL>), dim3(grid), dim3(256), 0, st, (const IO*)q, (const IO*)Dw,
                     (const IO*)Uw, t1, theta, g.Hq, g.N, g.C(), g.K, g.r, NB, items, g.nw);
  if (ev) hipEventRecord(ev[0], st);
  hipLaunchKernelGGL((score_topk_kernel<IO, D, NQ, NK, QCAL>), dim3(grid), dim3(256), 0, st, (const IO*)q,
                     (const IO*)Dw, (const IO*)Uw, planes, (const float*)theta, si, ss, g.Hq, g.N, g.C(), g.K, g.r,
                     NB, items, g.nw);
}

template <typename IO, int D>
static void launch_st_d(const Geom& g, const void* q, const void* Dw, const void* Uw, const uint16_t* planes,
                        const uint16_t* t1, float* theta, const float* bc, int32_t* si, float* ss, hipStream_t st,
                        hipEvent_t* ev) {
  constexpr bool F32 = io_traits<IO>::terms == 3;
  if (g.r > 0)
    launch_st<IO, D, F32 ? 3 : 2, F32 ? 3 : 2, true>(g, q, Dw, Uw, planes, t1, theta, bc, si, ss, st, ev);
  else
    launch_st<IO, D, F32 ? 3 : 1, F32 ? 3 : 2, false>(g, q, Dw, Uw, planes, t1, theta, bc, si, ss, st, ev);
}

template <int D>
static void launch_prep(const Geom& g, const float* kc, const float* bc, uint16_t* planes, uint16_t* t1,
                        hipStream_t st) {
  const int64_t rows = (int64_t)g.B * g.Hq * g.C();
  const int64_t rpb = 256 / (D / 8);
  const unsigned gs = (unsigned)std::min<int64_t>((rows + rpb - 1) / rpb, 16384);
  if (nk_of(g) == 3)
    hipLaunchKernelGGL((prep_kprime<D, 3>), dim3(gs), dim3(256), 0, st, kc, bc, planes, t1, rows);
  else
    hipLaunchKernelGGL((prep_kprime<D, 2>), dim3(gs), dim3(256), 0, st, kc, bc, planes, t1, rows);
}

hipError_t launch_score_topk(const Geom& g, const void* q, const void* Dw, const void* Uw, const float* kc,
                             const float* bc, int32_t* sel_idx, float* sel_score, void* ws, size_t ws_bytes,
                             hipStream_t st, hipEvent_t* ev) {
  if (ws_bytes < score_workspace_bytes(g)) return hipErrorInvalidValue;
  const ScoreWs w = score_ws(g);
  uint16_t* planes = (uint16_t*)((char*)ws + w.planes);
  uint16_t* t1 = (uint16_t*)((char*)ws + w.t1);
  float* theta = (float*)((char*)ws + w.theta);
  if (g.C() > 0) {
    if (g.d == 64)
      launch_prep<64>(g, kc, bc, planes, t1, st);
    else
      launch_prep<128>(g, kc, bc, planes, t1, st);
  }
  if (g.io == 0) {
    if (g.d == 64)
      launch_st_d<float, 64>(g, q, Dw, Uw, planes, t1, theta, bc, sel_idx, sel_score, st, ev);
    else
      launch_st_d<float, 128>(g, q, Dw, Uw, planes, t1, theta, bc, sel_idx, sel_score, st, ev);
  } else {
    if (g.d == 64)
      launch_st_d<bf16_t, 64>(g, q, Dw, Uw, planes, t1, theta, bc, sel_idx, sel_score, st, ev);
    else
      launch_st_d<bf16_t, 128>(g, q, Dw, Uw, planes, t1, theta, bc, sel_idx, sel_score, st, ev);
  }
  if (ev) hipEventRecord(ev[1], st);
  return hipGetLastError();
}

}  // namespace hils

// Dense causal attention: the baseline the sparse pass is measured against (hotpaper.ai
// abstract; ai-papers.net "Results": the speed-up over full attention grows with the
// context), built from the same MFMA tiles as the chunk attention so the comparison is
// between two kernels of one implementation.
//
//   o_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(d)) v_j      per (b, h), query head h
//                                                              reading KV head h / (Hq/Hkv)
//
// One workgroup per 128 consecutive queries of one (b, h), 32 per wave.  The keys are
// walked in 64-key tiles staged in LDS (K natural, V through transposing reads) and
// shared by the four waves; each wave keeps an online softmax (running max m, sum l and
// unnormalised O^T accumulators rescaled when m grows).  The G query heads of one KV
// head run as consecutive workgroups, so a K/V tile is fetched from HBM once and reused
// from L2; the longest (latest) query blocks start first.
#include "attn_tile.h"
#include "hils_common.h"
#include "kernels.h"

namespace hils {

constexpr int DN_ROWS = 128;  // query rows per workgroup

template <typename IO, int D>
__global__ void __launch_bounds__(256, 2) dense_attend(const IO* __restrict__ q, const IO* __restrict__ k,
                                                       const IO* __restrict__ v, IO* __restrict__ o, int Hq, int Hkv,
                                                       int N, int nqb) {
  constexpr int NT = io_traits<IO>::terms;
  constexpr int NKS = D / 16;
  constexpr int LDK = KVTile<IO, D, NT>::LDK, LDV = KVTile<IO, D, NT>::LDV;
  __shared__ KVTile<IO, D, NT> tile;
  const int G = Hq / Hkv;
  const int gi = blockIdx.x % G, rest = blockIdx.x / G;
  const int qb = nqb - 1 - rest % nqb, bkv = rest / nqb;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int64_t bh = (int64_t)b * Hq + kvh * G + gi;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5;
  const int r0 = qb * DN_ROWS;
  const int i = r0 + 32 * w + (lane & 31);  // this lane's query row (column of the tiles)
  const bool ok = i < N;
  const int wave_last = min(N - 1, r0 + 32 * w + 31);
  const int wave_first = r0 + 32 * w;
  const int64_t kv0 = ((int64_t)b * Hkv + kvh) * N;
  bf16x8_t qop[NT][NKS];
  load_q_operand<IO, D, NT>(q, (bh * N + (ok ? i : 0)) * D, ok, qop);
  const float tau = 1.0f / sqrtf((float)D);
  const float c = tau * 1.44269504088896340736f;  // tau log2(e)
  float m = -INFINITY, l = 0.f;
  f32x16_t acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
  const int ntile = (min(N, r0 + DN_ROWS) + 63) / 64;
  for (int t = 0; t < ntile; ++t) {
    const int key0 = 64 * t;
    __syncthreads();  // every wave is done with the previous tile
    stage_kv<IO, D, NT>(tile, k, v, kv0 + key0, min(64, N - key0), tid, 256);
    __syncthreads();
    if (key0 > wave_last) continue;  // past the diagonal of all this wave's rows
    f32x16_t s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = zero16();
      const int key = 32 * tt + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const bf16x8_t a = lds_op16(&tile.k[j][key * LDK + 16 * ks + 8 * hf]);
#pragma unroll
          for (int i2 = 0; i2 < NT; ++i2)
            if (i2 + j < NT) s[tt] = mfma32(a, qop[i2][ks], s[tt]);
        }
    }
    if (key0 + 63 > wave_first) {  // the tile crosses the diagonal: key j is used iff j <= i
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (key0 + 32 * tt + acc_row(rr, hf) > i) s[tt][rr] = -INFINITY;
    }
    float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int rr = 2; rr < 32; ++rr) mt = fmaxf(mt, s[rr >> 4][rr & 15]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // key 0 is in every row's first tile, so m is finite from then on; a later tile whose
    // keys are all masked for a row leaves mn = m (alpha = 1, p = 0)
    const float mn = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f((m - mn) * c);  // 0 on the first tile
    const float mc = mn * c;
    float lt = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[tt][rr], c, -mc));
        s[tt][rr] = p;
        lt += p;
      }
    lt += __shfl_xor(lt, 32);
    l = fmaf(l, alpha, lt);
    m = mn;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) acc[dt][rr] *= alpha;
    bf16x8_t pb[NT][4];
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      float pv[8];
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) pv[mm] = s[ks2 >> 1][8 * (ks2 & 1) + mm];
      u32x4_t tsp[NT];
      split8<NT>(pv, tsp);
#pragma unroll
      for (int j = 0; j < NT; ++j) pb[j][ks2] = __builtin_bit_cast(bf16x8_t, tsp[j]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const bf16x8_t a = vt_operand<LDV>(tile.v[j], dt, ks2, lane);
#pragma unroll
          for (int i2 = 0; i2 < NT; ++i2)
            if (i2 + j < NT) acc[dt] = mfma32(a, pb[i2][ks2], acc[dt]);
        }
  }
  if (!ok) return;
  const float inv = 1.0f / l;
  IO* dst = o + (bh * N + i) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int e = 32 * dt + 8 * g4 + 4 * hf;  // acc rows 4 g4 .. 4 g4 + 3 are dims e .. e + 3
      if constexpr (sizeof(IO) == 2) {
        u32x2_t pk;
        pk.x = pack_bf16x2(acc[dt][4 * g4 + 0] * inv, acc[dt][4 * g4 + 1] * inv);
        pk.y = pack_bf16x2(acc[dt][4 * g4 + 2] * inv, acc[dt][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(dst + e) = pk;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + e) =
            make_float4(acc[dt][4 * g4] * inv, acc[dt][4 * g4 + 1] * inv, acc[dt][4 * g4 + 2] * inv,
                        acc[dt][4 * g4 + 3] * inv);
      }
    }
}

template <typename IO, int D>
static hipError_t launch_dense_t(const Geom& g, const void* q, const void* k, const void* v, void* o,
                                 hipStream_t st) {
  const int nqb = (g.N + DN_ROWS - 1) / DN_ROWS;
  const int64_t grid = (int64_t)g.B * g.Hq * nqb;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dense_attend<IO, D>), dim3((unsigned)grid), dim3(256), 0, st, (const IO*)q, (const IO*)k,
                     (const IO*)v, (IO*)o, g.Hq, g.Hkv, g.N, nqb);
  return hipGetLastError();
}

hipError_t launch_dense(const Geom& g, const void* q, const void* k, const void* v, void* o, hipStream_t st) {
  if (g.io == 0)
    return g.d == 64 ? launch_dense_t<float, 64>(g, q, k, v, o, st) : launch_dense_t<float, 128>(g, q, k, v, o, st);
  return g.d == 64 ? launch_dense_t<bf16_t, 64>(g, q, k, v, o, st) : launch_dense_t<bf16_t, 128>(g, q, k, v, o, st);
}


// ------------------------------------------------------------------ dense decode
// The dense baseline of a decode step (bf16): for every sequence b and query head h, the
// query at position L_b - 1 attends to every cached key 0 .. L_b - 1, the full softmax
// the sparse step approximates.  Split over the sequence: one workgroup per (b, KV head,
// split of DD_SPLIT keys) holds the G query heads of that KV head and streams the split's
// K and V rows once.  A key row is read by D/8 threads (8 dims, 16 bytes each of K and V);
// the 256 / (D/8) row groups take consecutive keys, and each thread keeps per head an
// online softmax (running max and sum in base 2, unnormalised output of its 8 dims) over
// the keys of its row group, DD_UNR keys per step with the next step's rows in flight.
// The row groups are merged through LDS into one partial (output, max, sum) per split and
// head; dense_decode_merge combines a (b, h)'s splits.
constexpr int DD_SPLIT = 2048;  // keys per split
constexpr int DD_UNR = 4;       // keys per row group and step

// value of the lane at distance 1, 2 (quad permutations), mirrored in its 8-lane half row,
// and mirrored in its 16-lane row: four steps that sum a row of 16 lanes into every lane
template <int STEP>
HILS_DEV float dd_pair(float x) {
  constexpr int CTRL = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int D, int G>
__global__ void __launch_bounds__(256) dense_decode_part(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                         const bf16_t* __restrict__ v,
                                                         const int32_t* __restrict__ seq_lens, float* __restrict__ part,
                                                         int Hq, int Hkv, int N, int nsplit) {
  constexpr int TPR = D / 8;        // threads per key row
  constexpr int NRG = 256 / TPR;    // row groups (keys per pass)
  constexpr int LOG_TPR = D == 128 ? 4 : 3;
  static_assert(D == 64 || D == 128, "");
  __shared__ float s_o[G][NRG][D];
  __shared__ float s_m[G][NRG], s_l[G][NRG];
  const int sp = blockIdx.x % nsplit, bkv = blockIdx.x / nsplit;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int tid = threadIdx.x, rg = tid / TPR, ds = tid % TPR;
  const int L = min(seq_lens[b], N);
  const int j0 = sp * DD_SPLIT, j1 = min(L, j0 + DD_SPLIT);
  const int64_t bh0 = (int64_t)b * Hq + kvh * G;  // first query head of the group
  // the group's queries, this thread's 8 dims, scaled by log2(e) / sqrt(d)
  const float qs = 1.44269504088896340736f / sqrtf((float)D);
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(q + (bh0 + h) * D + 8 * ds);
    const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[h][2 * e] = __uint_as_float(wd[e] << 16) * qs;
      qv[h][2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u) * qs;
    }
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -3.0e38f;  // finite: exp2(m - m_new) stays defined before the first key
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  const bf16_t* kb = k + ((int64_t)b * Hkv + kvh) * N * D + 8 * ds;
  const bf16_t* vb = v + ((int64_t)b * Hkv + kvh) * N * D + 8 * ds;
  // every load is unconditional: keys past the split read its last key (in bounds) and
  // take zero weight
  u32x4_t kr[2][DD_UNR], vr[2][DD_UNR];
  auto issue = [&](int buf, int jb) {
#pragma unroll
    for (int u = 0; u < DD_UNR; ++u) {
      const int j = min(jb + u * NRG + rg, j1 - 1);
      kr[buf][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + (int64_t)j * D));
      vr[buf][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + (int64_t)j * D));
    }
  };
  auto consume = [&](int buf, int jb) {
    float s[G][DD_UNR];
#pragma unroll
    for (int u = 0; u < DD_UNR; ++u) {
      const uint32_t wd[4] = {kr[buf][u].x, kr[buf][u].y, kr[buf][u].z, kr[buf][u].w};
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = __uint_as_float(wd[e] << 16);
        kf[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
      }
      const bool live = jb + u * NRG + rg < j1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x = fmaf(qv[h][e], kf[e], x);
        x += dd_pair<0>(x);
        x += dd_pair<1>(x);
        x += dd_pair<2>(x);
        if constexpr (LOG_TPR == 4) x += dd_pair<3>(x);
        s[h][u] = live ? x : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = s[h][0];
#pragma unroll
      for (int u = 1; u < DD_UNR; ++u) mt = fmaxf(mt, s[h][u]);
      const float mn = fmaxf(m[h], mt);
      const float sc = __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
      l[h] *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= sc;
#pragma unroll
      for (int u = 0; u < DD_UNR; ++u) {
        const float pw = __builtin_amdgcn_exp2f(s[h][u] - mn);
        l[h] += pw;
        const uint32_t wd[4] = {vr[buf][u].x, vr[buf][u].y, vr[buf][u].z, vr[buf][u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[h][2 * e] = fmaf(pw, __uint_as_float(wd[e] << 16), o[h][2 * e]);
          o[h][2 * e + 1] = fmaf(pw, __uint_as_float(wd[e] & 0xffff0000u), o[h][2 * e + 1]);
        }
      }
    }
  };
  constexpr int STEP = DD_UNR * NRG;
  if (j0 < j1) {
    issue(0, j0);
    int jb = j0;
    for (; jb + STEP < j1; jb += 2 * STEP) {
      issue(1, jb + STEP);
      consume(0, jb);
      issue(0, jb + 2 * STEP);  // past the split: its last row again, from cache
      consume(1, jb + STEP);
    }
    if (jb < j1) consume(0, jb);
  }
  // merge the row groups: per head, the max over groups, then the rescaled sums
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[h][rg][8 * ds + e] = o[h][e];
    if (ds == 0) {
      s_m[h][rg] = m[h];
      s_l[h][rg] = l[h];
    }
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int h = x / D, e = x % D;
    float M = -3.0e38f;
    for (int r2 = 0; r2 < NRG; ++r2) M = fmaxf(M, s_m[h][r2]);
    float O = 0.f, Ls = 0.f;
    for (int r2 = 0; r2 < NRG; ++r2) {
      const float w = __builtin_amdgcn_exp2f(s_m[h][r2] - M);
      O = fmaf(w, s_o[h][r2][e], O);
      Ls = fmaf(w, s_l[h][r2], Ls);
    }
    float* dst = part + ((bh0 + h) * nsplit + sp) * (D + 2);
    dst[e] = O;
    if (e == 0) {
      dst[D] = M;
      dst[D + 1] = Ls;
    }
  }
}

// o[b,h] = the merge of the (b, h) splits' partials; one wave per (b, h), lanes over dims
template <int D>
__global__ void __launch_bounds__(256) dense_decode_merge(const float* __restrict__ part,
                                                          const int32_t* __restrict__ seq_lens,
                                                          bf16_t* __restrict__ out, int Hq, int nsplit, int64_t bhn) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= bhn) return;
  const int L = seq_lens[bh / Hq];
  const int ns = min(nsplit, (max(L, 0) + DD_SPLIT - 1) / DD_SPLIT);
  const float* pb = part + bh * nsplit * (D + 2);
  float M = -3.0e38f;
  for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, pb[s2 * (D + 2) + D]);
  float acc[EPL], Ls = 0.f;
#pragma unroll
  for (int u = 0; u < EPL; ++u) acc[u] = 0.f;
  for (int s2 = 0; s2 < ns; ++s2) {
    const float* ps = pb + s2 * (D + 2);
    const float w = __builtin_amdgcn_exp2f(ps[D] - M);
    Ls = fmaf(w, ps[D + 1], Ls);
#pragma unroll
    for (int u = 0; u < EPL; ++u) acc[u] = fmaf(w, ps[lane * EPL + u], acc[u]);
  }
  const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
  for (int u = 0; u < EPL; ++u) out[bh * D + lane * EPL + u].bits = f32_to_bf16(acc[u] * inv);
}

size_t dense_decode_workspace_bytes(const Geom& g) {
  const int64_t nsplit = (g.N + DD_SPLIT - 1) / DD_SPLIT;
  return (size_t)g.B * g.Hq * nsplit * (g.d + 2) * sizeof(float);
}

template <int D, int G>
static void launch_dd(const Geom& g, const void* q, const void* k, const void* v, const int32_t* seq_lens, void* o,
                      float* part, int nsplit, hipStream_t st) {
  hipLaunchKernelGGL((dense_decode_part<D, G>), dim3((unsigned)(g.B * g.Hkv * nsplit)), dim3(256), 0, st,
                     (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, seq_lens, part, g.Hq, g.Hkv, g.N, nsplit);
  const int64_t bhn = (int64_t)g.B * g.Hq;
  hipLaunchKernelGGL((dense_decode_merge<D>), dim3((unsigned)((bhn + 3) / 4)), dim3(256), 0, st, (const float*)part,
                     seq_lens, (bf16_t*)o, g.Hq, nsplit, bhn);
}

hipError_t launch_dense_decode(const Geom& g, const void* q, const void* k, const void* v, const int32_t* seq_lens,
                               void* o, void* ws, hipStream_t st) {
  const int nsplit = (g.N + DD_SPLIT - 1) / DD_SPLIT;
  float* part = (float*)ws;
  const int G = g.Hq / g.Hkv;
#define HILS_DD(D_, G_) \
  if (g.d == D_ && G == G_) { launch_dd<D_, G_>(g, q, k, v, seq_lens, o, part, nsplit, st); return hipGetLastError(); }
  HILS_DD(64, 1) HILS_DD(64, 2) HILS_DD(64, 4) HILS_DD(64, 8)
  HILS_DD(128, 1) HILS_DD(128, 2) HILS_DD(128, 4) HILS_DD(128, 8)
#undef HILS_DD
  return hipErrorNotSupported;
}

}  // namespace hils

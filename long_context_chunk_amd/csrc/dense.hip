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

}  // namespace hils

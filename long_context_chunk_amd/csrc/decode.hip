// One decode step: every sequence b has one new query per head at position
// L_b - 1 (L_b = seq_lens[b], the cache length including the current token).
//
//   1. decode_scan    s_c = q^ . k'_c / sqrt(d) + b'_c for every complete past
//                     chunk c < floor((L_b - 1)/S)  (fp32 GEMV, streams k' from HBM:
//                     the dominant traffic of a decode step)
//   2. decode_topk    exact top-K per (b, h) by radix selection on the ordered
//                     score bits; ties at the threshold go to the lower chunk id
//   3. decode_attend  one workgroup per (b, h, selected chunk) plus one for the
//                     own (causal) chunk: gathers the chunk's K/V rows (coalesced),
//                     softmax inside the chunk, o_c and its score (own: exact LSE)
//   4. decode_combine softmax over the chunk scores, fused output
// (aitrends.kr article, "Methodology" and "Main results": sparse KV access gives
// near-constant decode cost; hotpaper.ai abstract: chunk outputs fused by the
// retrieval scores.)
#include "hils_common.h"
#include "kernels.h"

namespace hils {

constexpr int DS_CHUNKS = 256;  // chunks scored per decode_scan workgroup

struct DecodeWs {
  size_t scores, sel_i, sel_s, nsel, part, sig, total;
};
static size_t al2(size_t x) { return (x + 255) / 256 * 256; }
static DecodeWs decode_ws(const Geom& g) {
  DecodeWs w;
  const size_t bh = (size_t)g.B * g.Hq;
  size_t off = 0;
  w.scores = off;
  off += al2(bh * g.C() * 4);
  w.sel_i = off;
  off += al2(bh * g.K * 4);
  w.sel_s = off;
  off += al2(bh * g.K * 4);
  w.nsel = off;
  off += al2(bh * 4);
  w.part = off;
  off += al2(bh * (g.K + 1) * g.d * 4);
  w.sig = off;
  off += al2(bh * (g.K + 1) * 4);
  w.total = off;
  return w;
}
size_t decode_workspace_bytes(const Geom& g) { return decode_ws(g).total; }

// q^ = q + U (D q) for one head into LDS (fp32).  256 threads.
template <typename IO, int D>
HILS_DEV void qhat_to_lds(const IO* __restrict__ qv, const IO* __restrict__ Dw, const IO* __restrict__ Uw, int h, int r,
                          float* qs, float* ts) {
  const int t = threadIdx.x;
  if (t < D) qs[t] = io_traits<IO>::load(qv, t);
  __syncthreads();
  if (r > 0) {
    if (t < r) {
      float a = 0.f;
      for (int e = 0; e < D; ++e) a = fmaf(io_traits<IO>::load(Dw, ((int64_t)h * r + t) * D + e), qs[e], a);
      ts[t] = a;
    }
    __syncthreads();
    float add = 0.f;
    if (t < D)
      for (int a = 0; a < r; ++a) add = fmaf(io_traits<IO>::load(Uw, ((int64_t)h * D + t) * r + a), ts[a], add);
    __syncthreads();
    if (t < D) qs[t] += add;
    __syncthreads();
  }
}

template <typename IO, int D>
__global__ void __launch_bounds__(256) decode_scan(const IO* __restrict__ q, const IO* __restrict__ Dw,
                                                   const IO* __restrict__ Uw, const float* __restrict__ kc,
                                                   const float* __restrict__ bc, const int32_t* __restrict__ seq_lens,
                                                   float* __restrict__ scores, int Hq, int C, int r, int nsplit) {
  __shared__ float qs[D];
  __shared__ float ts[32];
  const int sp = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;
  const int b = bh / Hq, h = bh % Hq;
  const int L = seq_lens[b];
  const int P = min(C, (L - 1) / 64);
  const int c_beg = sp * DS_CHUNKS, c_end = min(P, c_beg + DS_CHUNKS);
  if (c_beg >= c_end) return;
  qhat_to_lds<IO, D>(q + (int64_t)bh * D, Dw, Uw, h, r, qs, ts);
  constexpr int TPC = D / 4;        // threads per chunk (one float4 each)
  constexpr int CPP = 256 / TPC;    // chunks per pass
  const int t = threadIdx.x, sub = t % TPC, grp = t / TPC;
  const float4 qv = *reinterpret_cast<const float4*>(&qs[4 * sub]);
  const float tau = 1.0f / sqrtf((float)D);
  const float* kb = kc + (int64_t)bh * C * D;
  const float* bb = bc + (int64_t)bh * C;
  float* sb = scores + (int64_t)bh * C;
  constexpr int UNR = 4;
  for (int c0 = c_beg; c0 < c_end; c0 += CPP * UNR) {
    float4 kv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = c0 + u * CPP + grp;
      kv[u] = c < c_end ? *reinterpret_cast<const float4*>(kb + (int64_t)c * D + 4 * sub)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float s = qv.x * kv[u].x;
      s = fmaf(qv.y, kv[u].y, s);
      s = fmaf(qv.z, kv[u].z, s);
      s = fmaf(qv.w, kv[u].w, s);
#pragma unroll
      for (int o = TPC / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      const int c = c0 + u * CPP + grp;
      if (sub == 0 && c < c_end) sb[c] = fmaf(s, tau, bb[c]);
    }
  }
}

// exact top-K of the P scores of one (b, h); output in rank order.  The scores
// are staged in LDS once; four 8-bit radix passes on the ordered score bits find
// the K-th best value, then ties at that value are taken by ascending chunk id.
constexpr int TK_MAXC = 16384;  // largest chunk count decode_topk stages in LDS

__global__ void __launch_bounds__(256) decode_topk(const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                                                   int32_t* __restrict__ sel_i, float* __restrict__ sel_s,
                                                   int32_t* __restrict__ nsel_out, int32_t* __restrict__ sel_user,
                                                   int Hq, int C, int K) {
  __shared__ uint32_t ov[TK_MAXC];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_need;
  __shared__ uint32_t cnt_gt[256], cnt_eq[256];
  __shared__ uint64_t picked[32];
  const int bh = blockIdx.x, b = bh / Hq;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int L = seq_lens[b];
  const int P = min(C, (L - 1) / 64);
  const int n = min(K, P);
  const float* sb = scores + (int64_t)bh * C;
  for (int c = t; c < P; c += 256) ov[c] = order_f32(sb[c]);
  const int per = (P + 255) / 256;
  const int beg = min(P, t * per), end = min(P, beg + per);
  uint32_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)n;
  __syncthreads();
  if (n > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[t] = 0;
      __syncthreads();
      for (int c = t; c < P; c += 256) {
        const uint32_t o = ov[c];
        if ((o & mask) == prefix) atomicAdd(&hist[(o >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (w == 0) {
        // lane owns digits 4*lane .. 4*lane+3; suffix sums from the top digit down
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const uint32_t mine = h0 + h1 + h2 + h3;
        // inclusive suffix scan over lanes of `mine`; `above` = count of digits > 4*lane+3
        uint32_t suf = mine;
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t x = __shfl_down(suf, o);
          if (lane + o < 64) suf += x;
        }
        const uint32_t above = suf - mine;
        // the digit d with (count > d) < need <= (count >= d)
        const uint32_t c3 = above + h3, c2 = c3 + h2, c1 = c2 + h1, c0 = c1 + h0;
        int dg = -1;
        uint32_t cum = 0;
        if (above < need && c3 >= need) { dg = 4 * lane + 3; cum = above; }
        else if (c3 < need && c2 >= need) { dg = 4 * lane + 2; cum = c3; }
        else if (c2 < need && c1 >= need) { dg = 4 * lane + 1; cum = c2; }
        else if (c1 < need && c0 >= need) { dg = 4 * lane; cum = c1; }
        if (dg >= 0) {
          sh_prefix = prefix | ((uint32_t)dg << shift);
          sh_need = need - cum;
        }
      }
      __syncthreads();
      prefix = sh_prefix;
      need = sh_need;
      mask |= 255u << shift;
      __syncthreads();
    }
  }
  // prefix = ordered bits of the K-th best score; `need` of the elements equal to it are taken (lowest ids)
  uint32_t gt = 0, eq = 0;
  for (int c = beg; c < end; ++c) {
    const uint32_t o = ov[c];
    gt += o > prefix;
    eq += o == prefix;
  }
  cnt_gt[t] = gt;
  cnt_eq[t] = eq;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const uint32_t a = t >= o ? cnt_gt[t - o] : 0, e = t >= o ? cnt_eq[t - o] : 0;
    __syncthreads();
    cnt_gt[t] += a;
    cnt_eq[t] += e;
    __syncthreads();
  }
  if (n > 0 && (gt | eq)) {
    uint32_t pos_gt = cnt_gt[t] - gt;   // exclusive prefix
    uint32_t rank_eq = cnt_eq[t] - eq;
    const uint32_t ngt = cnt_gt[255];
    for (int c = beg; c < end; ++c) {
      const uint32_t o = ov[c];
      if (o > prefix) {
        picked[pos_gt++] = make_key(unorder_f32(o), c);
      } else if (o == prefix) {
        if (rank_eq < need) picked[ngt + rank_eq] = make_key(unorder_f32(o), c);
        ++rank_eq;
      }
    }
  }
  __syncthreads();
  if (t < K) {
    int32_t ci = -1;
    float cs = -INFINITY;
    int rk = t;
    if (t < n) {
      const uint64_t mine = picked[t];
      rk = 0;
      for (int j = 0; j < n; ++j) rk += picked[j] > mine;
      ci = key_chunk(mine);
      cs = key_score(mine);
    }
    sel_i[(int64_t)bh * K + rk] = ci;
    sel_s[(int64_t)bh * K + rk] = cs;
    if (sel_user) sel_user[(int64_t)bh * K + rk] = ci;
  }
  if (t == 0) nsel_out[bh] = n;
}

// slot s < nsel: selected chunk sel_i[s]; slot K: the own chunk.  Writes the
// normalised chunk output (fp32) and the chunk's fusion score.
template <typename IO, int D>
__global__ void __launch_bounds__(256) decode_attend(const IO* __restrict__ q, const IO* __restrict__ kcache,
                                                     const IO* __restrict__ vcache, const int32_t* __restrict__ seq_lens,
                                                     const int32_t* __restrict__ sel_i, const float* __restrict__ sel_s,
                                                     const int32_t* __restrict__ nsel, float* __restrict__ part,
                                                     float* __restrict__ sig, int Hq, int Hkv, int N, int K) {
  constexpr int NG = 256 / (D / 4);  // key groups for the value pass (4 head dims per thread)
  constexpr int KPG = 64 / NG;
  __shared__ float qs[D];
  __shared__ float z[64];
  __shared__ float ml[2];
  __shared__ float red[NG][D];
  const int slot = blockIdx.x % (K + 1), bh = blockIdx.x / (K + 1);
  const int b = bh / Hq, h = bh % Hq, kvh = h / (Hq / Hkv);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int L = seq_lens[b];
  int c, nk;
  if (slot == K) {
    c = (L - 1) / 64;
    nk = L - c * 64;
  } else {
    if (slot >= nsel[bh]) return;
    c = sel_i[(int64_t)bh * K + slot];
    nk = 64;
  }
  if (t < D) qs[t] = io_traits<IO>::load(q, (int64_t)bh * D + t);
  __syncthreads();
  const int64_t row0 = ((int64_t)b * Hkv + kvh) * N + (int64_t)c * 64;
  const float tau = 1.0f / sqrtf((float)D);
  {  // logits: 4 threads per key, each a quarter of the head dim (vector loads)
    const int key = t >> 2, qd = t & 3;
    float s = 0.f;
    if (key < nk) {
      const int64_t base = (row0 + key) * D + qd * (D / 4);
#pragma unroll
      for (int e = 0; e < D / 4; e += 4) {
        float x[4];
        io_traits<IO>::load4(kcache, base + e, x);
#pragma unroll
        for (int u = 0; u < 4; ++u) s = fmaf(qs[qd * (D / 4) + e + u], x[u], s);
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (qd == 0) z[key] = key < nk ? s * tau : -INFINITY;
  }
  __syncthreads();
  if (w == 0) {
    const float zz = z[lane];
    const float m = wave_max(zz);
    const float p = zz == -INFINITY ? 0.f : __expf(zz - m);
    const float l = wave_sum(p);
    z[lane] = p;
    if (lane == 0) {
      ml[0] = m;
      ml[1] = l;
    }
  }
  __syncthreads();
  {  // values: thread (4 head dims, key group)
    const int e4 = (t % (D / 4)) * 4, kg = t / (D / 4);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = kg * KPG; j < (kg + 1) * KPG; ++j) {
      if (j < nk) {
        float x[4];
        io_traits<IO>::load4(vcache, (row0 + j) * D + e4, x);
        const float pj = z[j];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = fmaf(pj, x[u], a[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) red[kg][e4 + u] = a[u];
  }
  __syncthreads();
  if (t < D) {
    float o = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) o += red[g2][t];
    part[((int64_t)bh * (K + 1) + slot) * D + t] = o / ml[1];
  }
  if (t == 0) sig[(int64_t)bh * (K + 1) + slot] = slot == K ? ml[0] + logf(ml[1]) : sel_s[(int64_t)bh * K + slot];
}

template <typename IO, int D>
__global__ void __launch_bounds__(128) decode_combine(const float* __restrict__ part, const float* __restrict__ sig,
                                                      const int32_t* __restrict__ nsel, IO* __restrict__ o, int K) {
  const int bh = blockIdx.x;
  const int n = nsel[bh];
  const float* sg = sig + (int64_t)bh * (K + 1);
  float M = sg[K];
  for (int s = 0; s < n; ++s) M = fmaxf(M, sg[s]);
  float Z = expf(sg[K] - M);
  for (int s = 0; s < n; ++s) Z += expf(sg[s] - M);
  const float inv = 1.0f / Z;
  for (int e = threadIdx.x; e < D; e += 128) {
    float a = expf(sg[K] - M) * part[((int64_t)bh * (K + 1) + K) * D + e];
    for (int s = 0; s < n; ++s) a = fmaf(expf(sg[s] - M), part[((int64_t)bh * (K + 1) + s) * D + e], a);
    io_traits<IO>::store(o, (int64_t)bh * D + e, a * inv);
  }
}

template <typename IO, int D>
static hipError_t launch_decode_t(const Geom& g, const void* q, const void* kcache, const void* vcache,
                                  const int32_t* seq_lens, const float* kc, const float* bc, const void* Dw,
                                  const void* Uw, int32_t* sel_user, void* o, char* ws, hipStream_t st,
                                  hipEvent_t* ev) {
  const DecodeWs w = decode_ws(g);
  float* scores = (float*)(ws + w.scores);
  int32_t* sel_i = (int32_t*)(ws + w.sel_i);
  float* sel_s = (float*)(ws + w.sel_s);
  int32_t* nsel = (int32_t*)(ws + w.nsel);
  float* part = (float*)(ws + w.part);
  float* sig = (float*)(ws + w.sig);
  const int C = g.C(), BH = g.B * g.Hq;
  const int nsplit = (C + DS_CHUNKS - 1) / DS_CHUNKS;
  if (ev) hipEventRecord(ev[0], st);
  if (nsplit > 0)
    hipLaunchKernelGGL((decode_scan<IO, D>), dim3(BH * nsplit), dim3(256), 0, st, (const IO*)q, (const IO*)Dw,
                       (const IO*)Uw, kc, bc, seq_lens, scores, g.Hq, C, g.r, nsplit);
  if (ev) hipEventRecord(ev[1], st);
  hipLaunchKernelGGL(decode_topk, dim3(BH), dim3(256), 0, st, scores, seq_lens, sel_i, sel_s, nsel, sel_user, g.Hq,
                     C, g.K);
  if (ev) hipEventRecord(ev[2], st);
  hipLaunchKernelGGL((decode_attend<IO, D>), dim3(BH * (g.K + 1)), dim3(256), 0, st, (const IO*)q, (const IO*)kcache,
                     (const IO*)vcache, seq_lens, sel_i, sel_s, nsel, part, sig, g.Hq, g.Hkv, g.N, g.K);
  if (ev) hipEventRecord(ev[3], st);
  hipLaunchKernelGGL((decode_combine<IO, D>), dim3(BH), dim3(128), 0, st, part, sig, nsel, (IO*)o, g.K);
  if (ev) hipEventRecord(ev[4], st);
  return hipGetLastError();
}

hipError_t launch_decode(const Geom& g, const void* q, const void* kcache, const void* vcache, const int32_t* seq_lens,
                         const float* kc, const float* bc, const void* Dw, const void* Uw, int32_t* sel_idx_out,
                         void* o, void* ws, size_t ws_bytes, hipStream_t st, hipEvent_t* ev) {
  if (ws_bytes < decode_workspace_bytes(g)) return hipErrorInvalidValue;
  char* w = (char*)ws;
  if (g.io == 0)
    return g.d == 64 ? launch_decode_t<float, 64>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev)
                     : launch_decode_t<float, 128>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev);
  return g.d == 64 ? launch_decode_t<bf16_t, 64>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev)
                   : launch_decode_t<bf16_t, 128>(g, q, kcache, vcache, seq_lens, kc, bc, Dw, Uw, sel_idx_out, o, w, st, ev);
}

}  // namespace hils

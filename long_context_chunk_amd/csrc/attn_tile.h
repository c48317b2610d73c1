// K/V chunk tiles in LDS and the per-wave MFMA attention of 32 query rows against one
// 64-key tile, shared by the chunk attention kernels and the dense baseline.
#pragma once
#include "hils_common.h"

namespace hils {

// ------------------------------------------------------ K/V chunk tile in LDS
// Both planes in natural [key][d] order, staged with 16-byte loads and stores.
// K (row stride D + 8) feeds the A operand of S^T = K Q^T, whose k-steps take 8
// consecutive head dimensions per lane half: one 16-byte LDS read per operand.
// V (row stride D + 32) feeds the A operand of O^T = V^T P^T (dims as rows, keys as k)
// through ds_read_b64_tr_b16 transposing reads: within a 16-lane group, lane j points at
// the 4 dims 4(j&3).. of key (j>>2) and lane i receives 4 consecutive keys of dim i.
// Keys at or beyond `nvalid` are stored as zeros.  NT bf16 terms per value.
// VPAD: V row padding; D + 32 suits the transposing reads, D + 8 whole-row reads.
template <typename IO, int D, int NT, int VPAD = 32>
struct alignas(16) KVTile {
  static constexpr int LDK = D + 8;
  static constexpr int LDV = D + VPAD;
  uint16_t k[NT][64 * LDK];
  uint16_t v[NT][64 * LDV];
};

template <typename IO, int D, int NT, int VPAD>
HILS_DEV void stage_kv(KVTile<IO, D, NT, VPAD>& tile, const IO* __restrict__ k, const IO* __restrict__ v, int64_t row0,
                       int nvalid, int tid, int nthreads) {
  constexpr int LDK = KVTile<IO, D, NT, VPAD>::LDK, LDV = KVTile<IO, D, NT, VPAD>::LDV;
  if constexpr (sizeof(IO) == 2 && NT == 1) {  // bf16 values are their own single term
    for (int i = tid * 8; i < 64 * D; i += nthreads * 8) {
      const int key = i / D, e = i % D;
      const int64_t off = (row0 + min(key, nvalid - 1)) * D + e;  // nvalid >= 1: in bounds; zeroed below
      const uint32_t keep = key < nvalid ? 0xffffffffu : 0u;
      u32x4_t kr = *reinterpret_cast<const u32x4_t*>(k + off), vr = *reinterpret_cast<const u32x4_t*>(v + off);
      kr.x &= keep, kr.y &= keep, kr.z &= keep, kr.w &= keep;
      vr.x &= keep, vr.y &= keep, vr.z &= keep, vr.w &= keep;
      *reinterpret_cast<u32x4_t*>(&tile.k[0][key * LDK + e]) = kr;
      *reinterpret_cast<u32x4_t*>(&tile.v[0][key * LDV + e]) = vr;
    }
    return;
  }
  for (int i = tid * 8; i < 64 * D; i += nthreads * 8) {
    const int key = i / D, e = i % D;
    float kx[8], vx[8];
    if (key < nvalid) {
      const int64_t off = (row0 + key) * D + e;
      io_traits<IO>::load4(k, off, *reinterpret_cast<float(*)[4]>(kx));
      io_traits<IO>::load4(k, off + 4, *reinterpret_cast<float(*)[4]>(kx + 4));
      io_traits<IO>::load4(v, off, *reinterpret_cast<float(*)[4]>(vx));
      io_traits<IO>::load4(v, off + 4, *reinterpret_cast<float(*)[4]>(vx + 4));
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) kx[u] = vx[u] = 0.f;
    }
    u32x4_t ks[NT], vs[NT];
    split8<NT>(kx, ks);
    split8<NT>(vx, vs);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      *reinterpret_cast<u32x4_t*>(&tile.k[j][key * LDK + e]) = ks[j];
      *reinterpret_cast<u32x4_t*>(&tile.v[j][key * LDV + e]) = vs[j];
    }
  }
}

// Staging of one 64-key K/V chunk by exactly NTH threads in two halves, so that the
// global loads of the next chunk are in flight while the current one is computed:
// load() issues the 16-byte loads of every element this thread stores (raw, in
// registers); store() splits them into NT bf16 terms and writes the tile.  Keys at or
// beyond nvalid read row nvalid - 1 (in bounds) and are stored as zeros.
template <typename IO, int D, int NT, int NTH>
struct KVPrefetch {
  static constexpr int NP = 64 * D / (8 * NTH);       // 8-element pieces per thread and plane
  static constexpr int W = sizeof(IO) / 2;             // 16-byte words per piece
  static_assert(NP >= 1 && NP * 8 * NTH == 64 * D, "the threads cover the chunk exactly");
  u32x4_t kr[NP][W], vr[NP][W];

  __device__ __forceinline__ void load(const IO* __restrict__ k, const IO* __restrict__ v, int64_t row0, int nvalid, int tid) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int i = (tid + p * NTH) * 8, key = i / D, e = i % D;
      const int64_t off = (row0 + min(key, nvalid - 1)) * D + e;
#pragma unroll
      for (int u = 0; u < W; ++u) {
        kr[p][u] = *reinterpret_cast<const u32x4_t*>(k + off + u * (16 / (int)sizeof(IO)));
        vr[p][u] = *reinterpret_cast<const u32x4_t*>(v + off + u * (16 / (int)sizeof(IO)));
      }
    }
  }

  __device__ __forceinline__ void store(KVTile<IO, D, NT>& tile, int nvalid, int tid) const {
    constexpr int LDK = KVTile<IO, D, NT>::LDK, LDV = KVTile<IO, D, NT>::LDV;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int i = (tid + p * NTH) * 8, key = i / D, e = i % D;
      const bool ok = key < nvalid;
      float kx[8], vx[8];
#pragma unroll
      for (int u = 0; u < W; ++u) {
        const uint32_t kw[4] = {kr[p][u].x, kr[p][u].y, kr[p][u].z, kr[p][u].w};
        const uint32_t vw[4] = {vr[p][u].x, vr[p][u].y, vr[p][u].z, vr[p][u].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if constexpr (sizeof(IO) == 2) {
            kx[2 * m] = __uint_as_float(kw[m] << 16);
            kx[2 * m + 1] = __uint_as_float(kw[m] & 0xffff0000u);
            vx[2 * m] = __uint_as_float(vw[m] << 16);
            vx[2 * m + 1] = __uint_as_float(vw[m] & 0xffff0000u);
          } else {
            kx[4 * u + m] = __uint_as_float(kw[m]);
            vx[4 * u + m] = __uint_as_float(vw[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        kx[m] = ok ? kx[m] : 0.f;
        vx[m] = ok ? vx[m] : 0.f;
      }
      u32x4_t ks[NT], vs[NT];
      split8<NT>(kx, ks);
      split8<NT>(vx, vs);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        *reinterpret_cast<u32x4_t*>(&tile.k[j][key * LDK + e]) = ks[j];
        *reinterpret_cast<u32x4_t*>(&tile.v[j][key * LDV + e]) = vs[j];
      }
    }
  }
};

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// A operand of O^T = V^T P^T for dim tile dt, key k-step ks2: lane l (dim 32 dt + (l & 31),
// half h = l >> 5) gets keys kperm(ks2, h, 0..7) of its dim, in two transposing reads
template <int LDV>
HILS_DEV bf16x8_t vt_operand(const uint16_t* vplane, int dt, int ks2, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int e = 32 * dt + 16 * (g & 1) + 4 * (j & 3);
  const int key = 16 * ks2 + 4 * (g >> 1) + (j >> 2);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vplane + key * LDV + e));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vplane + (key + 8) * LDV + e));
  u32x4_t u;
  u.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  u.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  u.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  u.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

HILS_DEV bf16x8_t lds_op16(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// One wave: 32 query rows (B operands qb, NT terms) against the staged chunk.
// Returns, per lane (row n = lane & 31, half hf), the O^T accumulators (unnormalised:
// P keeps its largest weight exactly 1 in bf16) and the row's softmax max m (of the
// scaled logits) and sum l.  MASK: key j is used iff j < key_lim
// (per row); otherwise all 64 keys are.  p = 2^((s - max s) tau log2 e) is one fma and
// one exp per logit; masked logits are -inf and give p = 0.
template <typename IO, int D, int NT, bool MASK>
HILS_DEV void wave_chunk_attention(const KVTile<IO, D, NT>& tile, const bf16x8_t (&qb)[NT][D / 16], int key_lim,
                                   f32x16_t (&o)[D / 32], float& m_out, float& l_out) {
  constexpr int NKS = D / 16;
  constexpr int LDK = KVTile<IO, D, NT>::LDK, LDV = KVTile<IO, D, NT>::LDV;
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float tau = 1.0f / sqrtf((float)D);
  const float c = tau * 1.44269504088896340736f;  // tau log2(e)
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
        for (int i = 0; i < NT; ++i)
          if (i + j < NT) s[tt] = mfma32(a, qb[i][ks], s[tt]);
      }
  }
  if constexpr (MASK) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        if (32 * tt + acc_row(rr, hf) >= key_lim) s[tt][rr] = -INFINITY;
  }
  float m = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int rr = 2; rr < 32; ++rr) m = fmaxf(m, s[rr >> 4][rr & 15]);
  m = fmaxf(m, __shfl_xor(m, 32));
  const float mc = m * c;
  float l = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[tt][rr], c, -mc));
      s[tt][rr] = p;
      l += p;
    }
  l += __shfl_xor(l, 32);
  // P^T as B operand: k-step ks2 (keys 16*ks2 ..), element mm = register 8*(ks2&1)+mm of tile ks2>>1
  bf16x8_t pb[NT][4];
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
    float pv[8];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) pv[mm] = s[ks2 >> 1][8 * (ks2 & 1) + mm];
    u32x4_t t[NT];
    split8<NT>(pv, t);
#pragma unroll
    for (int j = 0; j < NT; ++j) pb[j][ks2] = __builtin_bit_cast(bf16x8_t, t[j]);
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    o[dt] = zero16();
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8_t a = vt_operand<LDV>(tile.v[j], dt, ks2, lane);
#pragma unroll
        for (int i = 0; i < NT; ++i)
          if (i + j < NT) o[dt] = mfma32(a, pb[i][ks2], o[dt]);
      }
  }
  m_out = m * tau;
  l_out = l;
}

// One step of an online softmax over consecutive chunks: the wave's 32 query rows (B
// operands qb) against the staged chunk, folded into running O^T accumulators o, the
// running maximum m of the raw logits q.k (-inf before the first chunk) and sum l: the
// old state is scaled by 2^((m - m') tau log2 e) to the new maximum m' before the chunk's
// weights are added, so P keeps its largest weight at most 1 in bf16.  MASK: key j is
// used iff j < key_lim (per row); otherwise all 64 keys are.  Every row must keep at
// least one key.  The row's log-sum-exp is m tau + log l.
template <typename IO, int D, int NT, bool MASK>
HILS_DEV void wave_chunk_online(const KVTile<IO, D, NT>& tile, const bf16x8_t (&qb)[NT][D / 16], int key_lim,
                                f32x16_t (&o)[D / 32], float& m, float& l) {
  constexpr int NKS = D / 16;
  constexpr int LDK = KVTile<IO, D, NT>::LDK, LDV = KVTile<IO, D, NT>::LDV;
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float c = 1.44269504088896340736f / sqrtf((float)D);  // tau log2(e)
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
        for (int i = 0; i < NT; ++i)
          if (i + j < NT) s[tt] = mfma32(a, qb[i][ks], s[tt]);
      }
  }
  if constexpr (MASK) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        if (32 * tt + acc_row(rr, hf) >= key_lim) s[tt][rr] = -INFINITY;
  }
  float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int rr = 2; rr < 32; ++rr) mt = fmaxf(mt, s[rr >> 4][rr & 15]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float mn = fmaxf(m, mt);
  const float alpha = __builtin_amdgcn_exp2f((m - mn) * c);  // 0 on the first chunk
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
    for (int rr = 0; rr < 16; ++rr) o[dt][rr] *= alpha;
  bf16x8_t pb[NT][4];
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
    float pv[8];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) pv[mm] = s[ks2 >> 1][8 * (ks2 & 1) + mm];
    u32x4_t t[NT];
    split8<NT>(pv, t);
#pragma unroll
    for (int j = 0; j < NT; ++j) pb[j][ks2] = __builtin_bit_cast(bf16x8_t, t[j]);
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8_t a = vt_operand<LDV>(tile.v[j], dt, ks2, lane);
#pragma unroll
        for (int i = 0; i < NT; ++i)
          if (i + j < NT) o[dt] = mfma32(a, pb[i][ks2], o[dt]);
      }
}

// Loads query row `qrow_off` (element offset of the row) from global memory as NT-term B operands.
template <typename IO, int D, int NT>
HILS_DEV void load_q_operand(const IO* __restrict__ q, int64_t qrow_off, bool ok, bf16x8_t (&qb)[NT][D / 16]) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    float x[8];
    if (ok) {
      io_traits<IO>::load4(q, qrow_off + 16 * ks + 8 * hf, *reinterpret_cast<float(*)[4]>(x));
      io_traits<IO>::load4(q, qrow_off + 16 * ks + 8 * hf + 4, *reinterpret_cast<float(*)[4]>(x + 4));
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = 0.f;
    }
    u32x4_t t[NT];
    split8<NT>(x, t);
#pragma unroll
    for (int j = 0; j < NT; ++j) qb[j][ks] = __builtin_bit_cast(bf16x8_t, t[j]);
  }
}

// bf16 query row already staged in LDS (row stride LDQ elements) as the B operand.
template <int D>
HILS_DEV void lds_q_operand(const uint16_t* rowp, bf16x8_t (&qb)[1][D / 16]) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qb[0][ks] = lds_op16(rowp + 16 * ks + 8 * hf);
}

}  // namespace hils

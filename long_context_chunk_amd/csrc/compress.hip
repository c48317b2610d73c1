// Landmark compression: per (batch, landmark head, chunk) the landmark query
// attends the chunk's S keys; the softmax weights a_j give the compressed key
// k'_c = sum_j a_j k_j and the entropy bias b'_c = -sum_j a_j log a_j.
// (aitrends.kr article, "Key contributions" first item, "Methodology",
// "Technical details": O(S) work per chunk.)
//
// HBM-bound: each key tile is read once (coalesced 16-byte loads) and serves every
// landmark head of its KV head.
#include <algorithm>

#include "hils_common.h"
#include "kernels.h"

namespace hils {

// One wave per work item (b, KV head, chunk), all landmark heads of the KV head; the waves
// of a workgroup are independent (no workgroup barrier) and stride over the items, the
// next item's keys in flight in registers while the current one is computed.
//   * the 64 x D key tile goes to the wave's LDS region in its io type, rows padded by 16
//     bytes, so lane j reading row j with 16-byte reads is free of bank conflicts;
//   * logits: lane j owns key j; its row is read once and dotted with each landmark
//     query (bf16: v_dot2 of bf16 pairs with fp32 accumulation; fp32: fma), the query
//     broadcast from LDS;
//   * softmax, k'_c and b'_c per landmark head with wave reductions; for k'_c lane e owns
//     dimensions (2e, 2e+1) (D = 128) or e (D = 64) and reads one word of each key row,
//     shared by all landmark heads of the group (a_j taken from lane j with readlane).
constexpr int CP_WAVES = 4;    // waves per workgroup

// GP: landmark heads handled per pass over the key rows (4, 2 or 1, dividing the group)
template <typename IO, int D, int GP>
struct CompressLds {
  static constexpr int LDK = D + 16 / (int)sizeof(IO);   // elements per padded key row
  IO kt[64 * LDK];
  IO lq[GP][D];
};

template <typename IO, int D, int GP>
__global__ void __launch_bounds__(64 * CP_WAVES) compress_kernel(const IO* __restrict__ k, const IO* __restrict__ lmk,
                                                                float* __restrict__ kc, float* __restrict__ bc,
                                                                int Hkv, int Hl, int N, int C, int c_begin,
                                                                int nchunks, int64_t items, KvPages pg) {
  constexpr int S = 64;
  using L = CompressLds<IO, D, GP>;
  constexpr int LDK = L::LDK;
  constexpr int EPV = 16 / (int)sizeof(IO);    // elements per 16-byte piece
  constexpr int NL = S * D / EPV / 64;         // 16-byte pieces per lane for a whole tile
  constexpr int RW = D * (int)sizeof(IO) / 16; // 16-byte pieces per key row
  constexpr int DPL = D / 64;                  // k' dimensions per lane (1 or 2)
  __shared__ L lds[CP_WAVES];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  L& sm = lds[w];
  const int G = Hl / Hkv;
  const float tau = 1.0f / sqrtf((float)D);
  const int64_t stride = (int64_t)gridDim.x * CP_WAVES;
  int64_t item = (int64_t)blockIdx.x * CP_WAVES + w;
  if (item >= items) return;   // the whole wave: no barrier below waits for it

  // the keys of an item and the landmark queries of its first GP heads, in registers:
  // loaded one item ahead
  constexpr int LPL = (GP * RW + 63) / 64;  // 16-byte pieces of landmark queries per lane
  u32x4_t raw[NL], rawl[LPL];
  auto load_tile = [&](int64_t it) {
    const int cl = (int)(it % nchunks);
    const int64_t bk = it / nchunks;  // b * Hkv + kvh
    const int kvh = (int)(bk % Hkv), b = (int)(bk / Hkv);
    const IO* kt = k + pg.chunk_row(b, kvh, Hkv, N, c_begin + cl) * D;
#pragma unroll
    for (int u = 0; u < NL; ++u) raw[u] = *reinterpret_cast<const u32x4_t*>(kt + (u * 64 + lane) * EPV);
#pragma unroll
    for (int u = 0; u < LPL; ++u) {
      const int x = min(u * 64 + lane, GP * RW - 1);   // lanes past the last piece repeat it
      const int g = x / RW, pc = x % RW;
      const int64_t lrow = ((int64_t)b * Hl + kvh * G + g) * C + c_begin + cl;
      rawl[u] = *reinterpret_cast<const u32x4_t*>(lmk + lrow * D + pc * EPV);
    }
  };
  load_tile(item);
  for (;;) {
    const int cl = (int)(item % nchunks);
    const int64_t bk = item / nchunks;
    const int kvh = (int)(bk % Hkv), b = (int)(bk / Hkv);
    const int c = c_begin + cl;
    // this item's keys to LDS, then the next item's loads
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int e0 = (u * 64 + lane) * EPV;
      *reinterpret_cast<u32x4_t*>(&sm.kt[(e0 / D) * LDK + e0 % D]) = raw[u];
    }
#pragma unroll
    for (int u = 0; u < LPL; ++u) {
      const int x = u * 64 + lane;
      if (x < GP * RW) *reinterpret_cast<u32x4_t*>(&sm.lq[x / RW][(x % RW) * EPV]) = rawl[u];
    }
    const int64_t next = item + stride;
    if (next < items) load_tile(next);
    for (int g0 = 0; g0 < G; g0 += GP) {
      // the landmark queries of heads g0 .. g0+GP-1 to LDS (the first pass's came with the keys)
      if (g0 > 0) {
        for (int x = lane; x < GP * RW; x += 64) {
          const int g = x / RW, pc = x % RW;
          const int64_t lrow = ((int64_t)b * Hl + kvh * G + g0 + g) * C + c;
          *reinterpret_cast<u32x4_t*>(&sm.lq[g][pc * EPV]) =
              *reinterpret_cast<const u32x4_t*>(lmk + lrow * D + pc * EPV);
        }
      }
      // LDS operations of one wave execute in order: only the compiler must not move the
      // reads above the writes (a memory fence would also wait for the next item's loads)
      __builtin_amdgcn_wave_barrier();
      // logits z_g = tau L_g . k_j, lane j = key j
      u32x4_t kr[RW];
#pragma unroll
      for (int pc = 0; pc < RW; ++pc) kr[pc] = *reinterpret_cast<const u32x4_t*>(&sm.kt[lane * LDK + pc * EPV]);
      float a[GP], ent[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        {
          float z = 0.f;
#pragma unroll
          for (int pc = 0; pc < RW; ++pc) {
            const u32x4_t lv = *reinterpret_cast<const u32x4_t*>(&sm.lq[g][pc * EPV]);   // broadcast
            if constexpr (sizeof(IO) == 2) {
              // pairs taken with shufflevector from whole 8-element vectors (a bit cast of
              // one 32-bit element of a vector register was miscompiled to element 0)
              const bf16x8_t kv8 = __builtin_bit_cast(bf16x8_t, kr[pc]);
              const bf16x8_t lv8 = __builtin_bit_cast(bf16x8_t, lv);
              z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kv8, kv8, 0, 1),
                                                  __builtin_shufflevector(lv8, lv8, 0, 1), z, false);
              z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kv8, kv8, 2, 3),
                                                  __builtin_shufflevector(lv8, lv8, 2, 3), z, false);
              z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kv8, kv8, 4, 5),
                                                  __builtin_shufflevector(lv8, lv8, 4, 5), z, false);
              z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kv8, kv8, 6, 7),
                                                  __builtin_shufflevector(lv8, lv8, 6, 7), z, false);
            } else {
              z = fmaf(__uint_as_float(kr[pc].x), __uint_as_float(lv.x), z);
              z = fmaf(__uint_as_float(kr[pc].y), __uint_as_float(lv.y), z);
              z = fmaf(__uint_as_float(kr[pc].z), __uint_as_float(lv.z), z);
              z = fmaf(__uint_as_float(kr[pc].w), __uint_as_float(lv.w), z);
            }
          }
          z *= tau;
          const float m = wave_max(z);
          const float p = expf(z - m);
          const float Z = wave_sum(p);
          a[g] = p / Z;
          // -sum_j a_j log a_j, with log a_j = (z_j - m) - log Z
          ent[g] = logf(Z) - wave_sum(a[g] * (z - m));
        }
      }
      // k'_g = sum_j a_g[j] k_j: lane e owns dimensions DPL*e .. DPL*e+DPL-1
      float acc[GP][DPL];
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[g][x] = 0.f;
#pragma unroll 4
      for (int j = 0; j < S; ++j) {
        float kv[DPL];
        if constexpr (sizeof(IO) == 2 && DPL == 2) {
          const uint32_t wd = *reinterpret_cast<const uint32_t*>(&sm.kt[j * LDK + 2 * lane]);
          kv[0] = __uint_as_float(wd << 16);
          kv[1] = __uint_as_float(wd & 0xffff0000u);
        } else {
#pragma unroll
          for (int x = 0; x < DPL; ++x) kv[x] = io_traits<IO>::load(sm.kt, j * LDK + DPL * lane + x);
        }
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const float aj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[g]), j));
#pragma unroll
          for (int x = 0; x < DPL; ++x) acc[g][x] = fmaf(aj, kv[x], acc[g][x]);
        }
      }
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const int64_t row = ((int64_t)b * Hl + kvh * G + g0 + g) * C + c;
        if constexpr (DPL == 2)
          *reinterpret_cast<float2*>(kc + row * D + 2 * lane) = make_float2(acc[g][0], acc[g][1]);
        else
          kc[row * D + lane] = acc[g][0];
        if (lane == 0) bc[row] = ent[g];
      }
      // every lane is done reading this pass's landmark queries
      __builtin_amdgcn_wave_barrier();
    }
    if (next >= items) break;
    item = next;
    // every lane is done reading the key tile before it is rewritten
    __builtin_amdgcn_wave_barrier();
  }
}

template <typename IO, int D, int GP>
static void launch_cp(dim3 grid, hipStream_t st, const void* k, const void* lmk, float* kc, float* bc, int Hkv, int Hl,
                      int N, int C, int c_begin, int n, int64_t items, KvPages pg) {
  hipLaunchKernelGGL((compress_kernel<IO, D, GP>), grid, dim3(64 * CP_WAVES), 0, st, (const IO*)k, (const IO*)lmk, kc,
                     bc, Hkv, Hl, N, C, c_begin, n, items, pg);
}

template <typename IO>
hipError_t launch_compress_t(const void* k, const void* lmk, float* kc, float* bc, int B, int Hkv, int Hl, int N,
                             int d, int c_begin, int c_end, hipStream_t st, KvPages pg) {
  const int C = N / 64, n = c_end - c_begin;
  if (n <= 0) return hipSuccess;
  const int64_t items = (int64_t)B * Hkv * n;
  // enough waves to fill the chip several times over; each strides over the items
  const dim3 grid((unsigned)std::min<int64_t>((items + CP_WAVES - 1) / CP_WAVES, 256 * 16));
  const int G = Hl / Hkv;
  const int gp = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
#define HILS_CP(D_, GP_) launch_cp<IO, D_, GP_>(grid, st, k, lmk, kc, bc, Hkv, Hl, N, C, c_begin, n, items, pg)
  if (d == 64) {
    if (gp == 4) HILS_CP(64, 4);
    else if (gp == 2) HILS_CP(64, 2);
    else HILS_CP(64, 1);
  } else {
    if (gp == 4) HILS_CP(128, 4);
    else if (gp == 2) HILS_CP(128, 2);
    else HILS_CP(128, 1);
  }
#undef HILS_CP
  return hipGetLastError();
}

hipError_t launch_compress(int io, const void* k, const void* lmk, float* kc, float* bc, int B, int Hkv, int Hl,
                           int N, int d, int c_begin, int c_end, hipStream_t st, KvPages pg) {
  return io == 0 ? launch_compress_t<float>(k, lmk, kc, bc, B, Hkv, Hl, N, d, c_begin, c_end, st, pg)
                 : launch_compress_t<bf16_t>(k, lmk, kc, bc, B, Hkv, Hl, N, d, c_begin, c_end, st, pg);
}

}  // namespace hils

// Landmark compression: per (batch, landmark head, chunk) the landmark query
// attends the chunk's S keys; the softmax weights a_j give the compressed key
// k'_c = sum_j a_j k_j and the entropy bias b'_c = -sum_j a_j log a_j.
// (aitrends.kr article, "Key contributions" first item, "Methodology",
// "Technical details": O(S) work per chunk.)
//
// HBM-bound: each workgroup reads one S x d key tile once (coalesced, staged in
// LDS as fp32 with a padded row stride) and serves every landmark head of that
// KV head, one wave per landmark head.  Lane j of a wave owns key j for the
// logits and the softmax (wave shuffles), then lane e owns output dimension e.
#include "hils_common.h"
#include "kernels.h"

namespace hils {

template <typename IO, int D>
__global__ void __launch_bounds__(256) compress_kernel(const IO* __restrict__ k, const IO* __restrict__ lmk,
                                                        float* __restrict__ kc, float* __restrict__ bc, int Hkv,
                                                        int Hl, int N, int C, int c_begin, int nchunks, KvPages pg) {
  constexpr int S = 64;
  constexpr int LD = D + 1;  // padded fp32 row stride: lane j reading row j is conflict-free
  __shared__ float ks[S * LD];
  __shared__ float ls[4][D];
  __shared__ float as[4][S];

  const int item = blockIdx.x;
  const int cl = item % nchunks;
  const int bk = item / nchunks;  // b * Hkv + kvh
  const int c = c_begin + cl;
  const int kvh = bk % Hkv, b = bk / Hkv;
  const int G = Hl / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // stage the key tile (fp32 in LDS), 16-byte loads: the chunk's rows are consecutive
  const IO* kt = k + pg.chunk_row(b, kvh, Hkv, N, c) * D;
  constexpr int EPV = 16 / (int)sizeof(IO);  // elements per 16-byte load
  for (int i = tid * EPV; i < S * D; i += 256 * EPV) {
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(kt + i);
    float* dst = ks + (i / D) * LD + (i % D);
    if constexpr (sizeof(IO) == 2) {
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        dst[2 * m] = __uint_as_float(wd[m] << 16);
        dst[2 * m + 1] = __uint_as_float(wd[m] & 0xffff0000u);
      }
    } else {
      dst[0] = __uint_as_float(raw.x);
      dst[1] = __uint_as_float(raw.y);
      dst[2] = __uint_as_float(raw.z);
      dst[3] = __uint_as_float(raw.w);
    }
  }
  __syncthreads();

  const float tau = 1.0f / sqrtf((float)D);
  // every wave runs the same number of rounds so the barriers stay uniform
  for (int g0 = 0; g0 < G; g0 += 4) {
    const int g = g0 + w;
    const bool active = g < G;
    const int l = kvh * G + (active ? g : 0);
    const int64_t row = ((int64_t)b * Hl + l) * C + c;
    if (active) {
      const IO* lq = lmk + row * D;
      for (int e = lane; e < D; e += 64) ls[w][e] = io_traits<IO>::load(lq, e);
    }
    __syncthreads();
    float ent = 0.f;
    if (active) {
      float z = 0.f;
      const float* kr = ks + lane * LD;
#pragma unroll 8
      for (int e = 0; e < D; ++e) z = fmaf(ls[w][e], kr[e], z);
      z *= tau;
      const float m = wave_max(z);
      const float p = expf(z - m);
      const float Z = wave_sum(p);
      const float a = p / Z;
      // -sum_j a_j log a_j, with log a_j = (z_j - m) - log Z
      ent = logf(Z) - wave_sum(a * (z - m));
      as[w][lane] = a;
    }
    __syncthreads();
    if (active) {
      float* out = kc + row * D;
      for (int e = lane; e < D; e += 64) {
        float acc = 0.f;
#pragma unroll 8
        for (int j = 0; j < S; ++j) acc = fmaf(as[w][j], ks[j * LD + e], acc);
        out[e] = acc;
      }
      if (lane == 0) bc[row] = ent;
    }
    __syncthreads();
  }
}

template <typename IO>
hipError_t launch_compress_t(const void* k, const void* lmk, float* kc, float* bc, int B, int Hkv, int Hl, int N,
                             int d, int c_begin, int c_end, hipStream_t st, KvPages pg) {
  const int C = N / 64, n = c_end - c_begin;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((int64_t)B * Hkv * n)), block(256);
  if (d == 64)
    hipLaunchKernelGGL((compress_kernel<IO, 64>), grid, block, 0, st, (const IO*)k, (const IO*)lmk, kc, bc, Hkv,
                       Hl, N, C, c_begin, n, pg);
  else
    hipLaunchKernelGGL((compress_kernel<IO, 128>), grid, block, 0, st, (const IO*)k, (const IO*)lmk, kc, bc, Hkv,
                       Hl, N, C, c_begin, n, pg);
  return hipGetLastError();
}

hipError_t launch_compress(int io, const void* k, const void* lmk, float* kc, float* bc, int B, int Hkv, int Hl,
                           int N, int d, int c_begin, int c_end, hipStream_t st, KvPages pg) {
  return io == 0 ? launch_compress_t<float>(k, lmk, kc, bc, B, Hkv, Hl, N, d, c_begin, c_end, st, pg)
                 : launch_compress_t<bf16_t>(k, lmk, kc, bc, B, Hkv, Hl, N, d, c_begin, c_end, st, pg);
}

}  // namespace hils

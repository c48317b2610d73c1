// Device helpers shared by the HiLS kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define HILS_DEV static __device__ __forceinline__

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

namespace hils {

constexpr int WAVE = 64;

// ---------------------------------------------------------------- element types
// bf16 values are carried as their 16-bit patterns (uint16_t); fp32 as float.
struct bf16_t {
  uint16_t bits;
};

HILS_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// float -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32; NaN stays NaN)
HILS_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two floats -> packed bf16 pair (lo in bits 0..15), one instruction
HILS_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// two floats -> packed fp16 pair (lo in bits 0..15), round to nearest even, one instruction
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
HILS_DEV uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

HILS_DEV uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
HILS_DEV float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

template <typename T>
struct io_traits;
template <>
struct io_traits<float> {
  static constexpr int terms = 3;  // bf16 terms needed to carry an fp32 value exactly
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
  // four consecutive elements; i must be a multiple of 4
  static __device__ __forceinline__ void load4(const float* p, int64_t i, float (&v)[4]) {
    const float4 x = *reinterpret_cast<const float4*>(p + i);
    v[0] = x.x;
    v[1] = x.y;
    v[2] = x.z;
    v[3] = x.w;
  }
};
template <>
struct io_traits<bf16_t> {
  static constexpr int terms = 1;
  static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
  static __device__ __forceinline__ void load4(const bf16_t* p, int64_t i, float (&v)[4]) {
    const u32x2_t x = *reinterpret_cast<const u32x2_t*>(p + i);
    v[0] = __uint_as_float(x.x << 16);
    v[1] = __uint_as_float(x.x & 0xffff0000u);
    v[2] = __uint_as_float(x.y << 16);
    v[3] = __uint_as_float(x.y & 0xffff0000u);
  }
};

// Split x into NT bf16 terms whose sum carries x to ~8*NT mantissa bits
// (NT = 3 reproduces any fp32 value exactly).  Each residual is exact in fp32.
template <int NT>
HILS_DEV void split_bf16(float x, uint16_t (&t)[NT]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    t[i] = f32_to_bf16(x);
    x -= bf16_to_f32(t[i]);
  }
}

// The same for 8 values at once into NT packed MFMA operands (term j of element m in
// lane slot m of out[j]), with packed conversions.  x is consumed.
template <int NT>
HILS_DEV void split8(float (&x)[8], u32x4_t (&out)[NT]) {
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    u32x4_t u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    u.z = pack_bf16x2(x[4], x[5]);
    u.w = pack_bf16x2(x[6], x[7]);
    out[j] = u;
    if (j + 1 < NT) {
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[2 * m] -= __uint_as_float(w4[m] << 16);
        x[2 * m + 1] -= __uint_as_float(w4[m] & 0xffff0000u);
      }
    }
  }
}

// -------------------------------------------------------------------- MFMA 32x32x16
// D[32x32] += A[32x16] * B[16x32], bf16 inputs, fp32 accumulation.
// Operand lanes: A lane l supplies row (l & 31), B lane l supplies column (l & 31);
// lane half h = l >> 5 supplies 8 k-elements.  Every MFMA k-operand in this library
// uses the same (h, m) -> k mapping on both sides, so only the output layout
// matters: accumulator register r of lane l holds D[row = acc_row(r, h)][col = l & 31].
HILS_DEV f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
HILS_DEV constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// -------------------------------------------------------------------- MFMA 16x16x32
// D[16x16] += A[16x32] * B[32x16]: A lane l supplies row (l & 15) and B lane l column
// (l & 15), each with k-elements 8 (l >> 4) + m (m = 0..7); accumulator register i of
// lane l holds D[row = 4 (l >> 4) + i][col = l & 15].
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
HILS_DEV f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The k-permutation used for every MFMA k-operand: k-step ks (16 values), lane
// half h, element m (0..7) -> index 16*ks + 8*(m>>2) + 4*h + (m&3).  With it, the
// accumulator register r of an output tile t feeds k-step 2t + (r>>3), element
// r & 7 of a following MFMA without moving data between lanes.
HILS_DEV constexpr int kperm(int ks, int h, int m) { return 16 * ks + 8 * (m >> 2) + 4 * h + (m & 3); }

HILS_DEV bf16x8_t pack8(const uint16_t (&v)[8]) {
  u32x4_t u;
  u.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  u.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  u.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
  u.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}
HILS_DEV bf16x8_t pack8(u32x2_t lo, u32x2_t hi) {
  u32x4_t u;
  u.x = lo.x;
  u.y = lo.y;
  u.z = hi.x;
  u.w = hi.y;
  return __builtin_bit_cast(bf16x8_t, u);
}
HILS_DEV f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ------------------------------------------------------------------ wave helpers
HILS_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
HILS_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
HILS_DEV int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// --------------------------------------------------------- (score, chunk) ordering
// A candidate is packed into one 64-bit key: larger key = better candidate
// (higher score; equal scores -> lower chunk id).  Key 0 means "empty".
HILS_DEV uint32_t order_f32(float s) {
  uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
HILS_DEV float unorder_f32(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}
HILS_DEV uint64_t make_key(float s, int c) {
  return ((uint64_t)order_f32(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)c);
}
HILS_DEV float key_score(uint64_t k) { return unorder_f32((uint32_t)(k >> 32)); }
HILS_DEV int key_chunk(uint64_t k) { return (int)(0xffffffffu - (uint32_t)k); }
// the key with its halves swapped: larger = lower chunk id, whatever the scores (the
// empty key stays 0); applied twice it gives the key back.  Sorting swapped keys best
// first orders a list by ascending chunk id.
HILS_DEV uint64_t key_by_id(uint64_t k) { return (k << 32) | (k >> 32); }

// ------------------------------------------------------------- XCD-aware ordering
// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs (each
// with a private L2).  remap_xcd gives workgroup `bid` of `nblocks` a work index
// such that each XCD receives one contiguous range of work items, so items that
// share data (the same head) share an L2.  Correctness does not depend on it.
HILS_DEV int remap_xcd(int bid, int nblocks) {
  const int per = (nblocks + 7) >> 3;
  const int xcd = bid & 7, j = bid >> 3;
  return xcd * per + j;  // may be >= nblocks: the caller skips it
}

// Candidate chunks of the query at position i (chunks of 64 keys): the complete chunks
// before its local window of nw chunks (the own chunk and the nw - 1 before it), at
// most C.  nw = 1 leaves every complete past chunk a candidate.
HILS_DEV int candidate_chunks(int i, int C, int nw) { return min(C, max(0, (i >> 6) - nw + 1)); }

}  // namespace hils

// Sorted candidate lists of 64-bit selection keys (make_key: larger = better, equal
// scores -> lower chunk id; 0 = empty, sorts last), one key per lane in each 32-lane half
// of a wave, best first (lane j holds the j-th best).  A 64-entry list is two such
// registers: hi (ranks 0..31) and lo (ranks 32..63).  Used where the top-K may exceed 32.
#pragma once
#include "hils_common.h"

namespace hils {
namespace kl {

template <int CTRL>
HILS_DEV int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false);
}

// value of lane j ^ X within the half (X = 1, 2, 4, 8, 16), or of lane 31 - j (X = 31)
template <int X>
HILS_DEV uint32_t x32(uint32_t v, int j) {
  const int iv = (int)v;
  if constexpr (X == 1) {
    return (uint32_t)dpp<0xB1>(iv);  // quad_perm [1,0,3,2]
  } else if constexpr (X == 2) {
    return (uint32_t)dpp<0x4E>(iv);  // quad_perm [2,3,0,1]
  } else if constexpr (X == 4 || X == 8) {
    const int up = dpp<0x100 + X>(iv);  // row_shl: lane i <- lane i + X
    const int dn = dpp<0x110 + X>(iv);  // row_shr: lane i <- lane i - X
    return (uint32_t)((j & X) ? dn : up);
  } else if constexpr (X == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle(iv, 0x401F);  // xor 16 within 32 lanes
  } else {
    static_assert(X == 31, "");
    return (uint32_t)__builtin_amdgcn_ds_swizzle(iv, 0x7C1F);  // reverse within 32 lanes
  }
}
template <int X>
HILS_DEV uint64_t x64(uint64_t v, int j) {
  return ((uint64_t)x32<X>((uint32_t)(v >> 32), j) << 32) | x32<X>((uint32_t)v, j);
}
// compare-exchange with lane j ^ X: keep the larger key if keep_larger, else the smaller
template <int X>
HILS_DEV void cx(uint64_t& k, int j, bool keep_larger) {
  const uint64_t p = x64<X>(k, j);
  k = ((p > k) == keep_larger) ? p : k;
}

// bitonic sort, best first
HILS_DEV void sort(uint64_t& k, int j) {
#define HILS_KL_STAGE(K_, X_) cx<X_>(k, j, ((j & X_) == 0) == (((j & K_) == 0) || K_ == 32));
  HILS_KL_STAGE(2, 1)
  HILS_KL_STAGE(4, 2) HILS_KL_STAGE(4, 1)
  HILS_KL_STAGE(8, 4) HILS_KL_STAGE(8, 2) HILS_KL_STAGE(8, 1)
  HILS_KL_STAGE(16, 8) HILS_KL_STAGE(16, 4) HILS_KL_STAGE(16, 2) HILS_KL_STAGE(16, 1)
  HILS_KL_STAGE(32, 16) HILS_KL_STAGE(32, 8) HILS_KL_STAGE(32, 4) HILS_KL_STAGE(32, 2) HILS_KL_STAGE(32, 1)
#undef HILS_KL_STAGE
}
// a bitonic sequence (one rise and one fall) -> sorted best first
HILS_DEV void clean(uint64_t& k, int j) {
  cx<16>(k, j, (j & 16) == 0);
  cx<8>(k, j, (j & 8) == 0);
  cx<4>(k, j, (j & 4) == 0);
  cx<2>(k, j, (j & 2) == 0);
  cx<1>(k, j, (j & 1) == 0);
}
// a, b sorted -> a = the best 32 of both, sorted
HILS_DEV void top(uint64_t& a, uint64_t b, int j) {
  const uint64_t r = x64<31>(b, j);
  a = r > a ? r : a;
  clean(a, j);
}
// a, b sorted -> a = the best 32 of both, b = the other 32, both sorted (with b reversed,
// a ++ b is bitonic; position-wise max and min are its two halves)
HILS_DEV void split(uint64_t& a, uint64_t& b, int j) {
  const uint64_t r = x64<31>(b, j);
  const uint64_t mx = r > a ? r : a, mn = r > a ? a : r;
  a = mx;
  b = mn;
  clean(a, j);
  clean(b, j);
}
// (hi, lo) a sorted 64-list, b a sorted 32-list -> (hi, lo) = the best 64 of all, sorted:
// the best 32 of hi and b rank above everything else, the rest compete with lo
HILS_DEV void insert64(uint64_t& hi, uint64_t& lo, uint64_t b, int j) {
  split(hi, b, j);
  top(lo, b, j);
}
// two sorted 64-lists -> (hi, lo) = the best 64 of both, sorted
HILS_DEV void merge64(uint64_t& hi, uint64_t& lo, uint64_t hi2, uint64_t lo2, int j) {
  split(hi, hi2, j);
  top(hi2, lo, j);
  top(hi2, lo2, j);
  lo = hi2;
}
// the first m (m <= 64) keys of the sorted 64-list (hi, lo) of this lane's half, reordered
// by ascending chunk id (hi holds positions 0..31, lo 32..63), zero keys after them
HILS_DEV void ids_ascending(uint64_t& hi, uint64_t& lo, int m, int j) {
  hi = j < m ? key_by_id(hi) : 0ull;
  lo = 32 + j < m ? key_by_id(lo) : 0ull;
  sort(hi, j);
  sort(lo, j);
  split(hi, lo, j);
  hi = key_by_id(hi);
  lo = key_by_id(lo);
}
// The same networks on float keys with v_med3_f32: bnd = pinf keeps the larger of a pair,
// ninf the smaller (+-inf hidden from the compiler, so that the med3s stay med3s).
template <int X>
HILS_DEV void cxf(float& k, int j, float bnd) {
  k = __builtin_amdgcn_fmed3f(k, __uint_as_float(x32<X>(__float_as_uint(k), j)), bnd);
}
// bitonic sort, largest first
HILS_DEV void sortf(float& k, int j, float pinf, float ninf) {
#define HILS_KL_STAGE(K_, X_) cxf<X_>(k, j, (((j & X_) == 0) == (((j & K_) == 0) || K_ == 32)) ? pinf : ninf);
  HILS_KL_STAGE(2, 1)
  HILS_KL_STAGE(4, 2) HILS_KL_STAGE(4, 1)
  HILS_KL_STAGE(8, 4) HILS_KL_STAGE(8, 2) HILS_KL_STAGE(8, 1)
  HILS_KL_STAGE(16, 8) HILS_KL_STAGE(16, 4) HILS_KL_STAGE(16, 2) HILS_KL_STAGE(16, 1)
  HILS_KL_STAGE(32, 16) HILS_KL_STAGE(32, 8) HILS_KL_STAGE(32, 4) HILS_KL_STAGE(32, 2) HILS_KL_STAGE(32, 1)
#undef HILS_KL_STAGE
}
// a, b sorted -> a = the largest 32 of both, b = the other 32, both sorted
HILS_DEV void splitf(float& a, float& b, int j, float pinf, float ninf) {
  const float r = __uint_as_float(x32<31>(__float_as_uint(b), j));
  b = __builtin_amdgcn_fmed3f(a, r, ninf);
  a = __builtin_amdgcn_fmed3f(a, r, pinf);
#define HILS_KL_CLEAN(X_)                                  \
  cxf<X_>(a, j, (j & X_) == 0 ? pinf : ninf); \
  cxf<X_>(b, j, (j & X_) == 0 ? pinf : ninf);
  HILS_KL_CLEAN(16) HILS_KL_CLEAN(8) HILS_KL_CLEAN(4) HILS_KL_CLEAN(2) HILS_KL_CLEAN(1)
#undef HILS_KL_CLEAN
}

// key of rank p (p < 64) of the 64-list (hi, lo) of this lane's half
HILS_DEV uint64_t rank_key(uint64_t hi, uint64_t lo, int p, int lane) {
  const int src = (lane & 32) + (p & 31);
  return p < 32 ? __shfl(hi, src) : __shfl(lo, src);
}

}  // namespace kl
}  // namespace hils

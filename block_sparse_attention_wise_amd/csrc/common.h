// Shared device helpers of the WISE HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wise {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  Map hardware workgroup p to a logical work item so that
// every XCD walks one contiguous range of logical items: rows of the same head
// (which share K/V) then run on the same XCD and hit the same L2.
__device__ __forceinline__ int xcd_remap(int p, int n) {
  const int x = p & 7, idx = p >> 3;
  const int base = n >> 3, rem = n & 7;
  return x * base + (x < rem ? x : rem) + idx;
}

// Value held by lane l ^ 32 combined with this lane's via one permlane32 swap:
// the swap returns {own, other} (in some order), so max/sum of the pair are
// the cross-half max/sum.
__device__ __forceinline__ float halves_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// x of lane (l - n) within the same 16-lane row (0 for the first n lanes of a row).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, false));
}

// Sum over all 64 lanes, returned in every lane: DPP row shifts leave each 16-lane
// row's sum in its lane 15, and the four row sums are read back as scalars.
__device__ __forceinline__ float wave_sum(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  const int xi = __float_as_int(x);
  return (__int_as_float(__builtin_amdgcn_readlane(xi, 15)) + __int_as_float(__builtin_amdgcn_readlane(xi, 31))) +
         (__int_as_float(__builtin_amdgcn_readlane(xi, 47)) + __int_as_float(__builtin_amdgcn_readlane(xi, 63)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace wise

// 64-bit argmax keys: the order-preserving image of a float in the high word
// and the bit-inverted index in the low word.  The unsigned maximum of a set
// of keys is the largest value with the lowest index, whatever order the
// maximum is taken in, so reductions over them are exact and deterministic.
// -0.0 and +0.0 get the same key value; NaN is outside the contract.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace orthrus {

// Monotone map float -> uint32 (-0.0 and +0.0 map to the same key).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long make_key(float x, int idx) {
  return (static_cast<unsigned long long>(ordered_bits(x)) << 32) |
         static_cast<unsigned long long>(~static_cast<uint32_t>(idx));
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ int32_t key_index(unsigned long long k) {
  return static_cast<int32_t>(~static_cast<uint32_t>(k));
}

}  // namespace orthrus

// Wavefront reductions without LDS traffic: DPP row shifts (row_shr within
// each row of 16 lanes, gfx9 encoding 0x110 + n) and lane reads across the
// four rows, in a fixed order.  Every lane of the wavefront must be active.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

namespace orthrus {

constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

// v from the lane CTRL names within its row; lanes whose source lies outside
// the row keep `fill`.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v, float fill) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v), __float_as_int(fill)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v, double fill) {
  const int lo = dpp_i32<CTRL>(__double2loint(v), __double2loint(fill));
  const int hi = dpp_i32<CTRL>(__double2hiint(v), __double2hiint(fill));
  return __hiloint2double(hi, lo);
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v, unsigned long long fill) {
  const int lo = dpp_i32<CTRL>(static_cast<int>(static_cast<uint32_t>(v)), static_cast<int>(static_cast<uint32_t>(fill)));
  const int hi = dpp_i32<CTRL>(static_cast<int>(static_cast<uint32_t>(v >> 32)),
                               static_cast<int>(static_cast<uint32_t>(fill >> 32)));
  return (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                          __builtin_amdgcn_readlane(__double2loint(v), lane));
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int lane) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Sum over the wavefront (the rows' scans, then the four rows in order), the
// same value in every lane.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kRowShr1>(v, 0.0);
  v += dpp_f64<kRowShr2>(v, 0.0);
  v += dpp_f64<kRowShr4>(v, 0.0);
  v += dpp_f64<kRowShr8>(v, 0.0);
  return ((readlane_f64(v, 15) + readlane_f64(v, 31)) + readlane_f64(v, 47)) + readlane_f64(v, 63);
}

// Maxima over the wavefront, the same value in every lane.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kRowShr1>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowShr2>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowShr4>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowShr8>(v, -INFINITY));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_i32<kRowShr1>(v, INT_MIN));
  v = max(v, dpp_i32<kRowShr2>(v, INT_MIN));
  v = max(v, dpp_i32<kRowShr4>(v, INT_MIN));
  v = max(v, dpp_i32<kRowShr8>(v, INT_MIN));
  return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
             max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  auto mx = [](unsigned long long a, unsigned long long b) { return a > b ? a : b; };
  v = mx(v, dpp_u64<kRowShr1>(v, 0ull));
  v = mx(v, dpp_u64<kRowShr2>(v, 0ull));
  v = mx(v, dpp_u64<kRowShr4>(v, 0ull));
  v = mx(v, dpp_u64<kRowShr8>(v, 0ull));
  return mx(mx(readlane_u64(v, 15), readlane_u64(v, 31)), mx(readlane_u64(v, 47), readlane_u64(v, 63)));
}

}  // namespace orthrus

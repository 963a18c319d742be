// Keys and values of new rows in the e4m3 cache's format.
//
// An e4m3 cache stores code = e4m3(fp32(x) / scale[h]) for every element x of
// KV head h.  The block's own rows are converted the same way before both
// attention passes, so the verify pass reads a block key exactly as the cache
// will hold it after the commit, as plain decoding reads its own key back from
// the cache; that keeps the accepted tokens equal to greedy decoding's
// (gist.science technical summary of "Orthrus: Memory-Efficient Parallel Token
// Generation via Dual-View Diffusion", section 2.3 step 3).
//
// The rounding is written out rather than taken from a hardware conversion so
// that its rules are explicit: nearest e4m3 value, ties to the even code,
// magnitudes beyond the largest value (448) saturate, the sign of zero stays.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "check.h"
#include "launch.h"

namespace orthrus {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Finite fp32 -> OCP E4M3 code (1 sign, 4 exponent bits with bias 7, 3
// mantissa bits; exponent field 0 holds multiples of 2^-9).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float m = fabsf(x);
  uint32_t code;
  if (m >= 448.0f) {
    code = 0x7Eu;                                   // saturate at 448
  } else if (m < 0.015625f) {                       // below 2^-6: subnormal codes 0..8
    code = uint32_t(__builtin_rintf(m * 512.0f));   // exact scaling, ties to even
  } else {
    // rebias the exponent from 127 to 7, keep 3 of the 23 mantissa bits,
    // rounding to nearest even (a carry moves into the exponent by itself)
    const uint32_t v = __float_as_uint(m) - ((127u - 7u) << 23);
    code = (v + 0x7FFFFu + ((v >> 20) & 1u)) >> 20;
  }
  return sign | code;
}

struct QuantArgs {
  const uint16_t* k;
  const uint16_t* v;
  const float* k_scale;
  const float* v_scale;
  uint8_t* k_out;
  uint8_t* v_out;
  int64_t n8;   // 8-element groups per tensor
  int Hkv, D;
};

// One thread per 8 consecutive elements of K or V (16 bytes in, 8 bytes out).
__global__ __launch_bounds__(256) void quantize_kv_kernel(QuantArgs a) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < 2 * a.n8; u += stride) {
    const bool is_v = u >= a.n8;
    const int64_t w = is_v ? u - a.n8 : u;
    const int h = int((w * 8 / a.D) % a.Hkv);
    const float s = (is_v ? a.v_scale : a.k_scale)[h];
    const u32x4 x = *reinterpret_cast<const u32x4*>((is_v ? a.v : a.k) + w * 8);
    uint32_t q[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(x[i] << 16) / s;
      const float hi = __uint_as_float(x[i] & 0xFFFF0000u) / s;
      q[i >> 1] |= (e4m3_code(lo) | (e4m3_code(hi) << 8)) << (16 * (i & 1));
    }
    *reinterpret_cast<u32x2*>((is_v ? a.v_out : a.k_out) + w * 8) = u32x2{q[0], q[1]};
  }
}

}  // namespace

hipError_t launch_quantize_kv(const void* k, const void* v, const float* k_scale, const float* v_scale,
                              int rows, int Hkv, int D, void* k_out, void* v_out, hipStream_t stream) {
  QuantArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_out = static_cast<uint8_t*>(k_out);
  a.v_out = static_cast<uint8_t*>(v_out);
  a.n8 = int64_t(rows) * Hkv * D / 8;
  a.Hkv = Hkv;
  a.D = D;
  const int64_t threads = 2 * a.n8;
  const int64_t blocks = (threads + 255) / 256;
  const unsigned grid = unsigned(blocks < 4096 ? blocks : 4096);
  return launch_kernel(&quantize_kv_kernel, dim3(grid), dim3(256), stream, a);
}

}  // namespace orthrus

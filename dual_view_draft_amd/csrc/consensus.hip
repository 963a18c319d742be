// Consensus of the two views: vocabulary argmax and longest matching prefix.
//
// The drafted tokens are the argmax of the diffusion view's logits; the AR
// view's greedy tokens are the argmax of the verify pass's logits; drafted
// tokens are accepted left to right while they equal the AR tokens, and the
// AR token at the first mismatch is appended (gist.science technical summary
// of "Orthrus: Memory-Efficient Parallel Token Generation via Dual-View
// Diffusion", section 2.3 steps 1 and 3; Hacker News thread "Orthrus-Qwen3:
// up to 7.8x tokens/forward ...", post #21).
//
// Argmax is an HBM stream over fp32 logits.  Every row is cut into chunks
// processed by independent workgroups; each reduces its chunk to one 64-bit
// key (order-preserving image of the value in the high word, bit-inverted
// index in the low word).  The maximum key is the maximum value with the
// lowest index, whatever order the reduction runs in, so the result is
// deterministic and independent of the launch shape.  A small second kernel
// reduces the chunk keys of each row (argmax, one wavefront per row) or of
// each sequence's K rows and runs the prefix scan with one wavefront ballot
// (accept; there a small group of lanes reduces each row, so that one
// workgroup handles all K rows in a single pass).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "check.h"
#include "dpp.h"
#include "keys.h"
#include "launch.h"

namespace orthrus {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PartialArgs {
  const float* logits;  // [rows][V]
  unsigned long long* keys;  // [rows][nchunks]
  int rows, V, chunk, nchunks;
};

struct FinalArgs {
  const unsigned long long* keys;
  int32_t* out;
  int rows, nchunks;
};

struct AcceptArgs {
  const unsigned long long* keys;  // [B*K][nchunks]
  const int32_t* draft;            // [B][K]
  int32_t* a;
  int32_t* n_acc;
  int32_t* n_emit;
  int32_t* next_anchor;
  int B, K, nchunks, lpr;
};

// (the maximum of 64-bit keys does not depend on the order of reduction)
__device__ __forceinline__ unsigned long long wave_max(unsigned long long k) { return wave_max_u64(k); }

__global__ __launch_bounds__(256) void argmax_partial_kernel(PartialArgs a) {
  constexpr int UNR = 4;                         // float4 loads in flight per thread
  __shared__ unsigned long long red[4];
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const int lo = c * a.chunk;
  const int hi = min(lo + a.chunk, a.V);
  const float* base = a.logits + size_t(row) * a.V;
  unsigned long long best = 0ull;
  if ((a.V & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0) {
    const f32x4* b4 = reinterpret_cast<const f32x4*>(base);
    const int hi4 = hi >> 2;
    for (int v0 = (lo >> 2) + threadIdx.x; v0 < hi4; v0 += 256 * UNR) {
      f32x4 x[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int v4 = v0 + u * 256;
        x[u] = v4 < hi4 ? b4[v4] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int v4 = v0 + u * 256;
        if (v4 < hi4) {
          const int v = v4 * 4;
          best = umax64(best, make_key(x[u][0], v));
          best = umax64(best, make_key(x[u][1], v + 1));
          best = umax64(best, make_key(x[u][2], v + 2));
          best = umax64(best, make_key(x[u][3], v + 3));
        }
      }
    }
  } else {
    for (int v = lo + threadIdx.x; v < hi; v += 256) best = umax64(best, make_key(base[v], v));
  }
  best = wave_max(best);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    best = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
    a.keys[size_t(row) * a.nchunks + c] = best;
  }
}

// Lanes that reduce one row's chunk keys: a power of two (1..64) that leaves
// each lane kpl keys or fewer up to 64 kpl chunks, so a row costs one round
// trip of loads and log2(lanes) shuffle steps, and a wavefront reduces
// 64 / lanes rows at once.
int lanes_per_row(int nchunks, int kpl) {
  const int want = (nchunks + kpl - 1) / kpl;
  int lpr = 1;
  while (lpr < want && lpr < 64) lpr <<= 1;
  return lpr;
}

// Maximum over the aligned group of lpr lanes (lpr a power of two <= 64).
__device__ __forceinline__ unsigned long long group_max(unsigned long long k, int lpr) {
  for (int off = lpr >> 1; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(k), off);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(k >> 32), off);
    k = umax64(k, (static_cast<unsigned long long>(hi) << 32) | lo);
  }
  return k;
}

// One row's maximum key, reduced by the lpr lanes of its group (sub = this
// lane's place in the group); every lane of the group receives it.
template <int KPL>
__device__ __forceinline__ unsigned long long row_key(const unsigned long long* keys, int nchunks, int sub,
                                                      int lpr) {
  unsigned long long best = 0ull;
  for (int c0 = 0; c0 < nchunks; c0 += KPL * lpr) {
    unsigned long long k[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = c0 + j * lpr + sub;
      k[j] = c < nchunks ? keys[c] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j) best = umax64(best, k[j]);
  }
  return group_max(best, lpr);
}

// One wavefront per row (lane c reads chunks c, c + 64, ...): the rows of a
// call run side by side on many CUs.
__global__ __launch_bounds__(256) void argmax_final_kernel(FinalArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;                     // uniform per wavefront
  const int lane = threadIdx.x & 63;
  const unsigned long long* keys = a.keys + size_t(row) * a.nchunks;
  unsigned long long best = 0ull;
  for (int c = lane; c < a.nchunks; c += 64) best = umax64(best, keys[c]);
  best = wave_max(best);
  if (lane == 0) a.out[row] = key_index(best);
}

// One workgroup of THREADS threads per sequence: groups of lpr lanes reduce
// the K rows' chunk keys (THREADS / lpr rows at a time, KPL keys per lane
// and round trip), then wavefront 0 runs the prefix scan with lane i owning
// block row i (K <= 64).  256 threads serve when they cover all K rows in one
// pass (few chunks per row, as on the logits path); otherwise 1024.
template <int THREADS, int KPL>
__global__ __launch_bounds__(THREADS) void accept_kernel(AcceptArgs a) {
  __shared__ int32_t tok_s[64];
  const int b = blockIdx.x;
  const int sub = threadIdx.x % a.lpr;
  const int rows_per_pass = THREADS / a.lpr;
  for (int i0 = 0; i0 < a.K; i0 += rows_per_pass) {
    const int i = i0 + threadIdx.x / a.lpr;
    if (i < a.K) {                               // whole groups take the same branch
      const unsigned long long m =
          row_key<KPL>(a.keys + (size_t(b) * a.K + i) * a.nchunks, a.nchunks, sub, a.lpr);
      if (sub == 0) tok_s[i] = key_index(m);
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int i = threadIdx.x;
  int32_t tok = 0;
  bool mismatch = false;
  if (i < a.K) {
    const size_t row = size_t(b) * a.K + i;
    tok = tok_s[i];
    a.a[row] = tok;
    mismatch = a.draft[row] != tok;
  }
  const unsigned long long bad = __ballot(mismatch);
  const int n_acc = bad ? (__ffsll(static_cast<long long>(bad)) - 1) : a.K;
  const int n_emit = n_acc < a.K ? n_acc + 1 : a.K;
  const int32_t nxt = __shfl(tok, n_emit - 1);
  if (i == 0) {
    a.n_acc[b] = n_acc;
    a.n_emit[b] = n_emit;
    a.next_anchor[b] = nxt;
  }
}

hipError_t launch_partial(const ArgmaxPlan& p, const float* logits, void* ws, hipStream_t stream) {
  PartialArgs a{logits, static_cast<unsigned long long*>(ws), p.rows, p.V, p.chunk, p.nchunks};
  return launch_kernel(&argmax_partial_kernel, dim3(p.nchunks, p.rows), dim3(256), stream, a);
}

}  // namespace

hipError_t launch_argmax_keys(const unsigned long long* keys, int rows, int nchunks, int32_t* out,
                              hipStream_t stream) {
  FinalArgs f{keys, out, rows, nchunks};
  return launch_kernel(&argmax_final_kernel, dim3((rows + 3) / 4), dim3(256), stream, f);
}

hipError_t launch_accept_keys(const unsigned long long* keys, int nchunks, const int32_t* draft, int B,
                              int K, int32_t* a, int32_t* n_acc, int32_t* n_emit, int32_t* next_anchor,
                              hipStream_t stream) {
  // 256 threads when they cover the K rows in one pass, else 1024
  AcceptArgs x{keys, draft, a, n_acc, n_emit, next_anchor, B, K, nchunks, lanes_per_row(nchunks, 8)};
  if (K * x.lpr <= 256) return launch_kernel(&accept_kernel<256, 8>, dim3(B), dim3(256), stream, x);
  x.lpr = lanes_per_row(nchunks, 16);
  return launch_kernel(&accept_kernel<1024, 16>, dim3(B), dim3(1024), stream, x);
}

hipError_t launch_argmax(const ArgmaxPlan& p, const float* logits, int32_t* out, void* ws,
                         hipStream_t stream) {
  hipError_t e = launch_partial(p, logits, ws, stream);
  if (e != hipSuccess) return e;
  return launch_argmax_keys(static_cast<const unsigned long long*>(ws), p.rows, p.nchunks, out, stream);
}

hipError_t launch_accept(const ArgmaxPlan& p, const float* logits_a, const int32_t* draft, int B,
                         int K, int32_t* a, int32_t* n_acc, int32_t* n_emit, int32_t* next_anchor,
                         void* ws, hipStream_t stream) {
  hipError_t e = launch_partial(p, logits_a, ws, stream);
  if (e != hipSuccess) return e;
  return launch_accept_keys(static_cast<const unsigned long long*>(ws), p.nchunks, draft, B, K, a, n_acc,
                            n_emit, next_anchor, stream);
}

}  // namespace orthrus

// Consensus at temperature T > 0: sampling of the drafted tokens and the
// speculative-sampling acceptance of them.
//
// The pages fix the greedy rule only (gist.science technical summary of
// "Orthrus: Memory-Efficient Parallel Token Generation via Dual-View
// Diffusion", section 2.3 step 3) and state that the output distribution is
// the AR model's (Hacker News thread "Orthrus-Qwen3: up to 7.8x
// tokens/forward ...", post #21).  For T > 0 the rule here is standard
// speculative sampling: with q_i = softmax(z_d[i] / T) (draft view) and
// p_i = softmax(z_a[i] / T) (AR view), drafted token d_i is accepted when
// u_acc * q_i(d_i) < p_i(d_i); at the first rejection the emitted token is a
// draw of max(0, p_i - q_i) and the step ends.  Every draw is an inverse-CDF
// draw with a caller-supplied uniform: the smallest v whose cumulative weight
// exceeds u times the total.
//
// Work layout.  Rows are cut into vocabulary chunks; a statistics pass
// writes, per (row, chunk), the chunk's maximum logit m_c (fp32) and
// s_c = sum exp((z - m_c) / T) (fp64).  A row's maximum M and normaliser
// Z = sum_c s_c exp((m_c - M) / T) are then combined in chunk order.  A draw
// finds its chunk from the chunk sums in order and scans that chunk only.
// The exponentials and sums are fp64 so that every decision (a comparison
// with u times a probability or a cumulative weight) agrees with an exact
// evaluation except within about 1e-15 (relative) of its threshold.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "check.h"
#include "launch.h"

namespace orthrus {
namespace {

constexpr int kThreads = 256;

struct SeqState {      // per sequence, after the acceptance test
  double Za, Zd;       // normalisers of row j (AR, draft views)
  float Ma, Md;        // maxima of row j
  int j;               // first rejected row (K: none)
  int pad;
};

struct StatsArgs {
  const float* z0;     // rows [0, rows0) of the statistics
  const float* z1;     // rows [rows0, rows)
  float* cm;           // [rows][nchunks]
  double* cs;          // [rows][nchunks]
  int rows0, rows, V, chunk, nchunks;
  double inv_t;
};

struct SampleArgs {
  const float* z;
  const float* u;      // [rows]
  const float* cm;
  const double* cs;
  int32_t* out;        // [rows]
  int V, chunk, nchunks;
  double inv_t;
};

struct DecideArgs {
  const float* zd;     // [B*K][V] draft view
  const float* za;     // [B*K][V] AR view
  const int32_t* draft;
  const float* u_acc;  // [B][K]
  const float* cm;     // [2*B*K][nchunks]: draft rows, then AR rows
  const double* cs;
  int32_t* tokens;     // [B][K]
  int32_t* n_acc;
  int32_t* n_emit;
  int32_t* next_anchor;
  SeqState* seq;       // [B]
  int B, K, V, nchunks;
  double inv_t;
};

struct ResidualArgs {
  const float* zd;
  const float* za;
  const float* u_res;  // [B][K]
  const float* cm;
  const double* cs;
  const SeqState* seq;
  double* rs;          // [B][nchunks] residual chunk sums
  int32_t* tokens;
  int32_t* next_anchor;
  int B, K, V, chunk, nchunks;
  double inv_t;
};

__device__ __forceinline__ double wexp(float z, float m, double inv_t) {
  return exp((double(z) - double(m)) * inv_t);
}

// Sum (or max) over the workgroup in a fixed order: wavefront butterflies,
// then the four wavefront results in order.
__device__ double block_sum(double x, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ float block_max(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// A row's maximum and normaliser from its chunk statistics, in chunk order.
__device__ void row_norm(const float* cm, const double* cs, int nchunks, double inv_t, float* M, double* Z) {
  float m = -INFINITY;
  for (int c = 0; c < nchunks; ++c) m = fmaxf(m, cm[c]);
  double z = 0.0;
  for (int c = 0; c < nchunks; ++c) z += cs[c] * wexp(cm[c], m, inv_t);
  *M = m;
  *Z = z;
}

// Inverse-CDF draw over a row whose chunk weight sums are chunk_sum(c), with
// element weights weight(v): the smallest v whose cumulative weight exceeds
// u times the total.  Runs in one workgroup; every thread returns the token.
// The chunk is found from the chunk sums in order, then thread k of the
// workgroup sums its contiguous share of the chunk; the crossing thread
// rescans its share with the same sequence of additions, so it finds the
// crossing in its share.  If rounding leaves the target beyond every
// cumulative weight, the last element of positive weight is taken.
template <class ChunkSum, class Weight>
__device__ int draw(ChunkSum chunk_sum, Weight weight, int nchunks, int chunk, int V, double u) {
  __shared__ double part[kThreads];
  __shared__ int sel[3];                           // chunk, thread, fallback token
  __shared__ double rem_s;
  const int tid = threadIdx.x;
  if (tid == 0) {
    double total = 0.0;
    for (int c = 0; c < nchunks; ++c) total += chunk_sum(c);
    double target = u * total, before = 0.0;
    int cstar = -1, clast = 0;
    for (int c = 0; c < nchunks; ++c) {
      const double s = chunk_sum(c);
      if (s > 0.0) clast = c;
      if (cstar < 0 && before + s > target) cstar = c;
      if (cstar < 0) before += s;
    }
    sel[0] = cstar < 0 ? clast : cstar;
    // rounding at the very end of the row: no crossing, the last positive weight
    rem_s = cstar < 0 ? INFINITY : target - before;
  }
  __syncthreads();
  const int c = sel[0];
  const double rem = rem_s;
  const int v0 = c * chunk, v1 = min(v0 + chunk, V);
  const int per = (v1 - v0 + kThreads - 1) / kThreads;
  const int a0 = v0 + tid * per, a1 = min(a0 + per, v1);
  double mine = 0.0;
  int last_pos = -1;
  for (int v = a0; v < a1; ++v) {
    const double w = weight(v);
    mine += w;
    if (w > 0.0) last_pos = v;
  }
  part[tid] = mine;
  // the chunk's last positive weight, for the fallback
  int lp = last_pos;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lp = max(lp, __shfl_xor(lp, off));
  if (tid == 0) sel[2] = -1;
  __syncthreads();
  if ((tid & 63) == 0) atomicMax(&sel[2], lp);
  __syncthreads();
  if (tid == 0) {
    double before = 0.0;
    int t = -1;
    for (int k = 0; k < kThreads; ++k) {
      if (before + part[k] > rem) { t = k; break; }
      before += part[k];
    }
    sel[1] = t;
    part[0] = before;                              // the cumulative weight before thread t
  }
  __syncthreads();
  const int t = sel[1];
  int token = sel[2];
  __shared__ int tok_s;
  if (t >= 0 && tid == t) {
    const double before = part[0];
    double run = 0.0;                              // the additions of `mine`, in its order
    int found = -1;
    for (int v = a0; v < a1; ++v) {
      run += weight(v);
      if (before + run > rem) { found = v; break; }
    }
    tok_s = found >= 0 ? found : last_pos;          // (found always: before + mine > rem)
  }
  __syncthreads();
  if (t >= 0) token = tok_s;
  return token < 0 ? v0 : token;
}

// Chunk statistics of every row: m_c and s_c = sum exp((z - m_c) / T).
__global__ __launch_bounds__(kThreads) void sample_stats_kernel(StatsArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int row = blockIdx.y, c = blockIdx.x;
  const float* z = row < a.rows0 ? a.z0 + size_t(row) * a.V : a.z1 + size_t(row - a.rows0) * a.V;
  const int v0 = c * a.chunk, v1 = min(v0 + a.chunk, a.V);
  float m = -INFINITY;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) m = fmaxf(m, z[v]);
  m = block_max(m, redf);
  double s = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) s += wexp(z[v], m, a.inv_t);
  s = block_sum(s, redd);
  if (threadIdx.x == 0) {
    a.cm[size_t(row) * a.nchunks + c] = m;
    a.cs[size_t(row) * a.nchunks + c] = s;
  }
}

// One workgroup per row: out[row] = draw of softmax(z[row] / T) with u[row].
__global__ __launch_bounds__(kThreads) void sample_draw_kernel(SampleArgs a) {
  const int row = blockIdx.x;
  const float* cm = a.cm + size_t(row) * a.nchunks;
  const double* cs = a.cs + size_t(row) * a.nchunks;
  __shared__ float M_s;
  if (threadIdx.x == 0) {
    float M;
    double Z;
    row_norm(cm, cs, a.nchunks, a.inv_t, &M, &Z);
    M_s = M;
  }
  __syncthreads();
  const float M = M_s;
  const float* z = a.z + size_t(row) * a.V;
  const double inv_t = a.inv_t;
  const int tok = draw([&](int c) { return cs[c] * wexp(cm[c], M, inv_t); },
                       [&](int v) { return wexp(z[v], M, inv_t); }, a.nchunks, a.chunk, a.V, double(a.u[row]));
  if (threadIdx.x == 0) a.out[row] = tok;
}

// One wavefront per sequence, lane i = block row i: the acceptance test of
// every row, then the first rejection.
__global__ __launch_bounds__(64) void sample_decide_kernel(DecideArgs a) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int BK = a.B * a.K;
  bool reject = false;
  int32_t t = 0;
  double Za = 0.0, Zd = 0.0;
  float Ma = 0.f, Md = 0.f;
  if (i < a.K) {
    const size_t rd = size_t(b) * a.K + i, ra = BK + rd;
    row_norm(a.cm + rd * a.nchunks, a.cs + rd * a.nchunks, a.nchunks, a.inv_t, &Md, &Zd);
    row_norm(a.cm + ra * a.nchunks, a.cs + ra * a.nchunks, a.nchunks, a.inv_t, &Ma, &Za);
    t = a.draft[rd];
    double p = 0.0, q = 0.0;                       // a token outside the vocabulary has p = q = 0
    if (t >= 0 && t < a.V) {
      p = wexp(a.za[rd * a.V + t], Ma, a.inv_t) / Za;
      q = wexp(a.zd[rd * a.V + t], Md, a.inv_t) / Zd;
    }
    reject = !(double(a.u_acc[rd]) * q < p);
  }
  const unsigned long long bad = __ballot(reject);
  const int j = bad ? (__ffsll(static_cast<long long>(bad)) - 1) : a.K;
  if (i < a.K) a.tokens[size_t(b) * a.K + i] = i < j ? t : -1;
  if (i == 0) {
    a.n_acc[b] = j;
    a.n_emit[b] = j < a.K ? j + 1 : a.K;
    if (j == a.K) {
      a.next_anchor[b] = a.draft[size_t(b) * a.K + a.K - 1];
      a.seq[b] = SeqState{0.0, 0.0, 0.f, 0.f, a.K, 0};
    }
  }
  if (i == j) a.seq[b] = SeqState{Za, Zd, Ma, Md, j, 0};
}

struct Residual {
  const float* za;
  const float* zd;
  float Ma, Md;
  double Za, Zd, inv_t;
  __device__ double operator()(int v) const {
    const double p = wexp(za[v], Ma, inv_t) / Za;
    const double q = wexp(zd[v], Md, inv_t) / Zd;
    return p > q ? p - q : 0.0;
  }
};

// Chunk sums of the residual max(0, p - q) of each sequence's rejected row.
__global__ __launch_bounds__(kThreads) void residual_stats_kernel(ResidualArgs a) {
  __shared__ double redd[4];
  const int b = blockIdx.y, c = blockIdx.x;
  const SeqState st = a.seq[b];
  if (st.j >= a.K) return;                         // uniform: nothing rejected
  const size_t row = size_t(b) * a.K + st.j;
  const Residual r{a.za + row * a.V, a.zd + row * a.V, st.Ma, st.Md, st.Za, st.Zd, a.inv_t};
  const int v0 = c * a.chunk, v1 = min(v0 + a.chunk, a.V);
  double s = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) s += r(v);
  s = block_sum(s, redd);
  if (threadIdx.x == 0) a.rs[size_t(b) * a.nchunks + c] = s;
}

// One workgroup per sequence: the emitted token at the rejected row, a draw
// of max(0, p - q) (of p if the residual is empty, which only rounding can
// cause).
__global__ __launch_bounds__(kThreads) void residual_draw_kernel(ResidualArgs a) {
  const int b = blockIdx.x;
  const SeqState st = a.seq[b];
  if (st.j >= a.K) return;
  const size_t row = size_t(b) * a.K + st.j;
  const double* rs = a.rs + size_t(b) * a.nchunks;
  __shared__ int empty_s;
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int c = 0; c < a.nchunks; ++c) tot += rs[c];
    empty_s = !(tot > 0.0);
  }
  __syncthreads();
  const double u = double(a.u_res[row]);
  int tok;
  if (!empty_s) {
    const Residual r{a.za + row * a.V, a.zd + row * a.V, st.Ma, st.Md, st.Za, st.Zd, a.inv_t};
    tok = draw([&](int c) { return rs[c]; }, r, a.nchunks, a.chunk, a.V, u);
  } else {
    const size_t ra = size_t(a.B) * a.K + row;
    const float* cm = a.cm + ra * a.nchunks;
    const double* cs = a.cs + ra * a.nchunks;
    const float* z = a.za + row * a.V;
    const float M = st.Ma;
    const double inv_t = a.inv_t;
    tok = draw([&](int c) { return cs[c] * wexp(cm[c], M, inv_t); },
               [&](int v) { return wexp(z[v], M, inv_t); }, a.nchunks, a.chunk, a.V, u);
  }
  if (threadIdx.x == 0) {
    a.tokens[row] = tok;
    a.next_anchor[b] = tok;
  }
}

struct Ws {
  float* cm;
  double* cs;
  SeqState* seq;
  double* rs;
};

Ws carve(const SamplePlan& p, void* ws) {
  char* base = static_cast<char*>(ws);
  return Ws{reinterpret_cast<float*>(base + p.cm_off), reinterpret_cast<double*>(base + p.cs_off),
            reinterpret_cast<SeqState*>(base + p.seq_off), reinterpret_cast<double*>(base + p.rs_off)};
}

}  // namespace

static_assert(sizeof(SeqState) == kSampleSeqBytes, "per-sequence state size");

hipError_t launch_sample(const SamplePlan& p, const float* logits, float temperature, const float* u,
                         int32_t* out, void* ws, hipStream_t stream) {
  const Ws w = carve(p, ws);
  const double inv_t = 1.0 / double(temperature);
  StatsArgs s{logits, logits, w.cm, w.cs, p.rows, p.rows, p.V, p.chunk, p.nchunks, inv_t};
  hipError_t e = launch_kernel(&sample_stats_kernel, dim3(p.nchunks, p.rows), dim3(kThreads), stream, s);
  if (e != hipSuccess) return e;
  SampleArgs d{logits, u, w.cm, w.cs, out, p.V, p.chunk, p.nchunks, inv_t};
  return launch_kernel(&sample_draw_kernel, dim3(p.rows), dim3(kThreads), stream, d);
}

hipError_t launch_accept_sampled(const SamplePlan& p, const float* logits_d, const float* logits_a,
                                 const int32_t* draft, int B, int K, float temperature, const float* u_acc,
                                 const float* u_res, int32_t* tokens, int32_t* n_acc, int32_t* n_emit,
                                 int32_t* next_anchor, void* ws, hipStream_t stream) {
  const Ws w = carve(p, ws);
  const double inv_t = 1.0 / double(temperature);
  StatsArgs s{logits_d, logits_a, w.cm, w.cs, B * K, 2 * B * K, p.V, p.chunk, p.nchunks, inv_t};
  hipError_t e = launch_kernel(&sample_stats_kernel, dim3(p.nchunks, 2 * B * K), dim3(kThreads), stream, s);
  if (e != hipSuccess) return e;
  DecideArgs d{logits_d, logits_a, draft, u_acc, w.cm, w.cs, tokens, n_acc, n_emit, next_anchor, w.seq,
               B, K, p.V, p.nchunks, inv_t};
  e = launch_kernel(&sample_decide_kernel, dim3(B), dim3(64), stream, d);
  if (e != hipSuccess) return e;
  ResidualArgs r{logits_d, logits_a, u_res, w.cm, w.cs, w.seq, w.rs, tokens, next_anchor,
                 B, K, p.V, p.chunk, p.nchunks, inv_t};
  e = launch_kernel(&residual_stats_kernel, dim3(p.nchunks, B), dim3(kThreads), stream, r);
  if (e != hipSuccess) return e;
  return launch_kernel(&residual_draw_kernel, dim3(B), dim3(kThreads), stream, r);
}

}  // namespace orthrus

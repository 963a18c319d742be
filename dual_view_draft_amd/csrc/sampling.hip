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
// s_c = sum exp((z - m_c) / T) (fp64); a wavefront per row then forms the
// row maximum M, the chunk weights s_c exp((m_c - M) / T) and their sum Z in
// a fixed order.  A draw (one 1024-thread workgroup) finds its chunk from the
// chunk weights and then its entry inside that chunk, each time from a
// fixed-order prefix sum over contiguous per-thread shares.  The residual of
// a rejected row has its own, finer chunk sums.
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

constexpr int kThreads = 256;        // statistics kernels
constexpr int kDrawThreads = 1024;   // draw kernels (one workgroup per draw)

struct RowNorm {       // a row's maximum and normaliser
  double Z;
  float M;
  int pad;
};

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

struct NormArgs {
  const float* cm;
  const double* cs;
  double* cw;          // [rows][nchunks]: chunk weights relative to the row maximum
  RowNorm* rn;         // [rows]
  int rows, nchunks;
  double inv_t;
};

struct SampleArgs {
  const float* z;
  const float* u;      // [rows]
  const double* cw;
  const RowNorm* rn;
  int32_t* out;        // [rows]
  int V, chunk, nchunks;
  double inv_t;
};

struct DecideArgs {
  const float* zd;     // [B*K][V] draft view
  const float* za;     // [B*K][V] AR view
  const int32_t* draft;
  const float* u_acc;  // [B][K]
  const RowNorm* rn;   // [2*B*K]: draft rows, then AR rows
  int32_t* tokens;     // [B][K]
  int32_t* n_acc;
  int32_t* n_emit;
  int32_t* next_anchor;
  SeqState* seq;       // [B]
  int B, K, V;
  double inv_t;
};

struct ResidualArgs {
  const float* zd;
  const float* za;
  const float* u_res;  // [B][K]
  const double* cw;    // for the fallback draw from p
  const RowNorm* rn;
  const SeqState* seq;
  double* rs;          // [B][rchunks] residual chunk sums
  int32_t* tokens;
  int32_t* next_anchor;
  int B, K, V, chunk, nchunks, rchunk, rchunks;
  double inv_t;
};

__device__ __forceinline__ double wexp(float z, float m, double inv_t) {
  return exp((double(z) - double(m)) * inv_t);
}

// Sum (or max) over a 256-thread workgroup in a fixed order: wavefront
// butterflies, then the four wavefront results in order.
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

// Inclusive and exclusive prefix sums of one value per thread over a
// kDrawThreads workgroup, in a fixed order (a wavefront scan, then the
// wavefront totals in order).  incl of thread t is bitwise the excl of thread
// t+1, so "excl <= target < incl" holds for at most one thread.
__device__ void block_scan(double x, double* excl, double* incl, double* total) {
  __shared__ double wsum[kDrawThreads / 64];
  __shared__ double wpre[kDrawThreads / 64 + 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  double ve = __shfl_up(v, 1);
  if (lane == 0) ve = 0.0;
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double run = 0.0;
    for (int k = 0; k < kDrawThreads / 64; ++k) {
      wpre[k] = run;
      run = run + wsum[k];
    }
    wpre[kDrawThreads / 64] = run;
  }
  __syncthreads();
  *incl = lane == 63 ? wpre[w + 1] : wpre[w] + v;
  *excl = wpre[w] + ve;
  *total = wpre[kDrawThreads / 64];
  __syncthreads();
}

// Inverse-CDF draw in one kDrawThreads workgroup over a row whose chunk
// weights are chunk_w(c) (c < nchunks, chunks of `chunk` entries) and whose
// entry weights are weight(v): the smallest v whose cumulative weight exceeds
// u times the total.  Chunks, then the chosen chunk's entries, are split into
// contiguous per-thread shares; the one thread whose share holds the target
// rescans it in order.  If rounding leaves the target at or beyond the end
// of a share (or of the row), the share's last entry of positive weight is
// taken.  Every thread returns the token.
template <class ChunkW, class Weight>
__device__ int draw(ChunkW chunk_w, Weight weight, int nchunks, int chunk, int V, double u) {
  __shared__ int pick_s, last_s;
  __shared__ double rem_s;
  const int tid = threadIdx.x;
  if (tid == 0) { pick_s = -1; last_s = -1; }
  // ---- level 1: which chunk -------------------------------------------------
  const int cpt = (nchunks + kDrawThreads - 1) / kDrawThreads;
  const int c0 = min(tid * cpt, nchunks), c1 = min(c0 + cpt, nchunks);
  double x = 0.0;
  int lastc = -1;
  for (int c = c0; c < c1; ++c) {
    const double wc = chunk_w(c);
    x += wc;
    if (wc > 0.0) lastc = c;
  }
  double excl, incl, total;
  block_scan(x, &excl, &incl, &total);
  const double target = u * total;
  if (excl <= target && target < incl) {
    double cum = excl;
    int found = lastc;
    for (int c = c0; c < c1; ++c) {
      const double before = cum;
      cum += chunk_w(c);
      if (cum > target) { found = c; rem_s = target - before; break; }
      if (c == lastc) rem_s = target - before;     // fallback: the share's last positive chunk
    }
    pick_s = found;
  }
  if (lastc >= 0) atomicMax(&last_s, lastc);
  __syncthreads();
  int cstar = pick_s;
  double rem = rem_s;
  if (cstar < 0) { cstar = last_s < 0 ? 0 : last_s; rem = INFINITY; }   // target beyond the row
  __syncthreads();
  if (tid == 0) { pick_s = -1; last_s = -1; }
  __syncthreads();
  // ---- level 2: which entry of chunk cstar -----------------------------------
  // A thread's share (at most kMaxShare entries: chunks hold at most
  // kSampleMaxChunk entries) is loaded once, its weights kept in registers
  // for the rescan.
  constexpr int kMaxShare = kSampleMaxChunk / kDrawThreads;
  const int v0 = cstar * chunk, v1 = min(v0 + chunk, V);
  const int per = (v1 - v0 + kDrawThreads - 1) / kDrawThreads;
  const int a0 = min(v0 + tid * per, v1), a1 = min(a0 + per, v1);
  double wsh[kMaxShare];
  // per is the same in every thread: the blocks of 4 past it are skipped
  // by a uniform branch, so no masked-off exponential is issued
#pragma unroll
  for (int jb = 0; jb < kMaxShare; jb += 4) {
    if (jb >= per) break;
#pragma unroll
    for (int j = jb; j < jb + 4; ++j) wsh[j] = a0 + j < a1 ? weight(a0 + j) : 0.0;
  }
  double y = 0.0;
  int lastv = -1;
#pragma unroll
  for (int j = 0; j < kMaxShare; ++j) {
    if (a0 + j < a1) {
      y += wsh[j];
      if (wsh[j] > 0.0) lastv = a0 + j;
    }
  }
  double e2, i2, t2;
  block_scan(y, &e2, &i2, &t2);
  if (e2 <= rem && rem < i2) {
    double cum = e2;
    int found = lastv;
    bool hit = false;
#pragma unroll
    for (int j = 0; j < kMaxShare; ++j) {
      if (!hit && a0 + j < a1) {
        cum += wsh[j];
        if (cum > rem) {
          found = a0 + j;
          hit = true;
        }
      }
    }
    pick_s = found;
  }
  if (lastv >= 0) atomicMax(&last_s, lastv);
  __syncthreads();
  int tok = pick_s >= 0 ? pick_s : last_s;
  return tok < 0 ? v0 : tok;
}

// Chunk statistics of every row: m_c and s_c = sum exp((z - m_c) / T).
// PER entries per thread at most (chunk <= 256 PER), so that no exponential
// is issued for entries beyond the chunk.
template <int PER>
__global__ __launch_bounds__(kThreads) void sample_stats_kernel(StatsArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int row = blockIdx.y, c = blockIdx.x;
  const float* z = row < a.rows0 ? a.z0 + size_t(row) * a.V : a.z1 + size_t(row - a.rows0) * a.V;
  const int v0 = c * a.chunk, v1 = min(v0 + a.chunk, a.V);
  // thread t's entries v0 + t + 256 j, all loaded at once and kept in registers
  float x[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int v = v0 + threadIdx.x + j * kThreads;
    x[j] = v < v1 ? z[v] : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j) m = fmaxf(m, x[j]);
  m = block_max(m, redf);
  double s = 0.0;                                  // in increasing v, as the entries were read
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (v0 + int(threadIdx.x) + j * kThreads < v1) s += wexp(x[j], m, a.inv_t);
  s = block_sum(s, redd);
  if (threadIdx.x == 0) {
    a.cm[size_t(row) * a.nchunks + c] = m;
    a.cs[size_t(row) * a.nchunks + c] = s;
  }
}

// One wavefront per row: the row maximum M, every chunk's weight
// s_c exp((m_c - M) / T) and their sum Z (lane-strided, then a fixed butterfly).
__global__ __launch_bounds__(kThreads) void row_norm_kernel(NormArgs a) {
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= a.rows) return;                       // uniform per wavefront
  const int lane = threadIdx.x & 63;
  const float* cm = a.cm + size_t(row) * a.nchunks;
  const double* cs = a.cs + size_t(row) * a.nchunks;
  double* cw = a.cw + size_t(row) * a.nchunks;
  float m = -INFINITY;
  for (int c = lane; c < a.nchunks; c += 64) m = fmaxf(m, cm[c]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  double z = 0.0;
  for (int c = lane; c < a.nchunks; c += 64) {
    const double w = cs[c] * wexp(cm[c], m, a.inv_t);
    cw[c] = w;
    z += w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
  if (lane == 0) a.rn[row] = RowNorm{z, m, 0};
}

// One workgroup per row: out[row] = draw of softmax(z[row] / T) with u[row].
__global__ __launch_bounds__(kDrawThreads) void sample_draw_kernel(SampleArgs a) {
  const int row = blockIdx.x;
  const double* cw = a.cw + size_t(row) * a.nchunks;
  const float M = a.rn[row].M;
  const float* z = a.z + size_t(row) * a.V;
  const double inv_t = a.inv_t;
  const int tok = draw([&](int c) { return cw[c]; }, [&](int v) { return wexp(z[v], M, inv_t); },
                       a.nchunks, a.chunk, a.V, double(a.u[row]));
  if (threadIdx.x == 0) a.out[row] = tok;
}

// Draw with the row's normalisation done in the same workgroup: wavefront 0
// forms M, the chunk weights and Z exactly as row_norm_kernel does (the same
// lane-strided order and butterfly), into LDS; then the draw as in
// sample_draw_kernel.  One launch fewer for orthrus_sample, whose rows need
// no normaliser afterwards.
constexpr int kFusedMaxChunks = 1024;

struct NormDrawArgs {
  const float* z;
  const float* u;      // [rows]
  const float* cm;     // [rows][nchunks]
  const double* cs;
  int32_t* out;        // [rows]
  int V, chunk, nchunks;
  double inv_t;
};

__global__ __launch_bounds__(kDrawThreads) void sample_norm_draw_kernel(NormDrawArgs a) {
  __shared__ double cw_s[kFusedMaxChunks];
  __shared__ float m_s;
  const int row = blockIdx.x;
  if (threadIdx.x < 64) {                          // wavefront 0: row_norm_kernel's steps
    const int lane = threadIdx.x;
    const float* cm = a.cm + size_t(row) * a.nchunks;
    const double* cs = a.cs + size_t(row) * a.nchunks;
    float m = -INFINITY;
    for (int c = lane; c < a.nchunks; c += 64) m = fmaxf(m, cm[c]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    for (int c = lane; c < a.nchunks; c += 64) cw_s[c] = cs[c] * wexp(cm[c], m, a.inv_t);
    if (lane == 0) m_s = m;
  }
  __syncthreads();
  const float M = m_s;
  const float* z = a.z + size_t(row) * a.V;
  const double inv_t = a.inv_t;
  const int tok = draw([&](int c) { return cw_s[c]; }, [&](int v) { return wexp(z[v], M, inv_t); },
                       a.nchunks, a.chunk, a.V, double(a.u[row]));
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
  RowNorm nd{0.0, 0.f, 0}, na{0.0, 0.f, 0};
  if (i < a.K) {
    const size_t rd = size_t(b) * a.K + i;
    nd = a.rn[rd];
    na = a.rn[BK + rd];
    t = a.draft[rd];
    double p = 0.0, q = 0.0;                       // a token outside the vocabulary has p = q = 0
    if (t >= 0 && t < a.V) {
      p = wexp(a.za[rd * a.V + t], na.M, a.inv_t) / na.Z;
      q = wexp(a.zd[rd * a.V + t], nd.M, a.inv_t) / nd.Z;
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
  if (i == j) a.seq[b] = SeqState{na.Z, nd.Z, na.M, nd.M, j, 0};
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

// Sums of the residual max(0, p - q) of each sequence's rejected row over
// chunks of rchunk entries.
__global__ __launch_bounds__(kThreads) void residual_stats_kernel(ResidualArgs a) {
  __shared__ double redd[4];
  const int b = blockIdx.y, c = blockIdx.x;
  const SeqState st = a.seq[b];
  if (st.j >= a.K) return;                         // uniform: nothing rejected
  const size_t row = size_t(b) * a.K + st.j;
  const Residual r{a.za + row * a.V, a.zd + row * a.V, st.Ma, st.Md, st.Za, st.Zd, a.inv_t};
  const int v0 = c * a.rchunk, v1 = min(v0 + a.rchunk, a.V);
  double s = 0.0;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) s += r(v);
  s = block_sum(s, redd);
  if (threadIdx.x == 0) a.rs[size_t(b) * a.rchunks + c] = s;
}

// One workgroup per sequence: the emitted token at the rejected row, a draw
// of max(0, p - q) (of p if the residual is empty, which only rounding can
// cause).
__global__ __launch_bounds__(kDrawThreads) void residual_draw_kernel(ResidualArgs a) {
  const int b = blockIdx.x;
  const SeqState st = a.seq[b];
  if (st.j >= a.K) return;
  const size_t row = size_t(b) * a.K + st.j;
  const double* rs = a.rs + size_t(b) * a.rchunks;
  __shared__ double part[kDrawThreads / 64];
  double x = 0.0;
  for (int c = threadIdx.x; c < a.rchunks; c += kDrawThreads) x += rs[c];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  bool empty = true;
  for (int k = 0; k < kDrawThreads / 64; ++k) empty = empty && !(part[k] > 0.0);
  const double u = double(a.u_res[row]);
  int tok;
  if (!empty) {
    const Residual r{a.za + row * a.V, a.zd + row * a.V, st.Ma, st.Md, st.Za, st.Zd, a.inv_t};
    tok = draw([&](int c) { return rs[c]; }, r, a.rchunks, a.rchunk, a.V, u);
  } else {
    const double* cw = a.cw + (size_t(a.B) * a.K + row) * a.nchunks;
    const float* z = a.za + row * a.V;
    const float M = st.Ma;
    const double inv_t = a.inv_t;
    tok = draw([&](int c) { return cw[c]; }, [&](int v) { return wexp(z[v], M, inv_t); },
               a.nchunks, a.chunk, a.V, u);
  }
  if (threadIdx.x == 0) {
    a.tokens[row] = tok;
    a.next_anchor[b] = tok;
  }
}

struct Ws {
  float* cm;
  double* cs;
  double* cw;
  RowNorm* rn;
  SeqState* seq;
  double* rs;
};

Ws carve(const SamplePlan& p, void* ws) {
  char* base = static_cast<char*>(ws);
  return Ws{reinterpret_cast<float*>(base + p.cm_off), reinterpret_cast<double*>(base + p.cs_off),
            reinterpret_cast<double*>(base + p.cw_off), reinterpret_cast<RowNorm*>(base + p.rn_off),
            reinterpret_cast<SeqState*>(base + p.seq_off), reinterpret_cast<double*>(base + p.rs_off)};
}

hipError_t launch_stats_kernel(const SamplePlan& p, const StatsArgs& s, hipStream_t stream) {
  const dim3 grid(p.nchunks, p.rows);
  if (p.chunk <= 16 * kThreads) return launch_kernel(&sample_stats_kernel<16>, grid, dim3(kThreads), stream, s);
  if (p.chunk <= 32 * kThreads) return launch_kernel(&sample_stats_kernel<32>, grid, dim3(kThreads), stream, s);
  return launch_kernel(&sample_stats_kernel<kSampleMaxChunk / kThreads>, grid, dim3(kThreads), stream, s);
}

hipError_t launch_stats(const SamplePlan& p, const Ws& w, const float* z0, const float* z1, int rows0,
                        double inv_t, hipStream_t stream) {
  StatsArgs s{z0, z1, w.cm, w.cs, rows0, p.rows, p.V, p.chunk, p.nchunks, inv_t};
  hipError_t e = launch_stats_kernel(p, s, stream);
  if (e != hipSuccess) return e;
  NormArgs n{w.cm, w.cs, w.cw, w.rn, p.rows, p.nchunks, inv_t};
  return launch_kernel(&row_norm_kernel, dim3((p.rows + 3) / 4), dim3(kThreads), stream, n);
}

}  // namespace

static_assert(sizeof(SeqState) == kSampleSeqBytes, "per-sequence state size");
static_assert(sizeof(RowNorm) == kSampleRowBytes, "per-row state size");

hipError_t launch_sample(const SamplePlan& p, const float* logits, float temperature, const float* u,
                         int32_t* out, void* ws, hipStream_t stream) {
  const Ws w = carve(p, ws);
  const double inv_t = 1.0 / double(temperature);
  if (p.nchunks <= kFusedMaxChunks) {
    StatsArgs s{logits, logits, w.cm, w.cs, p.rows, p.rows, p.V, p.chunk, p.nchunks, inv_t};
    hipError_t e = launch_stats_kernel(p, s, stream);
    if (e != hipSuccess) return e;
    NormDrawArgs d{logits, u, w.cm, w.cs, out, p.V, p.chunk, p.nchunks, inv_t};
    return launch_kernel(&sample_norm_draw_kernel, dim3(p.rows), dim3(kDrawThreads), stream, d);
  }
  hipError_t e = launch_stats(p, w, logits, logits, p.rows, inv_t, stream);
  if (e != hipSuccess) return e;
  SampleArgs d{logits, u, w.cw, w.rn, out, p.V, p.chunk, p.nchunks, inv_t};
  return launch_kernel(&sample_draw_kernel, dim3(p.rows), dim3(kDrawThreads), stream, d);
}

hipError_t launch_accept_sampled(const SamplePlan& p, const float* logits_d, const float* logits_a,
                                 const int32_t* draft, int B, int K, float temperature, const float* u_acc,
                                 const float* u_res, int32_t* tokens, int32_t* n_acc, int32_t* n_emit,
                                 int32_t* next_anchor, void* ws, hipStream_t stream) {
  const Ws w = carve(p, ws);
  const double inv_t = 1.0 / double(temperature);
  hipError_t e = launch_stats(p, w, logits_d, logits_a, B * K, inv_t, stream);
  if (e != hipSuccess) return e;
  DecideArgs d{logits_d, logits_a, draft, u_acc, w.rn, tokens, n_acc, n_emit, next_anchor, w.seq,
               B, K, p.V, inv_t};
  e = launch_kernel(&sample_decide_kernel, dim3(B), dim3(64), stream, d);
  if (e != hipSuccess) return e;
  ResidualArgs r{logits_d, logits_a, u_res, w.cw, w.rn, w.seq, w.rs, tokens, next_anchor,
                 B, K, p.V, p.chunk, p.nchunks, p.rchunk, p.rchunks, inv_t};
  e = launch_kernel(&residual_stats_kernel, dim3(p.rchunks, B), dim3(kThreads), stream, r);
  if (e != hipSuccess) return e;
  return launch_kernel(&residual_draw_kernel, dim3(B), dim3(kDrawThreads), stream, r);
}

}  // namespace orthrus

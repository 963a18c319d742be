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
// Work layout.  Rows are cut into chunks of 1024 vocabulary entries (2048
// when the 1024-entry chunks would need more wavefronts than the GPU holds
// at once); a statistics pass (one wavefront per chunk, 16 or 32 entries per
// lane, wavefront reductions only) writes, per (row, chunk), the chunk's
// maximum logit m_c (fp32) and s_c = sum exp((z - m_c) / T) (fp64), and for
// the consensus the same over groups of four chunks.  The next kernel forms
// a row's maximum M, the chunk weights s_c exp((m_c - M) / T) and their sum Z
// in a fixed order, and then draws (orthrus_sample) or runs the acceptance
// test of a sequence's rows (consensus).  A draw (one 256-thread workgroup)
// finds its chunk from the chunk weights and then its entry inside that
// chunk (4 or 8 per thread), each time from a fixed-order prefix sum over
// contiguous per-thread shares.  The residual of a rejected row has its own
// chunk sums, taken in the acceptance test's launch: each workgroup of that
// launch repeats the sequence's test (the same arithmetic, so the same
// outcome everywhere) and then sums its share of the rejected row.
// (Handing the chunk results to the row's last workgroup within one launch
// was measured slower: a device-scope fence per workgroup, or device-scope
// atomics for the hand-over, cost more than the second launch.)
// The exponentials and sums are fp64 so that every decision (a comparison
// with u times a probability or a cumulative weight) agrees with an exact
// evaluation except within about 1e-15 (relative) of its threshold.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "check.h"
#include "dpp.h"
#include "fexp.h"
#include "launch.h"

namespace orthrus {
namespace {

constexpr int kThreads = 256;          // every sampling kernel but the acceptance test
constexpr int kMaxChunksInLds = 1024;  // chunk weights kept in LDS for a draw up to this many chunks

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
  float* gm;           // [rows][ngroups] the same over groups of kSampleGroup chunks (null: not wanted)
  double* gs;
  int rows0, rows, V, nchunks, ngroups;
  double tscale;
};

struct SampleArgs {
  const float* z;
  const float* u;      // [rows]
  const float* cm;
  const double* cs;
  double* cw;          // [rows][nchunks], used when the weights do not fit in LDS
  int32_t* out;        // [rows]
  int V, chunk, nchunks;
  double tscale;
};

struct DecideArgs {
  const float* zd;     // [B*K][V] draft view
  const float* za;     // [B*K][V] AR view
  const int32_t* draft;
  const float* u_acc;  // [B][K]
  const float* gm;     // group statistics rows: draft rows, then AR rows
  const double* gs;
  int32_t* tokens;     // [B][K]
  int32_t* n_acc;
  int32_t* n_emit;
  int32_t* next_anchor;
  SeqState* seq;       // [B]
  double* rs;          // [B][rchunks] residual chunk sums
  int B, K, V, ngroups, rchunk, rchunks, rcpw;
  double tscale;
};

struct ResidualArgs {
  const float* zd;
  const float* za;
  const float* u_res;  // [B][K]
  const float* cm;     // statistics of the AR rows, for the fallback draw from p
  const double* cs;
  const SeqState* seq;
  double* rs;          // [B][rchunks] residual chunk sums
  int32_t* tokens;
  int32_t* next_anchor;
  int B, K, V, chunk, nchunks, rchunk, rchunks;
  double tscale;
};

// Every kernel keeps the 2^(j/64) table of its exponential in LDS; a
// __syncthreads must separate this from the first use.
__device__ __forceinline__ void load_exp_table(double* tab) {
  if (threadIdx.x < 64) tab[threadIdx.x] = kExp2Frac[threadIdx.x];
}

// exp((z - m) / T) = 2^(t/64) with t = (z - m) tscale, tscale = 64 / (T ln2),
// for z <= m (every caller passes a maximum as m)
__device__ __forceinline__ double wexp(float z, float m, double tscale, const double* tab) {
  return exp2_64((double(z) - double(m)) * tscale, tab);
}

// ---- wavefront and workgroup reductions in a fixed order (dpp.h) ----------
__device__ __forceinline__ double wave_sum(double v) { return wave_sum_f64(v); }
__device__ __forceinline__ float wave_max(float v) { return wave_max_f32(v); }

// Sum (or max) over a 256-thread workgroup: the wavefront results, then the
// four of them in order.  One barrier: a second call on the same `red`
// needs a barrier between the two.
__device__ double block_sum(double x, double* red) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ float block_max(float x, float* red) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Inclusive and exclusive prefix sums of one value per thread over the
// workgroup, in a fixed order (the row scans, the rows of a wavefront in
// order, then the wavefront totals in order), and the workgroup's maximum of
// one int per thread.  incl of thread t is bitwise the excl of thread t+1,
// so "excl <= target < incl" holds for at most one thread.  One barrier: a
// second call needs a barrier between the two.
__device__ void block_scan(double x, int k, double* excl, double* incl, double* total, int* kmax) {
  __shared__ double wsum[kThreads / 64];
  __shared__ int wmax[kThreads / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double v = x;                                    // scan within the row of 16 lanes
  v += dpp_f64<kRowShr1>(v, 0.0);
  v += dpp_f64<kRowShr2>(v, 0.0);
  v += dpp_f64<kRowShr4>(v, 0.0);
  v += dpp_f64<kRowShr8>(v, 0.0);
  const double o1 = readlane_f64(v, 15);           // row offsets: the rows before, in order
  const double o2 = o1 + readlane_f64(v, 31);
  const double o3 = o2 + readlane_f64(v, 47);
  const int row = lane >> 4;
  const double off = row == 0 ? 0.0 : row == 1 ? o1 : row == 2 ? o2 : o3;
  v = off + v;                                     // lane 16r-1 ends as o_r exactly
  const double ve = dpp_f64<kRowShr1>(v, off);     // the previous lane's, o_r at a row start
  k = wave_max_i32(k);
  if (lane == 63) {
    wsum[w] = v;
    wmax[w] = k;
  }
  __syncthreads();
  double pre[kThreads / 64 + 1];
  pre[0] = 0.0;
#pragma unroll
  for (int q = 0; q < kThreads / 64; ++q) pre[q + 1] = pre[q] + wsum[q];
  double pw = pre[0], pw1 = pre[1];
#pragma unroll
  for (int q = 1; q < kThreads / 64; ++q) {
    pw = w == q ? pre[q] : pw;
    pw1 = w == q ? pre[q + 1] : pw1;
  }
  *incl = lane == 63 ? pw1 : pw + v;
  *excl = pw + ve;
  *total = pre[kThreads / 64];
  *kmax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

// Entries of a softmax row: weight exp((z - M) / T).
struct SoftmaxEntry {
  const float* z;
  float M;
  double tscale;
  const double* tab;
  __device__ float load(int v) const { return z[v]; }
  __device__ double weight(float zv) const { return wexp(zv, M, tscale, tab); }
};

// Entries of a residual row: weight max(0, p - q).
struct ResidualEntry {
  const float* za;
  const float* zd;
  float Ma, Md;
  double Za, Zd, tscale;
  const double* tab;
  __device__ float2 load(int v) const { return float2{za[v], zd[v]}; }
  __device__ double weight(float2 e) const {
    const double p = wexp(e.x, Ma, tscale, tab) / Za;
    const double q = wexp(e.y, Md, tscale, tab) / Zd;
    return p > q ? p - q : 0.0;
  }
};

// Inverse-CDF draw in one 256-thread workgroup over a row whose chunk
// weights are chunk_w(c) (c < nchunks, chunks of `chunk` entries, at most
// 256 SHARE) and whose entry weights are entry.weight(entry.load(v)): the
// smallest v whose cumulative weight exceeds u times the total.  Chunks,
// then the chosen chunk's entries, are split into contiguous per-thread
// shares; the one thread whose share holds the target rescans it in order.
// If rounding leaves the target at or beyond the end of a share (or of the
// row), the share's last entry of positive weight is taken.  Every thread
// returns the token.
template <int SHARE, class ChunkW, class Entry>
__device__ int draw(ChunkW chunk_w, const Entry& entry, int nchunks, int chunk, int V, double u) {
  __shared__ int pick_s, pick2_s;
  __shared__ double rem_s;
  const int tid = threadIdx.x;
  if (tid == 0) {                                  // (ordered before any write by block_scan's barrier)
    pick_s = -1;
    pick2_s = -1;
  }
  // ---- level 1: which chunk -------------------------------------------------
  const int cpt = (nchunks + kThreads - 1) / kThreads;
  const int c0 = min(tid * cpt, nchunks), c1 = min(c0 + cpt, nchunks);
  double x = 0.0;
  int lastc = -1;
  for (int c = c0; c < c1; ++c) {
    const double wc = chunk_w(c);
    x += wc;
    if (wc > 0.0) lastc = c;
  }
  double excl, incl, total;
  int lastc_all;
  block_scan(x, lastc, &excl, &incl, &total, &lastc_all);
  const double target = u * total;
  if (excl <= target && target < incl) {
    double cum = excl;
    int found = lastc;
    double r = 0.0;
    for (int c = c0; c < c1; ++c) {
      const double before = cum;
      cum += chunk_w(c);
      if (cum > target) { found = c; r = target - before; break; }
      if (c == lastc) r = target - before;         // fallback: the share's last positive chunk
    }
    pick_s = found;
    rem_s = r;
  }
  __syncthreads();
  int cstar = pick_s;
  double rem = rem_s;
  if (cstar < 0) { cstar = lastc_all < 0 ? 0 : lastc_all; rem = INFINITY; }   // target beyond the row
  // ---- level 2: which entry of chunk cstar -----------------------------------
  // A thread's share (at most SHARE entries) is loaded at once (addresses
  // clamped into the chunk, so that no load waits on a branch), its weights
  // kept in registers for the rescan.  per is the same in every thread: the
  // blocks of 4 past it are skipped by a uniform branch.
  const int v0 = cstar * chunk, v1 = min(v0 + chunk, V);
  const int per = (v1 - v0 + kThreads - 1) / kThreads;
  const int a0 = min(v0 + tid * per, v1), a1 = min(a0 + per, v1);
  decltype(entry.load(0)) raw[SHARE];
#pragma unroll
  for (int jb = 0; jb < SHARE; jb += 4) {
    if (jb >= per) break;
#pragma unroll
    for (int j = jb; j < jb + 4; ++j) raw[j] = entry.load(min(a0 + j, v1 - 1));
  }
  double wsh[SHARE];
  double y = 0.0;
  int lastv = -1;
#pragma unroll
  for (int jb = 0; jb < SHARE; jb += 4) {
    if (jb >= per) break;
#pragma unroll
    for (int j = jb; j < jb + 4; ++j) {
      const double w = entry.weight(raw[j]);       // (computed for clamped entries too: no branch)
      wsh[j] = a0 + j < a1 ? w : 0.0;
      y += wsh[j];
      if (wsh[j] > 0.0) lastv = a0 + j;
    }
  }
  double e2, i2, t2;
  int lastv_all;
  block_scan(y, lastv, &e2, &i2, &t2, &lastv_all);
  if (e2 <= rem && rem < i2) {
    double cum = e2;
    int found = lastv;
    bool hit = false;
#pragma unroll
    for (int jb = 0; jb < SHARE; jb += 4) {
      if (jb >= per) break;
#pragma unroll
      for (int j = jb; j < jb + 4; ++j) {
        if (!hit && a0 + j < a1) {
          cum += wsh[j];
          if (cum > rem) {
            found = a0 + j;
            hit = true;
          }
        }
      }
    }
    pick2_s = found;
  }
  __syncthreads();
  const int tok = pick2_s >= 0 ? pick2_s : lastv_all;
  return tok < 0 ? v0 : tok;
}

// Chunk statistics of every row: m_c and s_c = sum exp((z - m_c) / T), one
// wavefront per (row, chunk), lane l taking entries v0 + l + 64 j
// (j < PER, chunks of 64 PER entries), loaded in two stages (see below);
// the lane's and then the wavefront's sums are rescaled to the
// larger maximum (fixed order).  A workgroup holds kSampleGroup consecutive
// chunks of one row and also writes their combined statistics (in chunk
// order).
template <int PER>
__global__ __launch_bounds__(kThreads) void sample_stats_kernel(StatsArgs a) {
  __shared__ double tab[64];
  __shared__ float wm[kSampleGroup];
  __shared__ double ws[kSampleGroup];
  static_assert(kThreads == 64 * kSampleGroup, "a wavefront per chunk of the group");
  // Two stages of loads: four stages of 8 at PER = 32 measured 1 % faster at
  // 64 rows and 3 % slower at 512 and 1024 rows.
  constexpr int kStage = PER / 2;                  // entries per lane per stage of loads
  constexpr int S = PER / kStage;
  static_assert(PER % kStage == 0 && kStage % 4 == 0, "stages of whole blocks of 4");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // (uniform: scalar registers below)
  const int row = blockIdx.x / a.ngroups;
  const int g = blockIdx.x - row * a.ngroups;
  const int c = g * kSampleGroup + w;
  const bool live = c < a.nchunks;
  const float* z = row < a.rows0 ? a.z0 + size_t(row) * a.V : a.z1 + size_t(row - a.rows0) * a.V;
  const int v0 = c * (64 * PER), n = live ? min(64 * PER, a.V - v0) : 0;   // entries in the chunk
  // The chunk through a buffer descriptor of n entries: one address register
  // for all loads, and loads past the chunk's end return 0 (then -inf below).
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(z) + (live ? v0 : 0), 0, n * 4, 0x00020000);
  float x[PER];
#pragma unroll
  for (int j = 0; j < kStage; ++j)
    x[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane * 4, j * 256, 0));
  load_exp_table(tab);
  __syncthreads();
  // Stage st's loads are issued once stage st-1 has arrived (their offsets
  // wait on its data), and stage st-1's exponentials run while stage st is in
  // flight.  Each stage's sum is relative to the running maximum; the running
  // sum is rescaled when the maximum grows.  Entries past the chunk hold -inf
  // and add exp(-inf) = +0 exactly (no branch per entry); while the maximum
  // is still -inf (no entry yet) the NaN sums are replaced by 0, so a
  // wavefront past the last chunk ends with m = -inf, s = 0.  (The
  // exponentials go in blocks of 4, kept apart by scheduling barriers so that
  // the compiler does not interleave them all and raise the register count,
  // which would cut the wavefronts resident per SIMD.)
  const double tscale = a.tscale;
  float m2 = -INFINITY;                            // the lane's running maximum
  double sl = 0.0;                                 // and its sum, in increasing v
#pragma unroll
  for (int st = 0; st < S; ++st) {
    if (st + 1 < S) {
      int lb = lane * 4;
      asm volatile("" : "+v"(lb) : "v"(x[kStage * st + kStage - 1]));
#pragma unroll
      for (int j = kStage * (st + 1); j < kStage * (st + 2); ++j)
        x[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, lb, j * 256, 0));
    }
#pragma unroll
    for (int j = kStage * st; j < kStage * (st + 1); ++j) x[j] = lane + j * 64 < n ? x[j] : -INFINITY;
    float ms = m2;
#pragma unroll
    for (int j = kStage * st; j < kStage * (st + 1); ++j) ms = fmaxf(ms, x[j]);
    double ss = 0.0;
#pragma unroll
    for (int jb = kStage * st; jb < kStage * (st + 1); jb += 4) {
#pragma unroll
      for (int j = jb; j < jb + 4; ++j) ss += wexp(x[j], ms, tscale, tab);
      __builtin_amdgcn_sched_barrier(0);
    }
    ss = ms == -INFINITY ? 0.0 : ss;
    if (st == 0) sl = ss;                          // (the same as below with sl = 0, m2 = -inf)
    else sl = (m2 == ms ? sl : sl * wexp(m2, ms, tscale, tab)) + ss;
    m2 = ms;
  }
  const float m = wave_max(m2);
  const double sw = wave_sum(m2 == m ? sl : sl * wexp(m2, m, tscale, tab));
  if (lane == 0 && live) {
    a.cm[size_t(row) * a.nchunks + c] = m;
    a.cs[size_t(row) * a.nchunks + c] = sw;
  }
  if (a.gm == nullptr) return;                     // (uniform) no group statistics wanted
  if (lane == 0) {
    wm[w] = m;
    ws[w] = sw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {                          // chunk 0 of the group is always live
    const float gmax = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    double gsum = 0.0;
#pragma unroll
    for (int q = 0; q < kSampleGroup; ++q) gsum += wm[q] == gmax ? ws[q] : ws[q] * wexp(wm[q], gmax, tscale, tab);
    a.gm[size_t(row) * a.ngroups + g] = gmax;
    a.gs[size_t(row) * a.ngroups + g] = gsum;
  }
}

// One workgroup per row: the row maximum M, every chunk's weight
// s_c exp((m_c - M) / T) (into LDS, or global memory past kMaxChunksInLds
// chunks), then out[row] = draw of softmax(z[row] / T) with u[row].
template <int SHARE>
__global__ __launch_bounds__(kThreads) void sample_draw_kernel(SampleArgs a) {
  __shared__ float redf[4];
  __shared__ double tab[64];
  __shared__ double cw_s[kMaxChunksInLds];
  const int row = blockIdx.x;
  const float* cm = a.cm + size_t(row) * a.nchunks;
  const double* cs = a.cs + size_t(row) * a.nchunks;
  double* cw = a.cw + size_t(row) * a.nchunks;
  // every independent load first: the thread's first chunk, the uniform,
  // the exponential's table
  const int k0 = threadIdx.x;
  const float cm0 = k0 < a.nchunks ? cm[k0] : -INFINITY;
  const double cs0 = k0 < a.nchunks ? cs[k0] : 0.0;
  const double u = double(a.u[row]);
  load_exp_table(tab);
  float M = cm0;
  for (int k = k0 + kThreads; k < a.nchunks; k += kThreads) M = fmaxf(M, cm[k]);
  M = block_max(M, redf);                          // (its barriers also publish the table)
  const bool in_lds = a.nchunks <= kMaxChunksInLds;
  if (k0 < a.nchunks) {
    const double w = cs0 * wexp(cm0, M, a.tscale, tab);
    if (in_lds) cw_s[k0] = w;
    else cw[k0] = w;
  }
  for (int k = k0 + kThreads; k < a.nchunks; k += kThreads) {
    const double w = cs[k] * wexp(cm[k], M, a.tscale, tab);
    if (in_lds) cw_s[k] = w;
    else cw[k] = w;
  }
  // Up to one chunk per thread, the draw's first level reads only the
  // weight its own thread wrote; past that, shares span other threads' writes.
  if (a.nchunks > kThreads) __syncthreads();
  const int tok = draw<SHARE>([&](int k) { return in_lds ? cw_s[k] : cw[k]; },
                              SoftmaxEntry{a.z + size_t(row) * a.V, M, a.tscale, tab}, a.nchunks, a.chunk, a.V, u);
  if (threadIdx.x == 0) a.out[row] = tok;
}

// Acceptance test and residual chunk sums, one launch.  Workgroup (x, b)
// first recomputes what every workgroup of sequence b needs: the maximum and
// normaliser of each of its 2K statistics rows from their group statistics
// (a team of G threads per row, groups strided over the team, then a
// butterfly within it), then wavefront 0, lane i = block row i, runs the
// acceptance test of every row and finds the first rejection j (workgroup 0
// writes the sequence's outputs and state).  Then, if a row was rejected,
// the workgroup sums the residual max(0, p - q) of row j over its rcpw
// chunks of rchunk entries.  The test's arithmetic is the same in every
// workgroup, so all of them see the same j.
constexpr int kDecideThreads = 1024;

__global__ __launch_bounds__(kDecideThreads) void accept_residual_kernel(DecideArgs a) {
  __shared__ double tab[64];
  __shared__ RowNorm rn_s[2 * ORTHRUS_MAX_BLOCK];
  __shared__ SeqState st_s;
  __shared__ double redd[kDecideThreads / kThreads][4];
  constexpr int kReg = 16;                         // chunks per thread per batch of loads
  const int b = blockIdx.y;
  const int BK = a.B * a.K, R = 2 * a.K;
  // the table first, so that waiting for it does not wait for the loads below
  const double tab_v = threadIdx.x < 64 ? kExp2Frac[threadIdx.x] : 0.0;
  int G = 64;                                      // threads per row: a power of two, G * R <= 1024
  while (G * R > kDecideThreads) G >>= 1;
  const int r = threadIdx.x / G, gl = threadIdx.x % G;
  const bool has_row = r < R;                      // whole groups: G divides 64
  const size_t srow = (r < a.K ? size_t(b) * a.K + r : size_t(BK) + size_t(b) * a.K + (r - a.K));
  const float* cm = a.gm + (has_row ? srow : 0) * a.ngroups;
  const double* cs = a.gs + (has_row ? srow : 0) * a.ngroups;
  // every independent load first: the rows' first batch of statistics, and
  // for wavefront 0 (lane i = block row i) the drafted token, its uniform
  // and its logits
  const int i = threadIdx.x;
  const bool lane_row = i < a.K;
  const size_t rd = size_t(b) * a.K + (lane_row ? i : 0);
  const int32_t t = a.draft[rd];                   // (rd is a valid row for every lane: no branch)
  const float uacc = a.u_acc[rd];
  float mv[kReg];
  double sv[kReg];
#pragma unroll
  for (int q = 0; q < kReg; ++q) {
    const int k = gl + q * G;
    const bool ok = has_row && k < a.ngroups;
    mv[q] = ok ? cm[k] : -INFINITY;
    sv[q] = ok ? cs[k] : 0.0;
  }
  const bool in_vocab = lane_row && t >= 0 && t < a.V;
  const float zta = in_vocab ? a.za[rd * a.V + t] : 0.f;
  const float ztd = in_vocab ? a.zd[rd * a.V + t] : 0.f;
  if (threadIdx.x < 64) tab[threadIdx.x] = tab_v;
  __syncthreads();
  if (has_row) {
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < kReg; ++q) m = fmaxf(m, mv[q]);
    for (int k0 = gl + kReg * G; k0 < a.ngroups; k0 += kReg * G) {   // further batches (large vocabularies)
      float mb[kReg];
#pragma unroll
      for (int q = 0; q < kReg; ++q) mb[q] = k0 + q * G < a.ngroups ? cm[k0 + q * G] : -INFINITY;
#pragma unroll
      for (int q = 0; q < kReg; ++q) m = fmaxf(m, mb[q]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
      if (off < G) m = fmaxf(m, __shfl_xor(m, off));   // within the group: G is uniform
    double zs = 0.0;
#pragma unroll
    for (int q = 0; q < kReg; ++q)
      if (gl + q * G < a.ngroups) zs += sv[q] * wexp(mv[q], m, a.tscale, tab);   // uniform but for the last
    for (int k0 = gl + kReg * G; k0 < a.ngroups; k0 += kReg * G) {
      float mb[kReg];
      double sb[kReg];
#pragma unroll
      for (int q = 0; q < kReg; ++q) {
        const bool ok = k0 + q * G < a.ngroups;
        mb[q] = ok ? cm[k0 + q * G] : -INFINITY;
        sb[q] = ok ? cs[k0 + q * G] : 0.0;
      }
#pragma unroll
      for (int q = 0; q < kReg; ++q) {
        const double w = sb[q] * wexp(mb[q], m, a.tscale, tab);
        zs += k0 + q * G < a.ngroups ? w : 0.0;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
      if (off < G) zs += __shfl_xor(zs, off);
    if (gl == 0) rn_s[r] = RowNorm{zs, m, 0};
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    bool reject = false;
    RowNorm nd{0.0, 0.f, 0}, na{0.0, 0.f, 0};
    if (lane_row) {
      nd = rn_s[i];
      na = rn_s[a.K + i];
      double p = 0.0, q = 0.0;                     // a token outside the vocabulary has p = q = 0
      if (in_vocab) {
        p = wexp(zta, na.M, a.tscale, tab) / na.Z;
        q = wexp(ztd, nd.M, a.tscale, tab) / nd.Z;
      }
      reject = !(double(uacc) * q < p);
    }
    const unsigned long long bad = __ballot(reject);
    const int j = bad ? (__ffsll(static_cast<long long>(bad)) - 1) : a.K;
    const SeqState none{0.0, 0.0, 0.f, 0.f, a.K, 0};
    if (blockIdx.x == 0) {                         // the sequence's outputs, once
      if (lane_row) a.tokens[size_t(b) * a.K + i] = i < j ? t : -1;
      if (i == 0) {
        a.n_acc[b] = j;
        a.n_emit[b] = j < a.K ? j + 1 : a.K;
        if (j == a.K) {
          a.next_anchor[b] = a.draft[size_t(b) * a.K + a.K - 1];
          a.seq[b] = none;
        }
      }
      if (i == j) a.seq[b] = SeqState{na.Z, nd.Z, na.M, nd.M, j, 0};
    }
    if (i == 0 && j == a.K) st_s = none;
    if (i == j) st_s = SeqState{na.Z, nd.Z, na.M, nd.M, j, 0};
  }
  __syncthreads();
  // Residual chunk sums of the rejected row: the workgroup's rcpw chunks,
  // four at a time, each by one group of 256 threads (4 entries per thread
  // in order, then the group's four wavefront sums in order).
  const SeqState st = st_s;
  if (st.j >= a.K) return;                         // uniform: nothing rejected
  const size_t row = size_t(b) * a.K + st.j;
  const ResidualEntry res{a.za + row * a.V, a.zd + row * a.V, st.Ma, st.Md, st.Za, st.Zd, a.tscale, tab};
  const int grp = threadIdx.x / kThreads, gt = threadIdx.x % kThreads;
  const int c0 = blockIdx.x * a.rcpw;
  const int c1 = min(c0 + a.rcpw, a.rchunks);
  for (int cb = c0; cb < c1; cb += kDecideThreads / kThreads) {      // uniform
    const int c = cb + grp;
    double sum = 0.0;
    if (c < c1) {
      const int v0 = c * a.rchunk, v1 = min(v0 + a.rchunk, a.V);
      for (int v = v0 + gt; v < v1; v += kThreads) sum += res.weight(res.load(v));
    }
    sum = wave_sum(sum);
    if ((gt & 63) == 0) redd[grp][gt >> 6] = sum;
    __syncthreads();
    if (gt == 0 && c < c1) a.rs[size_t(b) * a.rchunks + c] = ((redd[grp][0] + redd[grp][1]) + redd[grp][2]) + redd[grp][3];
    __syncthreads();                               // redd is free for the next four chunks
  }
}

// One workgroup per sequence: the emitted token at the rejected row, a draw
// of max(0, p - q) (of p if the residual is empty, which only rounding can
// cause).
__global__ __launch_bounds__(kThreads) void residual_draw_kernel(ResidualArgs a) {
  __shared__ double tab[64];
  __shared__ double rs_s[kMaxChunksInLds];
  __shared__ float u_s[ORTHRUS_MAX_BLOCK];
  const int b = blockIdx.x;
  // every independent load first: the sequence's state, its residual chunk
  // sums (into LDS when they fit), the uniforms of all its rows
  const SeqState st = a.seq[b];
  const double* rs = a.rs + size_t(b) * a.rchunks;
  const bool in_lds = a.rchunks <= kMaxChunksInLds;
  bool pos = false;
  for (int k = threadIdx.x; k < a.rchunks; k += kThreads) {
    const double w = rs[k];
    if (in_lds) rs_s[k] = w;
    pos = pos || w > 0.0;
  }
  if (threadIdx.x < a.K) u_s[threadIdx.x] = a.u_res[size_t(b) * a.K + threadIdx.x];
  load_exp_table(tab);
  if (st.j >= a.K) return;                         // uniform: nothing rejected
  const bool nonempty = __syncthreads_or(pos);     // (also publishes the LDS copies)
  const size_t row = size_t(b) * a.K + st.j;
  const double u = double(u_s[st.j]);
  int tok;
  if (nonempty) {
    const ResidualEntry r{a.za + row * a.V, a.zd + row * a.V, st.Ma, st.Md, st.Za, st.Zd, a.tscale, tab};
    tok = draw<kResidualChunk / kThreads>([&](int k) { return in_lds ? rs_s[k] : rs[k]; }, r, a.rchunks,
                                          a.rchunk, a.V, u);
  } else {
    const size_t srow = size_t(a.B) * a.K + row;   // the AR view's statistics row
    const float* cm = a.cm + srow * a.nchunks;
    const double* cs = a.cs + srow * a.nchunks;
    const float M = st.Ma;
    const double tscale = a.tscale;
    tok = draw<kSampleChunkLarge / kThreads>([&](int k) { return cs[k] * wexp(cm[k], M, tscale, tab); },
                                           SoftmaxEntry{a.za + row * a.V, M, tscale, tab}, a.nchunks, a.chunk, a.V,
                                           u);
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
  float* gm;
  double* gs;
  SeqState* seq;
  double* rs;
};

Ws carve(const SamplePlan& p, void* ws) {
  char* base = static_cast<char*>(ws);
  return Ws{reinterpret_cast<float*>(base + p.cm_off), reinterpret_cast<double*>(base + p.cs_off),
            reinterpret_cast<double*>(base + p.cw_off), reinterpret_cast<float*>(base + p.gm_off),
            reinterpret_cast<double*>(base + p.gs_off), reinterpret_cast<SeqState*>(base + p.seq_off),
            reinterpret_cast<double*>(base + p.rs_off)};
}

hipError_t launch_stats(const SamplePlan& p, const StatsArgs& s, hipStream_t stream) {
  const dim3 grid(unsigned(int64_t(p.rows) * p.ngroups));
  if (p.chunk == kSampleChunk)
    return launch_kernel(&sample_stats_kernel<kSampleChunk / 64>, grid, dim3(kThreads), stream, s);
  return launch_kernel(&sample_stats_kernel<kSampleChunkLarge / 64>, grid, dim3(kThreads), stream, s);
}

}  // namespace

static_assert(sizeof(SeqState) == kSampleSeqBytes, "per-sequence state size");
static_assert(kResidualChunk % (4 * kThreads) == 0 && kSampleChunk % (4 * kThreads) == 0 &&
              kSampleChunkLarge % (4 * kThreads) == 0 && kSampleChunk == 64 * 16, "chunk shares");

hipError_t launch_sample(const SamplePlan& p, const float* logits, float temperature, const float* u,
                         int32_t* out, void* ws, hipStream_t stream) {
  const Ws w = carve(p, ws);
  const double tscale = kExp2Scale / double(temperature);   // 64 / (T ln2)
  hipError_t e = launch_stats(p, StatsArgs{logits, logits, w.cm, w.cs, nullptr, nullptr, p.rows, p.rows, p.V,
                                           p.nchunks, p.ngroups, tscale}, stream);
  if (e != hipSuccess) return e;
  const SampleArgs d{logits, u, w.cm, w.cs, w.cw, out, p.V, p.chunk, p.nchunks, tscale};
  if (p.chunk == kSampleChunk)
    return launch_kernel(&sample_draw_kernel<kSampleChunk / kThreads>, dim3(p.rows), dim3(kThreads), stream, d);
  return launch_kernel(&sample_draw_kernel<kSampleChunkLarge / kThreads>, dim3(p.rows), dim3(kThreads), stream, d);
}

hipError_t launch_accept_sampled(const SamplePlan& p, const float* logits_d, const float* logits_a,
                                 const int32_t* draft, int B, int K, float temperature, const float* u_acc,
                                 const float* u_res, int32_t* tokens, int32_t* n_acc, int32_t* n_emit,
                                 int32_t* next_anchor, void* ws, hipStream_t stream) {
  const Ws w = carve(p, ws);
  const double tscale = kExp2Scale / double(temperature);   // 64 / (T ln2)
  hipError_t e = launch_stats(p, StatsArgs{logits_d, logits_a, w.cm, w.cs, w.gm, w.gs, B * K, p.rows, p.V,
                                           p.nchunks, p.ngroups, tscale}, stream);
  if (e != hipSuccess) return e;
  const DecideArgs d{logits_d, logits_a, draft, u_acc, w.gm, w.gs, tokens, n_acc, n_emit, next_anchor, w.seq,
                     w.rs, B, K, p.V, p.ngroups, p.rchunk, p.rchunks, p.rcpw, tscale};
  e = launch_kernel(&accept_residual_kernel, dim3(unsigned((p.rchunks + p.rcpw - 1) / p.rcpw), unsigned(B)),
                    dim3(kDecideThreads), stream, d);
  if (e != hipSuccess) return e;
  const ResidualArgs r{logits_d, logits_a, u_res, w.cm, w.cs, w.seq, w.rs, tokens, next_anchor,
                       B, K, p.V, p.chunk, p.nchunks, p.rchunk, p.rchunks, tscale};
  return launch_kernel(&residual_draw_kernel, dim3(B), dim3(kThreads), stream, r);
}

}  // namespace orthrus

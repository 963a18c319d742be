// LM head and vocabulary argmax in one pass over the weights, without
// materialising the logits.
//
// Both Orthrus views end in the frozen model's shared LM head; the draft
// tokens and the AR view's greedy tokens are the argmax of its logits for
// every block row (gist.science technical summary of "Orthrus:
// Memory-Efficient Parallel Token Generation via Dual-View Diffusion",
// section 2.3 steps 1 and 3; Hacker News thread "Orthrus-Qwen3: up to
// 7.8x tokens/forward ...", post #26: the diffusion module shares the LM
// head).  For a few rows (B*K = 32 at B = 1) the product is a skinny matrix
// product bound by reading W [V, hidden] once: 1.24 GB at V = 151936,
// hidden = 4096, against 19 MB of fp32 logits that need not exist at all.
//
// Work decomposition: one workgroup (8 wavefronts) per contiguous vocabulary
// range [v0, v1) of about V/256 entries, for 32 query rows (grid.y walks row
// chunks).  The range is cut into blocks of 256 vocabulary rows; wavefront w
// owns block rows 32w .. 32w+31.  Tiles of 64 hidden elements of the block's
// weight rows (32 KiB) and of the query rows (4 KiB) stream HBM -> LDS through
// a 4-stage ring, three tiles in flight, with the same direct-to-LDS loads,
// fixed waits and zero tiles past the end as the attention kernel.  Per tile
// a wavefront does 4 MFMA 32x32x16 bf16 steps of
//     L^T[vocab][row] += W[vocab][k] . h[row][k]
// (A = weight rows from LDS, B = query rows from LDS), and at the end of a
// block turns its 32 x 32 fp32 logits into (value, index) keys (keys.h),
// keeping the best per row in registers.  The workgroup writes one key per
// row; the final argmax or acceptance kernel reduces the 256 keys of a row.
// Rows past the last one and vocabulary rows past the range are loaded as
// zeros and never become keys.  Every logit is one wavefront's sum over the
// hidden dimension in a fixed order, so the keys, and the tokens, do not
// depend on the launch shape or on how the maxima are combined.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "check.h"
#include "keys.h"
#include "launch.h"
#include "lds_ring.h"

namespace orthrus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16 zero bytes: the source of rows past the end.
__device__ __attribute__((aligned(16))) uint16_t g_lm_zero16[8] = {0, 0, 0, 0, 0, 0, 0, 0};

struct LmArgs {
  const uint16_t* h;         // [rows][hidden] bf16 (final norm applied)
  const uint16_t* w;         // [V][hidden] bf16
  float* logits;             // [rows][V] fp32, or null (not written)
  unsigned long long* keys;  // [rows][nwg]
  int rows, hidden, V, nwg, nrc;
};

// Workgroup -> (vocabulary range wg, row chunk rc).  Workgroups are dealt to
// the eight XCDs in turn (linear id mod 8).  The row chunks of one vocabulary
// range take consecutive slots on one XCD, so they stream the same weight
// rows at about the same time and share them through that XCD's L2 instead
// of each reading them from HBM.
__device__ __forceinline__ void lm_tile(const LmArgs& a, int* wg, int* rc) {
  const int L = blockIdx.x;
  if (a.nrc == 1 || (a.nwg & 7)) {
    *wg = L % a.nwg;
    *rc = L / a.nwg;
    return;
  }
  const int x = L & 7, m = L >> 3;
  *wg = (m / a.nrc) * 8 + x;
  *rc = m - (m / a.nrc) * a.nrc;
}

constexpr int VB = 256;               // vocabulary rows per block (8 wavefronts x 32)
constexpr int KT = kLmKTile;          // hidden elements per tile
constexpr int RC = kLmRowChunk;       // query rows per workgroup
constexpr int NS = 4;                 // ring stages
constexpr int W_ELEMS = VB * KT;      // 32 KiB of weights per tile
constexpr int H_ELEMS = RC * KT;      // 4 KiB of query rows per tile
constexpr int STAGE = W_ELEMS + H_ELEMS;
constexpr int LPT = 5;                // loads per wavefront per tile (4 weight + 1 query/sink)
static_assert(KT == 64, "8 granules of 16 bytes per tile row");

// Granule c (16 bytes) of tile row r sits at c ^ ((r >> 1) & 7): the 32
// rows one MFMA operand read touches fall on distinct LDS banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Per-lane best keys (query row col; lanes l and l^32 hold the same row) ->
// one key per row for the whole workgroup, written to keys[row][wg].  red is
// 2 KiB of LDS that no wavefront uses any more.
__device__ __forceinline__ void write_row_keys(const LmArgs& a, unsigned long long best, unsigned long long* red,
                                               int wg, int row0, int wave, int half, int col) {
  const auto lo = __builtin_amdgcn_permlane32_swap(uint32_t(best), uint32_t(best), false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(uint32_t(best >> 32), uint32_t(best >> 32), false, false);
  best = umax64((static_cast<unsigned long long>(hi[0]) << 32) | lo[0],
                (static_cast<unsigned long long>(hi[1]) << 32) | lo[1]);
  if (half == 0) red[wave * 32 + col] = best;
  __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): the LDS writes are done
  lds_barrier();
  if (wave == 0 && half == 0 && row0 + col < a.rows) {
    unsigned long long k = red[col];
#pragma unroll
    for (int w = 1; w < 8; ++w) k = umax64(k, red[w * 32 + col]);
    a.keys[size_t(row0 + col) * a.nwg + wg] = k;
  }
}

__global__ __launch_bounds__(512, 1) void lmhead_kernel(LmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ring[NS * STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t sink[512];   // target of the spare loads
  int wg, rc;
  lm_tile(a, &wg, &rc);
  const int row0 = rc * RC;
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int v0 = int((int64_t(a.V) * wg) / a.nwg);
  const int v1 = int((int64_t(a.V) * (wg + 1)) / a.nwg);
  const int nkt = a.hidden / KT;
  const int ntiles = ((v1 - v0 + VB - 1) / VB) * nkt;

  // Loads of tile t into stage st.  Weight rows: instruction i of wavefront
  // w covers block rows 32w + 8i .. +7, lane l row 32w + 8i + l/8, LDS granule
  // l%8.  Query rows: wavefronts 0..3, rows 8w + l/8; the others load zeros
  // into a sink.  Every wavefront issues LPT loads per tile (zeros for rows
  // outside the range and for tiles past the end), so the waits are fixed
  // counts.
  const int lr = lane >> 3, lp = lane & 7;
  auto issue_tile = [&](int t, uint16_t* st) {
    if (t >= ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) load_lds16(g_lm_zero16, lds_addr(st + (wave * 32 + i * 8) * KT));
      load_lds16(g_lm_zero16, lds_addr(wave < 4 ? st + W_ELEMS + wave * 8 * KT : sink));
      return;
    }
    const int blk = t / nkt;
    const int kt = t - blk * nkt;
    const int vbase = v0 + blk * VB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 32 + i * 8 + lr;
      const int v = vbase + r;
      const int c = lp ^ swz(r);
      const void* src = v < v1 ? static_cast<const void*>(a.w + size_t(v) * a.hidden + kt * KT + c * 8)
                               : static_cast<const void*>(g_lm_zero16);
      if (a.nrc == 1) load_lds16<true>(src, lds_addr(st + (wave * 32 + i * 8) * KT));   // read once
      else load_lds16(src, lds_addr(st + (wave * 32 + i * 8) * KT));
    }
    if (wave < 4) {
      const int r = wave * 8 + lr;
      const int hr = row0 + r;
      const int c = lp ^ swz(r);
      const void* src = hr < a.rows ? static_cast<const void*>(a.h + size_t(hr) * a.hidden + kt * KT + c * 8)
                                    : static_cast<const void*>(g_lm_zero16);
      load_lds16(src, lds_addr(st + W_ELEMS + wave * 8 * KT));
    } else {
      load_lds16(g_lm_zero16, lds_addr(sink));
    }
  };

#pragma unroll
  for (int k = 0; k < NS - 1; ++k) issue_tile(k, ring + k * STAGE);

  const int ra = wave * 32 + col;        // weight row of this lane's A operand
  f32x16 acc = f32x16{};
  unsigned long long best = 0ull;        // best key of row col over this lane's vocabulary
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<(NS - 2) * LPT>();        // tile t has landed for this wavefront
    lds_barrier();                       // ... for every wavefront; stage of t-1 is free
    const int tn = t + NS - 1;
    issue_tile(tn, ring + (tn % NS) * STAGE);
    const uint16_t* wt = ring + (t % NS) * STAGE;
    const uint16_t* ht = wt + W_ELEMS;
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      const int g = ks * 2 + half;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(wt + ra * KT + ((g ^ swz(ra)) * 8));
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(ht + col * KT + ((g ^ swz(col)) * 8));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
    const int blk = t / nkt;
    if (t - blk * nkt == nkt - 1) {      // uniform: the block's logits are complete
      // lane l, value v: vocabulary row 32w + 8(v/4) + 4 half + v%4 of the block, query row col
      const int vb = v0 + blk * VB + wave * 32 + 4 * half;
      const bool row_ok = row0 + col < a.rows;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int vi = vb + 8 * (v >> 2) + (v & 3);
        if (vi < v1) {
          best = umax64(best, make_key(acc[v], vi));
          if (a.logits && row_ok) a.logits[size_t(row0 + col) * a.V + vi] = acc[v];
        }
      }
      acc = f32x16{};
    }
  }

  wait_vmcnt<0>();                        // trailing zero-tile loads have landed
  lds_barrier();                          // every wavefront is done with the ring
  write_row_keys(a, best, reinterpret_cast<unsigned long long*>(ring), wg, row0, wave, half, col);
}

// GEMM-tiled variants for many query rows (batched decoding: B*K rows).
// There the product is no longer bound by one pass over the weights: it is a
// dense contraction (M = rows, N = vocabulary, K = hidden) whose weights
// every row tile must see.  Each workgroup (8 wavefronts) owns one output
// tile of VB vocabulary rows x RB query rows and runs the whole hidden
// dimension in tiles of GKT elements through an NS-stage LDS ring (the weight
// tile and the query tile per stage, NS - 1 tiles in flight).  The
// wavefronts form an NWV x NWR grid; each computes XB x YB blocks of
// 32x32x16 bf16 MFMA products (32 XB vocabulary rows x 32 YB query rows) per
// k-step.  The row tiles of one vocabulary tile are dealt to one XCD back to
// back (workgroup id mod 8 picks the XCD), so the weight tile comes from HBM
// once and from L2 for the other row tiles.  The epilogue turns each query
// row's VB logits into one (value, index) key per workgroup:
// keys[row][vocabulary tile].
//
// Two instances:
// - narrow: 256 x 128 tiles, 64 x 64 per wavefront, 64-element hidden tiles,
//   three 48 KiB stages;
// - wide: 256 x 256 tiles, 128 x 64 per wavefront, 32-element hidden tiles,
//   four 32 KiB stages.  It loads 1.5 times fewer bytes into LDS per product
//   and reads 6 operand blocks from LDS per 8 products instead of 4 per 4,
//   which makes a workgroup about 7 % cheaper per product.
// The host takes the one whose workgroups fill rounds of 256 CUs better;
// with a single row tile (at most 128 rows) it takes the narrow kernel's
// range mode (below).  Where several row tiles read the same weights, they
// keep the default cache policy, which leaves them in L2 for the other row
// tiles (the non-temporal policy cost 10 % at 512 and 768 rows).
// Every LM-head kernel here keeps one fp32 running sum per logit over
// 32x32x16 MFMA steps (A = 16 hidden elements of the weight row, B = the
// same elements of the query row) in increasing hidden order, so a row's
// logits are the same bits whatever kernel, tile or row count a call takes:
// the verify pass's B*K rows and greedy decoding's B rows agree.
template <int NWV_, int NWR_, int XB_, int YB_, int GKT_, int GNS_>
struct GemmCfg {
  static constexpr int NWV = NWV_, NWR = NWR_, XB = XB_, YB = YB_, GKT = GKT_, GNS = GNS_;
  static constexpr int VB = NWV * XB * 32, RB = NWR * YB * 32;
  static constexpr int ROWB = GKT * 2;                 // bytes per tile row
  static constexpr int GR = GKT / 8;                   // 16-byte granules per tile row
  static constexpr int RPL = 1024 / ROWB;              // tile rows per 1 KiB load instruction
  static constexpr int RPB = 256 / ROWB;               // tile rows per 256-byte bank row
  static constexpr int W = VB * GKT, H = RB * GKT;    // elements per stage
  static constexpr int STAGE = W + H;
  static constexpr int WCH = VB / RPL, HCH = RB / RPL; // 1 KiB chunks per stage
  static constexpr int LPT = (WCH + HCH) / 8;          // loads per wavefront per tile
  static constexpr int WLPT = WCH / 8;                 // ... of which weight loads
  static_assert(NWV * NWR == 8 && GKT % 16 == 0 && WCH % 8 == 0 && HCH % 8 == 0, "tile shape");
  static_assert(GNS >= 3, "ring depth");
  // Granule c of tile row r sits at c ^ ((r / RPB) mod GR): the 16 rows one
  // 16-lane group of an operand read touches fall on distinct LDS banks.
  static __device__ __forceinline__ int swz(int r) { return (r / RPB) % GR; }
};
using GemmNarrow = GemmCfg<4, 2, 2, 2, 64, 3>;
using GemmWide = GemmCfg<2, 4, 4, 2, 32, 4>;
static_assert(GemmNarrow::VB == kLmGemmVocabTile && GemmNarrow::RB == kLmGemmRowTile &&
              GemmWide::VB == kLmGemmWideVocabTile && GemmWide::RB == kLmGemmWideRowTile, "host tiles");

// RANGE (a single row tile, at most RB rows): workgroup wg takes the
// contiguous vocabulary range [V wg / nwg, V (wg + 1) / nwg) (nwg = 256, one
// per CU) and runs its blocks of VB rows back to back through the same ring,
// so the work is not cut into whole tiles that fill the CUs unevenly; no
// other workgroup reads its weights, so they take the non-temporal policy.
// Otherwise each workgroup owns one VB x RB output tile.
template <class C, bool RANGE>
__device__ __forceinline__ void lmhead_gemm_body(const LmArgs& a) {
  constexpr int NWV = C::NWV, NWR = C::NWR, XB = C::XB, YB = C::YB, GKT = C::GKT, GNS = C::GNS;
  __shared__ __attribute__((aligned(16))) uint16_t ring[GNS * C::STAGE];
  int slot, v0, v1, row0;                        // key slot, vocabulary range, first query row
  if constexpr (RANGE) {
    slot = blockIdx.x;
    v0 = int((int64_t(a.V) * slot) / a.nwg);
    v1 = int((int64_t(a.V) * (slot + 1)) / a.nwg);
    row0 = 0;
  } else {
    // workgroup -> (vocabulary tile, row tile); the grid is padded to a
    // multiple of 8 vocabulary tiles
    const int L = blockIdx.x;
    const int m = L >> 3;
    slot = (m / a.nrc) * 8 + (L & 7);
    const int rt = m - (m / a.nrc) * a.nrc;
    if (slot >= a.nwg) return;                   // uniform: padding
    v0 = slot * C::VB;
    v1 = min(v0 + C::VB, a.V);
    row0 = rt * C::RB;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % NWV, wr = wave / NWV;
  const int nkt = a.hidden / GKT;
  const int nblk = RANGE ? (v1 - v0 + C::VB - 1) / C::VB : 1;
  const int ntiles = RANGE ? nblk * nkt : nkt;   // (vocabulary block, hidden tile) pairs, block-major

  // Loads of tile t into stage st (tiles are issued in order; in a range,
  // tile t is block ib, hidden tile ik): wavefront w fills the 1 KiB chunks
  // w + 8i of the stage (weight rows first, then query rows), lane l row
  // RPL c + l / GR and granule l % GR of the LDS row, which holds logical
  // granule (l % GR) ^ swz(row).  Rows outside the range or past the last
  // query row, and tiles past the end, load the 16 zero bytes, so every step
  // issues LPT loads.
  const int lr = lane / C::GR, lp = lane % C::GR;
  int ib = 0, ik = 0;
  auto issue_tile = [&](int t, uint16_t* st) {
    bool live;
    int blk, kt;
    if constexpr (RANGE) {
      live = ib < nblk;
      blk = ib;
      kt = ik;
      if (++ik == nkt) { ik = 0; ++ib; }
    } else {
      live = t < nkt;
      blk = 0;
      kt = t;
    }
#pragma unroll
    for (int i = 0; i < C::LPT; ++i) {
      const int c = wave + 8 * i;
      const void* src = g_lm_zero16;
      if (i < C::WLPT) {
        const int r = c * C::RPL + lr;
        const int v = v0 + blk * C::VB + r;
        if (live && v < v1) src = a.w + size_t(v) * a.hidden + kt * GKT + (lp ^ C::swz(r)) * 8;
      } else {
        const int r = (c - C::WCH) * C::RPL + lr;
        const int hr = row0 + r;
        if (live && hr < a.rows) src = a.h + size_t(hr) * a.hidden + kt * GKT + (lp ^ C::swz(r)) * 8;
      }
      if (RANGE && i < C::WLPT) load_lds16<true>(src, lds_addr(st + c * C::RPL * GKT));   // i: unrolled constant
      else load_lds16(src, lds_addr(st + c * C::RPL * GKT));
    }
  };
#pragma unroll
  for (int k = 0; k < GNS - 1; ++k) issue_tile(k, ring + k * C::STAGE);

  f32x16 acc[XB][YB];
#pragma unroll
  for (int x = 0; x < XB; ++x)
#pragma unroll
    for (int y = 0; y < YB; ++y) acc[x][y] = f32x16{};
  unsigned long long best[YB];                   // best key of each of this lane's query rows
#pragma unroll
  for (int y = 0; y < YB; ++y) best[y] = 0ull;
  // Keys (and, on request, logits) of vocabulary block blk once its sums are
  // complete; the accumulators restart at zero.  Lane l, block (x, y), value
  // v: vocabulary row v0 + VB blk + 32 (XB wv + x) + 8(v/4) + 4 half + v%4,
  // query row row0 + 32 (YB wr + y) + col.
  auto block_keys = [&](int blk) __attribute__((always_inline)) {
#pragma unroll
    for (int y = 0; y < YB; ++y) {
      const int row = row0 + wr * YB * 32 + y * 32 + col;
      const bool row_ok = row < a.rows;
#pragma unroll
      for (int x = 0; x < XB; ++x) {
        const int vb = v0 + blk * C::VB + wv * XB * 32 + x * 32 + 4 * half;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int vi = vb + 8 * (v >> 2) + (v & 3);
          if (vi < v1) {
            best[y] = umax64(best[y], make_key(acc[x][y][v], vi));
            if (a.logits && row_ok) a.logits[size_t(row) * a.V + vi] = acc[x][y][v];
          }
        }
        acc[x][y] = f32x16{};
      }
    }
  };
  int cb = 0, ck = 0;                            // block and hidden tile of the tile being computed
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<(GNS - 2) * C::LPT>();    // tile t has landed for this wavefront
    lds_barrier();                       // ... for every wavefront; stage of t-1 is free
    const int tn = t + GNS - 1;
    issue_tile(tn, ring + (tn % GNS) * C::STAGE);
    const uint16_t* wt = ring + (t % GNS) * C::STAGE;
    const uint16_t* ht = wt + C::W;
    // All operand reads of the tile go out first, so their LDS latency is
    // paid once per tile rather than once per k-step (the scheduling barrier
    // keeps the compiler from sinking them between the products).
    constexpr int NKS = GKT / 16;
    bf16x8 av[NKS][XB], bv[NKS][YB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int g = ks * 2 + half;
#pragma unroll
      for (int x = 0; x < XB; ++x) {
        const int ra = wv * XB * 32 + x * 32 + col;
        av[ks][x] = *reinterpret_cast<const bf16x8*>(wt + ra * GKT + ((g ^ C::swz(ra)) * 8));
      }
#pragma unroll
      for (int y = 0; y < YB; ++y) {
        const int rb = wr * YB * 32 + y * 32 + col;
        bv[ks][y] = *reinterpret_cast<const bf16x8*>(ht + rb * GKT + ((g ^ C::swz(rb)) * 8));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int x = 0; x < XB; ++x)
#pragma unroll
        for (int y = 0; y < YB; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks][x], bv[ks][y], acc[x][y], 0, 0, 0);

    if constexpr (RANGE) {
      if (++ck == nkt) {                 // uniform: block cb's logits are complete
        block_keys(cb);
        ck = 0;
        ++cb;
      }
    }
  }
  if constexpr (!RANGE) block_keys(0);

  wait_vmcnt<0>();                        // trailing zero-tile loads have landed
  lds_barrier();                          // every wavefront is done with the ring
  unsigned long long* red = reinterpret_cast<unsigned long long*>(ring);   // [NWV vocabulary groups][RB rows]
#pragma unroll
  for (int y = 0; y < YB; ++y) {
    unsigned long long k = best[y];
    const auto lo = __builtin_amdgcn_permlane32_swap(uint32_t(k), uint32_t(k), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(uint32_t(k >> 32), uint32_t(k >> 32), false, false);
    k = umax64((static_cast<unsigned long long>(hi[0]) << 32) | lo[0],
               (static_cast<unsigned long long>(hi[1]) << 32) | lo[1]);
    if (half == 0) red[wv * C::RB + wr * YB * 32 + y * 32 + col] = k;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): the LDS writes are done
  lds_barrier();
  if (tid < C::RB && row0 + tid < a.rows) {
    unsigned long long k = red[tid];
#pragma unroll
    for (int g = 1; g < NWV; ++g) k = umax64(k, red[g * C::RB + tid]);
    a.keys[size_t(row0 + tid) * a.nwg + slot] = k;
  }
}

__global__ __launch_bounds__(512, 1) void lmhead_gemm_kernel(LmArgs a) {
  lmhead_gemm_body<GemmNarrow, false>(a);
}

__global__ __launch_bounds__(512, 1) void lmhead_gemm_range_kernel(LmArgs a) {
  lmhead_gemm_body<GemmNarrow, true>(a);
}

__global__ __launch_bounds__(512, 1) void lmhead_gemm_wide_kernel(LmArgs a) {
  lmhead_gemm_body<GemmWide, false>(a);
}

}  // namespace

hipError_t launch_lmhead(const LmHeadPlan& p, const void* hidden, const void* weight, float* logits,
                         void* ws, hipStream_t stream) {
  LmArgs a{static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(weight), logits,
           static_cast<unsigned long long*>(ws), p.rows, p.hidden, p.V, p.nwg, p.nrc};
  if (p.gemm) {
    const dim3 grid(unsigned((int64_t(p.nwg) + 7) / 8 * 8 * p.nrc));
    if (p.gemm == 2) return launch_kernel(&lmhead_gemm_wide_kernel, grid, dim3(512), stream, a);
    if (p.gemm == 3) return launch_kernel(&lmhead_gemm_range_kernel, dim3(p.nwg), dim3(512), stream, a);
    return launch_kernel(&lmhead_gemm_kernel, grid, dim3(512), stream, a);
  }
  const dim3 grid(unsigned(int64_t(p.nwg) * p.nrc));
  return launch_kernel(&lmhead_kernel, grid, dim3(512), stream, a);
}

}  // namespace orthrus

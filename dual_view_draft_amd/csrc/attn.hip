// Dual-view block attention over one shared paged KV cache, for gfx950.
//
// Both Orthrus views attend to the single cache that the AR view wrote
// (gist.science technical summary of "Orthrus: Memory-Efficient Parallel
// Token Generation via Dual-View Diffusion", section 2.1).  The draft pass
// (diffusion view) lets every block row see the whole cache and every other
// block row (section 2.2, block mask); the verify pass (AR view) is causal
// inside the block (section 2.3 step 2).  Both are this kernel with a
// compile-time mask.
//
// Work decomposition (flash-decoding style split context):
//   one workgroup per (context split s, sequence b, KV head g, row chunk),
//   (b, g, chunk) fastest so that all splits of a head share an XCD; one
//   8-wavefront workgroup per CU.  A workgroup owns the G*K query rows of KV
//   head g (up to 128 rows per chunk) and streams the keys/values at absolute
//   positions [s*split, (s+1)*split) in 64-token tiles (4 pages), so every K/V
//   byte is read from HBM once and shared by all rows of the group.  Positions
//   < L_b come from the pages via the block table, positions L_b .. L_b+K-1
//   from the block's own k_blk/v_blk, later positions are zero.  Splits and
//   tiles sit at fixed absolute positions, so a row's arithmetic does not
//   depend on K or on the other rows present.
//
// Memory path: tiles go HBM -> LDS directly (16-byte global_load_lds per lane,
// 1 KiB per wavefront instruction) through a 5-stage LDS ring (9 stages for
// the e4m3 cache): while tile t's P.V and tile t+1's scores are computed,
// three tiles (96 KiB for bf16 head_dim 128) are in flight.  Each wavefront
// fetches half of one page of K and of V per tile; page ids come from the
// block table once per split.
//
// Compute per tile (wavefront w: rows 32*(w%4)+0..31, tokens 32*(w/4)+0..31):
//   S^T[token][row] = K . Q^T   32x32x16 bf16 MFMA, A = K from LDS, B = Q in
//                               registers; a lane holds one query row, so the
//                               softmax max/sum are in-lane plus one exchange
//                               with lane l^32 (v_permlane32_swap).
//   O^T[d][row]    += V^T . P^T  A = V^T read transposed from LDS with
//                               ds_read_b64_tr_b16, B = P (bf16) taken straight
//                               from the S^T accumulators.
//   Online softmax in fp32 with exp2 (log2 e folded into the scale).  The two
//   token halves keep separate states, merged in LDS at the end of the split.
// Each split stores O/l as bf16 plus (m, l) in fp32; a second kernel merges
// the splits in a fixed order and writes bf16.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>

#include "check.h"
#include "launch.h"
#include "lds_ring.h"

namespace orthrus {
namespace {

// f(std::integral_constant<int, k>) for k = 0 .. N-1, expanded at compile time.
template <typename F, int... Ks>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Ks...>) {
  (f(std::integral_constant<int, Ks>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef const int32_t __attribute__((address_space(4)))* cptr_i32;
typedef const float __attribute__((address_space(4)))* cptr_f32;
typedef const void __attribute__((address_space(1)))* gptr_void;
typedef void __attribute__((address_space(3)))* lptr_void;
typedef bf16x4 __attribute__((address_space(3)))* lptr_bf16x4;
typedef i32x2 __attribute__((address_space(3)))* lptr_i32x2;

// 16 zero bytes: the source of tile rows past the last key.
__device__ __attribute__((aligned(16))) uint16_t g_zero16[8] = {0, 0, 0, 0, 0, 0, 0, 0};

struct AttnArgs {
  const void* k_pages;   // bf16 or e4m3 [num_pages][Hkv][16][D]
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* k_scale;   // e4m3 cache: [Hkv]
  const float* v_scale;
  const uint16_t* q;
  const void* k_blk;     // same element type as the pages
  const void* v_blk;
  uint16_t* part_o;  // [B][Hkv][nchunks][nsplit][rpc][D] bf16: O / l of the split
  float* part_ml;    // [B][Hkv][nchunks][nsplit][rpc][2]: m (log2 units), l
  unsigned int* err; // the device error word (ORTHRUS_DEVERR_* bits)
  int B, K, Hq, Hkv, G, num_pages, maxp, max_ctx, split, nsplit, rows, nchunks, rpc;
  float scale_log2;
};

struct CombineArgs {
  const uint16_t* part_o;
  const float* part_ml;
  const int32_t* seq_lens;
  uint16_t* out;  // [B][K][Hq][D] bf16
  int B, K, Hq, G, max_ctx, split, nsplit, nchunks, rpc;
};

__device__ __forceinline__ int clamp_len(int L, int max_ctx) {
  return L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
}

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Combine a value with the one in lane l ^ 32 (v_permlane32_swap): both
// halves receive the pair, so max and sum come out bitwise identical in
// lanes l and l ^ 32 (the low half's value is always the first operand).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Tile geometry of the split kernel for head_dim D and the cache's element
// type (bf16, or e4m3 bytes when FP8).
template <int D, bool FP8>
struct SplitCfg {
  static constexpr int RB = FP8 ? D : 2 * D;       // bytes per key/value row
  static constexpr int KG = RB / 16;               // 16-byte granules per row
  static constexpr int NS = FP8 ? 9 : 5;           // LDS ring stages
  static constexpr int TILE_BYTES = kTile * RB;    // one K (or V) tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int RPI = 1024 / RB;            // tile rows per 1 KiB wave-wide LDS load
  static constexpr int LPR = 8 / RPI;              // such loads per 8 rows of one tensor
  static constexpr int LPT = 2 * LPR;              // loads per wavefront per tile (K and V)
  static_assert(LPR >= 1, "a wavefront's 8 rows fill at least one 1 KiB load");

  // Physical 16-byte granule of logical granule c in tile row t is c ^ swizzle(t).
  // LDS has 64 four-byte banks; a 16-byte read serves 16 consecutive lanes per
  // cycle and an 8-byte (transposing) read 32 consecutive lanes.
  // K: the 16 rows read by 16 consecutive lanes (one per row, same logical
  // granule) land on distinct banks.  V: granule pairs stay together (the
  // transposing reads take 8 or 16 bytes of one pair), and the 4 rows that 32
  // lanes of one transposing read gather (64 bytes of d each) land on distinct
  // banks: with 256-byte rows (bf16, head_dim 128) each row's 4 granules move
  // to their own quarter of the row.
  __device__ static __forceinline__ int kswz(int t) { return FP8 ? (t >> 1) & 7 : t & (KG - 1); }
  __device__ static __forceinline__ int vswz(int t) {
    if constexpr (FP8) return 2 * (((t >> 1) & 1) | ((t >> 2) & 2));
    return KG == 16 ? 4 * (t & 3) : 2 * (t & 3);
  }
};

// Eight e4m3 codes (two dwords, lowest byte first) -> eight bf16 values.
// Every e4m3 value is exactly representable in bf16; the scale operand of the
// conversion is 1, so this is a pure change of format.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int D, bool VERIFY, bool FP8>
__global__ __launch_bounds__(512, 1) void attn_split_kernel(AttnArgs a) {
  using C = SplitCfg<D, FP8>;
  constexpr int RB = C::RB, KG = C::KG, NS = C::NS, TILE_BYTES = C::TILE_BYTES;
  constexpr int STAGE_BYTES = C::STAGE_BYTES, RPI = C::RPI, LPR = C::LPR, LPT = C::LPT;
  constexpr int KS = D / 16;                    // MFMA k-steps of Q.K
  constexpr int DB = D / 32;                    // 32-wide d blocks of O
  static_assert(!FP8 || D == 128, "the e4m3 cache is built for head_dim 128");
  // The ring is one array; a stage is always addressed with a compile-time
  // stage number.  Tiles arrive by asynchronous DMA whose completion is
  // tracked with explicit counter waits.
  __shared__ __attribute__((aligned(16))) char ring[NS * STAGE_BYTES];
  auto stage = [&](int k) { return ring + k * STAGE_BYTES; };

  // Linear workgroup id -> (split s, sequence b, KV head g, row chunk).  The
  // (b, g, chunk) index runs fastest, so with the 8 KV heads of the 8B shape
  // every split of head g gets an id = g (mod 8): the dispatcher deals ids to
  // the eight XCDs in turn, so one XCD streams one head and the Q rows and
  // page ids that all splits of the head read come from that XCD's L2.
  const int ny = a.Hkv * a.nchunks * a.B;
  const int s = blockIdx.x / ny;
  const int yz = blockIdx.x - s * ny;
  const int b = yz / (a.Hkv * a.nchunks);
  const int yy = yz - b * (a.Hkv * a.nchunks);
  const int g = yy / a.nchunks;
  const int chunk = yy - g * a.nchunks;
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
  const int rg = wave & 3, th = wave >> 2;      // row group, token half

  // The K/V stream is read once: the bf16 cache's tiles load with the
  // non-temporal policy (faster); for the e4m3 cache, whose pass is bound by
  // arithmetic, it measured no better, and the default policy stays.
  constexpr bool kStreamNT = !FP8;
  const int start = s * a.split;
  // Table index of this wavefront's page of tile t_idx, clamped to the row so
  // it can be read before the sequence length is known.
  auto page_index = [&](int t_idx) { return min((start >> 4) + 4 * t_idx + (wave >> 1), a.maxp - 1); };
  const int32_t* trow = a.block_table + size_t(b) * a.maxp;

  // ---- prologue, part 1: one memory round trip ---------------------------
  // Scalar loads: the sequence length, the page ids of the first NS-1 tiles
  // and (e4m3 cache) this KV head's two scales.  Vector loads: the page ids
  // of every tile of the split (lane i: tile i, clamped only when used) and
  // this lane's query row.  All of them are waited for before any tile load
  // is issued: a register value still in flight when the tile loop starts
  // makes the compiler drain the whole memory queue, tile loads included, at
  // the loop entry.
  int pg0[NS - 1];
  int L_raw;
  float k_scale = 1.0f, v_scale = 1.0f;
  {
    const cptr_i32 strow = (cptr_i32)(a.block_table) + size_t(b) * a.maxp;
    L_raw = ((cptr_i32)(a.seq_lens))[b];
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) pg0[k] = strow[page_index(k)];
    if constexpr (FP8) {
      k_scale = ((cptr_f32)(a.k_scale))[g];
      v_scale = ((cptr_f32)(a.v_scale))[g];
    }
  }
  static_assert(kMaxSplitTiles <= 64, "one lane per tile of a split");
  const int page_ids = trow[page_index(lane)];   // lane i: this wavefront's page of tile i
  const bool wave_rows = rg * kRowsPerWave < a.rpc;            // wave-uniform
  const int r = chunk * kMaxRowsPerCta + rg * kRowsPerWave + col;
  const bool row_ok = wave_rows && r < a.rows;
  const int i_row = row_ok ? r / a.G : 0;
  const int gg = row_ok ? r - i_row * a.G : 0;
  // Q^T operand of k-step ks: 8 values of this lane's query row.  bf16 cache:
  // d = 16 ks + 8 half + 0..7.  e4m3 cache: d = 32 (ks/2) + 16 half + 8 (ks%2)
  // + 0..7, matching the 16-byte K reads below (one read feeds two k-steps).
  u32x4 qraw[KS];
  {
    const uint16_t* qp = a.q + ((size_t(b) * a.K + i_row) * a.Hq + size_t(g) * a.G + gg) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = FP8 ? 32 * (ks >> 1) + 16 * half + 8 * (ks & 1) : 16 * ks + 8 * half;
      qraw[ks] = u32x4{0u, 0u, 0u, 0u};
      if (row_ok) qraw[ks] = *reinterpret_cast<const u32x4*>(qp + d0);
    }
  }
  // The empty asm takes the scalar results as operands and clobbers memory:
  // the compiler can move none of these loads past it, so all of them are in
  // flight together before the single wait below.
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) asm volatile("" ::"s"(pg0[k]));
  if constexpr (FP8) asm volatile("" ::"s"(k_scale), "s"(v_scale));
  asm volatile("" ::"s"(L_raw) : "memory");
  __builtin_amdgcn_s_waitcnt(0);                 // vmcnt(0) expcnt(0) lgkmcnt(0)

  const int L = clamp_len(L_raw, a.max_ctx);
  const int N = L + a.K;                         // keys that exist for this sequence
  if (start >= N) return;                        // uniform across the workgroup
  const int end = min(start + a.split, N);
  const int ntiles = (end - start + kTile - 1) / kTile;   // <= kMaxSplitTiles
  {
    // Device-side preconditions: the length, and this wavefront's page of
    // every tile of the split whose rows hold cached positions (lane i: tile
    // i, rows start + 64 i + 8 wave ...).  A violation is clamped below and
    // flagged in the error word (no cost when all hold but this check).
    const bool bad_page = lane < ntiles && start + kTile * lane + 8 * wave < L &&
                          static_cast<unsigned>(page_ids) >= static_cast<unsigned>(a.num_pages);
    const unsigned bad = (L_raw != L ? ORTHRUS_DEVERR_SEQ_LEN : 0u) | (__ballot(bad_page) ? ORTHRUS_DEVERR_PAGE_ID : 0u);
    if (bad && lane == 0) atomicOr(a.err, bad);
  }

  // ---- where this wavefront's share of each tile comes from ---------------
  // Wavefront w fetches tile rows 8w .. 8w+7 (half of page w/2) of K and V.
  // Lane l of a 1 KiB load fills physical granule l % KG of one row, so it
  // fetches the logical granule that the swizzle puts there.
  const size_t page_bytes = size_t(a.Hkv) * ORTHRUS_PAGE_SIZE * RB;
  const size_t blk_row = size_t(a.Hkv) * RB;
  const int lrow = lane / KG;                    // row within one 1 KiB load
  const int lgran = lane % KG;                   // physical granule this lane fills
  uint32_t koff[LPR], voff[LPR];                 // byte offsets inside the half page
  int trow_of[LPR];
#pragma unroll
  for (int j = 0; j < LPR; ++j) {
    const int t = 8 * wave + j * RPI + lrow;     // tile row
    trow_of[j] = t;
    koff[j] = uint32_t((t & 15) * RB + (lgran ^ C::kswz(t)) * 16);
    voff[j] = uint32_t((t & 15) * RB + (lgran ^ C::vswz(t)) * 16);
  }
  const char* kpool = reinterpret_cast<const char*>(a.k_pages) + size_t(g) * ORTHRUS_PAGE_SIZE * RB;
  const char* vpool = reinterpret_cast<const char*>(a.v_pages) + size_t(g) * ORTHRUS_PAGE_SIZE * RB;
  const char* kblk = reinterpret_cast<const char*>(a.k_blk) + (size_t(b) * a.K * a.Hkv + g) * RB;
  const char* vblk = reinterpret_cast<const char*>(a.v_blk) + (size_t(b) * a.K * a.Hkv + g) * RB;

  auto issue_tile = [&](int ts, int page, char* sbuf) {
    const char* kbase = kpool + size_t(page) * page_bytes;
    const char* vbase = vpool + size_t(page) * page_bytes;
    char* dst = sbuf + wave * LPR * 1024;
    if (ts + kTile <= L) {                       // uniform: whole tile from the cache
#pragma unroll
      for (int j = 0; j < LPR; ++j) {
        load_lds16<kStreamNT>(kbase + koff[j], lds_addr(dst + j * 1024));
        load_lds16<kStreamNT>(vbase + voff[j], lds_addr(dst + TILE_BYTES + j * 1024));
      }
    } else {
#pragma unroll
      for (int j = 0; j < LPR; ++j) {
        const int p = ts + trow_of[j];
        const void* ks = kbase + koff[j];
        const void* vs = vbase + voff[j];
        if (p >= L) {
          const int t = trow_of[j];
          ks = p < N ? static_cast<const void*>(kblk + (p - L) * blk_row + (lgran ^ C::kswz(t)) * 16) : g_zero16;
          vs = p < N ? static_cast<const void*>(vblk + (p - L) * blk_row + (lgran ^ C::vswz(t)) * 16) : g_zero16;
        }
        load_lds16<kStreamNT>(ks, lds_addr(dst + j * 1024));
        load_lds16<kStreamNT>(vs, lds_addr(dst + TILE_BYTES + j * 1024));
      }
    }
  };
  // A tile past the end of the split: the same number of loads, all from the
  // 16 zero bytes, so that every step of the ring issues the same count and
  // the waits below are fixed numbers.
  auto issue_dummy = [&](char* sbuf) {
    char* dst = sbuf + wave * LPR * 1024;
#pragma unroll
    for (int j = 0; j < LPR; ++j) {
      load_lds16(g_zero16, lds_addr(dst + j * 1024));
      load_lds16(g_zero16, lds_addr(dst + TILE_BYTES + j * 1024));
    }
  };
  auto clamp_page = [&](int p) { return min(max(p, 0), a.num_pages - 1); };

  // ---- prologue, part 2: the first NS-1 tiles -----------------------------
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) {
    if (k < ntiles) issue_tile(start + k * kTile, clamp_page(pg0[k]), stage(k));
    else issue_dummy(stage(k));
  }

  // ---- running softmax state (per lane = per query row, this token half) --
  // m_run is a lazily raised reference maximum (log2 units): it only moves
  // when a score exceeds it by more than 2^8, so P <= 256 and O is rarely
  // rescaled.  The result depends only on this row's own scores.
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const int row_limit = VERIFY ? (L + i_row) : (N - 1);  // last visible position
  // e4m3 cache: a key's value is code * k_scale, so the scale joins the score scale
  const float c = FP8 ? a.scale_log2 * k_scale : a.scale_log2;
  // Transposing V reads (A = V^T of the P.V product).  Lane l of the MFMA
  // operand holds d = l % 32 and the 8 tokens whose probabilities lane l's
  // P^T operand holds: 16 k2 + 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..7.
  const int trk = lane & 15;
  const int tr_dofs = 16 * ((lane >> 4) & 1) + 4 * (trk & 3);   // bf16 (+ db*32)
  const int tr_tofs = 4 * half + (trk >> 2);                      // bf16 (+ th*32 + 16*k2, + 8)
  // e4m3: lane trk of each 16-lane group names one 8-byte piece of the 8x16
  // byte block the read transposes: row trk/2 (a token), bytes 8 (trk%2)
  // of d = 16 ((lane/16) % 2) + 32 db .. +15; lane trk receives column trk.
  const int jr8 = trk >> 1;
  const int tr8_tok = 8 * (jr8 >> 2) + 4 * half + (jr8 & 3);     // + th*32 + 16*k2
  const int tr8_gran = (lane >> 4) & 1;                           // + 2*db
  const int tr8_byte = 8 * (trk & 1);

  // Raw scores S^T of one tile for this wavefront: this lane's query row
  // against 16 of the 32 tokens of its half (A = K rows from LDS, B = Q).
  auto qk = [&](const char* ks) {
    const int tok = th * 32 + col;
    bf16x8 kf[KS];
    if constexpr (FP8) {
#pragma unroll
      for (int m = 0; m < KS / 2; ++m) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(ks + tok * RB + (((2 * m + half) ^ C::kswz(tok)) * 16));
        kf[2 * m] = e4m3x8_to_bf16(raw[0], raw[1]);
        kf[2 * m + 1] = e4m3x8_to_bf16(raw[2], raw[3]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int gk = kk * 2 + half;
        kf[kk] = *reinterpret_cast<const bf16x8*>(ks + tok * RB + ((gk ^ C::kswz(tok)) * 16));
      }
    }
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], __builtin_bit_cast(bf16x8, qraw[kk]), acc, 0, 0, 0);
    return acc;
  };

  // Software pipeline: iteration t holds the raw scores of tile t on entry,
  // takes its softmax statistics, waits for tile t+1, and then computes the
  // scores of tile t+1 (matrix cores) together with P of tile t (vector
  // ALU) before P.V of tile t.  The stage of tile t-1 is free once tile t+1
  // has landed, and tile t-1+NS goes there, so NS-2 tiles stay in flight.
  wait_vmcnt<(NS - 2) * LPT>();                                  // tile 0 has landed
  lds_barrier();
  f32x16 sacc = f32x16{};
  if (wave_rows) sacc = qk(stage(0));

  // One step of the ring: returns false past the last tile.  The NS steps of
  // a pass are unrolled so that every stage number is a constant; for the
  // e4m3 ring (NS = 9) the compiler keeps a plain loop rolled, so there they
  // are expanded by template.
  auto step = [&](const int t0, const int k) __attribute__((always_inline)) -> bool {
      const int t = t0 + k;
      if (t >= ntiles) return false;                               // uniform
      const int ts = start + t * kTile;
      float m_use = 0.f;
      if (wave_rows) {
        // mask what this row may not see (raw scores; the scale is positive)
        const int tok0 = ts + th * 32;
        if (tok0 + 31 > row_limit) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int pos = tok0 + 8 * (v >> 2) + 4 * half + (v & 3);
            if (pos > row_limit) sacc[v] = -__builtin_inff();
          }
        }
        float tmax = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[v]);
        tmax = xor32_max(tmax) * c;
        const float m_new = tmax > m_run + 8.0f ? tmax : m_run;
        m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
        if (__any(m_new != m_run)) {
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
        m_run = m_new;
      }
      // Tile t+1 (a zero tile after the last one) has landed for this
      // wavefront; waiting also on the last step keeps the wait count the
      // same on every path, which the compiler's own wait insertion needs.
      wait_vmcnt<(NS - 3) * LPT>();
      if (t + 1 < ntiles) {                                        // uniform
        lds_barrier();                                             // ... for every wavefront
        if (t - 1 + NS < ntiles)
          issue_tile(ts + (NS - 1) * kTile, clamp_page(__builtin_amdgcn_readlane(page_ids, t - 1 + NS)),
                     stage((k + NS - 1) % NS));
        else
          issue_dummy(stage((k + NS - 1) % NS));
      }
      if (wave_rows) {
        // scores of tile t+1 (after the last tile: stale LDS, never used)
        const f32x16 snext = qk(stage((k + 1) % NS));
        float lsum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], c, -m_use));
          sacc[v] = pv;
          lsum += pv;
        }
        l_run += lsum;
        const char* vs = stage(k) + TILE_BYTES;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          bf16x8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(sacc[8 * k2 + j]);
          bf16x8 vf[DB];
          if constexpr (FP8) {
            const int t1 = th * 32 + 16 * k2 + tr8_tok;
            const int sw = C::vswz(t1);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int off = t1 * RB + ((2 * db + tr8_gran) ^ sw) * 16 + tr8_byte;
              const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lptr_i32x2)(vs + off));
              vf[db] = e4m3x8_to_bf16(uint32_t(raw[0]), uint32_t(raw[1]));
            }
          } else {
            const int t1 = th * 32 + 16 * k2 + tr_tofs;        // rows t1 and t1 + 8
            const int sw = C::vswz(t1);                         // same for t1 + 8
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int d = db * 32 + tr_dofs;
              const int off = (((d >> 3) ^ sw) * 8 + (d & 4)) * 2;
              const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lptr_bf16x4)(vs + t1 * RB + off));
              const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lptr_bf16x4)(vs + (t1 + 8) * RB + off));
              vf[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
          }
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pb, oacc[db], 0, 0, 0);
        }
        sacc = snext;
      }
      return true;
  };
  for (int t0 = 0; t0 < ntiles; t0 += NS) {
    if constexpr (FP8) {
      static_for<NS>([&](auto kc) { step(t0, decltype(kc)::value); });
    } else {
#pragma unroll
      for (int k = 0; k < NS; ++k)
        if (!step(t0, k)) break;
    }
  }

  // ---- merge the two token halves of each row group through LDS ----------
  l_run = xor32_sum(l_run);
  wait_vmcnt<0>();                                 // trailing zero-tile loads have landed
  lds_barrier();                                   // every wavefront is done with the ring
  // rows padded by 4 floats: lane col writes row col, and the padding puts
  // consecutive rows on different LDS banks
  constexpr int XS = D + 4;
  constexpr int XREGION = kRowsPerWave * XS + 2 * kRowsPerWave;   // floats per row group
  static_assert(4 * XREGION * 4 <= NS * STAGE_BYTES, "the exchange fits in the ring");
  float* xo = reinterpret_cast<float*>(ring) + rg * XREGION;
  float* xml = xo + kRowsPerWave * XS;
  if (wave_rows && th == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 o4 = {oacc[db][4 * j + 0], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]};
        *reinterpret_cast<f32x4*>(xo + col * XS + db * 32 + 8 * j + 4 * half) = o4;
      }
    if (half == 0) {
      xml[col] = m_run;
      xml[kRowsPerWave + col] = l_run;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): exchange writes done
  lds_barrier();
  if (!wave_rows || th == 1) return;
  const float m_b = xml[col], l_b = xml[kRowsPerWave + col];
  const float M = fmaxf(m_run, m_b);
  const float M_use = (M == -__builtin_inff()) ? 0.f : M;
  const float wa = __builtin_amdgcn_exp2f(m_run - M_use);
  const float wb = __builtin_amdgcn_exp2f(m_b - M_use);
  const float l_tot = wa * l_run + wb * l_b;
  // e4m3 cache: a value is code * v_scale, so the scale multiplies the output
  const float inv = l_tot > 0.f ? (FP8 ? v_scale : 1.0f) / l_tot : 0.f;
  const size_t part = ((size_t(b) * a.Hkv + g) * a.nchunks + chunk) * a.nsplit + s;
  const size_t prow = part * a.rpc + rg * kRowsPerWave + col;
  uint16_t* po = a.part_o + prow * D;
  // All of the other half's values first (one LDS round trip), then the
  // merged, normalised bf16 values: lane half h holds d = 32 db + 8 j + 4 h
  // + 0..3.  Pairs of lanes l, l^32 then trade 8-byte pieces so that every
  // lane writes 16 consecutive bytes (8 values).
  f32x4 ob[DB * 4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ob[db * 4 + j] = *reinterpret_cast<const f32x4*>(xo + col * XS + db * 32 + 8 * j + 4 * half);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      uint32_t w[2][2];                            // [j - 2 jp][pair]
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * jp + jj;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (wa * oacc[db][4 * j + i] + wb * ob[db * 4 + j][i]) * inv;
        w[jj][0] = pack_bf16x2(o[0], o[1]);
        w[jj][1] = pack_bf16x2(o[2], o[3]);
      }
      // half 0 keeps j = 2jp (d 0..3 of the 16) and sends j = 2jp+1; half 1
      // keeps j = 2jp+1 (d 12..15) and sends j = 2jp
      const bool hi = half != 0;
      u32x4 out4;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t x = hi ? w[0][q] : w[1][q];
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        const uint32_t other = hi ? r[0] : r[1];          // the partner's sent piece
        out4[q] = hi ? other : w[0][q];
        out4[2 + q] = hi ? w[1][q] : other;
      }
      *reinterpret_cast<u32x4*>(po + db * 32 + 16 * jp + 8 * half) = out4;
    }
  if (half == 0) *reinterpret_cast<f32x2*>(a.part_ml + prow * 2) = f32x2{M, l_tot};
}

// Sum of x over the lanes l, l ^ off (off a power of two <= 32): the pair is
// added in the same order in both lanes, so they hold the same bits.
__device__ __forceinline__ float pair_sum(float x, int off) {
  if (off == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const float y = __shfl_xor(x, off);
  return (threadIdx.x & off) ? y + x : x + y;
}
__device__ __forceinline__ float pair_max(float x, int off) {
  if (off == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return fmaxf(x, __shfl_xor(x, off));
}

// Merge the split partials of every output row:
//   out = sum_s w_s l_s Ohat_s / sum_s w_s l_s,  w_s = 2^(m_s - M),  M = max_s m_s,
// with Ohat_s = O_s / l_s (bf16).  One wavefront per output row: D/8 lanes
// cover the row (8 values, 16 bytes each) and the 64/(D/8) lane groups take
// interleaved splits, U per group and batch.  Every lane loads the (m, l) of
// its own splits with their partial rows, so a row with up to U splits per
// lane group costs one memory round trip, and takes the weights in the lane;
// the maximum and the group sums cross lanes only in log2(groups) swap steps
// (permlane swaps for lane distances 16 and 32).  Batches after the first
// rescale the running sums when the maximum grows.  Splits a row cannot see
// contribute exact zeros, so the result does not depend on how many splits
// the call had.  U is 2 when the call has at most 2 SG splits (batched
// decoding, whose many rows would otherwise issue 4 times the loads they
// use), else 8; a row's splits meet in the same lanes and order either way.
template <int D, int U>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineArgs a) {
  constexpr int TPR = D / 8;      // lanes per row slice
  constexpr int SG = 64 / TPR;    // split groups per wavefront
  constexpr int BATCH = U * SG;   // splits per batch
  const int lane = threadIdx.x & 63;
  // Workgroup -> (sequence b, KV head g) = id mod (B * Hkv), and 4 of that
  // head's G*K rows: the merge of head g runs on the XCD whose L2 took the
  // head's partial results (as in the split kernel's mapping).
  const int Hkv = a.Hq / a.G;
  const int nbg = a.B * Hkv;
  const int bg = blockIdx.x % nbg;
  const int rr = (blockIdx.x / nbg) * 4 + (threadIdx.x >> 6);   // row of head (b, g): i * G + gg
  if (rr >= a.K * a.G) return;                                   // uniform per wavefront
  const int orow = ((bg / Hkv) * a.K + rr / a.G) * a.Hq + (bg % Hkv) * a.G + rr % a.G;   // (b, i, h) flattened
  const int sg = lane / TPR;
  const int d0 = (lane % TPR) * 8;
  const int h = orow % a.Hq;
  const int bi = orow / a.Hq;
  const int i = bi % a.K;
  const int b = bi / a.K;
  const int g = h / a.G;
  const int r = i * a.G + (h - g * a.G);
  const int chunk = r / kMaxRowsPerCta;
  const int rl = r - chunk * kMaxRowsPerCta;
  const size_t prow0 = ((size_t(b) * Hkv + g) * a.nchunks + chunk) * a.nsplit * a.rpc + rl;
  const float* ml = a.part_ml + prow0 * 2;
  const uint16_t* po = a.part_o + prow0 * D + d0;
  const size_t ml_stride = size_t(a.rpc) * 2, o_stride = size_t(a.rpc) * D;

  // Loads read slots of the call's splits only (indices past the last one
  // read the last one again); slots of splits >= ns hold nothing of this
  // call and are skipped (never multiplied: they may hold any bits).
  f32x2 e[U];
  u32x4 raw[U];
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = size_t(min(j0 + u * SG + sg, a.nsplit - 1));
      e[u] = *reinterpret_cast<const f32x2*>(ml + j * ml_stride);
      raw[u] = *reinterpret_cast<const u32x4*>(po + j * o_stride);
    }
  };
  const int L_raw = a.seq_lens[b];
  load_batch(0);
  // The empty asm statements take the loaded values as operands: the first
  // batch is in flight together with the sequence length (one round trip)
  // instead of being issued once the length is known.
#pragma unroll
  for (int u = 0; u < U; ++u) asm volatile("" ::"v"(e[u]), "v"(raw[u]));
  asm volatile("" ::"v"(L_raw) : "memory");
  const int L = clamp_len(L_raw, a.max_ctx);
  const int ns = (L + a.K + a.split - 1) / a.split;

  float M = -__builtin_inff();     // running maximum of m_s over the batches so far
  float lsum = 0.f;                // this lane's sum of w_s l_s, relative to M
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < ns; j0 += BATCH) {
    if (j0 > 0) load_batch(j0);
    float mb = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u * SG + sg < ns) mb = fmaxf(mb, e[u][0]);
#pragma unroll
    for (int off = TPR; off < 64; off <<= 1) mb = pair_max(mb, off);
    const float Mn = fmaxf(M, mb);
    const float Mu = (Mn == -__builtin_inff()) ? 0.f : Mn;
    if (j0 > 0 && M != -__builtin_inff() && Mn != M) {      // uniform: rescale earlier batches
      const float sc = __builtin_amdgcn_exp2f(M - Mu);
      lsum *= sc;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] *= sc;
    }
    M = Mn;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u * SG + sg < ns) {
        const float w = __builtin_amdgcn_exp2f(e[u][0] - Mu) * e[u][1];
        lsum += w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += w * bf16_lo(raw[u][q]);
          acc[2 * q + 1] += w * bf16_hi(raw[u][q]);
        }
      }
    }
  }
  // sum the lane groups: lanes l and l ^ off hold the same d
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
    lsum = pair_sum(lsum, off);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = pair_sum(acc[q], off);
  }
  if (sg != 0) return;
  const float inv = 1.0f / lsum;
  const u32x4 packed = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                        pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4*>(a.out + size_t(orow) * D + d0) = packed;
}

template <int D, bool VERIFY, bool FP8>
hipError_t launch_split(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(unsigned(int64_t(a.nsplit) * a.Hkv * a.nchunks * a.B));
  return launch_kernel(&attn_split_kernel<D, VERIFY, FP8>, grid, dim3(512), stream, a);
}

}  // namespace

// Scratch of orthrus_attn_verify_noalloc: the split partials live in this
// file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends; in host code
// the name is only a stand-in, so host code uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
namespace {
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_attn_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attention(const AttnPlan& p, const orthrus_kv& kv, const void* q,
                            const void* k_blk, const void* v_blk, void* out, float scale,
                            bool verify, void* ws, hipStream_t stream) {
  AttnArgs a;
  a.k_pages = kv.k_pages;
  a.v_pages = kv.v_pages;
  a.block_table = kv.block_table;
  a.seq_lens = kv.seq_lens;
  a.k_scale = kv.k_scale;
  a.v_scale = kv.v_scale;
  a.q = static_cast<const uint16_t*>(q);
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.part_o = static_cast<uint16_t*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_o_bytes);
  a.B = p.B; a.K = p.K; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G;
  a.num_pages = kv.num_pages; a.maxp = kv.max_pages_per_seq; a.max_ctx = p.max_ctx;
  {
    hipError_t e = device_error_word(&a.err);
    if (e != hipSuccess) return e;
  }
  a.split = p.split; a.nsplit = p.nsplit; a.rows = p.rows; a.nchunks = p.nchunks;
  a.rpc = p.rows_per_chunk;
  a.scale_log2 = float(double(scale) * 1.4426950408889634);

  hipError_t e;
  if (kv.kv_dtype == ORTHRUS_KV_FP8_E4M3)   // head_dim 128 (checked on the host)
    e = verify ? launch_split<128, true, true>(a, stream) : launch_split<128, false, true>(a, stream);
  else if (p.D == 128)
    e = verify ? launch_split<128, true, false>(a, stream) : launch_split<128, false, false>(a, stream);
  else
    e = verify ? launch_split<64, true, false>(a, stream) : launch_split<64, false, false>(a, stream);
  if (e != hipSuccess) return e;

  CombineArgs c;
  c.part_o = a.part_o; c.part_ml = a.part_ml; c.seq_lens = kv.seq_lens;
  c.out = static_cast<uint16_t*>(out);
  c.B = p.B; c.K = p.K; c.Hq = p.Hq; c.G = p.G; c.max_ctx = p.max_ctx;
  c.split = p.split; c.nsplit = p.nsplit; c.nchunks = p.nchunks; c.rpc = p.rows_per_chunk;
  dim3 grid(unsigned((int64_t(p.K) * p.G + 3) / 4 * p.B * p.Hkv));
  if (p.D == 128)
    return p.nsplit <= 2 * 4 ? launch_kernel(&attn_combine_kernel<128, 2>, grid, dim3(256), stream, c)
                             : launch_kernel(&attn_combine_kernel<128, 8>, grid, dim3(256), stream, c);
  return p.nsplit <= 2 * 8 ? launch_kernel(&attn_combine_kernel<64, 2>, grid, dim3(256), stream, c)
                           : launch_kernel(&attn_combine_kernel<64, 8>, grid, dim3(256), stream, c);
}

}  // namespace orthrus

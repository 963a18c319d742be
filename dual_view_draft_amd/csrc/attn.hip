// Dual-view block attention over one shared paged KV cache, for gfx950.
//
// Both Orthrus views attend to the single cache that the AR view wrote
// (gist.science technical summary of "Orthrus: Memory-Efficient Parallel
// Token Generation via Dual-View Diffusion", section 2.1).  The draft pass
// (diffusion view) lets every block row see the whole cache and every other
// block row (section 2.2, block mask); the verify pass (AR view) is causal
// inside the block (section 2.3 step 2).  Both are the same kernel with a
// compile-time mask.
//
// Work decomposition (flash-decoding style split context):
//   grid = (context split s, KV head g x row chunk, sequence b)
//   Each workgroup owns the G*K query rows of KV head g (up to 128 rows per
//   chunk, 32 rows per wavefront) and streams the keys/values at absolute
//   positions [s*split, (s+1)*split) through LDS in 64-token tiles (4 pages),
//   so every K/V byte is read from HBM once and shared by all rows of the
//   group.  Positions < L_b come from the pages via the block table, positions
//   L_b .. L_b+K-1 from the block's own k_blk/v_blk, later positions are zero.
//   Split boundaries and tiles are fixed in absolute position, so a row's
//   arithmetic is independent of K and of the other rows present.
//
// Per tile and wavefront (S^T formulation, 32x32x16 bf16 MFMA, fp32 accum):
//   S^T[token][row] = K_tile . Q^T     A = K tile from LDS, B = Q in registers
//     -> lane l holds one query row (l % 32) and 32 of the tile's 64 scores,
//        so the softmax max/sum are in-lane plus one exchange with lane l^32.
//   O^T[d][row]    += V^T . P^T        A = V^T tile from LDS, B = P (bf16)
//     -> P^T comes straight out of the S^T accumulator registers; the V tile is
//        transposed while being written to LDS, in the token order that matches.
//   Online softmax in fp32 with exp2 (log2(e) folded into the scale).
// The partial (m, l, O) of every split goes to the workspace; a second kernel
// merges the splits in fixed order and writes bf16.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "check.h"
#include "launch.h"

namespace orthrus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef const int32_t __attribute__((address_space(4)))* cptr_i32;
typedef const void __attribute__((address_space(1)))* gptr_void;
typedef void __attribute__((address_space(3)))* lptr_void;
typedef bf16x4 __attribute__((address_space(3)))* lptr_bf16x4;

// 16 zero bytes: the source of tile rows past the last key.
__device__ __attribute__((aligned(16))) uint16_t g_zero16[8] = {0, 0, 0, 0, 0, 0, 0, 0};

struct AttnArgs {
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* q;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  float* part_o;   // [B][Hkv][nchunks][nsplit][rpc][D]
  float* part_ml;  // [B][Hkv][nchunks][nsplit][rpc][2]  (running max m in log2 units, sum l)
  int B, K, Hq, Hkv, G, num_pages, maxp, max_ctx, split, nsplit, rows, nchunks, rpc;
  float scale_log2;
};

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* seq_lens;
  uint16_t* out;  // [B][K][Hq][D] bf16
  int B, K, Hq, G, max_ctx, split, nsplit, nchunks, rpc;
};

__device__ __forceinline__ int clamp_len(int L, int max_ctx) {
  return L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
}

template <int D, bool VERIFY>
__global__ __launch_bounds__(256, 2) void attn_split_kernel(AttnArgs a) {
  constexpr int KG = D / 8;                     // 16-byte granules per key/value row
  constexpr int KS = D / 16;                    // MFMA k-steps of Q.K
  constexpr int DB = D / 32;                    // 32-wide d blocks of O
  constexpr int RPI = 512 / D;                  // rows per 1 KiB wave-wide LDS load
  constexpr int LPW = KG / 4;                   // LDS loads per wavefront per tile (each of K, V)
  constexpr int TILE_ELEMS = kTile * D;         // bf16 values per K (or V) tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2 * TILE_ELEMS];

  const int s = blockIdx.x;
  const int g = blockIdx.y / a.nchunks;
  const int chunk = blockIdx.y - g * a.nchunks;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;

  const int L = clamp_len(a.seq_lens[b], a.max_ctx);
  const int N = L + a.K;                         // keys that exist for this sequence
  const int start = s * a.split;
  if (start >= N) return;                        // uniform across the workgroup
  const int end = min(start + a.split, N);
  const int ntiles = (end - start + kTile - 1) / kTile;

  // ---- this lane's query row ---------------------------------------------
  const bool wave_rows = wave * kRowsPerWave < a.rpc;          // wave-uniform
  const int r = chunk * kMaxRowsPerCta + wave * kRowsPerWave + col;
  const bool row_ok = wave_rows && r < a.rows;
  const int i_row = row_ok ? r / a.G : 0;
  const int gg = row_ok ? r - i_row * a.G : 0;

  bf16x8 qreg[KS];
  {
    const uint16_t* qp = a.q + ((size_t(b) * a.K + i_row) * a.Hq + size_t(g) * a.G + gg) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + ks * 16);
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- tile loads: HBM -> LDS directly (16 bytes per lane, 1 KiB per
  // wavefront instruction).  Wavefront w loads tile rows 16w .. 16w+15, i.e.
  // exactly one cache page, whose id comes through the scalar cache.
  // K rows keep granule c at c ^ (t % KG); V rows keep it at c ^ 2(t % (KG/2))
  // (pairs of granules stay together for the transposing reads).
  const cptr_i32 trow = (cptr_i32)(a.block_table) + size_t(b) * a.maxp;
  const size_t head_off = size_t(g) * ORTHRUS_PAGE_SIZE * D;
  const size_t page_stride = size_t(a.Hkv) * ORTHRUS_PAGE_SIZE * D;
  const size_t blk_row = size_t(a.Hkv) * D;
  const uint16_t* kblk = a.k_blk + (size_t(b) * a.K * a.Hkv + g) * D;
  const uint16_t* vblk = a.v_blk + (size_t(b) * a.K * a.Hkv + g) * D;
  const int lrow = lane / KG;                    // row within one wave load
  const int lgran = lane % KG;                   // physical granule this lane fills

  auto issue_tile = [&](int ts, int buf) {
    const int pidx = min((ts >> 4) + wave, a.maxp - 1);
    const int page = min(max(trow[pidx], 0), a.num_pages - 1);
    const uint16_t* kpage = a.k_pages + size_t(page) * page_stride + head_off;
    const uint16_t* vpage = a.v_pages + size_t(page) * page_stride + head_off;
    const bool full = ts + kTile <= L;           // uniform: whole tile from the cache
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int t = 16 * wave + j * RPI + lrow;  // tile row of this lane
      const int ck = lgran ^ (t & (KG - 1));
      const int cv = lgran ^ (2 * (t & (KG / 2 - 1)));
      const uint16_t* ksrc = kpage + (t & 15) * D + ck * 8;
      const uint16_t* vsrc = vpage + (t & 15) * D + cv * 8;
      if (!full) {
        const int p = ts + t;
        if (p >= L) {
          if (p < N) {
            ksrc = kblk + (p - L) * blk_row + ck * 8;
            vsrc = vblk + (p - L) * blk_row + cv * 8;
          } else {
            ksrc = g_zero16;
            vsrc = g_zero16;
          }
        }
      }
      const int n = wave * LPW + j;              // 1 KiB slot of this load
      __builtin_amdgcn_global_load_lds((const gptr_void)ksrc,
                                       (lptr_void)(&lds[buf][n * 512]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const gptr_void)vsrc,
                                       (lptr_void)(&lds[buf][TILE_ELEMS + n * 512]), 16, 0, 0);
    }
  };

  // ---- running softmax state (per lane = per query row) ------------------
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const int row_limit = VERIFY ? (L + i_row) : (N - 1);  // last visible position

  // lane constants of the transposing V reads: lane (group G = lane/16, k = lane%16)
  const int trk = lane & 15;
  const int tr_dofs = 16 * ((lane >> 4) & 1) + 4 * (trk & 3);   // + db*32
  const int tr_tofs = 4 * half + (trk >> 2);                      // + tb*32 + 16*k2 (+8)

  issue_tile(start, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this wave's loads landed
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const int ts = start + t * kTile;
    if (t + 1 < ntiles) issue_tile(ts + kTile, cur ^ 1);

    if (wave_rows) {
      const uint16_t* ks = lds[cur];
      const uint16_t* vs = lds[cur] + TILE_ELEMS;
      f32x16 sacc[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        sacc[tb] = f32x16{};
        const int tok = tb * 32 + col;
        bf16x8 kf[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int gk = kk * 2 + half;
          kf[kk] = *reinterpret_cast<const bf16x8*>(ks + tok * D + ((gk ^ (tok & (KG - 1))) * 8));
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          sacc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qreg[kk], sacc[tb], 0, 0, 0);
      }
      // scores in log2 units; mask what this row may not see
      const bool need_mask = ts + kTile - 1 > row_limit;   // per lane
      float tmax = -__builtin_inff();
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float sc = sacc[tb][v] * a.scale_log2;
          if (need_mask) {
            const int pos = ts + tb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if (pos > row_limit) sc = -__builtin_inff();
          }
          sacc[tb][v] = sc;
          tmax = fmaxf(tmax, sc);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = __builtin_amdgcn_exp2f(sacc[tb][v] - m_use);
          sacc[tb][v] = pv;
          lsum += pv;
        }
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (__any(alpha != 1.0f)) {        // skipped once no row's maximum moves
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      }

#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          bf16x8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(sacc[tb][8 * k2 + j]);
          const int t1 = tb * 32 + 16 * k2 + tr_tofs;       // rows t1 and t1 + 8
          const int sw = 2 * (t1 & (KG / 2 - 1));            // same for t1 + 8
          bf16x8 vf[DB];
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + tr_dofs;
            const int off = ((((d >> 3) ^ sw) * 8) + (d & 4));
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lptr_bf16x4)(vs + t1 * D + off));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lptr_bf16x4)(vs + (t1 + 8) * D + off));
            vf[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pb, oacc[db], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): next tile's loads landed
    __syncthreads();
  }

  if (!wave_rows) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const size_t part = ((size_t(b) * a.Hkv + g) * a.nchunks + chunk) * a.nsplit + s;
  const size_t prow = part * a.rpc + wave * kRowsPerWave + col;
  float* po = a.part_o + prow * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 o4 = {oacc[db][4 * j + 0], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]};
      *reinterpret_cast<f32x4*>(po + db * 32 + 8 * j + 4 * half) = o4;
    }
  }
  if (half == 0) {
    a.part_ml[prow * 2 + 0] = m_run;
    a.part_ml[prow * 2 + 1] = l_tot;
  }
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;  // NaN stays NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Merge the split partials of every output row:
//   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
// One wavefront per output row: D/4 lanes cover the row (4 values each) and
// the 64/(D/4) lane groups take interleaved splits s = group, group + SG, ...
// in increasing order; the group sums are then added in group order.  Splits
// a row cannot see contribute exact zeros, so the result does not depend on
// how many splits the call had.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineArgs a) {
  constexpr int TPR = D / 4;      // lanes per row slice
  constexpr int SG = 64 / TPR;    // split groups per wavefront
  const int lane = threadIdx.x & 63;
  const int orow = blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, i, h) flattened
  if (orow >= a.B * a.K * a.Hq) return;                    // uniform per wavefront
  const int sg = lane / TPR;
  const int d0 = (lane % TPR) * 4;
  const int h = orow % a.Hq;
  const int bi = orow / a.Hq;
  const int i = bi % a.K;
  const int b = bi / a.K;
  const int g = h / a.G;
  const int r = i * a.G + (h - g * a.G);
  const int chunk = r / kMaxRowsPerCta;
  const int rl = r - chunk * kMaxRowsPerCta;
  const int L = clamp_len(a.seq_lens[b], a.max_ctx);
  const int ns = (L + a.K + a.split - 1) / a.split;
  const int Hkv = a.Hq / a.G;
  const size_t prow0 = ((size_t(b) * Hkv + g) * a.nchunks + chunk) * a.nsplit * a.rpc + rl;
  const float* ml = a.part_ml + prow0 * 2;
  const float* po = a.part_o + prow0 * D + d0;
  const size_t ml_stride = size_t(a.rpc) * 2, o_stride = size_t(a.rpc) * D;

  float M = -__builtin_inff();
#pragma unroll 4
  for (int s = sg; s < ns; s += SG) M = fmaxf(M, ml[s * ml_stride]);
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll 4
  for (int s = sg; s < ns; s += SG) {
    const float w = __builtin_amdgcn_exp2f(ml[s * ml_stride] - M);
    const f32x4 o = *reinterpret_cast<const f32x4*>(po + s * o_stride);
    acc += w * o;
    lsum += w * ml[s * ml_stride + 1];
  }
  f32x4 tot = {0.f, 0.f, 0.f, 0.f};
  float ltot = 0.f;
#pragma unroll
  for (int k = 0; k < SG; ++k) {
    const int src = (lane % TPR) + k * TPR;
    tot[0] += __shfl(acc[0], src);
    tot[1] += __shfl(acc[1], src);
    tot[2] += __shfl(acc[2], src);
    tot[3] += __shfl(acc[3], src);
    ltot += __shfl(lsum, src);
  }
  if (sg != 0) return;
  const float inv = 1.0f / ltot;
  u32x2 packed = {bf16_rne_bits(tot[0] * inv) | (bf16_rne_bits(tot[1] * inv) << 16),
                  bf16_rne_bits(tot[2] * inv) | (bf16_rne_bits(tot[3] * inv) << 16)};
  *reinterpret_cast<u32x2*>(a.out + size_t(orow) * D + d0) = packed;
}

template <int D, bool VERIFY>
hipError_t launch_split(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.nsplit, a.Hkv * a.nchunks, a.B);
  return launch_kernel(&attn_split_kernel<D, VERIFY>, grid, dim3(256), stream, a);
}

}  // namespace

hipError_t launch_attention(const AttnPlan& p, const orthrus_kv& kv, const void* q,
                            const void* k_blk, const void* v_blk, void* out, float scale,
                            bool verify, void* ws, hipStream_t stream) {
  AttnArgs a;
  a.k_pages = static_cast<const uint16_t*>(kv.k_pages);
  a.v_pages = static_cast<const uint16_t*>(kv.v_pages);
  a.block_table = kv.block_table;
  a.seq_lens = kv.seq_lens;
  a.q = static_cast<const uint16_t*>(q);
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_o_bytes);
  a.B = p.B; a.K = p.K; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G;
  a.num_pages = kv.num_pages; a.maxp = kv.max_pages_per_seq; a.max_ctx = p.max_ctx;
  a.split = p.split; a.nsplit = p.nsplit; a.rows = p.rows; a.nchunks = p.nchunks;
  a.rpc = p.rows_per_chunk;
  a.scale_log2 = float(double(scale) * 1.4426950408889634);

  hipError_t e;
  if (p.D == 128) e = verify ? launch_split<128, true>(a, stream) : launch_split<128, false>(a, stream);
  else e = verify ? launch_split<64, true>(a, stream) : launch_split<64, false>(a, stream);
  if (e != hipSuccess) return e;

  CombineArgs c;
  c.part_o = a.part_o; c.part_ml = a.part_ml; c.seq_lens = kv.seq_lens;
  c.out = static_cast<uint16_t*>(out);
  c.B = p.B; c.K = p.K; c.Hq = p.Hq; c.G = p.G; c.max_ctx = p.max_ctx;
  c.split = p.split; c.nsplit = p.nsplit; c.nchunks = p.nchunks; c.rpc = p.rows_per_chunk;
  const int64_t rows = int64_t(p.B) * p.K * p.Hq;
  dim3 grid(unsigned((rows + 3) / 4));
  return p.D == 128 ? launch_kernel(&attn_combine_kernel<128>, grid, dim3(256), stream, c)
                    : launch_kernel(&attn_combine_kernel<64>, grid, dim3(256), stream, c);
}

}  // namespace orthrus

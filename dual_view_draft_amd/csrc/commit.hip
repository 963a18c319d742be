// Commit of the accepted prefix into the single shared KV cache.
//
// Only the AR view writes the cache; after consensus the cache holds exactly
// the confirmed prefix (gist.science technical summary of "Orthrus:
// Memory-Efficient Parallel Token Generation via Dual-View Diffusion",
// section 2.3 step 3, and section 3 on keeping no redundant drafter cache).
// The verify pass's block K/V rows 0 .. n_emit-1 are copied bit for bit to
// positions L .. L+n_emit-1 of every layer's paged pool; the draft pass's
// K/V are never stored.  One workgroup per (block row, sequence, layer); each
// thread moves one 16-byte granule of one KV head's K or V row.  The copy is
// the same for every element type of the cache (bf16, or e4m3 codes that
// orthrus_quantize_kv produced for the block).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "check.h"
#include "launch.h"

namespace orthrus {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CommitArgs {
  char* k_pages;
  char* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const char* k_blk;
  const char* v_blk;
  const int32_t* n_emit;
  int32_t* seq_lens_out;
  int64_t pool_stride, blk_stride;   // bytes per layer
  unsigned int* err;                 // the device error word (ORTHRUS_DEVERR_* bits)
  int B, K, Hkv, RB, num_pages, maxp;   // RB: bytes per head row
};

__global__ __launch_bounds__(256) void commit_kernel(CommitArgs a) {
  const int r = blockIdx.x;
  const int b = blockIdx.y;
  const int layer = blockIdx.z;
  // A length beyond what the block table can address is clamped first, so
  // L + r stays far below 2^31.
  // Violated device-side preconditions are clamped and flagged in the error
  // word (by one thread per sequence, or per row and layer 0).
  const int L_raw = a.seq_lens[b];
  const int L = int(min(int64_t(max(L_raw, 0)), int64_t(a.maxp) * ORTHRUS_PAGE_SIZE));
  const int e_raw = a.n_emit[b];
  const int e = e_raw < 0 ? 0 : (e_raw > a.K ? a.K : e_raw);
  if (r == 0 && layer == 0 && threadIdx.x == 0) {
    a.seq_lens_out[b] = L + e;
    const unsigned bad = (L_raw != L ? ORTHRUS_DEVERR_SEQ_LEN : 0u) | (e_raw != e ? ORTHRUS_DEVERR_N_EMIT : 0u);
    if (bad) atomicOr(a.err, bad);
  }
  if (r >= e) return;
  const int p = L + r;
  const int pi = p >> 4;
  const int page = pi < a.maxp ? a.block_table[size_t(b) * a.maxp + pi] : -1;
  if (static_cast<unsigned>(page) >= static_cast<unsigned>(a.num_pages)) {
    if (layer == 0 && threadIdx.x == 0) atomicOr(a.err, ORTHRUS_DEVERR_PAGE_ID);
    return;
  }
  const int slot = p & 15;
  const int G16 = a.RB / 16;               // granules per head row
  const int per_tensor = a.Hkv * G16;
  for (int u = threadIdx.x; u < 2 * per_tensor; u += 256) {
    const bool is_v = u >= per_tensor;
    const int w = is_v ? u - per_tensor : u;
    const int g = w / G16, c = w - g * G16;
    const char* src = (is_v ? a.v_blk : a.k_blk) + layer * a.blk_stride +
                      ((size_t(b) * a.K + r) * a.Hkv + g) * a.RB + c * 16;
    char* dst = (is_v ? a.v_pages : a.k_pages) + layer * a.pool_stride +
                ((size_t(page) * a.Hkv + g) * ORTHRUS_PAGE_SIZE + slot) * a.RB + c * 16;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

}  // namespace

hipError_t launch_commit(const orthrus_kv& kv, int layers, int64_t pool_layer_stride,
                         const void* k_blk, const void* v_blk, int64_t blk_layer_stride,
                         const int32_t* n_emit, int B, int K, int32_t* seq_lens_out,
                         hipStream_t stream) {
  CommitArgs a;
  const int es = kv_elem_bytes(kv);
  a.k_pages = static_cast<char*>(kv.k_pages);
  a.v_pages = static_cast<char*>(kv.v_pages);
  a.block_table = kv.block_table;
  a.seq_lens = kv.seq_lens;
  a.k_blk = static_cast<const char*>(k_blk);
  a.v_blk = static_cast<const char*>(v_blk);
  a.n_emit = n_emit;
  a.seq_lens_out = seq_lens_out;
  a.pool_stride = pool_layer_stride * es;
  a.blk_stride = blk_layer_stride * es;
  a.B = B; a.K = K; a.Hkv = kv.num_kv_heads; a.RB = kv.head_dim * es;
  a.num_pages = kv.num_pages; a.maxp = kv.max_pages_per_seq;
  hipError_t e = device_error_word(&a.err);
  if (e != hipSuccess) return e;
  return launch_kernel(&commit_kernel, dim3(K, B, layers), dim3(256), stream, a);
}

}  // namespace orthrus

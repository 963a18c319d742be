// Host-side argument checking and launch planning (see check.h).
#include "check.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>

namespace orthrus {
namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int fail(std::string* err, int code, const char* msg) {
  if (err) *err = msg;
  return code;
}

// need_scales: the call reads values (attention), not only bit patterns (commit).
int check_kv(const orthrus_kv* kv, bool need_scales, std::string* err) {
  if (!kv) return fail(err, ORTHRUS_ERR_INVALID_ARG, "kv descriptor is null");
  if (!kv->k_pages || !kv->v_pages || !kv->block_table || !kv->seq_lens)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "kv: null k_pages/v_pages/block_table/seq_lens");
  if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "kv: page pools must be 16-byte aligned");
  if (kv->page_size != ORTHRUS_PAGE_SIZE)
    return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "kv: page_size must be 16");
  if (kv->kv_dtype != ORTHRUS_KV_BF16 && kv->kv_dtype != ORTHRUS_KV_FP8_E4M3)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "kv: kv_dtype must be ORTHRUS_KV_BF16 or ORTHRUS_KV_FP8_E4M3");
  if (kv->kv_dtype == ORTHRUS_KV_FP8_E4M3) {
    if (kv->head_dim != 128)
      return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "kv: an e4m3 cache needs head_dim 128");
    if (need_scales && (!kv->k_scale || !kv->v_scale || !aligned4(kv->k_scale) || !aligned4(kv->v_scale)))
      return fail(err, ORTHRUS_ERR_INVALID_ARG, "kv: an e4m3 cache needs 4-byte aligned k_scale and v_scale");
  }
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "kv: head_dim must be 64 or 128");
  if (kv->num_kv_heads < 1 || kv->num_pages < 1 || kv->max_pages_per_seq < 1)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "kv: num_kv_heads, num_pages, max_pages_per_seq must be >= 1");
  return ORTHRUS_OK;
}

}  // namespace

const char* status_string(int status) {
  switch (status) {
    case ORTHRUS_OK: return "ORTHRUS_OK";
    case ORTHRUS_ERR_INVALID_ARG: return "ORTHRUS_ERR_INVALID_ARG";
    case ORTHRUS_ERR_UNSUPPORTED_SHAPE: return "ORTHRUS_ERR_UNSUPPORTED_SHAPE";
    case ORTHRUS_ERR_WORKSPACE_TOO_SMALL: return "ORTHRUS_ERR_WORKSPACE_TOO_SMALL";
    case ORTHRUS_ERR_CAPACITY: return "ORTHRUS_ERR_CAPACITY";
    case ORTHRUS_ERR_HIP: return "ORTHRUS_ERR_HIP";
    default: return "ORTHRUS_ERR_UNKNOWN";
  }
}

int attn_split_tokens(int B, int Hkv, int max_ctx) {
  if (B < 1 || Hkv < 1 || max_ctx < 0) return kTile * 4;
  // One 8-wavefront workgroup fills a CU (256 CUs).  A single sequence is cut
  // into about one split per CU.  A batch, whose lengths the host does not
  // know, is cut into about four splits per CU if every sequence had the
  // longest length (about two per CU for lengths spread evenly below it);
  // the dispatcher starts a workgroup whenever a CU frees up, and longer
  // splits carry the fixed cost of a split (the page-table round trip, the
  // half merge, the partial stores, their merge) over more tokens.  On the
  // 16-sequence ragged batch (lengths 1K-32K) splits of 3072-4096 tokens
  // measured within 5 % of each other and 8-25 % faster than 1024-2560.
  const int64_t work = int64_t(B) * Hkv * (int64_t(max_ctx) + kTile);
  const int64_t target = B == 1 ? 256 : 1024;
  int64_t s = round_up(ceil_div(work, target), kTile);
  if (s < 2 * kTile) s = 2 * kTile;
  if (s > kMaxSplitTiles * kTile) s = kMaxSplitTiles * kTile;
  return int(s);
}

bool plan_attention_shape(int B, int K, int Hq, int Hkv, int D, int max_ctx, int split_tokens,
                          AttnPlan* p, std::string* why) {
  auto no = [&](const char* m) { if (why) *why = m; return false; };
  if (B < 0) return no("batch must be >= 0");
  if (K < 1 || K > ORTHRUS_MAX_BLOCK) return no("block_k must be in [1, 64]");
  if (Hkv < 1 || Hq < 1 || Hq % Hkv) return no("num_q_heads must be a positive multiple of num_kv_heads");
  if (Hq / Hkv > kMaxGroup) return no("group size num_q_heads/num_kv_heads must be <= 16");
  if (D != 64 && D != 128) return no("head_dim must be 64 or 128");
  if (max_ctx < 0 || max_ctx > (1 << 30)) return no("max_ctx out of range");
  if (split_tokens < 0 || split_tokens % kTile || split_tokens > kMaxSplitTiles * kTile)
    return no("split_tokens must be 0 or a multiple of 64 up to 4096");
  p->B = B; p->K = K; p->Hq = Hq; p->Hkv = Hkv; p->G = Hq / Hkv; p->D = D;
  p->max_ctx = max_ctx;
  p->split = split_tokens ? split_tokens : attn_split_tokens(B, Hkv, max_ctx);
  p->nsplit = int(ceil_div(int64_t(max_ctx) + K, p->split));
  p->rows = p->G * K;
  p->nchunks = int(ceil_div(p->rows, kMaxRowsPerCta));
  p->rows_per_chunk = p->rows > kMaxRowsPerCta ? kMaxRowsPerCta : int(round_up(p->rows, kRowsPerWave));
  // one workgroup per (split, sequence, KV head, row chunk) in a 1-D grid
  if (int64_t(B) * Hkv * p->nchunks * p->nsplit > int64_t(INT32_MAX))
    return no("batch * num_kv_heads * context splits too large for one launch");
  const int64_t parts = int64_t(B) * Hkv * p->nchunks * p->nsplit * p->rows_per_chunk;
  p->part_o_bytes = size_t(round_up(parts * D * 2, 256));   // bf16 O / l per split row
  p->part_ml_bytes = size_t(round_up(parts * 2 * 4, 256));
  p->ws_bytes = p->part_o_bytes + p->part_ml_bytes;
  return true;
}

int check_attention(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk,
                    const void* out, int B, int K, int Hq, float scale, int max_ctx,
                    int split_tokens, const void* ws, size_t ws_bytes, AttnPlan* plan,
                    std::string* err) {
  int rc = check_kv(kv, true, err);
  if (rc) return rc;
  std::string why;
  if (!plan_attention_shape(B, K, Hq, kv->num_kv_heads, kv->head_dim, max_ctx, split_tokens, plan, &why)) {
    if (err) *err = why;
    return (B < 0 || max_ctx < 0 || split_tokens < 0 || split_tokens % kTile ||
            split_tokens > kMaxSplitTiles * kTile)
               ? ORTHRUS_ERR_INVALID_ARG : ORTHRUS_ERR_UNSUPPORTED_SHAPE;
  }
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (int64_t(kv->max_pages_per_seq) * ORTHRUS_PAGE_SIZE < int64_t(max_ctx) + K)
    return fail(err, ORTHRUS_ERR_CAPACITY, "block table shorter than max_ctx + block_k positions");
  if (B == 0) return ORTHRUS_OK;
  if (!q || !k_blk || !v_blk || !out)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "null q/k_blk/v_blk/out");
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(out))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "q/k_blk/v_blk/out must be 16-byte aligned");
  if (!ws || !aligned16(ws)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "workspace null or misaligned");
  if (ws_bytes < plan->ws_bytes)
    return fail(err, ORTHRUS_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than orthrus_attn_workspace_bytes()");
  return ORTHRUS_OK;
}

bool plan_argmax(int rows, int V, ArgmaxPlan* p) {
  if (rows < 0 || V < 1) return false;
  p->rows = rows;
  p->V = V;
  // about 2048 workgroups over the whole matrix, each at least 4096 values
  int64_t chunk = round_up(ceil_div(int64_t(V) * (rows > 0 ? rows : 1), 2048), 1024);
  if (chunk < 4096) chunk = 4096;
  if (chunk > V) chunk = round_up(V, 4);
  p->chunk = int(chunk);
  p->nchunks = int(ceil_div(V, chunk));
  p->ws_bytes = size_t(round_up(int64_t(rows > 0 ? rows : 1) * p->nchunks * 8, 256));
  return true;
}

int check_argmax(const float* logits, int rows, int V, const int32_t* out, const void* ws,
                 size_t ws_bytes, ArgmaxPlan* plan, std::string* err) {
  if (rows < 0 || V < 1) return fail(err, ORTHRUS_ERR_INVALID_ARG, "rows must be >= 0 and vocab >= 1");
  if (rows > 65535) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "at most 65535 rows per call");
  if (V > kMaxVocab) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "vocab must be <= 2^30");
  plan_argmax(rows, V, plan);
  if (rows == 0) return ORTHRUS_OK;
  if (!logits || !out) return fail(err, ORTHRUS_ERR_INVALID_ARG, "null logits/out");
  if (!ws || !aligned16(ws)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "workspace null or misaligned");
  if (ws_bytes < plan->ws_bytes)
    return fail(err, ORTHRUS_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than orthrus_argmax_workspace_bytes()");
  return ORTHRUS_OK;
}

int check_accept(const float* logits_a, const int32_t* draft, int B, int K, int V,
                 const int32_t* a, const int32_t* n_acc, const int32_t* n_emit,
                 const int32_t* next_anchor, const void* ws, size_t ws_bytes, ArgmaxPlan* plan,
                 std::string* err) {
  if (B < 0) return fail(err, ORTHRUS_ERR_INVALID_ARG, "batch must be >= 0");
  if (K < 1 || K > ORTHRUS_MAX_BLOCK) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "block_k must be in [1, 64]");
  if (V < 1) return fail(err, ORTHRUS_ERR_INVALID_ARG, "vocab must be >= 1");
  if (int64_t(B) * K > (int64_t(1) << 30)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "batch * block_k too large");
  int rc = check_argmax(logits_a, B * K, V, a, ws, ws_bytes, plan, err);
  if (rc) return rc;
  if (B == 0) return ORTHRUS_OK;
  if (!draft || !n_acc || !n_emit || !next_anchor)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "null draft/n_acc/n_emit/next_anchor");
  return ORTHRUS_OK;
}

bool plan_lmhead(int rows, int hidden, int V, LmHeadPlan* p, std::string* why) {
  auto no = [&](const char* m) { if (why) *why = m; return false; };
  if (rows < 0) return no("rows must be >= 0");
  if (V < 1) return no("vocab must be >= 1");
  if (V > kMaxVocab) return no("vocab must be <= 2^30");
  if (hidden < kLmKTile || hidden % kLmKTile || hidden > (1 << 20))
    return no("hidden must be a multiple of 64 in [64, 2^20]");
  if (int64_t(rows) * V > (int64_t(1) << 40)) return no("rows * vocab too large");
  p->rows = rows; p->hidden = hidden; p->V = V;
  p->gemm = 0;
  if (rows > kLmGemmRows) {
    // Both GEMM kernels run one workgroup per CU (256 CUs).  A wide tile does
    // twice a narrow tile's work in about 1.87 times its time (measured at
    // hidden 4096, vocabulary 151936), so the wide kernel is chosen only
    // where its workgroups fill the rounds of 256 better.
    const int64_t narrow = ceil_div(V, kLmGemmVocabTile) * ceil_div(rows, kLmGemmRowTile);
    const int64_t wide = ceil_div(V, kLmGemmWideVocabTile) * ceil_div(rows, kLmGemmWideRowTile);
    p->gemm = ceil_div(wide, 256) * 187 < ceil_div(narrow, 256) * 100 ? 2 : 1;
    // one row tile (33-128 rows): contiguous vocabulary ranges, one
    // workgroup per CU (at 64 rows 1.3 times faster than two 32-row chunks
    // of the streaming kernel)
    if (p->gemm == 1 && rows <= kLmGemmRowTile) p->gemm = 3;
  }
  if (p->gemm == 3) {
    p->nwg = V < kLmWorkgroups ? V : kLmWorkgroups;
    p->nrc = 1;
  } else if (p->gemm == 2) {
    p->nwg = int(ceil_div(V, kLmGemmWideVocabTile));
    p->nrc = int(ceil_div(rows, kLmGemmWideRowTile));
  } else if (p->gemm == 1) {
    p->nwg = int(ceil_div(V, kLmGemmVocabTile));
    p->nrc = int(ceil_div(rows, kLmGemmRowTile));
  } else {
    p->nwg = V < kLmWorkgroups ? V : kLmWorkgroups;
    p->nrc = int(ceil_div(rows, kLmRowChunk));
  }
  p->ws_bytes = size_t(round_up(int64_t(rows > 0 ? rows : 1) * p->nwg * 8, 256));
  return true;
}

int check_lmhead(const void* hidden_states, const void* weight, int rows, int hidden, int V,
                 const int32_t* out, const void* ws, size_t ws_bytes, LmHeadPlan* plan, std::string* err) {
  std::string why;
  if (!plan_lmhead(rows, hidden, V, plan, &why)) {
    if (err) *err = why;
    return (rows < 0 || V < 1) ? ORTHRUS_ERR_INVALID_ARG : ORTHRUS_ERR_UNSUPPORTED_SHAPE;
  }
  if (rows > 65535 * kLmRowChunk) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "too many rows per call");
  if (rows == 0) return ORTHRUS_OK;
  if (!hidden_states || !weight || !out) return fail(err, ORTHRUS_ERR_INVALID_ARG, "null hidden/weight/out");
  if (!aligned16(hidden_states) || !aligned16(weight))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "hidden/weight must be 16-byte aligned");
  if (!ws || !aligned16(ws)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "workspace null or misaligned");
  if (ws_bytes < plan->ws_bytes)
    return fail(err, ORTHRUS_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than orthrus_lmhead_workspace_bytes()");
  return ORTHRUS_OK;
}

int check_lmhead_accept(const void* hidden_states, const void* weight, const int32_t* draft, int B, int K,
                        int hidden, int V, const int32_t* a, const int32_t* n_acc, const int32_t* n_emit,
                        const int32_t* next_anchor, const void* ws, size_t ws_bytes, LmHeadPlan* plan,
                        std::string* err) {
  if (B < 0) return fail(err, ORTHRUS_ERR_INVALID_ARG, "batch must be >= 0");
  if (K < 1 || K > ORTHRUS_MAX_BLOCK) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "block_k must be in [1, 64]");
  if (int64_t(B) * K > (int64_t(1) << 30)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "batch * block_k too large");
  int rc = check_lmhead(hidden_states, weight, B * K, hidden, V, a, ws, ws_bytes, plan, err);
  if (rc) return rc;
  if (B == 0) return ORTHRUS_OK;
  if (!draft || !n_acc || !n_emit || !next_anchor)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "null draft/n_acc/n_emit/next_anchor");
  return ORTHRUS_OK;
}

int check_commit(const orthrus_kv* kv, int layers, int64_t pool_layer_stride, const void* k_blk,
                 const void* v_blk, int64_t blk_layer_stride, const int32_t* n_emit, int B, int K,
                 const int32_t* seq_lens_out, std::string* err) {
  int rc = check_kv(kv, false, err);
  if (rc) return rc;
  if (layers < 1) return fail(err, ORTHRUS_ERR_INVALID_ARG, "num_layers must be >= 1");
  if (B < 0) return fail(err, ORTHRUS_ERR_INVALID_ARG, "batch must be >= 0");
  if (K < 1 || K > ORTHRUS_MAX_BLOCK) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "block_k must be in [1, 64]");
  const int64_t pool_elems = int64_t(kv->num_pages) * kv->num_kv_heads * ORTHRUS_PAGE_SIZE * kv->head_dim;
  const int64_t blk_elems = int64_t(B) * K * kv->num_kv_heads * kv->head_dim;
  if (layers > 1 && (pool_layer_stride < pool_elems || blk_layer_stride < blk_elems))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "layer strides smaller than one layer");
  const int64_t es = kv_elem_bytes(*kv);
  if (layers > 1 && ((pool_layer_stride * es) % 16 || (blk_layer_stride * es) % 16))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "layer strides must keep 16-byte alignment");
  if (B == 0) return ORTHRUS_OK;
  if (!k_blk || !v_blk || !n_emit || !seq_lens_out)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "null k_blk/v_blk/n_emit/seq_lens_out");
  if (!aligned16(k_blk) || !aligned16(v_blk))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "k_blk/v_blk must be 16-byte aligned");
  if (seq_lens_out == kv->seq_lens)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "seq_lens_out must not alias kv->seq_lens");
  return ORTHRUS_OK;
}

bool plan_sample(int stat_rows, int B, int V, SamplePlan* p) {
  if (stat_rows < 0 || B < 0 || V < 1) return false;
  p->rows = stat_rows;
  p->B = B;
  p->V = V;
  const int64_t rows1 = stat_rows > 0 ? stat_rows : 1;
  const int64_t waves = rows1 * round_up(ceil_div(V, kSampleChunk), kSampleGroup);
  p->chunk = waves <= kSampleResidentWaves ? kSampleChunk : kSampleChunkLarge;
  p->nchunks = int(ceil_div(V, p->chunk));
  p->ngroups = int(ceil_div(p->nchunks, kSampleGroup));
  p->rchunk = kResidualChunk;
  p->rchunks = B > 0 ? int(ceil_div(V, kResidualChunk)) : 0;
  // every workgroup of the acceptance launch repeats the sequence's test, so
  // the chunks are spread over at most one workgroup per CU
  p->rcpw = int(std::max<int64_t>(1, ceil_div(int64_t(B) * p->rchunks, kResidualWorkgroups)));
  const int64_t cells = rows1 * p->nchunks, gcells = rows1 * p->ngroups;
  p->cm_off = 0;
  p->cs_off = p->cm_off + size_t(round_up(cells * 4, 256));
  p->cw_off = p->cs_off + size_t(round_up(cells * 8, 256));
  p->gm_off = p->cw_off + size_t(round_up(cells * 8, 256));
  p->gs_off = p->gm_off + size_t(round_up(gcells * 4, 256));
  p->seq_off = p->gs_off + size_t(round_up(gcells * 8, 256));
  p->rs_off = p->seq_off + size_t(round_up(int64_t(B > 0 ? B : 1) * kSampleSeqBytes, 256));
  p->ws_bytes = p->rs_off + size_t(round_up(int64_t(B > 0 ? B : 1) * (p->rchunks > 0 ? p->rchunks : 1) * 8, 256));
  return true;
}

int check_sample(const float* logits, int rows, int V, float temperature, const float* u, const int32_t* out,
                 const void* ws, size_t ws_bytes, SamplePlan* plan, std::string* err) {
  if (rows < 0 || V < 1) return fail(err, ORTHRUS_ERR_INVALID_ARG, "rows must be >= 0 and vocab >= 1");
  if (rows > 65535) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "at most 65535 rows per call");
  if (V > kMaxVocab) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "vocab must be <= 2^30");
  if (!(std::isfinite(temperature) && temperature > 0.f))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "temperature must be finite and > 0");
  plan_sample(rows, 0, V, plan);
  if (int64_t(rows) * plan->nchunks > kMaxSampleCells)
    return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "rows * (statistics chunks per row) must be <= 2^30");
  if (rows == 0) return ORTHRUS_OK;
  if (!logits || !u || !out) return fail(err, ORTHRUS_ERR_INVALID_ARG, "null logits/u/out");
  if (!ws || !aligned16(ws)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "workspace null or misaligned");
  if (ws_bytes < plan->ws_bytes)
    return fail(err, ORTHRUS_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than orthrus_sample_workspace_bytes()");
  return ORTHRUS_OK;
}

int check_accept_sampled(const float* logits_d, const float* logits_a, const int32_t* draft, int B, int K,
                         int V, float temperature, const float* u_acc, const float* u_res,
                         const int32_t* tokens, const int32_t* n_acc, const int32_t* n_emit,
                         const int32_t* next_anchor, const void* ws, size_t ws_bytes, SamplePlan* plan,
                         std::string* err) {
  if (B < 0) return fail(err, ORTHRUS_ERR_INVALID_ARG, "batch must be >= 0");
  if (K < 1 || K > ORTHRUS_MAX_BLOCK) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "block_k must be in [1, 64]");
  if (V < 1) return fail(err, ORTHRUS_ERR_INVALID_ARG, "vocab must be >= 1");
  if (V > kMaxVocab) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "vocab must be <= 2^30");
  if (int64_t(B) * K * 2 > 65535) return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "2 * batch * block_k must be <= 65535");
  if (!(std::isfinite(temperature) && temperature > 0.f))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "temperature must be finite and > 0");
  plan_sample(2 * B * K, B, V, plan);
  if (int64_t(2 * B * K) * plan->nchunks > kMaxSampleCells)
    return fail(err, ORTHRUS_ERR_UNSUPPORTED_SHAPE, "2 * batch * block_k * (statistics chunks per row) must be <= 2^30");
  if (B == 0) return ORTHRUS_OK;
  if (!logits_d || !logits_a || !draft || !u_acc || !u_res || !tokens || !n_acc || !n_emit || !next_anchor)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "null pointer argument");
  if (!ws || !aligned16(ws)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "workspace null or misaligned");
  if (ws_bytes < plan->ws_bytes)
    return fail(err, ORTHRUS_ERR_WORKSPACE_TOO_SMALL,
                "workspace smaller than orthrus_accept_sampled_workspace_bytes()");
  return ORTHRUS_OK;
}

int check_quantize(const void* k, const void* v, const float* k_scale, const float* v_scale, int rows,
                   int Hkv, int D, const void* k_out, const void* v_out, std::string* err) {
  if (rows < 0 || Hkv < 1 || D < 16 || D % 16)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "rows >= 0, num_kv_heads >= 1, head_dim a multiple of 16");
  if (int64_t(rows) * Hkv * D > (int64_t(1) << 40)) return fail(err, ORTHRUS_ERR_INVALID_ARG, "too many elements");
  if (rows == 0) return ORTHRUS_OK;
  if (!k || !v || !k_scale || !v_scale || !k_out || !v_out)
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "null k/v/k_scale/v_scale/k_out/v_out");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out) || !aligned4(k_scale) ||
      !aligned4(v_scale))
    return fail(err, ORTHRUS_ERR_INVALID_ARG, "k/v/k_out/v_out must be 16-byte aligned, scales 4-byte");
  return ORTHRUS_OK;
}

}  // namespace orthrus

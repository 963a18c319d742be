// Host-side argument checking and launch planning for the Orthrus C ABI.
// Pure C++ (no HIP headers): it is compiled into the library and, separately,
// into a host-only test driver built with sanitizers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "orthrus.h"

namespace orthrus {

constexpr int kTile = 64;          // tokens per attention tile (4 pages)
constexpr int kRowsPerWave = 32;   // query rows per wavefront (one 32x32 MFMA block)
constexpr int kMaxRowsPerCta = 128;
constexpr int kMaxGroup = 16;
constexpr int kMaxSplitTiles = 64;  // a context split covers at most 64 tiles (4096 tokens)
// Largest vocabulary: chunk bounds (start + chunk length) stay below 2^31 in
// the kernels' int32 index arithmetic.
constexpr int kMaxVocab = 1 << 30;

// Bytes of the static device scratch behind orthrus_attn_verify_noalloc
// (one copy per GPU): the split partials of any call whose workspace query
// is at most this size (every single-sequence call with 8 KV heads needs
// about 8.6 MB).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;

// Geometry of one attention call, all derived on the host.
struct AttnPlan {
  int B = 0, K = 0, Hq = 0, Hkv = 0, G = 0, D = 0;
  int max_ctx = 0;
  int split = 0;           // tokens per context split (multiple of kTile)
  int nsplit = 0;          // splits covering max_ctx + K positions
  int rows = 0;            // G*K query rows per KV head
  int nchunks = 0;         // row chunks of <= 128 rows
  int rows_per_chunk = 0;  // multiple of 32
  size_t part_o_bytes = 0, part_ml_bytes = 0, ws_bytes = 0;
};

struct ArgmaxPlan {
  int rows = 0, V = 0, chunk = 0, nchunks = 0;
  size_t ws_bytes = 0;
};

// LM head + argmax: one workgroup per contiguous vocabulary range (one per
// CU of an MI355X), query rows in chunks of 32, hidden in tiles of 64.
constexpr int kLmWorkgroups = 256;
constexpr int kLmRowChunk = 32;
constexpr int kLmKTile = 64;

constexpr int kLmGemmRows = 32;       // more rows than this take a GEMM-tiled kernel
constexpr int kLmGemmVocabTile = 256;
constexpr int kLmGemmRowTile = 128;
constexpr int kLmGemmWideVocabTile = 256;
constexpr int kLmGemmWideRowTile = 256;

struct LmHeadPlan {
  int rows = 0, hidden = 0, V = 0;
  int gemm = 0;          // 0: rows kernel; GEMM: 1 256 x 128 tiles, 2 256 x 256 tiles, 3 vocabulary ranges
  int nwg = 0;           // vocabulary ranges (or tiles) = argmax key chunks per row
  int nrc = 0;           // row chunks of kLmRowChunk rows (or row tiles)
  size_t ws_bytes = 0;   // keys [rows][nwg] (8 bytes each)
};

int attn_split_tokens(int B, int Hkv, int max_ctx);

// Shape-only planning (no pointers); false if the shape is unsupported.
bool plan_attention_shape(int B, int K, int Hq, int Hkv, int D, int max_ctx, int split_tokens,
                          AttnPlan* plan, std::string* why);

// Full check of an attention call; returns an orthrus_status.
int check_attention(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk,
                    const void* out, int B, int K, int Hq, float scale, int max_ctx,
                    int split_tokens, const void* ws, size_t ws_bytes, AttnPlan* plan,
                    std::string* err);

bool plan_argmax(int rows, int V, ArgmaxPlan* plan);

int check_argmax(const float* logits, int rows, int V, const int32_t* out, const void* ws,
                 size_t ws_bytes, ArgmaxPlan* plan, std::string* err);

int check_accept(const float* logits_a, const int32_t* draft, int B, int K, int V,
                 const int32_t* a, const int32_t* n_acc, const int32_t* n_emit,
                 const int32_t* next_anchor, const void* ws, size_t ws_bytes, ArgmaxPlan* plan,
                 std::string* err);

bool plan_lmhead(int rows, int hidden, int V, LmHeadPlan* plan, std::string* why);

int check_lmhead(const void* hidden_states, const void* weight, int rows, int hidden, int V,
                 const int32_t* out, const void* ws, size_t ws_bytes, LmHeadPlan* plan, std::string* err);

int check_lmhead_accept(const void* hidden_states, const void* weight, const int32_t* draft, int B, int K,
                        int hidden, int V, const int32_t* a, const int32_t* n_acc, const int32_t* n_emit,
                        const int32_t* next_anchor, const void* ws, size_t ws_bytes, LmHeadPlan* plan,
                        std::string* err);

int check_commit(const orthrus_kv* kv, int layers, int64_t pool_layer_stride, const void* k_blk,
                 const void* v_blk, int64_t blk_layer_stride, const int32_t* n_emit, int B, int K,
                 const int32_t* seq_lens_out, std::string* err);

// Temperature sampling and the speculative-sampling consensus: vocabulary
// chunks of every row with statistics (m fp32, s fp64 per chunk), the
// per-sequence acceptance state and the residual chunk sums.
constexpr int kSampleSeqBytes = 32;
constexpr int kResidualChunk = 1024;   // entries per residual chunk
constexpr int kResidualWorkgroups = 256;   // residual workgroups per call at most (one per CU)
// Statistics chunks: one wavefront each, 16 entries per lane (1024), or 32
// per lane (2048) when the 1024-entry chunks would need more wavefronts than
// the GPU holds at once; four consecutive chunks of a row form a group.
constexpr int kSampleChunk = 1024;
constexpr int kSampleChunkLarge = 2048;
constexpr int kSampleGroup = 4;
constexpr int64_t kSampleResidentWaves = 7168;   // 256 CUs x 4 SIMDs x 7 wavefronts
constexpr int64_t kMaxSampleCells = int64_t(1) << 30;   // statistics rows x chunks per call at most

struct SamplePlan {
  int rows = 0;          // rows with chunk statistics
  int B = 0, V = 0, chunk = 0, nchunks = 0;
  int ngroups = 0;               // groups of kSampleGroup chunks per row
  int rchunk = 0, rchunks = 0;   // residual chunks (consensus only)
  int rcpw = 0;                  // residual chunks per workgroup of the acceptance launch
  size_t cm_off = 0, cs_off = 0, cw_off = 0, gm_off = 0, gs_off = 0, seq_off = 0, rs_off = 0, ws_bytes = 0;
};

// stat_rows: rows of orthrus_sample, or 2*B*K for the consensus (B sequences).
bool plan_sample(int stat_rows, int B, int V, SamplePlan* plan);

int check_sample(const float* logits, int rows, int V, float temperature, const float* u, const int32_t* out,
                 const void* ws, size_t ws_bytes, SamplePlan* plan, std::string* err);

int check_accept_sampled(const float* logits_d, const float* logits_a, const int32_t* draft, int B, int K,
                         int V, float temperature, const float* u_acc, const float* u_res,
                         const int32_t* tokens, const int32_t* n_acc, const int32_t* n_emit,
                         const int32_t* next_anchor, const void* ws, size_t ws_bytes, SamplePlan* plan,
                         std::string* err);

int check_quantize(const void* k, const void* v, const float* k_scale, const float* v_scale, int rows,
                   int Hkv, int D, const void* k_out, const void* v_out, std::string* err);

// Bytes per cached element (2 for bf16, 1 for e4m3).
inline int kv_elem_bytes(const orthrus_kv& kv) { return kv.kv_dtype == ORTHRUS_KV_FP8_E4M3 ? 1 : 2; }

const char* status_string(int status);

}  // namespace orthrus

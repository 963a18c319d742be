// extern "C" entry points of liborthrus (declared in include/orthrus.h):
// host-side checks (check.cpp), then kernel launches (launch.h).  No C++
// exception escapes; failures return a status and set a thread-local message.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "check.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int rc, const std::string& msg) {
  g_last_error = msg;
  return rc;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ORTHRUS_OK;
  return fail(ORTHRUS_ERR_HIP, std::string("HIP: ") + hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int attention(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk, void* out,
              int B, int K, int Hq, float scale, int max_ctx, int split_tokens, void* ws,
              size_t ws_bytes, void* stream, bool verify) {
  try {
    orthrus::AttnPlan plan;
    std::string err;
    const int rc = orthrus::check_attention(kv, q, k_blk, v_blk, out, B, K, Hq, scale, max_ctx,
                                            split_tokens, ws, ws_bytes, &plan, &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (B == 0) return ORTHRUS_OK;
    return hip_status(orthrus::launch_attention(plan, *kv, q, k_blk, v_blk, out, scale, verify,
                                                ws, as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

}  // namespace

extern "C" {

int orthrus_abi_version(void) { return ORTHRUS_ABI_VERSION; }

const char* orthrus_status_string(int status) { return orthrus::status_string(status); }

const char* orthrus_last_error(void) { return g_last_error.c_str(); }

int orthrus_device_errors(uint32_t* flags, int clear, void* stream) {
  try {
    if (!flags || (reinterpret_cast<uintptr_t>(flags) & 3u))
      return fail(ORTHRUS_ERR_INVALID_ARG, "flags must be a non-null, 4-byte aligned device pointer");
    return hip_status(orthrus::launch_device_errors(flags, clear, as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

int orthrus_attn_split_tokens(int batch, int num_kv_heads, int max_ctx) {
  return orthrus::attn_split_tokens(batch, num_kv_heads, max_ctx);
}

size_t orthrus_attn_workspace_bytes(int batch, int block_k, int num_q_heads, int num_kv_heads,
                                    int head_dim, int max_ctx, int split_tokens) {
  orthrus::AttnPlan plan;
  if (!orthrus::plan_attention_shape(batch, block_k, num_q_heads, num_kv_heads, head_dim, max_ctx,
                                     split_tokens, &plan, nullptr))
    return 0;
  return plan.ws_bytes;
}

int orthrus_attn_draft(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk,
                       void* out, int batch, int block_k, int num_q_heads, float scale,
                       int max_ctx, int split_tokens, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return attention(kv, q, k_blk, v_blk, out, batch, block_k, num_q_heads, scale, max_ctx,
                   split_tokens, workspace, workspace_bytes, stream, false);
}

int orthrus_attn_verify(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk,
                        void* out, int batch, int block_k, int num_q_heads, float scale,
                        int max_ctx, int split_tokens, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return attention(kv, q, k_blk, v_blk, out, batch, block_k, num_q_heads, scale, max_ctx,
                   split_tokens, workspace, workspace_bytes, stream, true);
}

int orthrus_attn_verify_noalloc(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk,
                                void* out, int batch, int block_k, int num_q_heads, float scale,
                                int max_ctx, int split_tokens, void* stream) {
  try {
    if (!kv) return fail(ORTHRUS_ERR_INVALID_ARG, "kv descriptor is null");
    orthrus::AttnPlan plan;
    std::string why;
    if (orthrus::plan_attention_shape(batch, block_k, num_q_heads, kv->num_kv_heads, kv->head_dim, max_ctx,
                                      split_tokens, &plan, &why) &&
        plan.ws_bytes > orthrus::kStaticScratchBytes)
      return fail(ORTHRUS_ERR_WORKSPACE_TOO_SMALL,
                  "call needs " + std::to_string(plan.ws_bytes) + " bytes of scratch; the static scratch of "
                  "orthrus_attn_verify_noalloc holds " + std::to_string(orthrus::kStaticScratchBytes));
    void* scratch = nullptr;
    const hipError_t e = orthrus::static_attn_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e);
    return attention(kv, q, k_blk, v_blk, out, batch, block_k, num_q_heads, scale, max_ctx, split_tokens,
                     scratch, orthrus::kStaticScratchBytes, stream, true);
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

size_t orthrus_argmax_workspace_bytes(int rows, int vocab) {
  orthrus::ArgmaxPlan plan;
  if (!orthrus::plan_argmax(rows, vocab, &plan)) return 0;
  return plan.ws_bytes;
}

int orthrus_argmax(const float* logits, int rows, int vocab, int32_t* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  try {
    orthrus::ArgmaxPlan plan;
    std::string err;
    const int rc = orthrus::check_argmax(logits, rows, vocab, out, workspace, workspace_bytes,
                                         &plan, &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (rows == 0) return ORTHRUS_OK;
    return hip_status(orthrus::launch_argmax(plan, logits, out, workspace, as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

int orthrus_accept(const float* logits_a, const int32_t* draft, int batch, int block_k, int vocab,
                   int32_t* ar_tokens, int32_t* n_acc, int32_t* n_emit, int32_t* next_anchor,
                   void* workspace, size_t workspace_bytes, void* stream) {
  try {
    orthrus::ArgmaxPlan plan;
    std::string err;
    const int rc = orthrus::check_accept(logits_a, draft, batch, block_k, vocab, ar_tokens, n_acc,
                                         n_emit, next_anchor, workspace, workspace_bytes, &plan,
                                         &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (batch == 0) return ORTHRUS_OK;
    return hip_status(orthrus::launch_accept(plan, logits_a, draft, batch, block_k, ar_tokens,
                                             n_acc, n_emit, next_anchor, workspace,
                                             as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

size_t orthrus_lmhead_workspace_bytes(int rows, int hidden, int vocab) {
  orthrus::LmHeadPlan plan;
  if (!orthrus::plan_lmhead(rows, hidden, vocab, &plan, nullptr)) return 0;
  return plan.ws_bytes;
}

int orthrus_lmhead_argmax(const void* hidden_states, const void* weight, int rows, int hidden, int vocab,
                          int32_t* out, float* logits, void* workspace, size_t workspace_bytes,
                          void* stream) {
  try {
    orthrus::LmHeadPlan plan;
    std::string err;
    const int rc = orthrus::check_lmhead(hidden_states, weight, rows, hidden, vocab, out, workspace,
                                         workspace_bytes, &plan, &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (rows == 0) return ORTHRUS_OK;
    hipStream_t s = as_stream(stream);
    hipError_t e = orthrus::launch_lmhead(plan, hidden_states, weight, logits, workspace, s);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(orthrus::launch_argmax_keys(static_cast<const unsigned long long*>(workspace), rows,
                                                  plan.nwg, out, s));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

int orthrus_lmhead_accept(const void* hidden_states, const void* weight, const int32_t* draft, int batch,
                          int block_k, int hidden, int vocab, int32_t* ar_tokens, int32_t* n_acc,
                          int32_t* n_emit, int32_t* next_anchor, void* workspace, size_t workspace_bytes,
                          void* stream) {
  try {
    orthrus::LmHeadPlan plan;
    std::string err;
    const int rc = orthrus::check_lmhead_accept(hidden_states, weight, draft, batch, block_k, hidden, vocab,
                                                ar_tokens, n_acc, n_emit, next_anchor, workspace,
                                                workspace_bytes, &plan, &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (batch == 0) return ORTHRUS_OK;
    hipStream_t s = as_stream(stream);
    hipError_t e = orthrus::launch_lmhead(plan, hidden_states, weight, nullptr, workspace, s);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(orthrus::launch_accept_keys(static_cast<const unsigned long long*>(workspace), plan.nwg,
                                                  draft, batch, block_k, ar_tokens, n_acc, n_emit,
                                                  next_anchor, s));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

int orthrus_commit_kv(const orthrus_kv* kv, int num_layers, int64_t pool_layer_stride,
                      const void* k_blk, const void* v_blk, int64_t blk_layer_stride,
                      const int32_t* n_emit, int batch, int block_k, int32_t* seq_lens_out,
                      void* stream) {
  try {
    std::string err;
    const int rc = orthrus::check_commit(kv, num_layers, pool_layer_stride, k_blk, v_blk,
                                         blk_layer_stride, n_emit, batch, block_k, seq_lens_out,
                                         &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (batch == 0) return ORTHRUS_OK;
    return hip_status(orthrus::launch_commit(*kv, num_layers, pool_layer_stride, k_blk, v_blk,
                                             blk_layer_stride, n_emit, batch, block_k,
                                             seq_lens_out, as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

size_t orthrus_sample_workspace_bytes(int rows, int vocab) {
  orthrus::SamplePlan plan;
  if (!orthrus::plan_sample(rows, 0, vocab, &plan)) return 0;
  return plan.ws_bytes;
}

int orthrus_sample(const float* logits, int rows, int vocab, float temperature, const float* u, int32_t* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  try {
    orthrus::SamplePlan plan;
    std::string err;
    const int rc = orthrus::check_sample(logits, rows, vocab, temperature, u, out, workspace, workspace_bytes,
                                         &plan, &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (rows == 0) return ORTHRUS_OK;
    return hip_status(orthrus::launch_sample(plan, logits, temperature, u, out, workspace, as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

size_t orthrus_accept_sampled_workspace_bytes(int batch, int block_k, int vocab) {
  orthrus::SamplePlan plan;
  if (batch < 0 || block_k < 1 || int64_t(batch) * block_k * 2 > 65535) return 0;
  if (!orthrus::plan_sample(2 * batch * block_k, batch, vocab, &plan)) return 0;
  return plan.ws_bytes;
}

int orthrus_accept_sampled(const float* logits_d, const float* logits_a, const int32_t* draft, int batch,
                           int block_k, int vocab, float temperature, const float* u_acc, const float* u_res,
                           int32_t* tokens, int32_t* n_acc, int32_t* n_emit, int32_t* next_anchor,
                           void* workspace, size_t workspace_bytes, void* stream) {
  try {
    orthrus::SamplePlan plan;
    std::string err;
    const int rc = orthrus::check_accept_sampled(logits_d, logits_a, draft, batch, block_k, vocab, temperature,
                                                 u_acc, u_res, tokens, n_acc, n_emit, next_anchor, workspace,
                                                 workspace_bytes, &plan, &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (batch == 0) return ORTHRUS_OK;
    return hip_status(orthrus::launch_accept_sampled(plan, logits_d, logits_a, draft, batch, block_k,
                                                     temperature, u_acc, u_res, tokens, n_acc, n_emit,
                                                     next_anchor, workspace, as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

int orthrus_quantize_kv(const void* k, const void* v, const float* k_scale, const float* v_scale, int rows,
                        int num_kv_heads, int head_dim, void* k_out, void* v_out, void* stream) {
  try {
    std::string err;
    const int rc = orthrus::check_quantize(k, v, k_scale, v_scale, rows, num_kv_heads, head_dim, k_out,
                                           v_out, &err);
    if (rc != ORTHRUS_OK) return fail(rc, err);
    if (rows == 0) return ORTHRUS_OK;
    return hip_status(orthrus::launch_quantize_kv(k, v, k_scale, v_scale, rows, num_kv_heads, head_dim, k_out,
                                                  v_out, as_stream(stream)));
  } catch (...) {
    return fail(ORTHRUS_ERR_HIP, "internal error");
  }
}

}  // extern "C"

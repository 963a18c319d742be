/*
 * orthrus.h - C ABI of the Orthrus draft/verify decode step on AMD MI355X (gfx950).
 *
 * Orthrus ("Orthrus: Memory-Efficient Parallel Token Generation via
 * Dual-View Diffusion") adds a diffusion view to a frozen autoregressive (AR)
 * Transformer.  Both views read ONE KV cache that only the AR view writes
 * (gist.science technical summary, section 2.1; paper abstract).  One decode
 * step of a sequence whose cache holds positions 0 .. L-1 and whose last
 * emitted token (the anchor) sits at position L:
 *
 *   1. draft:  the diffusion view runs the block [anchor, <mask> x (K-1)] at
 *              positions L .. L+K-1 in one forward pass; every block row sees
 *              the whole cache and every other block row (section 2.2, the
 *              block mask; section 2.3 step 1).  Its argmax gives K drafted
 *              tokens d[0..K-1].                -> orthrus_attn_draft, orthrus_argmax
 *   2. verify: the AR view runs [anchor, d[0] .. d[K-2]] in one forward pass,
 *              causal inside the block (section 2.3 step 2; Hacker News thread
 *              "Orthrus-Qwen3: up to 7.8x tokens/forward ...", post #21).
 *                                               -> orthrus_attn_verify
 *   3. accept: left to right, keep drafted tokens while they equal the AR
 *              view's greedy token; at the first mismatch append the AR token
 *              (section 2.3 step 3).            -> orthrus_accept
 *   4. commit: append the AR view's K/V of the emitted rows to the cache and
 *              advance L (section 2.3 step 3, the cache is cut back to the
 *              accepted prefix).                -> orthrus_commit_kv
 *
 * Indexing convention: draft row i and verify row i predict position L+i+1.
 * n_acc = length of the matched prefix; n_emit = n_acc+1 if n_acc < K else K;
 * emitted tokens a[0 .. n_emit-1]; next anchor a[n_emit-1].
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `kv` and the workspace size arguments is a
 *    DEVICE pointer unless stated; `kv` itself is a host struct whose fields
 *    are device pointers.  The caller owns all memory; the library allocates
 *    nothing and keeps no state between calls.
 *  - bf16 tensors are raw 16-bit bfloat16 bit patterns; all tensors are dense,
 *    row-major, in the shapes given, 16-byte aligned.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising.  Calls on one stream run in order;
 *    calls that share a workspace must not overlap.
 *  - Return value: ORTHRUS_OK (0) or a negative orthrus_status.  Arguments are
 *    checked on the host before anything is enqueued; a failed check enqueues
 *    nothing.  orthrus_last_error() gives a thread-local message about the last
 *    failure.  No C++ exception crosses this interface.
 *  - Device-side contents (page ids, sequence lengths, emitted counts) are
 *    preconditions the host cannot see.  Kernels clamp them so that no access
 *    leaves the buffers described here, but results are unspecified when they
 *    are violated; each violation met also sets a bit of the GPU's device
 *    error word (orthrus_device_errors).
 */
#ifndef ORTHRUS_H
#define ORTHRUS_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ORTHRUS_API __attribute__((visibility("default")))
#else
#define ORTHRUS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define ORTHRUS_ABI_VERSION 2
#define ORTHRUS_PAGE_SIZE 16   /* tokens per KV page */
#define ORTHRUS_MAX_BLOCK 64   /* largest block K */

typedef enum orthrus_status {
    ORTHRUS_OK = 0,
    ORTHRUS_ERR_INVALID_ARG = -1,        /* null/misaligned pointer, negative size, aliasing */
    ORTHRUS_ERR_UNSUPPORTED_SHAPE = -2,  /* head_dim, page size, block size, group size */
    ORTHRUS_ERR_WORKSPACE_TOO_SMALL = -3,
    ORTHRUS_ERR_CAPACITY = -4,           /* block table too short for max_ctx + K */
    ORTHRUS_ERR_HIP = -5                 /* a HIP runtime call failed (launch error) */
} orthrus_status;

/* Element type of the cached keys and values (orthrus_kv.kv_dtype). */
#define ORTHRUS_KV_BF16 0
#define ORTHRUS_KV_FP8_E4M3 1   /* OCP 8-bit E4M3 codes with per-KV-head fp32 scales */

/*
 * Paged KV cache of ONE layer (the shared cache of both views).
 *  k_pages, v_pages : [num_pages][num_kv_heads][page_size][head_dim] elements
 *                     of kv_dtype.  One page of one KV head is a contiguous
 *                     slab of page_size * head_dim elements.
 *  block_table      : int32 [batch][max_pages_per_seq]; position p of sequence
 *                     b lives in page block_table[b][p / 16], slot p % 16.
 *  seq_lens         : int32 [batch]; L_b, the number of cached positions.
 *  kv_dtype         : ORTHRUS_KV_BF16 (bf16 bit patterns) or
 *                     ORTHRUS_KV_FP8_E4M3 (one byte per element).
 *  k_scale, v_scale : ORTHRUS_KV_FP8_E4M3 only: fp32 [num_kv_heads], device.
 *                     The key (value) of KV head h that a code c stands for
 *                     is e4m3(c) * k_scale[h] (v_scale[h]); finite, > 0.
 *                     Ignored for bf16 (may be NULL).
 *  page_size must be 16; head_dim 64 or 128 (bf16) or 128 (e4m3).
 *
 * The e4m3 cache is not described by the method's pages: it halves the bytes
 * the attention streams.  Every key and value the attention reads is in the
 * cache's format, the block's own rows included (orthrus_quantize_kv), so the
 * verify pass sees a block key exactly as the cache will hold it and Orthrus
 * still emits greedy decoding's tokens.
 */
typedef struct orthrus_kv {
    void* k_pages;
    void* v_pages;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int32_t num_pages;
    int32_t page_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t max_pages_per_seq;
    int32_t kv_dtype;
    const float* k_scale;
    const float* v_scale;
} orthrus_kv;

/* Version of this interface (ORTHRUS_ABI_VERSION). */
ORTHRUS_API int orthrus_abi_version(void);

/* Static, human-readable name of a status code. */
ORTHRUS_API const char* orthrus_status_string(int status);

/* Thread-local detail of the most recent failed call on this thread ("" if none). */
ORTHRUS_API const char* orthrus_last_error(void);

/*
 * Device error word: one 32-bit word per GPU, zero when the library is first
 * used on it, into which kernels OR these bits when they meet a violated
 * device-side precondition (and clamp the value so that every access stays
 * in bounds):
 *  ORTHRUS_DEVERR_SEQ_LEN : a sequence length below 0, above max_ctx
 *                           (attention) or beyond the block table (commit);
 *  ORTHRUS_DEVERR_PAGE_ID : a page id outside [0, num_pages) where a cached
 *                           position (attention) or a committed row (commit)
 *                           needs it, or a committed row past the block table;
 *  ORTHRUS_DEVERR_N_EMIT  : an emitted count outside [0, block_k] (commit).
 * orthrus_device_errors enqueues, on `stream`, a copy of the current device's
 * word into flags (device memory, one uint32) and, if clear != 0, resets the
 * word to zero.  It sees what kernels earlier on the same stream set; kernels
 * on other streams of the GPU may set bits at any time.  Allocates nothing.
 */
#define ORTHRUS_DEVERR_SEQ_LEN 1u
#define ORTHRUS_DEVERR_PAGE_ID 2u
#define ORTHRUS_DEVERR_N_EMIT 4u
ORTHRUS_API int orthrus_device_errors(uint32_t* flags, int clear, void* stream);

/*
 * Context split size in tokens chosen when split_tokens == 0 is passed to the
 * attention calls: a multiple of 64 that depends only on (batch,
 * num_kv_heads, max_ctx).  Attention splits sit at fixed absolute positions
 * [s * split, (s+1) * split), so a row's result never depends on K or on
 * which other rows are in the block.
 */
ORTHRUS_API int orthrus_attn_split_tokens(int batch, int num_kv_heads, int max_ctx);

/*
 * Bytes of device workspace the attention calls need (fp32 partial results of
 * every context split).  split_tokens: 0 = orthrus_attn_split_tokens(...).
 * Returns 0 for invalid arguments.
 */
ORTHRUS_API size_t orthrus_attn_workspace_bytes(int batch, int block_k, int num_q_heads, int num_kv_heads,
                                    int head_dim, int max_ctx, int split_tokens);

/*
 * Draft-pass attention (diffusion view, block-bidirectional mask).
 *
 * For sequence b, block row i (position L_b + i) and query head h (KV head
 * g = h / (num_q_heads / num_kv_heads)):
 *   out[b][i][h] = sum_j softmax_j(scale * q[b][i][h] . key_j) value_j
 * over every cached position j < L_b (keys/values from the pages, KV head g)
 * and every block row r < K (k_blk[b][r][g], v_blk[b][r][g]).  No key is
 * masked.  The block K/V are read, never written to the cache.
 *
 *  q            : bf16 [batch][block_k][num_q_heads][head_dim]   (post-RoPE)
 *  k_blk, v_blk : [batch][block_k][num_kv_heads][head_dim] in the cache's
 *                 element type (post-RoPE; e4m3 codes from orthrus_quantize_kv
 *                 for an e4m3 cache, read with the cache's scales)
 *  out          : bf16 [batch][block_k][num_q_heads][head_dim]   (written)
 *  scale        : score scale, normally 1/sqrt(head_dim); finite, > 0
 *  max_ctx      : host-known upper bound on every L_b (sizes the grid; no
 *                 device->host read is needed).  L_b > max_ctx is clamped.
 *  split_tokens : context split size (multiple of 64, at most 4096), 0 = automatic
 *  workspace    : device scratch of >= orthrus_attn_workspace_bytes(...) bytes,
 *                 16-byte aligned; contents on entry do not matter.
 *
 * Requirements: 1 <= block_k <= 64; num_q_heads % num_kv_heads == 0 with a
 * group size of at most 16; head_dim in {64, 128}; page_size 16;
 * max_pages_per_seq * 16 >= max_ctx + block_k; batch >= 0 (0 = no-op).
 * Arithmetic: bf16 MFMA products with fp32 accumulation, fp32 online
 * softmax, bf16 output rounded to nearest even.  An e4m3 cache's codes are
 * widened to bf16 exactly; k_scale joins the score scale and v_scale
 * multiplies the output.
 */
ORTHRUS_API int orthrus_attn_draft(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk,
                       void* out, int batch, int block_k, int num_q_heads, float scale,
                       int max_ctx, int split_tokens, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Verify-pass attention (AR view, causal inside the block): as
 * orthrus_attn_draft, except that block row i sees block rows r <= i only
 * (every cached position stays visible).  With block_k = 1 this is ordinary
 * single-token decode attention; with L_b = 0 it is causal self-attention of
 * the block (chunked prefill).
 */
ORTHRUS_API int orthrus_attn_verify(const orthrus_kv* kv, const void* q, const void* k_blk, const void* v_blk,
                        void* out, int batch, int block_k, int num_q_heads, float scale,
                        int max_ctx, int split_tokens, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * orthrus_attn_verify without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and errors are
 * those of orthrus_attn_verify, computed by the same kernels; the split
 * partial results go to a static scratch array that the library holds on
 * each GPU (16 MiB per GPU, kept until the process ends; its address is
 * looked up once per device on the first call there).  The call allocates
 * nothing.  A call whose orthrus_attn_workspace_bytes(...) exceeds 16 MiB
 * returns ORTHRUS_ERR_WORKSPACE_TOO_SMALL (every single-sequence call with
 * 8 KV heads needs about 8.6 MB).  All calls on one GPU share the scratch:
 * calls that may overlap on one GPU (other streams, other threads) race and
 * must be ordered by the caller.
 */
ORTHRUS_API int orthrus_attn_verify_noalloc(const orthrus_kv* kv, const void* q, const void* k_blk,
                                const void* v_blk, void* out, int batch, int block_k, int num_q_heads,
                                float scale, int max_ctx, int split_tokens, void* stream);

/* Bytes of device workspace for orthrus_argmax / orthrus_accept (0 if invalid). */
ORTHRUS_API size_t orthrus_argmax_workspace_bytes(int rows, int vocab);

/*
 * Vocabulary argmax: out[r] = smallest v with logits[r][v] == max_v logits[r][v]
 * (fp32 comparisons; -0.0 == +0.0).  This gives the drafted tokens d from the
 * draft logits (section 2.3 step 1).
 *  logits : fp32 [rows][vocab], finite (NaN is outside the contract)
 *  out    : int32 [rows]
 * 0 <= rows <= 65535 (0 = no-op), 1 <= vocab <= 2^30.
 */
ORTHRUS_API int orthrus_argmax(const float* logits, int rows, int vocab, int32_t* out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Consensus (section 2.3 step 3): AR greedy tokens and the longest matching
 * prefix.
 *  logits_a    : fp32 [batch][block_k][vocab], the verify pass's logits
 *  draft       : int32 [batch][block_k], drafted tokens d
 *  ar_tokens   : int32 [batch][block_k] (written) a[b][i] = argmax logits_a[b][i]
 *  n_acc       : int32 [batch] (written) largest m with d[b][i] == a[b][i] for i < m
 *  n_emit      : int32 [batch] (written) n_acc + 1 if n_acc < block_k else block_k
 *  next_anchor : int32 [batch] (written) a[b][n_emit - 1]
 * workspace: >= orthrus_argmax_workspace_bytes(batch * block_k, vocab).
 */
ORTHRUS_API int orthrus_accept(const float* logits_a, const int32_t* draft, int batch, int block_k, int vocab,
                   int32_t* ar_tokens, int32_t* n_acc, int32_t* n_emit, int32_t* next_anchor,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * LM head fused with the vocabulary argmax (the greedy token of every row),
 * without materialising the logits.  Both views end in the frozen model's
 * shared LM head (section 2.3 steps 1 and 3; Hacker News thread
 * "Orthrus-Qwen3: up to 7.8x tokens/forward ...", post #26: the diffusion
 * module adds only attention projections).
 *
 *   logits[r][v] = sum_k hidden_states[r][k] * weight[v][k]
 *                  (bf16 products, fp32 accumulation over k in a fixed order)
 *   out[r]       = smallest v with logits[r][v] == max_v logits[r][v]
 *
 *  hidden_states : bf16 [rows][hidden], the final hidden states (final norm
 *                  applied)
 *  weight        : bf16 [vocab][hidden], the LM-head weight (row v = token v)
 *  out           : int32 [rows] (written)
 *  logits        : NULL, or fp32 [rows][vocab] to also receive the logits the
 *                  argmax was taken over (bit-identical values; for checking
 *                  and for callers that need them)
 *  workspace     : >= orthrus_lmhead_workspace_bytes(rows, hidden, vocab)
 *                  bytes, 16-byte aligned; contents on entry do not matter.
 * Requirements: hidden a multiple of 64 in [64, 2^20]; 1 <= vocab <= 2^30;
 * 0 <= rows <= 65535 * 32 (0 = no-op).  The weights are read once per 32
 * rows (rows beyond 32 re-read them).  NaN logits are outside the contract.
 */
ORTHRUS_API size_t orthrus_lmhead_workspace_bytes(int rows, int hidden, int vocab);

ORTHRUS_API int orthrus_lmhead_argmax(const void* hidden_states, const void* weight, int rows, int hidden,
                          int vocab, int32_t* out, float* logits, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Consensus from the verify pass's final hidden states: as orthrus_accept,
 * with the AR tokens a[b][i] computed by the fused LM head + argmax of
 * orthrus_lmhead_argmax from hidden_states [batch][block_k][hidden].
 * workspace: >= orthrus_lmhead_workspace_bytes(batch * block_k, hidden, vocab).
 */
ORTHRUS_API int orthrus_lmhead_accept(const void* hidden_states, const void* weight, const int32_t* draft,
                          int batch, int block_k, int hidden, int vocab, int32_t* ar_tokens,
                          int32_t* n_acc, int32_t* n_emit, int32_t* next_anchor, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Commit (section 2.3 step 3; the single shared cache keeps only what the AR
 * view confirmed): for every layer l, sequence b and row r < n_emit[b], copy
 * the verify pass's k_blk/v_blk row [l][b][r] (all KV heads) bit for bit to
 * position L_b + r, i.e. page block_table[b][(L_b + r) / 16], slot
 * (L_b + r) % 16, of layer l's pool.  Then seq_lens_out[b] = L_b + n_emit[b].
 * No other pool slot is written.
 *
 *  kv                 : layer 0's cache; layer l's pools start
 *                       l * pool_layer_stride elements after kv->k_pages / v_pages
 *  k_blk, v_blk       : [num_layers][batch][block_k][num_kv_heads][head_dim] in
 *                       the cache's element type, with layer stride
 *                       blk_layer_stride elements
 *  n_emit             : int32 [batch], each in [1, block_k]
 *  seq_lens_out       : int32 [batch] (written); must not alias kv->seq_lens
 * The block table must already cover positions L_b .. L_b + n_emit[b] - 1.
 */
ORTHRUS_API int orthrus_commit_kv(const orthrus_kv* kv, int num_layers, int64_t pool_layer_stride,
                      const void* k_blk, const void* v_blk, int64_t blk_layer_stride,
                      const int32_t* n_emit, int batch, int block_k, int32_t* seq_lens_out,
                      void* stream);

/*
 * Consensus at temperature T > 0.  The pages give the acceptance rule for
 * greedy decoding only (section 2.3 step 3) and state that the output
 * distribution is the AR model's (Hacker News thread, post #21); for T > 0
 * this library takes the standard speculative-sampling rule.  Every random
 * choice is an inverse-CDF draw with a caller-supplied uniform u in [0, 1):
 * the smallest token v whose cumulative weight exceeds u times the total
 * weight.  Probabilities, exponentials and cumulative weights are evaluated
 * in fp64 from the fp32 logits, so a draw agrees with an exact evaluation
 * except when u lies within about 1e-15 (relative) of a threshold.
 */

/* Bytes of device workspace for orthrus_sample (0 if invalid). */
ORTHRUS_API size_t orthrus_sample_workspace_bytes(int rows, int vocab);

/*
 * Temperature sampling (the drafted tokens at T > 0): out[r] = draw of
 * softmax(logits[r] / temperature) with uniform u[r].
 *  logits : fp32 [rows][vocab], finite
 *  u      : fp32 [rows], each in [0, 1)
 *  out    : int32 [rows] (written)
 * 0 <= rows <= 65535 (0 = no-op); 1 <= vocab <= 2^30; rows * ceil(vocab / 1024)
 * <= 2^30 (ORTHRUS_ERR_UNSUPPORTED_SHAPE beyond); temperature finite and > 0.
 * The workspace holds per-call results only; its contents need no
 * initialisation and are not read across calls.
 */
ORTHRUS_API int orthrus_sample(const float* logits, int rows, int vocab, float temperature, const float* u,
                   int32_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace for orthrus_accept_sampled (0 if invalid). */
ORTHRUS_API size_t orthrus_accept_sampled_workspace_bytes(int batch, int block_k, int vocab);

/*
 * Speculative-sampling consensus.  With q_i = softmax(logits_d[b][i] / T)
 * (draft view) and p_i = softmax(logits_a[b][i] / T) (AR view, the verify
 * pass), left to right: drafted token d_i is accepted when
 * u_acc[b][i] * q_i(d_i) < p_i(d_i); at the first row j that fails, the
 * emitted token is a draw of max(0, p_j - q_j) (normalised) with u_res[b][j]
 * and the step ends.  If every row passes, the K drafted tokens are emitted.
 * The emitted tokens follow the AR view's distribution whatever q is; as
 * T -> 0 this is orthrus_accept's greedy rule.
 *  logits_d, logits_a : fp32 [batch][block_k][vocab], finite
 *  draft              : int32 [batch][block_k], the drafted tokens
 *  u_acc, u_res       : fp32 [batch][block_k], each in [0, 1)
 *  tokens             : int32 [batch][block_k] (written) emitted tokens in
 *                       [0, n_emit), -1 after
 *  n_acc, n_emit, next_anchor : int32 [batch] (written), as in orthrus_accept
 * 1 <= block_k <= 64; 2 * batch * block_k <= 65535; 1 <= vocab <= 2^30;
 * 2 * batch * block_k * ceil(vocab / 1024) <= 2^30; temperature finite, > 0.
 * A drafted token outside [0, vocab) counts as probability 0 in both views
 * (always rejected).  The workspace needs no initialisation.
 */
ORTHRUS_API int orthrus_accept_sampled(const float* logits_d, const float* logits_a, const int32_t* draft,
                           int batch, int block_k, int vocab, float temperature, const float* u_acc,
                           const float* u_res, int32_t* tokens, int32_t* n_acc, int32_t* n_emit,
                           int32_t* next_anchor, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Keys and values of new rows in an e4m3 cache's format: for every element x
 * of KV head h,
 *   k_out = e4m3(fp32(x) / k_scale[h]),   v_out = e4m3(fp32(x) / v_scale[h])
 * with the fp32 division rounded to nearest even, then the nearest e4m3 value
 * (ties to the even code; magnitudes beyond 448 give +-448; a zero result
 * keeps x's sign).  The block's rows go through this before both attention
 * passes and the commit, exactly as a token's K/V are written to and read
 * back from the cache in plain decoding.
 *  k, v             : bf16 [rows][num_kv_heads][head_dim], finite
 *  k_scale, v_scale : fp32 [num_kv_heads], finite, > 0
 *  k_out, v_out     : uint8 [rows][num_kv_heads][head_dim] (written)
 * 0 <= rows (0 = no-op); head_dim a multiple of 16.
 */
ORTHRUS_API int orthrus_quantize_kv(const void* k, const void* v, const float* k_scale,
                        const float* v_scale, int rows, int num_kv_heads, int head_dim,
                        void* k_out, void* v_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ORTHRUS_H */

"""Orthrus draft/verify hot path on AMD MI355X (gfx950).

The compute lives in liborthrus.so (hand-written HIP kernels behind a C ABI,
include/orthrus.h); `binding` marshals torch tensors into it; `toy` and
`model` run Qwen3-style models (a small one, and one of Qwen3-8B's shape)
through the Orthrus loop and plain greedy decoding.
"""
from .binding import (ORTHRUS_KV_BF16, ORTHRUS_KV_FP8_E4M3, ORTHRUS_MAX_BLOCK,  # noqa: F401
                      ORTHRUS_PAGE_SIZE, OrthrusError, PagedKV, argmax_workspace, attn_workspace,
                      library_path, lmhead_workspace, load_library, orthrus_abi_version,
                      orthrus_accept, orthrus_argmax, orthrus_argmax_workspace_bytes,
                      orthrus_attn_draft, orthrus_attn_split_tokens, orthrus_attn_verify,
                      orthrus_attn_verify_noalloc,
                      orthrus_attn_workspace_bytes, orthrus_commit_kv, orthrus_last_error,
                      orthrus_lmhead_accept, orthrus_lmhead_argmax, orthrus_lmhead_workspace_bytes,
                      orthrus_quantize_kv, orthrus_status_string, orthrus_sample,
                      orthrus_sample_workspace_bytes, orthrus_accept_sampled,
                      orthrus_accept_sampled_workspace_bytes, orthrus_device_errors, device_errors,
                      DEVERR_SEQ_LEN, DEVERR_PAGE_ID, DEVERR_N_EMIT)

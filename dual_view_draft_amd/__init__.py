"""Orthrus draft/verify hot path on AMD MI355X (gfx950).

The compute lives in liborthrus.so (hand-written HIP kernels behind a C ABI,
include/orthrus.h); `binding` marshals torch tensors into it, and `toy` runs a
small Qwen3-style model through the Orthrus loop and plain greedy decoding.
"""
from .binding import (ORTHRUS_MAX_BLOCK, ORTHRUS_PAGE_SIZE, OrthrusError, PagedKV,  # noqa: F401
                      argmax_workspace, attn_workspace, library_path, lmhead_workspace,
                      load_library, orthrus_lmhead_accept, orthrus_lmhead_argmax,
                      orthrus_lmhead_workspace_bytes,
                      orthrus_abi_version, orthrus_accept, orthrus_argmax,
                      orthrus_argmax_workspace_bytes, orthrus_attn_draft,
                      orthrus_attn_split_tokens, orthrus_attn_verify,
                      orthrus_attn_workspace_bytes, orthrus_commit_kv, orthrus_last_error,
                      orthrus_status_string)

"""Python binding of liborthrus (the C ABI in include/orthrus.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream, every computation runs in the library's HIP kernels.  Each function
has the name of the C entry point it calls.  There is no fallback: if the
library is not built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liborthrus.so")
_lib = None

ORTHRUS_PAGE_SIZE = 16
ORTHRUS_MAX_BLOCK = 64
ORTHRUS_KV_BF16 = 0
ORTHRUS_KV_FP8_E4M3 = 1
_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)   # e4m3 codes, raw or typed


class OrthrusError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load_library()
        name = lib.orthrus_status_string(status).decode()
        detail = lib.orthrus_last_error().decode()
        super().__init__(f"{where}: {name} ({status}): {detail}")
        self.status = status


class orthrus_kv(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


EXPORTS = {
    # name: (restype, argtypes)
    "orthrus_abi_version": (ctypes.c_int, []),
    "orthrus_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "orthrus_last_error": (ctypes.c_char_p, []),
    "orthrus_device_errors": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "orthrus_attn_split_tokens": (ctypes.c_int, [ctypes.c_int] * 3),
    "orthrus_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 7),
    "orthrus_attn_draft": (ctypes.c_int, [ctypes.POINTER(orthrus_kv)] + [ctypes.c_void_p] * 4 +
                           [ctypes.c_int] * 3 + [ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "orthrus_attn_verify": None,  # same signature as orthrus_attn_draft
    "orthrus_attn_verify_noalloc": (ctypes.c_int, [ctypes.POINTER(orthrus_kv)] + [ctypes.c_void_p] * 4 +
                                    [ctypes.c_int] * 3 + [ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                          ctypes.c_void_p]),
    "orthrus_argmax_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 2),
    "orthrus_argmax": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "orthrus_accept": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 3 +
                       [ctypes.c_void_p] * 4 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "orthrus_lmhead_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 3),
    "orthrus_lmhead_argmax": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 3 +
                              [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                               ctypes.c_void_p]),
    "orthrus_lmhead_accept": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 +
                              [ctypes.c_void_p] * 4 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "orthrus_commit_kv": (ctypes.c_int, [ctypes.POINTER(orthrus_kv), ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]),
    "orthrus_quantize_kv": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3),
    "orthrus_sample_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 2),
    "orthrus_sample": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]),
    "orthrus_accept_sampled_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 3),
    "orthrus_accept_sampled": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_float] +
                               [ctypes.c_void_p] * 6 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
}
EXPORTS["orthrus_attn_verify"] = EXPORTS["orthrus_attn_draft"]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load liborthrus.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                               "(python -m dual_view_draft_amd.build)")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(rc: int, where: str):
    if rc != 0:
        raise OrthrusError(rc, where)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclasses.dataclass
class PagedKV:
    """One layer's view of the shared paged cache (tensors, device memory).

    k_pages, v_pages: [num_pages, Hkv, 16, D], bf16, or e4m3 codes (uint8 or
    float8_e4m3fn) with k_scale, v_scale fp32 [Hkv]; block_table: int32
    [B, max_pages]; seq_lens: int32 [B]."""
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None

    @property
    def is_fp8(self) -> bool:
        return self.k_pages.dtype in _FP8_DTYPES

    def c_struct(self) -> orthrus_kv:
        elem = self.k_pages.dtype if self.is_fp8 else torch.bfloat16
        for t, dt in ((self.v_pages, elem), (self.block_table, torch.int32), (self.seq_lens, torch.int32)):
            if t.dtype != dt:
                raise ValueError(f"expected {dt}, got {t.dtype}")
        if self.k_pages.dtype != elem:
            raise ValueError(f"k_pages must be bfloat16 or e4m3 codes, got {self.k_pages.dtype}")
        n, hkv, p, d = self.k_pages.shape
        if tuple(self.v_pages.shape) != (n, hkv, p, d):
            raise ValueError("k_pages and v_pages shapes differ")
        # the library rejects an e4m3 cache without scales where it reads
        # values (attention); the commit copies codes and needs none
        for t in (self.k_scale, self.v_scale):
            if t is not None and (t.dtype != torch.float32 or t.numel() != hkv):
                raise ValueError("k_scale and v_scale must be float32 with num_kv_heads entries")
        scales = (_ptr(self.k_scale), _ptr(self.v_scale)) if self.is_fp8 else (None, None)
        return orthrus_kv(_ptr(self.k_pages), _ptr(self.v_pages), _ptr(self.block_table),
                          _ptr(self.seq_lens), n, p, hkv, d, self.block_table.shape[1],
                          ORTHRUS_KV_FP8_E4M3 if self.is_fp8 else ORTHRUS_KV_BF16, *scales)

    @property
    def head_dim(self) -> int:
        return int(self.k_pages.shape[3])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pages.shape[1])


# ---------------------------------------------------------------------------
def orthrus_abi_version() -> int:
    return load_library().orthrus_abi_version()


def orthrus_status_string(status: int) -> str:
    return load_library().orthrus_status_string(status).decode()


def orthrus_last_error() -> str:
    return load_library().orthrus_last_error().decode()


def orthrus_attn_split_tokens(batch: int, num_kv_heads: int, max_ctx: int) -> int:
    return load_library().orthrus_attn_split_tokens(batch, num_kv_heads, max_ctx)


def orthrus_attn_workspace_bytes(batch, block_k, num_q_heads, num_kv_heads, head_dim, max_ctx,
                                 split_tokens=0) -> int:
    return load_library().orthrus_attn_workspace_bytes(batch, block_k, num_q_heads, num_kv_heads,
                                                       head_dim, max_ctx, split_tokens)


def attn_workspace(kv: PagedKV, q: torch.Tensor, max_ctx: int, split_tokens: int = 0) -> torch.Tensor:
    B, K, Hq, D = q.shape
    n = orthrus_attn_workspace_bytes(B, K, Hq, kv.num_kv_heads, D, max_ctx, split_tokens)
    if n == 0:
        raise ValueError("unsupported attention shape")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def _attention(fn_name, kv, q, k_blk, v_blk, out, max_ctx, scale, split_tokens, workspace, stream):
    B, K, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = attn_workspace(kv, q, max_ctx, split_tokens)
    kvs = kv.c_struct()
    rc = getattr(load_library(), fn_name)(
        ctypes.byref(kvs), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(out), B, K, Hq,
        float(scale), int(max_ctx), int(split_tokens), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, fn_name)
    return out


def orthrus_attn_draft(kv: PagedKV, q, k_blk, v_blk, out, *, max_ctx: int, scale=None,
                       split_tokens: int = 0, workspace=None, stream=None):
    """Draft pass (diffusion view): every block row sees the cache and the whole block."""
    return _attention("orthrus_attn_draft", kv, q, k_blk, v_blk, out, max_ctx, scale,
                      split_tokens, workspace, stream)


def orthrus_attn_verify(kv: PagedKV, q, k_blk, v_blk, out, *, max_ctx: int, scale=None,
                        split_tokens: int = 0, workspace=None, stream=None):
    """Verify pass (AR view): block row i sees the cache and block rows 0..i."""
    return _attention("orthrus_attn_verify", kv, q, k_blk, v_blk, out, max_ctx, scale,
                      split_tokens, workspace, stream)


def orthrus_attn_verify_noalloc(kv: PagedKV, q, k_blk, v_blk, out, *, max_ctx: int, scale=None,
                                split_tokens: int = 0, stream=None):
    """orthrus_attn_verify with the library's static scratch instead of a
    workspace (no device allocation)."""
    B, K, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kvs = kv.c_struct()
    rc = load_library().orthrus_attn_verify_noalloc(
        ctypes.byref(kvs), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(out), B, K, Hq, float(scale),
        int(max_ctx), int(split_tokens), _stream(stream))
    _check(rc, "orthrus_attn_verify_noalloc")
    return out


def orthrus_argmax_workspace_bytes(rows: int, vocab: int) -> int:
    return load_library().orthrus_argmax_workspace_bytes(rows, vocab)


def argmax_workspace(rows: int, vocab: int, device) -> torch.Tensor:
    return torch.empty(orthrus_argmax_workspace_bytes(rows, vocab), dtype=torch.uint8, device=device)


def orthrus_argmax(logits: torch.Tensor, out: torch.Tensor, *, workspace=None, stream=None):
    """out[r] = lowest index of the maximum of logits[r] (logits fp32 [..., V])."""
    if logits.dtype != torch.float32 or out.dtype != torch.int32:
        raise ValueError("logits must be float32 and out int32")
    V = logits.shape[-1]
    rows = logits.numel() // V
    if workspace is None:
        workspace = argmax_workspace(rows, V, logits.device)
    rc = load_library().orthrus_argmax(_ptr(logits), rows, V, _ptr(out), _ptr(workspace),
                                       workspace.numel(), _stream(stream))
    _check(rc, "orthrus_argmax")
    return out


def orthrus_accept(logits_a: torch.Tensor, draft: torch.Tensor, ar_tokens, n_acc, n_emit,
                   next_anchor, *, workspace=None, stream=None):
    """Consensus: AR argmax of logits_a [B,K,V] and the longest prefix where draft matches."""
    if logits_a.dtype != torch.float32:
        raise ValueError("logits_a must be float32")
    for t in (draft, ar_tokens, n_acc, n_emit, next_anchor):
        if t.dtype != torch.int32:
            raise ValueError("token and count tensors must be int32")
    B, K, V = logits_a.shape
    if workspace is None:
        workspace = argmax_workspace(B * K, V, logits_a.device)
    rc = load_library().orthrus_accept(_ptr(logits_a), _ptr(draft), B, K, V, _ptr(ar_tokens),
                                       _ptr(n_acc), _ptr(n_emit), _ptr(next_anchor),
                                       _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "orthrus_accept")


def orthrus_lmhead_workspace_bytes(rows: int, hidden: int, vocab: int) -> int:
    return load_library().orthrus_lmhead_workspace_bytes(rows, hidden, vocab)


def lmhead_workspace(rows: int, hidden: int, vocab: int, device) -> torch.Tensor:
    n = orthrus_lmhead_workspace_bytes(rows, hidden, vocab)
    if n == 0:
        raise ValueError("unsupported LM-head shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def orthrus_lmhead_argmax(hidden_states: torch.Tensor, weight: torch.Tensor, out: torch.Tensor, *,
                          logits=None, workspace=None, stream=None):
    """out[r] = greedy token of hidden_states[r] (bf16 [..., hidden]) under the LM head
    weight (bf16 [V, hidden]); logits (fp32 [rows, V]) optionally receives the logits."""
    if hidden_states.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise ValueError("hidden_states and weight must be bfloat16")
    if out.dtype != torch.int32 or (logits is not None and logits.dtype != torch.float32):
        raise ValueError("out must be int32 and logits float32")
    V, Hd = weight.shape
    rows = hidden_states.numel() // Hd
    if workspace is None:
        workspace = lmhead_workspace(rows, Hd, V, hidden_states.device)
    rc = load_library().orthrus_lmhead_argmax(_ptr(hidden_states), _ptr(weight), rows, Hd, V, _ptr(out),
                                              _ptr(logits) if logits is not None else None,
                                              _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "orthrus_lmhead_argmax")
    return out


def orthrus_lmhead_accept(hidden_states: torch.Tensor, weight: torch.Tensor, draft: torch.Tensor,
                          ar_tokens, n_acc, n_emit, next_anchor, *, workspace=None, stream=None):
    """Consensus from the verify pass's final hidden states [B, K, hidden] (bf16)."""
    if hidden_states.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise ValueError("hidden_states and weight must be bfloat16")
    for t in (draft, ar_tokens, n_acc, n_emit, next_anchor):
        if t.dtype != torch.int32:
            raise ValueError("token and count tensors must be int32")
    B, K, Hd = hidden_states.shape
    V = weight.shape[0]
    if workspace is None:
        workspace = lmhead_workspace(B * K, Hd, V, hidden_states.device)
    rc = load_library().orthrus_lmhead_accept(_ptr(hidden_states), _ptr(weight), _ptr(draft), B, K, Hd, V,
                                              _ptr(ar_tokens), _ptr(n_acc), _ptr(n_emit), _ptr(next_anchor),
                                              _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "orthrus_lmhead_accept")


def orthrus_commit_kv(kv_layer0: PagedKV, k_blk: torch.Tensor, v_blk: torch.Tensor,
                      n_emit: torch.Tensor, seq_lens_out: torch.Tensor, *,
                      pool_layer_stride: int = 0, stream=None):
    """Append the accepted rows' K/V (k_blk, v_blk: [layers,B,K,Hkv,D] in the
    cache's element type) to the cache.

    kv_layer0 describes layer 0's pools; layer l's pools start pool_layer_stride
    elements later (pass the stride of a [layers, num_pages, Hkv, 16, D] pool)."""
    layers, B, K = k_blk.shape[:3]
    kvs = kv_layer0.c_struct()
    blk_stride = k_blk.stride(0) if layers > 1 else 0
    rc = load_library().orthrus_commit_kv(ctypes.byref(kvs), layers, int(pool_layer_stride),
                                          _ptr(k_blk), _ptr(v_blk), int(blk_stride), _ptr(n_emit),
                                          B, K, _ptr(seq_lens_out), _stream(stream))
    _check(rc, "orthrus_commit_kv")


def orthrus_quantize_kv(k: torch.Tensor, v: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                        k_out: torch.Tensor, v_out: torch.Tensor, *, stream=None):
    """e4m3 codes of bf16 K and V rows [..., Hkv, D] with per-head fp32 scales
    (k_out, v_out: uint8 or float8_e4m3fn of the same shape)."""
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("k and v must be bfloat16")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32:
        raise ValueError("scales must be float32")
    if k_out.dtype not in _FP8_DTYPES or v_out.dtype not in _FP8_DTYPES:
        raise ValueError("k_out and v_out must be uint8 or float8_e4m3fn")
    if k.shape != v.shape or k_out.shape != k.shape or v_out.shape != k.shape:
        raise ValueError("k, v, k_out and v_out must have one shape")
    Hkv, D = k.shape[-2], k.shape[-1]
    if k_scale.numel() != Hkv or v_scale.numel() != Hkv:
        raise ValueError("one scale per KV head")
    rows = k.numel() // (Hkv * D)
    rc = load_library().orthrus_quantize_kv(_ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), rows, Hkv, D,
                                            _ptr(k_out), _ptr(v_out), _stream(stream))
    _check(rc, "orthrus_quantize_kv")


def orthrus_sample_workspace_bytes(rows: int, vocab: int) -> int:
    return load_library().orthrus_sample_workspace_bytes(rows, vocab)


def orthrus_sample(logits: torch.Tensor, temperature: float, u: torch.Tensor, out: torch.Tensor, *,
                   workspace=None, stream=None):
    """out[r] = inverse-CDF draw of softmax(logits[r] / temperature) with uniform u[r]
    (logits fp32 [..., V]; u fp32 and out int32 with one entry per row)."""
    if logits.dtype != torch.float32 or u.dtype != torch.float32 or out.dtype != torch.int32:
        raise ValueError("logits and u must be float32, out int32")
    V = logits.shape[-1]
    rows = logits.numel() // V
    if u.numel() != rows or out.numel() != rows:
        raise ValueError("one uniform and one output per row")
    if workspace is None:
        workspace = torch.empty(orthrus_sample_workspace_bytes(rows, V), dtype=torch.uint8, device=logits.device)
    rc = load_library().orthrus_sample(_ptr(logits), rows, V, float(temperature), _ptr(u), _ptr(out),
                                       _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "orthrus_sample")
    return out


def orthrus_accept_sampled_workspace_bytes(batch: int, block_k: int, vocab: int) -> int:
    return load_library().orthrus_accept_sampled_workspace_bytes(batch, block_k, vocab)


def orthrus_accept_sampled(logits_d: torch.Tensor, logits_a: torch.Tensor, draft: torch.Tensor,
                           temperature: float, u_acc: torch.Tensor, u_res: torch.Tensor, tokens, n_acc, n_emit,
                           next_anchor, *, workspace=None, stream=None):
    """Speculative-sampling consensus of the draft and AR views' logits [B, K, V] (fp32)."""
    if logits_d.dtype != torch.float32 or logits_a.dtype != torch.float32:
        raise ValueError("logits must be float32")
    if u_acc.dtype != torch.float32 or u_res.dtype != torch.float32:
        raise ValueError("uniforms must be float32")
    for t in (draft, tokens, n_acc, n_emit, next_anchor):
        if t.dtype != torch.int32:
            raise ValueError("token and count tensors must be int32")
    B, K, V = logits_a.shape
    if tuple(logits_d.shape) != (B, K, V):
        raise ValueError("logits_d and logits_a shapes differ")
    if workspace is None:
        n = orthrus_accept_sampled_workspace_bytes(B, K, V)
        if n == 0:
            raise ValueError("unsupported consensus shape")
        workspace = torch.empty(n, dtype=torch.uint8, device=logits_a.device)
    rc = load_library().orthrus_accept_sampled(_ptr(logits_d), _ptr(logits_a), _ptr(draft), B, K, V,
                                               float(temperature), _ptr(u_acc), _ptr(u_res), _ptr(tokens),
                                               _ptr(n_acc), _ptr(n_emit), _ptr(next_anchor), _ptr(workspace),
                                               workspace.numel(), _stream(stream))
    _check(rc, "orthrus_accept_sampled")


DEVERR_SEQ_LEN, DEVERR_PAGE_ID, DEVERR_N_EMIT = 1, 2, 4


def orthrus_device_errors(out: torch.Tensor, *, clear: bool = True, stream=None) -> torch.Tensor:
    """Copy the GPU's device error word (ORTHRUS_DEVERR_* bits) into `out`
    (int32 or uint32-sized, one element, on the device), in stream order, and
    reset it if `clear`."""
    if out.numel() != 1 or out.element_size() != 4:
        raise ValueError("out must hold one 32-bit element")
    rc = load_library().orthrus_device_errors(_ptr(out), 1 if clear else 0, _stream(stream))
    _check(rc, "orthrus_device_errors")
    return out


def device_errors(clear: bool = True) -> int:
    """The current device's error word (synchronises the current stream)."""
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    orthrus_device_errors(out, clear=clear, stream=torch.cuda.current_stream())
    return int(out.item())

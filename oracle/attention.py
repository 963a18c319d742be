"""Oracle: dual-view block attention over one shared paged KV cache (fp64).

TEST INFRASTRUCTURE ONLY - see the package docstring.

What is computed.  Both views of Orthrus attend to the same KV cache, which the
frozen AR view built [gist §2.1; abstract; HN #21].  A decode step processes a
block of K rows at positions L .. L+K-1 of a sequence whose cache holds
positions 0 .. L-1:

* draft pass (diffusion view): every block row sees the whole cached context
  and, bidirectionally, every row of its own block [gist §2.2, the M_diff block
  mask: causal to the clean context before the block anchor, bidirectional
  inside the block].  At inference the whole cache precedes the anchor, so no
  key is masked at all.
* verify pass (AR view): the filled block is run through the frozen AR
  attention, which is causal: block row i sees the cache and block rows
  0 .. i [gist §2.3 step 2; HN #21 "second pass"].

For query head h the KV head is floor(h / G), G = Hq / Hkv (grouped-query
attention with contiguous groups); the score scale is 1/sqrt(D).  The block
rows' own keys and values are inputs (k_blk, v_blk); the draft pass's block
K/V are never written to the cache.

Pinned by (tests/test_oracle_attention.py): a pure-Python brute force with
math.exp on tiny inputs; torch scaled_dot_product_attention in fp64 on the
CPU with an explicit boolean mask; K = 1 (both masks reduce to single-token
decode attention); L = 0 (plain bidirectional / plain causal attention);
constant V; a dominant needle key; page-table permutation invariance;
softmax weights summing to one; draft == verify exactly on the last block row.
"""
from __future__ import annotations

import numpy as np

MODES = ("draft", "verify")


def from_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of
    an IEEE float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def gather_context(k_pages, v_pages, block_table, b: int, L: int, page_size: int):
    """Walk sequence b's block table and return its cached keys and values,
    [L, Hkv, D] each, in position order.  Position p lives in page
    block_table[b, p // page_size] at slot p % page_size; pages are laid out
    [num_pages, Hkv, page_size, D]."""
    Hkv, D = k_pages.shape[1], k_pages.shape[3]
    kc = np.zeros((L, Hkv, D), dtype=np.float64)
    vc = np.zeros((L, Hkv, D), dtype=np.float64)
    for p in range(L):
        page = int(block_table[b, p // page_size])
        slot = p % page_size
        kc[p] = k_pages[page, :, slot, :]
        vc[p] = v_pages[page, :, slot, :]
    return kc, vc


def _visible(mode: str, L: int, K: int) -> np.ndarray:
    """[K, L+K] boolean: may block row i attend key j (j < L: cached
    position j; j >= L: block row j - L)."""
    vis = np.ones((K, L + K), dtype=bool)
    if mode == "verify":
        for i in range(K):
            vis[i, L + i + 1:] = False
    elif mode != "draft":
        raise ValueError(f"mode must be one of {MODES}")
    return vis


def attention_weights(q, k_blk, v_blk, k_pages, v_pages, block_table, seq_lens,
                      mode: str, b: int, h: int, scale: float | None = None,
                      page_size: int = 16):
    """Softmax weights [K, L_b+K] of query head h of sequence b (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    B, K, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    g = h // (Hq // Hkv)
    L = int(seq_lens[b])
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    kc, _ = gather_context(k_pages, v_pages, block_table, b, L, page_size)
    keys = np.concatenate([kc[:, g], np.asarray(k_blk, np.float64)[b, :, g]], axis=0)
    s = (q[b, :, h] @ keys.T) * scale
    s = np.where(_visible(mode, L, K), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return w / w.sum(axis=1, keepdims=True)


def block_attention(q, k_blk, v_blk, k_pages, v_pages, block_table, seq_lens,
                    mode: str, scale: float | None = None, page_size: int = 16):
    """Attention output [B, K, Hq, D] in fp64 for one layer.

    q [B,K,Hq,D]; k_blk, v_blk [B,K,Hkv,D]; k_pages, v_pages
    [num_pages,Hkv,page_size,D]; block_table [B, max_pages]; seq_lens [B].
    Inputs may be any float dtype (bf16 data should first go through
    from_bf16); everything is computed in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    k_pages = np.asarray(k_pages, dtype=np.float64)
    v_pages = np.asarray(v_pages, dtype=np.float64)
    B, K, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.zeros((B, K, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        kc, vc = gather_context(k_pages, v_pages, block_table, b, L, page_size)
        vis = _visible(mode, L, K)
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([kc[:, g], k_blk[b, :, g]], axis=0)   # [L+K, D]
            vals = np.concatenate([vc[:, g], v_blk[b, :, g]], axis=0)   # [L+K, D]
            s = (q[b, :, h] @ keys.T) * scale                          # [K, L+K]
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w = w / w.sum(axis=1, keepdims=True)
            out[b, :, h] = w @ vals
    return out

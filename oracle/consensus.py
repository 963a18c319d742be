"""Oracle: consensus (argmax + longest matching prefix) and cache commit.

TEST INFRASTRUCTURE ONLY - see the package docstring.

What is computed [gist §2.3 steps 1 and 3; HN #21]:

* The diffusion view drafts K candidate tokens in one pass; the AR view's
  greedy prediction at every block position comes from the same verify pass.
  Both are vocabulary argmaxes (ties go to the lowest index; -0.0 equals +0.0).
* Acceptance runs strictly left to right: a drafted token is kept only while
  it equals the AR view's greedy token.  At the first mismatch, index j, the
  matched prefix 0 .. j-1 is kept, the AR view's own token at j is appended as
  the correction, and the cache is cut back to that point.

Reading used here (the pages leave the exact indexing open).  Draft row i
and verify row i both predict position L+i+1; the verify block is
[anchor, d_0, ..., d_{K-2}].  With n_acc the length of the matched prefix,
n_emit = n_acc + 1 if n_acc < K else K, the emitted tokens are a[0 : n_emit],
the next anchor is a[n_emit - 1], and the committed cache rows are the verify
pass's (AR view's) K/V of block rows 0 .. n_emit-1, written at positions
L .. L+n_emit-1.  Nothing else in the pool changes.

Pinned by (tests/test_oracle_consensus.py): brute-force argmax loops, planted
maxima and planted ties; hand-worked acceptance cases in tests/golden/; the
K = 1 case (every step emits exactly the AR token: greedy decoding); commit
checked by gathering back through the block table and by sentinel slots.
"""
from __future__ import annotations

import numpy as np


def argmax_rows(logits) -> np.ndarray:
    """Index of the maximum of every row of logits[..., V]; the lowest index
    wins among equal values.  Values are compared exactly as given (float32
    logits are compared in float32); -0.0 and +0.0 compare equal."""
    x = np.asarray(logits)
    m = x.max(axis=-1, keepdims=True)
    hit = x == m
    return hit.argmax(axis=-1).astype(np.int32)   # first True along the row


def accept(d, a):
    """Longest matching prefix per sequence.

    d, a: [B, K] draft tokens and AR greedy tokens.  Returns
    (n_acc, n_emit, next_anchor), each [B] int32.
    """
    d = np.asarray(d)
    a = np.asarray(a)
    B, K = a.shape
    n_acc = np.zeros(B, np.int32)
    n_emit = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        j = 0
        while j < K and int(d[b, j]) == int(a[b, j]):
            j += 1
        n_acc[b] = j
        n_emit[b] = j + 1 if j < K else K
        nxt[b] = a[b, n_emit[b] - 1]
    return n_acc, n_emit, nxt


def commit_kv(k_pages, v_pages, block_table, seq_lens, k_blk, v_blk, n_emit,
              page_size: int = 16):
    """Append the accepted rows' K/V to the cache.

    k_pages, v_pages: [layers, num_pages, Hkv, page_size, D] (any dtype; bit
    patterns are copied unchanged).  k_blk, v_blk: [layers, B, K, Hkv, D], the
    verify pass's block K/V.  Returns (new_k_pages, new_v_pages, seq_lens_out);
    the inputs are not modified.
    """
    k_new = np.array(k_pages, copy=True)
    v_new = np.array(v_pages, copy=True)
    layers = k_new.shape[0]
    B = len(seq_lens)
    out_lens = np.zeros(B, np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        for r in range(int(n_emit[b])):
            p = L + r
            page = int(block_table[b, p // page_size])
            slot = p % page_size
            for layer in range(layers):
                k_new[layer, page, :, slot, :] = k_blk[layer, b, r]
                v_new[layer, page, :, slot, :] = v_blk[layer, b, r]
        out_lens[b] = L + int(n_emit[b])
    return k_new, v_new, out_lens

"""Oracle: LM-head projection and vocabulary argmax (greedy token) per row.

TEST INFRASTRUCTURE ONLY - see the package docstring.

What is computed.  Both views end in the frozen model's shared LM head: the
diffusion view's draft tokens and the AR view's greedy tokens are the argmax
over the vocabulary of the LM-head logits of each block row [gist §2.3 steps
1 and 3].  The diffusion module adds only its own attention projections and
shares everything else with the AR model, the LM head included [HN #26].
For the final hidden state h_r of row r (after the final norm) and the LM-head
weight W [V, hidden]:

    logits[r, v] = sum_k h_r[k] * W[v, k]
    token[r]     = the smallest v with logits[r, v] = max_v logits[r, v]

Here h and W are bf16 bit patterns widened exactly to fp64; every product of
two bf16 values is exact in fp64, and the sum is taken by numpy's matrix
product in fp64.

Pinned by (tests/test_oracle_lmhead.py): exactly rounded sums (math.fsum) of
the products on small cases; a planted row of W that makes a known token win
by a wide margin; permutation of the vocabulary; invariance of the argmax
under positive scaling of h; duplicated maximal rows (lowest index wins).
"""
from __future__ import annotations

import numpy as np

from .attention import from_bf16


def lm_logits(hidden_bits, weight_bits) -> np.ndarray:
    """fp64 logits [R, V] = h [R, hidden] . W[V, hidden]^T from bf16 bits."""
    h = from_bf16(hidden_bits)
    w = from_bf16(weight_bits)
    return h @ w.T


def lm_argmax(hidden_bits, weight_bits) -> np.ndarray:
    """Greedy token of every row: first index of the row maximum of the fp64
    logits (int32 [R])."""
    x = lm_logits(hidden_bits, weight_bits)
    m = x.max(axis=-1, keepdims=True)
    return (x == m).argmax(axis=-1).astype(np.int32)

"""Oracle: Orthrus consensus at temperature > 0 (TEST INFRASTRUCTURE ONLY).

The pages state that Orthrus keeps the output distribution of the AR model
[HN #21, "identical output distribution"; abstract, lossless consensus] and
report speedups at several sampling temperatures [gist §4], but they give the
acceptance rule only for greedy decoding (keep the longest prefix of drafted
tokens that equal the AR view's greedy tokens, then append the AR token
[gist §2.3 step 3]).  For temperature T > 0 this oracle takes the standard
speculative-sampling rule (Leviathan, Kalman, Matias, "Fast Inference from
Transformers via Speculative Decoding", 2023; Chen et al., "Accelerating
Large Language Model Decoding with Speculative Sampling", 2023) as a stated
reading:

* the draft view's distribution of row i is q_i = softmax(z_d[i] / T) and the
  drafted token d_i is a sample of q_i (rows are drawn independently, as the
  diffusion view proposes all K tokens in one pass);
* the AR view's distribution of row i is p_i = softmax(z_a[i] / T), computed
  by the verify pass on the block [anchor, d_0 .. d_{K-2}];
* left to right, d_i is accepted when u_acc[i] * q_i(d_i) < p_i(d_i) (that is
  u < min(1, p/q) for a uniform u in [0, 1)); at the first rejection the
  emitted token is a sample of the residual distribution
  max(0, p_i - q_i) / sum(max(0, p_i - q_i)) drawn with u_res[i], and the step
  ends.  If all K are accepted, the K drafted tokens are emitted (no bonus
  token, the same reading as the greedy rule's: the verify block holds K rows).
  As T -> 0 every distribution becomes one-hot and the rule is the greedy one.

Every sample is an inverse-CDF draw with one uniform u in [0, 1) per draw:
the token is the smallest v whose cumulative weight exceeds u times the total
weight.  The uniforms are inputs (the caller's random numbers), so a GPU
implementation can be compared draw for draw.

Pinned by (tests/test_oracle_sampling.py): hand-worked inverse-CDF draws and
the u = 0 edge; the T -> 0 limit equals the greedy oracle (accept) exactly;
a draft equal to the AR distribution is always accepted; and the emitted
token's distribution, integrated over a uniform grid of every random input,
equals the AR view's p_i at the first row and, after an acceptance, at the
next row (the property that makes the method lossless).
"""
from __future__ import annotations

import numpy as np


def softmax_t(z, T: float) -> np.ndarray:
    """softmax(z / T) over the last axis in fp64 (T > 0)."""
    z = np.asarray(z, dtype=np.float64)
    if not T > 0:
        raise ValueError("temperature must be > 0")
    s = (z - z.max(axis=-1, keepdims=True)) / T
    w = np.exp(s)
    return w / w.sum(axis=-1, keepdims=True)


def inverse_cdf(weights, u: float) -> int:
    """Smallest v with cumsum(weights)[v] > u * sum(weights); weights >= 0,
    not all zero, u in [0, 1)."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    target = u * c[-1]
    v = int(np.searchsorted(c, target, side="right"))
    return min(v, int(np.flatnonzero(w > 0)[-1]))


def sample_rows(logits, T: float, u) -> np.ndarray:
    """One inverse-CDF sample of softmax(logits[r] / T) per row with uniform u[r]."""
    z = np.asarray(logits, dtype=np.float64)
    V = z.shape[-1]
    rows = z.reshape(-1, V)
    uu = np.asarray(u, dtype=np.float64).reshape(-1)
    out = np.empty(rows.shape[0], dtype=np.int32)
    for r in range(rows.shape[0]):
        out[r] = inverse_cdf(softmax_t(rows[r], T), float(uu[r]))
    return out.reshape(z.shape[:-1])


def speculative_accept(logits_d, logits_a, d, T: float, u_acc, u_res):
    """Consensus at temperature T for a batch.

    logits_d, logits_a: [B, K, V] (draft view, AR view); d: int [B, K] drafted
    tokens; u_acc, u_res: [B, K] uniforms in [0, 1).  Returns (tokens [B, K]
    int32, n_acc [B], n_emit [B], next_anchor [B]); tokens[b, :n_emit[b]] are
    the emitted tokens (entries past n_emit are -1)."""
    zd = np.asarray(logits_d, dtype=np.float64)
    za = np.asarray(logits_a, dtype=np.float64)
    d = np.asarray(d)
    B, K, V = za.shape
    tokens = np.full((B, K), -1, dtype=np.int32)
    n_acc = np.zeros(B, np.int32)
    n_emit = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        j = K
        for i in range(K):
            p = softmax_t(za[b, i], T)
            q = softmax_t(zd[b, i], T)
            t = int(d[b, i])
            if float(u_acc[b, i]) * q[t] < p[t]:
                tokens[b, i] = t
                continue
            r = np.maximum(p - q, 0.0)
            if not r.sum() > 0:          # p == q: a rejection cannot happen; kept total
                r = p
            tokens[b, i] = inverse_cdf(r, float(u_res[b, i]))
            j = i
            break
        n_acc[b] = j
        n_emit[b] = j + 1 if j < K else K
        nxt[b] = tokens[b, n_emit[b] - 1]
    return tokens, n_acc, n_emit, nxt

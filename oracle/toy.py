"""Oracle: a tiny fp64 Qwen3-style decoder with a diffusion view, the Orthrus
decode loop and plain greedy decoding.

TEST INFRASTRUCTURE ONLY - see the package docstring.

Model [gist §2.1; HN #21 and the parameter discussion in post #26 of the same
thread]: a frozen AR Transformer (RMSNorm, q/k/v/o projections with per-head
QK RMSNorm and rotary embeddings, SwiGLU FFN, untied LM head) plus, in every
layer, a diffusion attention module with its own q/k/v/o projections.  The two
views share embeddings, norms, FFN, LM head and - the point of the method -
the single KV cache, which only the AR view writes.  The <mask> token is one
extra embedding row.

Loop [gist §2.3]: prefill the prompt with the AR view; the last prompt row's
greedy token is the first anchor.  Each step drafts K tokens in one diffusion
forward over [anchor, <mask> x (K-1)] (draft mask), verifies the filled block
[anchor, d_0 .. d_{K-2}] in one AR forward (causal mask), accepts the longest
matching prefix plus the AR correction, and commits the AR K/V of the emitted
rows.  Greedy decoding is the same AR forward with a block of one row.  The
pages state that the output equals the base model's greedy output exactly
[gist §2.3 step 3, §3; HN thread title]; tests/test_oracle_toy.py checks that
invariant with three drafters.

Every linear layer is evaluated row by row, so a row's result never depends
on how many rows share the forward pass.
"""
from __future__ import annotations

import numpy as np

from .attention import block_attention, from_bf16
from .consensus import accept, argmax_rows, commit_kv


class ToyModel:
    def __init__(self, cfg, weight_bits: dict, page_size: int = 16):
        self.cfg = cfg
        self.w = {k: from_bf16(v) for k, v in weight_bits.items()}
        self.P = page_size
        half = cfg.D // 2
        self.inv_freq = cfg.rope_base ** (-np.arange(half, dtype=np.float64) * 2.0 / cfg.D)

    # ---- building blocks -------------------------------------------------
    @staticmethod
    def linear(x, w):
        return np.stack([x[i] @ w for i in range(x.shape[0])])

    def rmsnorm(self, x, w):
        ms = np.mean(x * x, axis=-1, keepdims=True)
        return x / np.sqrt(ms + self.cfg.rms_eps) * w

    def rope(self, x, positions):
        """x [n, heads, D]; rotate-half rotary embedding at absolute positions."""
        ang = positions[:, None].astype(np.float64) * self.inv_freq[None, :]   # [n, D/2]
        cos = np.cos(ang)[:, None, :]
        sin = np.sin(ang)[:, None, :]
        half = self.cfg.D // 2
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)

    # ---- cache -------------------------------------------------------------
    def new_cache(self, capacity: int, seed: int = 0):
        c = self.cfg
        n_pages = -(-capacity // self.P)
        perm = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
        shape = (c.layers, n_pages, c.Hkv, self.P, c.D)
        return {"k": np.zeros(shape), "v": np.zeros(shape),
                "table": perm[None, :], "L": 0}

    # ---- one forward over a block of rows ---------------------------------
    def forward(self, tokens, cache, view: str, mode: str):
        """Run the block `tokens` (positions L .. L+n-1) through the model.

        view "ar" uses the frozen projections; view "diff" the diffusion
        module's.  mode is the attention mask ("draft" or "verify").  Returns
        (logits [n, V], k_rows [layers, n, Hkv, D], v_rows [layers, n, Hkv, D]).
        """
        c = self.cfg
        n = len(tokens)
        L = cache["L"]
        pos = np.arange(L, L + n)
        x = self.w["embed"][np.asarray(tokens)]
        sfx = "" if view == "ar" else "_diff"
        ks, vs = [], []
        for i in range(c.layers):
            p = f"l{i}."
            h = self.rmsnorm(x, self.w[p + "attn_norm"])
            q = self.linear(h, self.w[p + "wq" + sfx]).reshape(n, c.Hq, c.D)
            k = self.linear(h, self.w[p + "wk" + sfx]).reshape(n, c.Hkv, c.D)
            v = self.linear(h, self.w[p + "wv" + sfx]).reshape(n, c.Hkv, c.D)
            q = self.rope(self.rmsnorm(q, self.w[p + "q_norm"]), pos)
            k = self.rope(self.rmsnorm(k, self.w[p + "k_norm"]), pos)
            o = block_attention(q[None], k[None], v[None], cache["k"][i], cache["v"][i],
                                cache["table"], np.array([L]), mode, page_size=self.P)[0]
            x = x + self.linear(o.reshape(n, c.Hq * c.D), self.w[p + "wo" + sfx])
            h = self.rmsnorm(x, self.w[p + "ffn_norm"])
            gate = self.linear(h, self.w[p + "w_gate"])
            up = self.linear(h, self.w[p + "w_up"])
            x = x + self.linear(gate / (1.0 + np.exp(-gate)) * up, self.w[p + "w_down"])
            ks.append(k)
            vs.append(v)
        logits = self.linear(self.rmsnorm(x, self.w["final_norm"]), self.w["lm_head"])
        return logits, np.stack(ks), np.stack(vs)

    def commit(self, cache, k_rows, v_rows, n_emit: int):
        kn, vn, lens = commit_kv(cache["k"], cache["v"], cache["table"], np.array([cache["L"]]),
                                 k_rows[:, None], v_rows[:, None], np.array([n_emit]),
                                 page_size=self.P)
        cache["k"], cache["v"], cache["L"] = kn, vn, int(lens[0])

    def prefill(self, prompt, cache):
        """AR view over the whole prompt (causal); returns the first token."""
        logits, k, v = self.forward(prompt, cache, "ar", "verify")
        self.commit(cache, k, v, len(prompt))
        return int(argmax_rows(logits[-1:])[0])


# ---- drafters ----------------------------------------------------------------

class DiffusionDrafter:
    """The model's own diffusion view over [anchor, <mask> x (K-1)]."""

    def __call__(self, model, cache, anchor, emitted, K):
        block = [anchor] + [model.cfg.mask_id] * (K - 1)
        logits, _, _ = model.forward(block, cache, "diff", "draft")
        return argmax_rows(logits)


class TeacherDrafter:
    """Proposes the known greedy continuation, corrupted at a geometric position,
    so that every accepted length 0..K occurs."""

    def __init__(self, reference, p: float, seed: int, vocab: int):
        self.ref = list(reference)
        self.rng = np.random.default_rng(seed)
        self.p, self.V = p, vocab

    def __call__(self, model, cache, anchor, emitted, K):
        e = len(emitted)
        d = np.array([self.ref[e + i] for i in range(K)], dtype=np.int32)
        m = min(int(self.rng.geometric(self.p)) - 1, K)
        if m < K:
            d[m] = (d[m] + 1) % self.V
        return d


class WrongDrafter:
    """Every drafted token is wrong, so each step emits exactly one token."""

    def __init__(self, reference, vocab: int):
        self.ref, self.V = list(reference), vocab

    def __call__(self, model, cache, anchor, emitted, K):
        e = len(emitted)
        return np.array([(self.ref[e + i] + 1) % self.V for i in range(K)], dtype=np.int32)


# ---- loops -------------------------------------------------------------------

def greedy_generate(model: ToyModel, prompt, n: int):
    cache = model.new_cache(len(prompt) + n + 1)
    out = [model.prefill(prompt, cache)]
    while len(out) < n:
        logits, k, v = model.forward([out[-1]], cache, "ar", "verify")
        model.commit(cache, k, v, 1)
        out.append(int(argmax_rows(logits)[0]))
    return out


def orthrus_generate(model: ToyModel, prompt, n: int, K: int, drafter):
    """Returns (tokens[:n], list of n_emit per step)."""
    cache = model.new_cache(len(prompt) + n + 2 * K)
    out = [model.prefill(prompt, cache)]
    anchor = out[0]
    emits = []
    while len(out) < n:
        d = np.asarray(drafter(model, cache, anchor, out, K), dtype=np.int32)
        block = [anchor] + [int(t) for t in d[:K - 1]]
        logits, k, v = model.forward(block, cache, "ar", "verify")
        a = argmax_rows(logits)
        n_acc, n_emit, nxt = accept(d[None], a[None])
        e = int(n_emit[0])
        model.commit(cache, k, v, e)
        out.extend(int(t) for t in a[:e])
        anchor = int(nxt[0])
        emits.append(e)
    return out[:n], emits

"""A small Qwen3-style decoder with a diffusion view, decoded on the GPU with
the Orthrus loop and with plain greedy decoding.

The model follows the dual-view construction (gist.science technical summary
of "Orthrus: Memory-Efficient Parallel Token Generation via Dual-View
Diffusion", section 2.1; Hacker News thread "Orthrus-Qwen3: up to 7.8x
tokens/forward ...", posts #21 and #26): a frozen AR decoder (RMSNorm,
q/k/v/o projections with per-head QK RMSNorm and rotary embeddings, SwiGLU
FFN, untied LM head) plus a diffusion attention module (its own q/k/v/o
projections) in every layer.  Both views read one paged KV cache that only
the AR view writes; the <mask> token is one extra embedding row.

Every step of the decode hot path runs in liborthrus: block attention (draft
and verify masks), vocabulary argmax, acceptance and the multi-layer KV
commit.  The dense layers around it (norms, projections, FFN, LM head) are
plain torch float64 matrix products evaluated at a fixed shape of 64 rows, so
a row's result never depends on how many real rows a call has; combined with
the attention kernel's fixed absolute-position split grid this makes the
Orthrus loop reproduce greedy decoding bit for bit.
"""
from __future__ import annotations

import dataclasses
import time

import numpy as np
import torch

from . import binding as ob

PAD_ROWS = 64          # every dense layer runs on exactly this many rows
PAGE = ob.ORTHRUS_PAGE_SIZE


def _dev_bf16_bits_to_f64(bits: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch.bfloat16).to(torch.float64)


@dataclasses.dataclass
class DecodeStats:
    tokens: list
    steps: int
    emitted_per_step: list
    seconds: float

    @property
    def mean_accepted(self) -> float:
        return float(np.mean(self.emitted_per_step)) if self.emitted_per_step else 0.0

    @property
    def tokens_per_s(self) -> float:
        return len(self.tokens) / self.seconds if self.seconds > 0 else 0.0


class PagedCache:
    """All layers' pools [layers, pages, Hkv, 16, D] (bf16) plus one sequence's
    block table (a seeded permutation of the pool) and two length buffers that
    alternate as input and output of the commit."""

    def __init__(self, cfg, capacity: int, device, seed: int = 0):
        n_pages = -(-capacity // PAGE)
        shape = (cfg.layers, n_pages, cfg.Hkv, PAGE, cfg.D)
        self.k = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.v = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        perm = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
        self.table = torch.from_numpy(perm[None, :]).to(device)
        self.lens = [torch.zeros(1, dtype=torch.int32, device=device),
                     torch.zeros(1, dtype=torch.int32, device=device)]
        self.cur = 0
        self.L = 0                                  # host copy of the cached length
        self.capacity = n_pages * PAGE

    def layer(self, i: int) -> ob.PagedKV:
        return ob.PagedKV(self.k[i], self.v[i], self.table, self.lens[self.cur])

    def commit(self, k_rows, v_rows, n_emit: torch.Tensor, n_emit_host: int):
        """k_rows, v_rows: bf16 [layers, 1, K, Hkv, D] of the AR view."""
        out = self.lens[1 - self.cur]
        ob.orthrus_commit_kv(self.layer(0), k_rows, v_rows, n_emit, out,
                             pool_layer_stride=self.k.stride(0))
        self.cur = 1 - self.cur
        self.L += n_emit_host


class ToyOrthrus:
    def __init__(self, cfg, weight_bits: dict, device="cuda", max_block: int = 32):
        self.cfg = cfg
        self.device = torch.device(device)
        self.w = {k: _dev_bf16_bits_to_f64(v, self.device) for k, v in weight_bits.items()}
        half = cfg.D // 2
        self.inv_freq = cfg.rope_base ** (-torch.arange(half, dtype=torch.float64, device=self.device)
                                          * 2.0 / cfg.D)
        self.max_block = max_block
        self.ws = None

    # ---- dense building blocks (fixed 64-row shape) ------------------------
    def _lin(self, x, w):
        n = x.shape[0]
        xp = torch.zeros((PAD_ROWS, x.shape[1]), dtype=x.dtype, device=x.device)
        xp[:n] = x
        return (xp @ w)[:n]

    def _rms(self, x, w):
        return x * torch.rsqrt(torch.mean(x * x, dim=-1, keepdim=True) + self.cfg.rms_eps) * w

    def _rope(self, x, pos):
        ang = pos[:, None].to(torch.float64) * self.inv_freq[None, :]
        cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        h = self.cfg.D // 2
        x1, x2 = x[..., :h], x[..., h:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)

    def _workspace(self, cache: PagedCache, n: int):
        # one max_ctx for every call on this cache: the attention's split grid
        # depends on it, and greedy and Orthrus decoding must share that grid
        max_ctx = cache.capacity - PAD_ROWS
        need = ob.orthrus_attn_workspace_bytes(1, n, self.cfg.Hq, self.cfg.Hkv, self.cfg.D, max_ctx)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device=self.device)
        return max_ctx

    # ---- one forward over a block of rows ----------------------------------
    def forward(self, tokens: torch.Tensor, cache: PagedCache, view: str, mode: str):
        """tokens: int64 [n] at positions L .. L+n-1.  Returns (fp32 logits [n, V],
        k_rows, v_rows bf16 [layers, 1, n, Hkv, D])."""
        c = self.cfg
        n = tokens.shape[0]
        assert n <= PAD_ROWS
        pos = torch.arange(cache.L, cache.L + n, device=self.device)
        x = self.w["embed"][tokens]
        sfx = "" if view == "ar" else "_diff"
        max_ctx = self._workspace(cache, n)
        ks, vs = [], []
        for i in range(c.layers):
            p = f"l{i}."
            h = self._rms(x, self.w[p + "attn_norm"])
            q = self._lin(h, self.w[p + "wq" + sfx]).view(n, c.Hq, c.D)
            k = self._lin(h, self.w[p + "wk" + sfx]).view(n, c.Hkv, c.D)
            v = self._lin(h, self.w[p + "wv" + sfx]).view(n, c.Hkv, c.D)
            q = self._rope(self._rms(q, self.w[p + "q_norm"]), pos)
            k = self._rope(self._rms(k, self.w[p + "k_norm"]), pos)
            qb = q.to(torch.bfloat16).contiguous()[None]
            kb = k.to(torch.bfloat16).contiguous()[None]
            vb = v.to(torch.bfloat16).contiguous()[None]
            o = torch.empty_like(qb)
            fn = ob.orthrus_attn_draft if mode == "draft" else ob.orthrus_attn_verify
            fn(cache.layer(i), qb, kb, vb, o, max_ctx=max_ctx, workspace=self.ws)
            x = x + self._lin(o[0].to(torch.float64).reshape(n, c.Hq * c.D), self.w[p + "wo" + sfx])
            h = self._rms(x, self.w[p + "ffn_norm"])
            gate = self._lin(h, self.w[p + "w_gate"])
            up = self._lin(h, self.w[p + "w_up"])
            x = x + self._lin(torch.nn.functional.silu(gate) * up, self.w[p + "w_down"])
            ks.append(kb)
            vs.append(vb)
        logits = self._lin(self._rms(x, self.w["final_norm"]), self.w["lm_head"])
        return logits.to(torch.float32).contiguous(), torch.stack(ks), torch.stack(vs)

    def argmax(self, logits: torch.Tensor) -> torch.Tensor:
        out = torch.empty(logits.shape[0], dtype=torch.int32, device=self.device)
        ob.orthrus_argmax(logits, out)
        return out

    # ---- decoding ---------------------------------------------------------
    def new_cache(self, prompt_len: int, n_new: int, seed: int = 0) -> PagedCache:
        return PagedCache(self.cfg, prompt_len + n_new + 2 * self.max_block + PAD_ROWS + PAGE,
                          self.device, seed)

    def prefill(self, prompt: torch.Tensor, cache: PagedCache) -> int:
        """Causal AR pass over the prompt in blocks of up to 64 rows; returns the
        first generated token."""
        last = None
        for s0 in range(0, prompt.shape[0], PAD_ROWS):
            blk = prompt[s0:s0 + PAD_ROWS]
            logits, k, v = self.forward(blk, cache, "ar", "verify")
            n = torch.full((1,), blk.shape[0], dtype=torch.int32, device=self.device)
            cache.commit(k, v, n, blk.shape[0])
            last = logits[-1:]
        return int(self.argmax(last).item())

    def greedy(self, prompt: torch.Tensor, n: int, seed: int = 0) -> DecodeStats:
        cache = self.new_cache(prompt.shape[0], n, seed)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = [self.prefill(prompt, cache)]
        one = torch.ones(1, dtype=torch.int32, device=self.device)
        steps = 0
        while len(out) < n:
            tok = torch.tensor([out[-1]], dtype=torch.int64, device=self.device)
            logits, k, v = self.forward(tok, cache, "ar", "verify")
            a = self.argmax(logits)
            cache.commit(k, v, one, 1)
            out.append(int(a.item()))
            steps += 1
        torch.cuda.synchronize()
        return DecodeStats(out, steps, [1] * steps, time.perf_counter() - t0)

    def orthrus(self, prompt: torch.Tensor, n: int, K: int = 32, drafter=None,
                seed: int = 0) -> DecodeStats:
        """drafter(emitted_tokens, K) -> host int32 [K] overrides the diffusion
        view's draft (for exercising every accepted length); None uses the
        model's own diffusion view."""
        assert 1 <= K <= self.max_block
        cfg = self.cfg
        cache = self.new_cache(prompt.shape[0], n, seed)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = [self.prefill(prompt, cache)]
        anchor = torch.tensor([out[0]], dtype=torch.int64, device=self.device)
        mask_row = torch.full((K - 1,), cfg.mask_id, dtype=torch.int64, device=self.device)
        a = torch.empty((1, K), dtype=torch.int32, device=self.device)
        n_acc, n_emit, nxt = (torch.empty(1, dtype=torch.int32, device=self.device) for _ in range(3))
        emits = []
        while len(out) < n:
            if drafter is None:
                logits_d, _, _ = self.forward(torch.cat([anchor, mask_row]), cache, "diff", "draft")
                d = self.argmax(logits_d)
            else:
                d = torch.from_numpy(np.asarray(drafter(out, K), dtype=np.int32)).to(self.device)
            block = torch.cat([anchor, d[:K - 1].to(torch.int64)])
            logits_a, k, v = self.forward(block, cache, "ar", "verify")
            ob.orthrus_accept(logits_a[None], d[None].contiguous(), a, n_acc, n_emit, nxt)
            e = int(n_emit.item())
            cache.commit(k, v, n_emit, e)
            out.extend(int(t) for t in a[0, :e].tolist())
            anchor = nxt.to(torch.int64)
            emits.append(e)
        torch.cuda.synchronize()
        return DecodeStats(out[:n], len(emits), emits, time.perf_counter() - t0)

"""A Qwen3-shaped decoder with a diffusion view, at full size, decoded on one GPU
with the Orthrus loop and with plain greedy decoding.

The model follows the dual-view construction (gist.science technical summary
of "Orthrus: Memory-Efficient Parallel Token Generation via Dual-View
Diffusion", sections 2.1 and 2.3; Hacker News thread "Orthrus-Qwen3: up to
7.8x tokens/forward ...", posts #21 and #26): a frozen AR decoder (RMSNorm,
fused q/k/v and o projections with per-head QK RMSNorm and rotary embeddings,
SwiGLU FFN, untied LM head) plus, in every layer, the diffusion view's own
q/k/v/o projections.  Both views read the one paged KV cache that only the AR
view writes; the <mask> token is one extra embedding row.  Weights are random
(no trained weights exist here): this class times the whole step and checks
that the Orthrus loop reproduces greedy decoding.

What runs where: block attention (both masks), the LM head fused with the
argmax, acceptance, the all-layer commit and (for an e4m3 cache) the
quantisation of each layer's new K/V rows are liborthrus kernels; the dense
layers are bf16 matrix products in torch (hipBLASLt) with fp32 accumulation,
always on exactly 64 rows, so that a row's result never depends on how many
real rows a call has; the RMSNorm reductions run on the same fixed shape;
rotary embeddings and SiLU are torch elementwise ops in fp32; the residual
stream is fp32.  Every step is device-side (no host
synchronisation), so a whole step can be captured in a HIP graph.
"""
from __future__ import annotations

import time

import numpy as np
import torch

from . import binding as ob

PAD_ROWS = 64
PAGE = ob.ORTHRUS_PAGE_SIZE


class ModelCache:
    """All layers' K/V pools [layers, pages, Hkv, 16, D] (bf16, or e4m3 codes
    with per-layer, per-KV-head fp32 scales [layers, Hkv]), one sequence's
    block table (a seeded permutation of the pool) and two device length
    buffers that alternate as input and output of the commit."""

    def __init__(self, cfg, capacity: int, device, seed: int = 0, kv_scales=None):
        n_pages = -(-capacity // PAGE)
        shape = (cfg.layers, n_pages, cfg.Hkv, PAGE, cfg.D)
        self.fp8 = kv_scales is not None
        dt = torch.uint8 if self.fp8 else torch.bfloat16
        self.k = torch.zeros(shape, dtype=dt, device=device)
        self.v = torch.zeros(shape, dtype=dt, device=device)
        self.k_scale, self.v_scale = kv_scales if self.fp8 else (None, None)
        perm = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
        self.table = torch.from_numpy(perm[None, :]).to(device)
        self.lens = [torch.zeros(1, dtype=torch.int32, device=device),
                     torch.zeros(1, dtype=torch.int32, device=device)]
        self.cur = 0
        self.capacity = n_pages * PAGE

    @property
    def length(self) -> torch.Tensor:
        return self.lens[self.cur]

    def layer(self, i: int) -> ob.PagedKV:
        if self.fp8:
            return ob.PagedKV(self.k[i], self.v[i], self.table, self.lens[self.cur],
                              k_scale=self.k_scale[i], v_scale=self.v_scale[i])
        return ob.PagedKV(self.k[i], self.v[i], self.table, self.lens[self.cur])

    def fill_random(self, L: int, seed: int = 0):
        """Synthetic cache state of L tokens (N(0, 1) K/V, or e4m3 codes of
        magnitude below 8 with random signs) for timing."""
        gen = torch.Generator(device=self.k.device).manual_seed(seed)
        for t in (self.k, self.v):
            for i in range(t.shape[0]):
                if self.fp8:
                    code = torch.randint(0, 0x50, t[i].shape, generator=gen, device=t.device, dtype=torch.int32)
                    sign = torch.randint(0, 2, t[i].shape, generator=gen, device=t.device, dtype=torch.int32)
                    t[i].copy_((code | (sign << 7)).to(torch.uint8))
                else:
                    t[i].copy_(torch.randn(t[i].shape, generator=gen, device=t.device))
        self.lens[self.cur].fill_(L)

    def commit(self, k_rows, v_rows, n_emit: torch.Tensor):
        """k_rows, v_rows: [layers, 1, K, Hkv, D] of the AR view, in the cache's
        element type."""
        ob.orthrus_commit_kv(self.layer(0), k_rows, v_rows, n_emit, self.lens[1 - self.cur],
                             pool_layer_stride=self.k.stride(0))
        self.cur = 1 - self.cur


class DualViewModel:
    def __init__(self, cfg, weights: dict, device="cuda", max_block: int = 32):
        self.cfg = cfg
        self.w = weights
        self.device = torch.device(device)
        self.max_block = max_block
        half = cfg.D // 2
        self.inv_freq = (cfg.rope_base ** (-torch.arange(half, dtype=torch.float64, device=self.device)
                                           * 2.0 / cfg.D)).to(torch.float32)
        self.xpad = {}
        self.ws_attn = None
        self.ws_lm = ob.lmhead_workspace(PAD_ROWS, cfg.hidden, cfg.vocab, self.device)
        self.one = torch.ones(1, dtype=torch.int32, device=self.device)
        self.mask_row = torch.full((max_block - 1,), cfg.mask_id, dtype=torch.int64, device=self.device)

    # ---- building blocks ----------------------------------------------------
    def _lin(self, x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
        """x [n, in] bf16 @ w [in, out] bf16 on a fixed 64-row shape."""
        n, d_in = x.shape
        buf = self.xpad.get(d_in)
        if buf is None:
            buf = self.xpad[d_in] = torch.zeros((PAD_ROWS, d_in), dtype=torch.bfloat16, device=self.device)
        buf[:n].copy_(x)
        return torch.matmul(buf, w)[:n]

    def _rms(self, x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
        """RMSNorm over the last dimension in fp32, on a fixed 64-row shape: the
        reduction kernel torch picks (and so the order of the sum) depends on
        the tensor's shape, and a row's result must not depend on how many
        rows the call has."""
        n = x.shape[0]
        key = ("rms",) + tuple(x.shape[1:])
        buf = self.xpad.get(key)
        if buf is None:
            buf = self.xpad[key] = torch.zeros((PAD_ROWS,) + tuple(x.shape[1:]), dtype=torch.float32,
                                               device=self.device)
        buf[:n].copy_(x)
        y = buf * torch.rsqrt(buf.pow(2).mean(dim=-1, keepdim=True) + self.cfg.rms_eps) * w.float()
        return y[:n]

    def _rope(self, x: torch.Tensor, pos: torch.Tensor) -> torch.Tensor:
        ang = pos[:, None].float() * self.inv_freq[None, :]
        cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        h = self.cfg.D // 2
        x1, x2 = x[..., :h], x[..., h:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)

    def max_ctx(self, cache: ModelCache) -> int:
        # one max_ctx for every call on a cache: the attention's split grid
        # depends on it, and greedy and Orthrus decoding must share that grid
        return cache.capacity - PAD_ROWS

    def _attn_ws(self, cache: ModelCache, n: int):
        c = self.cfg
        need = ob.orthrus_attn_workspace_bytes(1, n, c.Hq, c.Hkv, c.D, self.max_ctx(cache))
        if self.ws_attn is None or self.ws_attn.numel() < need:
            self.ws_attn = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device=self.device)
        return self.ws_attn

    # ---- one forward over a block of rows -----------------------------------
    def forward(self, tokens: torch.Tensor, cache: ModelCache, view: str, mode: str):
        """tokens: int64 [n] (device) at positions L .. L+n-1, L = cache.length.
        Returns (final hidden states bf16 [n, hidden], k_rows, v_rows
        [layers, 1, n, Hkv, D] of this view in the cache's element type)."""
        c = self.cfg
        n = tokens.shape[0]
        assert n <= PAD_ROWS
        pos = cache.length.to(torch.int64) + torch.arange(n, device=self.device)
        x = self.w["embed"][tokens].float()
        sfx = "" if view == "ar" else "_diff"
        ws = self._attn_ws(cache, n)
        max_ctx = self.max_ctx(cache)
        fn = ob.orthrus_attn_draft if mode == "draft" else ob.orthrus_attn_verify
        qd, kd = c.Hq * c.D, c.Hkv * c.D
        ks, vs = [], []
        for i in range(c.layers):
            p = f"l{i}."
            h = self._rms(x, self.w[p + "attn_norm"]).to(torch.bfloat16)
            qkv = self._lin(h, self.w[p + "wqkv" + sfx])
            q = qkv[:, :qd].view(n, c.Hq, c.D)
            k = qkv[:, qd:qd + kd].view(n, c.Hkv, c.D)
            v = qkv[:, qd + kd:].reshape(1, n, c.Hkv, c.D)
            q = self._rope(self._rms(q, self.w[p + "q_norm"]), pos).to(torch.bfloat16)[None].contiguous()
            k = self._rope(self._rms(k, self.w[p + "k_norm"]), pos).to(torch.bfloat16)[None].contiguous()
            v = v.contiguous()
            if cache.fp8:
                # the block's rows in the cache's format: attention reads, and
                # the commit stores, exactly these codes
                k8 = torch.empty(k.shape, dtype=torch.uint8, device=self.device)
                v8 = torch.empty_like(k8)
                ob.orthrus_quantize_kv(k, v, cache.k_scale[i], cache.v_scale[i], k8, v8)
                k, v = k8, v8
            o = torch.empty_like(q)
            fn(cache.layer(i), q, k, v, o, max_ctx=max_ctx, workspace=ws)
            x = x + self._lin(o[0].view(n, qd), self.w[p + "wo" + sfx]).float()
            h = self._rms(x, self.w[p + "ffn_norm"]).to(torch.bfloat16)
            gu = self._lin(h, self.w[p + "w_gate_up"]).float()
            act = (torch.nn.functional.silu(gu[:, :c.ffn]) * gu[:, c.ffn:]).to(torch.bfloat16)
            x = x + self._lin(act, self.w[p + "w_down"]).float()
            ks.append(k)
            vs.append(v)
        hidden = self._rms(x, self.w["final_norm"]).to(torch.bfloat16).contiguous()
        return hidden, torch.stack(ks), torch.stack(vs)

    def greedy_token(self, hidden: torch.Tensor, out: torch.Tensor):
        ob.orthrus_lmhead_argmax(hidden, self.w["lm_head"], out, workspace=self.ws_lm)
        return out

    # ---- decode steps (device-side, capturable) -------------------------------
    def greedy_step(self, cache: ModelCache, tok: torch.Tensor, out: torch.Tensor):
        """tok: int64 [1], the last token (not cached yet); out: int32 [1] <- next token."""
        hidden, k, v = self.forward(tok, cache, "ar", "verify")
        self.greedy_token(hidden, out)
        cache.commit(k, v, self.one)

    def orthrus_step(self, cache: ModelCache, anchor: torch.Tensor, K: int, d: torch.Tensor,
                     a: torch.Tensor, n_acc, n_emit, nxt, draft_override=None):
        """anchor: int64 [1].  d, a: int32 [1, K]; n_acc, n_emit, nxt: int32 [1]."""
        hd, _, _ = self.forward(torch.cat([anchor, self.mask_row[:K - 1]]), cache, "diff", "draft")
        self.greedy_token(hd, d[0])
        if draft_override is not None:
            d[0].copy_(draft_override)
        block = torch.cat([anchor, d[0, :K - 1].to(torch.int64)])
        hv, k, v = self.forward(block, cache, "ar", "verify")
        ob.orthrus_lmhead_accept(hv[None], self.w["lm_head"], d, a, n_acc, n_emit, nxt, workspace=self.ws_lm)
        cache.commit(k, v, n_emit)

    # ---- host-driven decoding (tests) -----------------------------------------
    def new_cache(self, prompt_len: int, n_new: int, seed: int = 0, kv_scales=None) -> ModelCache:
        return ModelCache(self.cfg, prompt_len + n_new + 2 * self.max_block + PAD_ROWS + PAGE, self.device, seed,
                          kv_scales=kv_scales)

    def calibrate_kv_scales(self, prompt: torch.Tensor, headroom: float = 2.0):
        """Per-layer, per-KV-head e4m3 scales from the AR view's K/V on the first
        (up to 64) prompt tokens: amax * headroom / 448 (static scales, as a
        serving system calibrates them once)."""
        blk = prompt[:PAD_ROWS]
        cache = ModelCache(self.cfg, blk.shape[0] + PAD_ROWS + PAGE, self.device)
        _, k, v = self.forward(blk, cache, "ar", "verify")
        scales = []
        for t in (k, v):                                      # [layers, 1, n, Hkv, D]
            amax = t.float().abs().amax(dim=(1, 2, 4))        # [layers, Hkv]
            scales.append((amax.clamp_min(1e-3) * headroom / 448.0).contiguous())
        return tuple(scales)

    def prefill(self, prompt: torch.Tensor, cache: ModelCache) -> int:
        out = torch.empty(1, dtype=torch.int32, device=self.device)
        for s0 in range(0, prompt.shape[0], PAD_ROWS):
            blk = prompt[s0:s0 + PAD_ROWS]
            hidden, k, v = self.forward(blk, cache, "ar", "verify")
            cache.commit(k, v, torch.full((1,), blk.shape[0], dtype=torch.int32, device=self.device))
        self.greedy_token(hidden[-1:], out)
        return int(out.item())

    def greedy(self, prompt: torch.Tensor, n: int, seed: int = 0, kv_scales=None):
        cache = self.new_cache(prompt.shape[0], n, seed, kv_scales)
        return self.decode_greedy(cache, self.prefill(prompt, cache), n)

    def decode_greedy(self, cache: ModelCache, first: int, n: int):
        """Plain greedy decoding from the cache's current state: `first` is the
        last emitted token (not cached yet); returns n tokens starting with it."""
        toks = [int(first)]
        out = torch.empty(1, dtype=torch.int32, device=self.device)
        t0 = time.perf_counter()
        while len(toks) < n:
            self.greedy_step(cache, torch.tensor([toks[-1]], device=self.device), out)
            toks.append(int(out.item()))
        return toks, time.perf_counter() - t0

    def orthrus(self, prompt: torch.Tensor, n: int, K: int = 32, drafter=None, seed: int = 0, kv_scales=None):
        """drafter(emitted_tokens, K) -> host int32 [K] overrides the diffusion
        view's draft (the draft pass still runs).  kv_scales (k, v fp32
        [layers, Hkv]) selects an e4m3 cache."""
        cache = self.new_cache(prompt.shape[0], n, seed, kv_scales)
        return self.decode_orthrus(cache, self.prefill(prompt, cache), n, K, drafter)

    def decode_orthrus(self, cache: ModelCache, first: int, n: int, K: int = 32, drafter=None):
        """The Orthrus loop from the cache's current state (as decode_greedy);
        returns (n tokens, emitted tokens per step, seconds)."""
        toks = [int(first)]
        anchor = torch.tensor([toks[0]], device=self.device)
        d, a = (torch.empty((1, K), dtype=torch.int32, device=self.device) for _ in range(2))
        n_acc, n_emit, nxt = (torch.empty(1, dtype=torch.int32, device=self.device) for _ in range(3))
        emits = []
        t0 = time.perf_counter()
        while len(toks) < n:
            over = None
            if drafter is not None:
                over = torch.from_numpy(np.asarray(drafter(toks, K), dtype=np.int32)).to(self.device)
            self.orthrus_step(cache, anchor, K, d, a, n_acc, n_emit, nxt, draft_override=over)
            e = int(n_emit.item())
            toks.extend(int(t) for t in a[0, :e].tolist())
            anchor = nxt.to(torch.int64)
            emits.append(e)
        return toks[:n], emits, time.perf_counter() - t0

    def block_logits(self, tokens: torch.Tensor, cache: ModelCache, view: str, mode: str,
                     commit: bool = False) -> torch.Tensor:
        """fp32 logits [n, V] of one block (the fused LM head's own logits, the
        values its argmax reduces); with commit, the block's K/V (AR view)
        are appended to the cache afterwards."""
        hidden, k, v = self.forward(tokens, cache, view, mode)
        n = tokens.shape[0]
        logits = torch.empty((n, self.cfg.vocab), dtype=torch.float32, device=self.device)
        out = torch.empty(n, dtype=torch.int32, device=self.device)
        ob.orthrus_lmhead_argmax(hidden, self.w["lm_head"], out, logits=logits, workspace=self.ws_lm)
        if commit:
            cache.commit(k, v, torch.full((1,), n, dtype=torch.int32, device=self.device))
        return logits

"""Seeded generators for every workload of the Orthrus draft/verify step.

Everything here is random-number drawing and memory layout only.  The method's
arithmetic (attention, argmax, acceptance, commit) lives on the two sides that
are compared: ``oracle/`` and the HIP library.  Generated tensors are handed
over as raw bit patterns (``uint16`` for bf16, ``float32``, ``int32``) so both
sides read identical bytes.

Layouts (one layer unless stated):

* ``q``            ``[B, K, Hq, D]``  bf16 bits
* ``k_blk, v_blk`` ``[B, K, Hkv, D]`` bf16 bits (block rows, post-RoPE)
* ``k_pages, v_pages`` ``[layers, num_pages, Hkv, page_size, D]`` bf16 bits
* ``block_table``  ``[B, max_pages]`` int32, a random permutation of the pool
* ``seq_lens``     ``[B]`` int32, cached length ``L_b``
* logits           ``[B, K, V]`` float32
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "BF16_NAN", "BF16_SENTINEL", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "PagedCase", "make_paged_case", "make_block_qkv", "ConsensusCase", "make_consensus_case",
    "draw_accept_lengths", "make_tie_logits", "ToyConfig", "TOY_CFG5", "QWEN3_8B",
    "make_model_weights_device",
    "TOY_TINY", "TOY_CHECK", "make_toy_weights", "make_prompt", "WORKLOADS",
]

BF16_NAN = 0x7FC0        # quiet NaN: poison for slots no kernel may read
BF16_SENTINEL = 0x7F7F   # largest finite bf16: marks slots commit must not touch


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Paged KV + block Q/K/V
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PagedCase:
    B: int
    K: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    layers: int
    q: np.ndarray
    k_blk: np.ndarray
    v_blk: np.ndarray
    k_pages: np.ndarray
    v_pages: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    num_pages: int
    fill_bits: int
    needles: list  # (b, g, position, row i, q-head offset gg, score lift)

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def _normal_bf16(rng, shape, std):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def make_paged_case(seed: int, B: int, K: int, Hq: int, Hkv: int, D: int,
                    seq_lens, *, layers: int = 1, page_size: int = 16,
                    slack_pages: int = 1, std: float | None = None,
                    sharp: bool = False, fill: str = "nan",
                    extra_pages_per_seq: int = 0) -> PagedCase:
    """Draw one paged-attention workload.

    ``std`` is the standard deviation of Q, K and V (default 1/sqrt(D), the
    scaling of the Qwen3-8B-shaped workloads).  ``sharp`` draws unscaled
    N(0,1) values and plants needle keys whose score for one chosen query row
    is lifted 8-12 above the background; needles sit at page boundaries, the
    first and last cached position, the block rows and random positions, so a
    dropped page, wrong mask, wrong head map or bad split merge shows up.

    Each sequence owns ceil((L_b + K) / page_size) + extra_pages_per_seq pages
    drawn from a random permutation of the pool; the slots at positions >= L_b
    (where this step's block K/V would be committed) and every slack page hold
    ``fill`` (``"nan"`` poison or the finite ``"sentinel"``).  Unused
    block-table entries point at a slack page.
    """
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    if std is None:
        std = 1.0 / math.sqrt(D)
    val_std = 1.0 if sharp else std
    fill_bits = BF16_NAN if fill == "nan" else BF16_SENTINEL
    G = Hq // Hkv

    q = _normal_bf16(rng, (B, K, Hq, D), val_std)
    k_blk = _normal_bf16(rng, (B, K, Hkv, D), val_std)
    v_blk = _normal_bf16(rng, (B, K, Hkv, D), val_std)

    need = [-(-(int(L) + K) // page_size) + extra_pages_per_seq for L in seq_lens]
    max_pages = max(need)
    num_pages = int(sum(need)) + max(1, slack_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    poison_page = int(perm[-1])  # one slack page that no sequence owns
    table = np.full((B, max_pages), poison_page, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]

    k_pages = np.full((layers, num_pages, Hkv, page_size, D), fill_bits, dtype=np.uint16)
    v_pages = np.full_like(k_pages, fill_bits)
    needles = []
    for layer in range(layers):
        for b in range(B):
            L = int(seq_lens[b])
            kc = rng.standard_normal((L, Hkv, D), dtype=np.float32) * np.float32(val_std)
            vc = _normal_bf16(rng, (L, Hkv, D), val_std)
            if sharp and layer == 0:
                kc, kb = _plant_needles(rng, q, k_blk, kc, b, L, K, G, Hkv, D,
                                        page_size, needles)
                k_blk[b] = kb
            kc = f32_to_bf16_bits(kc)
            for p0 in range(0, L, page_size):
                n = min(page_size, L - p0)
                page = table[b, p0 // page_size]
                k_pages[layer, page, :, :n, :] = kc[p0:p0 + n].transpose(1, 0, 2)
                v_pages[layer, page, :, :n, :] = vc[p0:p0 + n].transpose(1, 0, 2)
    return PagedCase(B, K, Hq, Hkv, D, page_size, layers, q, k_blk, v_blk,
                     k_pages, v_pages, table, seq_lens, num_pages, fill_bits, needles)


def make_block_qkv(seed: int, B: int, K: int, Hq: int, Hkv: int, D: int, std: float | None = None):
    """Another set of block rows (q [B,K,Hq,D], k_blk, v_blk [B,K,Hkv,D], bf16
    bits): the verify pass uses the AR view's projections, which differ from
    the draft pass's diffusion-view projections."""
    rng = np.random.default_rng(seed)
    std = 1.0 / math.sqrt(D) if std is None else std
    return (_normal_bf16(rng, (B, K, Hq, D), std), _normal_bf16(rng, (B, K, Hkv, D), std),
            _normal_bf16(rng, (B, K, Hkv, D), std))


def _plant_needles(rng, q_bits, k_blk_bits, kc, b, L, K, G, Hkv, D, P, needles):
    """Add beta * q_row to chosen keys so that row's score rises by 8..12."""
    q = bf16_bits_to_f32(q_bits[b])          # [K, Hq, D]
    kb = bf16_bits_to_f32(k_blk_bits[b])     # [K, Hkv, D]
    n_total = L + K
    edge = {0, P - 1, P, L - 1, L, L + K - 1, L + K // 2}
    edge |= {p for p in range(P, L, 37 * P)}  # page starts across the context
    edge |= set(int(x) for x in rng.integers(0, n_total, size=8))
    positions = sorted(p for p in edge if 0 <= p < n_total)
    for g in range(Hkv):
        for p in positions:
            i = int(rng.integers(0, K))
            gg = int(rng.integers(0, G))
            lift = float(rng.uniform(8.0, 12.0))
            qrow = q[i, g * G + gg].astype(np.float64)
            beta = lift * math.sqrt(D) / float(qrow @ qrow)
            if p < L:
                kc[p, g] = (kc[p, g] + beta * qrow).astype(np.float32)
            else:
                kb[p - L, g] = (kb[p - L, g] + beta * qrow).astype(np.float32)
            needles.append((b, g, p, i, gg, lift))
    return kc, f32_to_bf16_bits(kb)


# --------------------------------------------------------------------------
# Consensus logits with planted argmax
# --------------------------------------------------------------------------

@dataclasses.dataclass
class ConsensusCase:
    logits_d: np.ndarray   # [B, K, V] float32, draft-view logits
    logits_a: np.ndarray   # [B, K, V] float32, AR-view logits
    d: np.ndarray          # [B, K] int32, planted argmax of logits_d
    a: np.ndarray          # [B, K] int32, planted argmax of logits_a
    n_acc: np.ndarray      # [B] int32, the drawn forced-match prefix length


def draw_accept_lengths(rng, B: int, K: int, dist: str, p: float = 0.15) -> np.ndarray:
    """Forced-match prefix lengths.

    ``"uniform"``: j uniform in {0..K} (inclusive: j = K means all K match).
    ``"geometric"``: min(G - 1, K) with G ~ Geometric(p) on {1, 2, ...}: each
    position independently mismatches with probability p.
    """
    if dist == "uniform":
        return rng.integers(0, K + 1, size=B).astype(np.int32)
    if dist == "geometric":
        return np.minimum(rng.geometric(p, size=B) - 1, K).astype(np.int32)
    raise ValueError(dist)


def make_consensus_case(seed: int, B: int, K: int, V: int, *, dist: str = "geometric",
                        p: float = 0.15, n_acc=None) -> ConsensusCase:
    """Logits N(0,1) clipped to [-8, 8] with one planted maximum per row in
    (8.5, 10]; the planted indices make the draft agree with the AR view on
    exactly the first n_acc positions (the next position is forced to differ)."""
    rng = np.random.default_rng(seed)
    n = draw_accept_lengths(rng, B, K, dist, p) if n_acc is None else \
        np.asarray(n_acc, dtype=np.int32).reshape(B)
    a = rng.integers(0, V, size=(B, K)).astype(np.int32)
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    for b in range(B):
        j = int(n[b])
        d[b, :j] = a[b, :j]
        if j < K:
            d[b, j] = (a[b, j] + 1 + rng.integers(0, V - 1)) % V
    logits = []
    for planted in (d, a):
        x = rng.standard_normal((B, K, V), dtype=np.float32)
        np.clip(x, -8.0, 8.0, out=x)
        top = rng.uniform(8.5, 10.0, size=(B, K)).astype(np.float32)
        bi, ki = np.meshgrid(np.arange(B), np.arange(K), indexing="ij")
        x[bi, ki, planted] = top
        logits.append(x)
    return ConsensusCase(logits[0], logits[1], d, a, n)


def make_tie_logits(seed: int, rows: int, V: int, n_ties: int = 3, signed_zero: bool = False):
    """Rows whose maximum occurs ``n_ties`` times (bitwise-equal values) at
    random positions; returns (logits [rows, V] float32, sorted tie positions
    [rows, n_ties]).  With ``signed_zero`` every value is <= 0 and the maxima
    are a mix of -0.0 and +0.0 (they compare equal)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, V), dtype=np.float32)
    pos = np.stack([np.sort(rng.choice(V, size=n_ties, replace=False)) for _ in range(rows)])
    if signed_zero:
        x = -np.abs(x) - np.float32(0.5)
        for r in range(rows):
            for t, c in enumerate(pos[r]):
                x[r, c] = np.float32(-0.0) if t % 2 == 0 else np.float32(0.0)
    else:
        np.clip(x, -8.0, 8.0, out=x)
        top = rng.uniform(8.5, 10.0, size=rows).astype(np.float32)
        for r in range(rows):
            x[r, pos[r]] = top[r]
    return x, pos.astype(np.int64)


# --------------------------------------------------------------------------
# Toy Qwen3-style decoder + diffusion module weights
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ToyConfig:
    layers: int
    hidden: int
    Hq: int
    Hkv: int
    D: int
    ffn: int
    vocab: int
    rope_base: float
    weight_std: float = 0.02
    rms_eps: float = 1e-6

    @property
    def mask_id(self) -> int:
        """The <mask> token: one extra embedding row owned by the diffusion module."""
        return self.vocab


TOY_CFG5 = ToyConfig(layers=4, hidden=1024, Hq=16, Hkv=4, D=64, ffn=2816,
                     vocab=32000, rope_base=1e6)
# Qwen3-8B shape (36 layers, hidden 4096, 32/8 heads of 128, SwiGLU 12288,
# vocabulary 151936): random weights only, for timing the whole step
QWEN3_8B = ToyConfig(layers=36, hidden=4096, Hq=32, Hkv=8, D=128, ffn=12288,
                     vocab=151936, rope_base=1e6)
TOY_TINY = ToyConfig(layers=2, hidden=64, Hq=4, Hkv=2, D=16, ffn=96,
                     vocab=97, rope_base=1e4, weight_std=0.3)
# a small config that both the GPU models and the fp64 oracle decoder run:
# the attention and LM-head kernels' shape limits (head_dim 64, hidden a
# multiple of 64), Qwen3's RoPE base, several 64-row prefill blocks
TOY_CHECK = ToyConfig(layers=2, hidden=256, Hq=8, Hkv=2, D=64, ffn=512,
                      vocab=2048, rope_base=1e6, weight_std=0.05)


def make_toy_weights(seed: int, cfg: ToyConfig) -> dict:
    """bf16 bit patterns for every weight; matrices are [in, out].  Norm weights
    are ones (the usual random init of an RMSNorm gain)."""
    rng = np.random.default_rng(seed)
    H, Hq, Hkv, D, F = cfg.hidden, cfg.Hq, cfg.Hkv, cfg.D, cfg.ffn
    s = cfg.weight_std
    ones = lambda n: f32_to_bf16_bits(np.ones(n, np.float32))  # noqa: E731
    w = {"embed": _normal_bf16(rng, (cfg.vocab + 1, H), s),
         "final_norm": ones(H),
         "lm_head": _normal_bf16(rng, (H, cfg.vocab), s)}
    for i in range(cfg.layers):
        p = f"l{i}."
        w[p + "attn_norm"] = ones(H)
        w[p + "ffn_norm"] = ones(H)
        w[p + "q_norm"] = ones(D)
        w[p + "k_norm"] = ones(D)
        w[p + "wq"] = _normal_bf16(rng, (H, Hq * D), s)
        w[p + "wk"] = _normal_bf16(rng, (H, Hkv * D), s)
        w[p + "wv"] = _normal_bf16(rng, (H, Hkv * D), s)
        w[p + "wo"] = _normal_bf16(rng, (Hq * D, H), s)
        w[p + "w_gate"] = _normal_bf16(rng, (H, F), s)
        w[p + "w_up"] = _normal_bf16(rng, (H, F), s)
        w[p + "w_down"] = _normal_bf16(rng, (F, H), s)
        # the diffusion view's own attention projections
        w[p + "wq_diff"] = _normal_bf16(rng, (H, Hq * D), s)
        w[p + "wk_diff"] = _normal_bf16(rng, (H, Hkv * D), s)
        w[p + "wv_diff"] = _normal_bf16(rng, (H, Hkv * D), s)
        w[p + "wo_diff"] = _normal_bf16(rng, (Hq * D, H), s)
    return w


def make_model_weights_device(seed: int, cfg: ToyConfig, device) -> dict:
    """The same set of weights as make_toy_weights, drawn on the GPU (bf16
    torch tensors; tens of GB at the 8B shape are impractical to draw on the
    host).  Matrices are [in, out] except the LM head, [vocab, hidden] (row v =
    token v); q/k/v projections come fused as one [hidden, (Hq + 2 Hkv) D]
    matrix per view, gate and up as one [hidden, 2 ffn] matrix."""
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    H, Hq, Hkv, D, F = cfg.hidden, cfg.Hq, cfg.Hkv, cfg.D, cfg.ffn
    s = cfg.weight_std

    def normal(*shape):
        return torch.randn(shape, generator=gen, device=device).mul_(s).to(torch.bfloat16)

    ones = lambda n: torch.ones(n, dtype=torch.bfloat16, device=device)  # noqa: E731
    w = {"embed": normal(cfg.vocab + 1, H), "final_norm": ones(H), "lm_head": normal(cfg.vocab, H)}
    for i in range(cfg.layers):
        p = f"l{i}."
        w[p + "attn_norm"], w[p + "ffn_norm"] = ones(H), ones(H)
        w[p + "q_norm"], w[p + "k_norm"] = ones(D), ones(D)
        w[p + "wqkv"] = normal(H, (Hq + 2 * Hkv) * D)
        w[p + "wo"] = normal(Hq * D, H)
        w[p + "w_gate_up"] = normal(H, 2 * F)
        w[p + "w_down"] = normal(F, H)
        w[p + "wqkv_diff"] = normal(H, (Hq + 2 * Hkv) * D)
        w[p + "wo_diff"] = normal(Hq * D, H)
    return w


def make_prompt(seed: int, n: int, vocab: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, vocab, size=n).astype(np.int64)


# --------------------------------------------------------------------------
# Named workloads (sizes and seeds)
# --------------------------------------------------------------------------
# LM head (final hidden states x vocabulary weights)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LmHeadCase:
    hidden: np.ndarray   # [R, hidden] bf16 bits (after the final norm)
    weight: np.ndarray   # [V, hidden] bf16 bits
    targets: np.ndarray  # [R] int32 planted token per row, -1 if none


def make_lmhead_case(seed: int, R: int, hidden: int, V: int, *, plant: bool = True,
                     lift: float = 30.0, w_std: float = 0.02, dup_rows: int = 0) -> LmHeadCase:
    """Hidden states N(0,1) and LM-head weights N(0, w_std) rounded to bf16.

    With ``plant``, row r gets a target token t_r (distinct across rows when
    V >= R): W[t_r] += lift * h_r / |h_r|^2 before rounding, which raises that
    logit by about ``lift`` (the background logits have standard deviation
    w_std * sqrt(hidden), 1.28 at hidden 4096).  ``dup_rows`` copies the
    weight row of each of the first ``dup_rows`` targets to a random lower
    vocabulary index, so the maximum is attained twice."""
    rng = np.random.default_rng(seed)
    h32 = rng.standard_normal((R, hidden), dtype=np.float32)
    h_bits = f32_to_bf16_bits(h32)
    w32 = rng.standard_normal((V, hidden), dtype=np.float32) * np.float32(w_std)
    targets = np.full(R, -1, dtype=np.int32)
    if plant:
        t = rng.choice(V, size=R, replace=V < R).astype(np.int32)
        hf = bf16_bits_to_f32(h_bits)
        for r in range(R):
            w32[t[r]] += np.float32(lift) * hf[r] / np.float32(np.dot(hf[r], hf[r]))
        targets = t
    w_bits = f32_to_bf16_bits(w32)
    taken = set(int(x) for x in targets)
    for r in range(min(dup_rows, R)):
        free = [v for v in range(int(targets[r])) if v not in taken] if targets[r] > 0 else []
        if free:
            lower = int(free[int(rng.integers(0, len(free)))])
            w_bits[lower] = w_bits[targets[r]]
            taken.add(lower)
            targets[r] = lower
    return LmHeadCase(h_bits, w_bits, targets)


__all__ += ["LmHeadCase", "make_lmhead_case"]


# --------------------------------------------------------------------------

WORKLOADS = {
    # tiny CPU-checkable case
    "tiny": dict(seed=1, B=1, K=8, Hq=2, Hkv=1, D=64, seq_lens=[256], V=1024,
                 accept="uniform", hidden=128),
    # Qwen3-8B attention shape, 4K context
    "qwen3_8b_4k": dict(seed=2, B=1, K=32, Hq=32, Hkv=8, D=128, seq_lens=[4096],
                        V=151936, accept="geometric", hidden=4096),
    # same shape at 40960-token context
    "qwen3_8b_40k": dict(seed=3, B=1, K=32, Hq=32, Hkv=8, D=128, seq_lens=[40960],
                         V=151936, accept="geometric", hidden=4096),
    # batched ragged serving step, 16 sequences, L_b ~ U[1024, 32768]
    "qwen3_8b_ragged16": dict(seed=4, B=16, K=32, Hq=32, Hkv=8, D=128, seq_lens=None,
                              V=151936, accept="geometric", hidden=4096),
}


def ragged_lengths(seed: int, B: int, lo: int = 1024, hi: int = 32768) -> np.ndarray:
    return np.random.default_rng(seed + 1000).integers(lo, hi + 1, size=B).astype(np.int32)


__all__ += ["ragged_lengths"]

"""Pins for the oracle's dual-view block attention (CPU only).

Each check ties the oracle to something other than itself: a brute force
written independently with scalar loops, torch's scaled_dot_product_attention
in fp64 with an explicit mask, closed-form special cases and invariants.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_weights, block_attention, from_bf16, gather_context
from synth import make_paged_case


def _case(seed=0, B=2, K=3, Hq=4, Hkv=2, D=8, lens=(5, 19), P=4, sharp=False, std=1.0):
    # page_size 4 spreads even tiny contexts over several pages
    c = make_paged_case(seed, B, K, Hq, Hkv, D, list(lens), page_size=P, std=std,
                        sharp=sharp)
    return dict(q=from_bf16(c.q), k_blk=from_bf16(c.k_blk), v_blk=from_bf16(c.v_blk),
                k_pages=from_bf16(c.k_pages[0]), v_pages=from_bf16(c.v_pages[0]),
                block_table=c.block_table, seq_lens=c.seq_lens, page_size=P), c


def _brute(x, mode):
    """Scalar loops: walk the page table, exp with math.exp, sum in order."""
    q, kb, vb, kp, vp = x["q"], x["k_blk"], x["v_blk"], x["k_pages"], x["v_pages"]
    B, K, Hq, D = q.shape
    Hkv = kp.shape[1]
    P = x["page_size"]
    out = np.zeros_like(q)
    for b in range(B):
        L = int(x["seq_lens"][b])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(K):
                keys, vals = [], []
                for p in range(L):
                    pg, sl = x["block_table"][b][p // P], p % P
                    keys.append(kp[pg, g, sl]); vals.append(vp[pg, g, sl])
                last = K - 1 if mode == "draft" else i
                for r in range(last + 1):
                    keys.append(kb[b, r, g]); vals.append(vb[b, r, g])
                sc = [sum(q[b, i, h, d] * kk[d] for d in range(D)) / math.sqrt(D) for kk in keys]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                tot = sum(e)
                for d in range(D):
                    out[b, i, h, d] = sum(e[j] * vals[j][d] for j in range(len(e))) / tot
    return out


def _run(x, mode, **kw):
    return block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_pages"], x["v_pages"],
                           x["block_table"], x["seq_lens"], mode, page_size=x["page_size"], **kw)


@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_matches_scalar_brute_force(mode):
    x, _ = _case()
    np.testing.assert_allclose(_run(x, mode), _brute(x, mode), rtol=1e-12, atol=1e-13)


def _sdpa(x, mode):
    """torch SDPA in fp64 with an explicit boolean mask, per (b, h)."""
    q = torch.from_numpy(x["q"])
    B, K, Hq, D = q.shape
    Hkv = x["k_pages"].shape[1]
    out = torch.zeros_like(q)
    for b in range(B):
        L = int(x["seq_lens"][b])
        kc, vc = gather_context(x["k_pages"], x["v_pages"], x["block_table"], b, L, x["page_size"])
        mask = torch.ones(K, L + K, dtype=torch.bool)
        if mode == "verify":
            mask[:, L:] = torch.tril(torch.ones(K, K, dtype=torch.bool))
        for h in range(Hq):
            g = h // (Hq // Hkv)
            k = torch.cat([torch.from_numpy(kc[:, g]), torch.from_numpy(x["k_blk"][b, :, g])])
            v = torch.cat([torch.from_numpy(vc[:, g]), torch.from_numpy(x["v_blk"][b, :, g])])
            out[b, :, h] = torch.nn.functional.scaled_dot_product_attention(
                q[b, :, h][None, None], k[None, None], v[None, None], attn_mask=mask)[0, 0]
    return out.numpy()


@pytest.mark.parametrize("mode", ["draft", "verify"])
@pytest.mark.parametrize("lens,K,P", [((5, 19), 3, 4), ((0, 33), 8, 16), ((64, 1), 5, 16)])
def test_matches_torch_sdpa_fp64(mode, lens, K, P):
    x, _ = _case(seed=3, K=K, lens=lens, P=P, D=16)
    np.testing.assert_allclose(_run(x, mode), _sdpa(x, mode), rtol=1e-11, atol=1e-12)


def test_k1_is_single_token_decode():
    x, _ = _case(seed=4, K=1, lens=(9, 30), D=16)
    dr, ve = _run(x, "draft"), _run(x, "verify")
    assert np.array_equal(dr, ve)
    q = torch.from_numpy(x["q"])
    for b in range(2):
        L = int(x["seq_lens"][b])
        kc, vc = gather_context(x["k_pages"], x["v_pages"], x["block_table"], b, L, 4)
        for h in range(4):
            g = h // 2
            k = torch.cat([torch.from_numpy(kc[:, g]), torch.from_numpy(x["k_blk"][b, :, g])])
            v = torch.cat([torch.from_numpy(vc[:, g]), torch.from_numpy(x["v_blk"][b, :, g])])
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[b, :, h][None, None], k[None, None], v[None, None])[0, 0]
            np.testing.assert_allclose(dr[b, :, h], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_empty_cache_reduces_to_plain_attention():
    x, _ = _case(seed=5, K=7, lens=(0, 0), D=16)
    q = torch.from_numpy(x["q"]).permute(0, 2, 1, 3)              # [B, Hq, K, D]
    k = torch.from_numpy(x["k_blk"]).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    v = torch.from_numpy(x["v_blk"]).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    full = torch.nn.functional.scaled_dot_product_attention(q, k, v).permute(0, 2, 1, 3)
    causal = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).permute(0, 2, 1, 3)
    np.testing.assert_allclose(_run(x, "draft"), full.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(_run(x, "verify"), causal.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_constant_values_give_the_constant(mode):
    x, _ = _case(seed=6, lens=(21, 3))
    x["v_pages"][:] = 0.375
    x["v_blk"][:] = 0.375
    np.testing.assert_allclose(_run(x, mode), 0.375, rtol=0, atol=1e-14)


def test_dominant_needle_returns_its_value():
    x, _ = _case(seed=7, lens=(40, 12), K=4, D=16, std=0.1)
    b, h, i, p = 0, 3, 2, 17
    g = h // 2
    page, slot = x["block_table"][b][p // 4], p % 4
    x["k_pages"][page, g, slot] = 4000.0 * x["q"][b, i, h] / np.linalg.norm(x["q"][b, i, h])
    for mode in ("draft", "verify"):
        o = _run(x, mode)
        np.testing.assert_allclose(o[b, i, h], x["v_pages"][page, g, slot], atol=1e-9)


def test_page_permutation_invariance():
    x, _ = _case(seed=8, lens=(37, 22), K=5)
    n = x["k_pages"].shape[0]
    perm = np.random.default_rng(1).permutation(n)
    inv = np.argsort(perm)
    y = dict(x)
    y["k_pages"] = x["k_pages"][perm]
    y["v_pages"] = x["v_pages"][perm]
    y["block_table"] = inv[x["block_table"]].astype(np.int32)
    for mode in ("draft", "verify"):
        assert np.array_equal(_run(x, mode), _run(y, mode))


def test_weights_sum_to_one_and_respect_mask():
    x, c = _case(seed=9, lens=(13, 6), K=4)
    args = (x["q"], x["k_blk"], x["v_blk"], x["k_pages"], x["v_pages"], x["block_table"], x["seq_lens"])
    for b in range(2):
        L = int(x["seq_lens"][b])
        for h in range(4):
            wd = attention_weights(*args, "draft", b, h, page_size=4)
            wv = attention_weights(*args, "verify", b, h, page_size=4)
            np.testing.assert_allclose(wd.sum(1), 1.0, atol=1e-14)
            np.testing.assert_allclose(wv.sum(1), 1.0, atol=1e-14)
            assert np.all(wd > 0)
            for i in range(4):
                assert np.all(wv[i, L + i + 1:] == 0) and np.all(wv[i, :L + i + 1] > 0)


def test_draft_equals_verify_only_on_last_row():
    x, _ = _case(seed=10, lens=(25, 9), K=6)
    dr, ve = _run(x, "draft"), _run(x, "verify")
    assert np.array_equal(dr[:, -1], ve[:, -1])
    assert np.all(np.abs(dr[:, :-1] - ve[:, :-1]).max(axis=-1) > 0)


def test_verify_row_ignores_later_block_rows_draft_does_not():
    x, _ = _case(seed=11, lens=(10, 30), K=6)
    y = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    y["k_blk"][:, 3:] += 1.0
    y["v_blk"][:, 3:] -= 2.0
    ve_x, ve_y = _run(x, "verify"), _run(y, "verify")
    assert np.array_equal(ve_x[:, :3], ve_y[:, :3])
    assert not np.allclose(_run(x, "draft")[:, :3], _run(y, "draft")[:, :3])


def test_gqa_head_groups_are_contiguous():
    # with Hq=4, Hkv=2 heads 0,1 read KV head 0 and heads 2,3 read KV head 1:
    # zeroing KV head 1's values must zero heads 2,3 only
    x, _ = _case(seed=12, lens=(11, 4), K=3)
    x["v_pages"][:, 1] = 0.0
    x["v_blk"][:, :, 1] = 0.0
    o = _run(x, "draft")
    assert np.all(o[:, :, 2:] == 0) and np.all(np.abs(o[:, :, :2]).max(axis=-1) > 0)

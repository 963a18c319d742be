"""Pins for the oracle's consensus (argmax + acceptance) and commit (CPU only)."""
import os

import numpy as np
import pytest

from oracle import accept, argmax_rows, commit_kv, gather_context
from synth import (BF16_SENTINEL, make_consensus_case, make_paged_case, make_tie_logits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_cases.txt")


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, d, a, exp = (s.strip() for s in line.split("|"))
            cases.append((name, [int(t) for t in d.split()], [int(t) for t in a.split()],
                          [int(t) for t in exp.split()]))
    return cases


@pytest.mark.parametrize("name,d,a,exp", _golden_cases(), ids=[c[0] for c in _golden_cases()])
def test_accept_golden(name, d, a, exp):
    n_acc, n_emit, nxt = accept(np.array([d]), np.array([a]))
    assert [int(n_acc[0]), int(n_emit[0]), int(nxt[0])] == exp


def test_accept_batch_matches_per_sequence_and_cumprod():
    rng = np.random.default_rng(0)
    B, K = 64, 16
    a = rng.integers(0, 4, size=(B, K))
    d = np.where(rng.random((B, K)) < 0.8, a, rng.integers(0, 4, size=(B, K)))
    n_acc, n_emit, nxt = accept(d, a)
    # independent statement: length of the leading run of equalities
    run = np.cumprod(d == a, axis=1).sum(axis=1)
    assert np.array_equal(n_acc, run)
    assert np.array_equal(n_emit, np.minimum(run + 1, K))
    assert np.array_equal(nxt, a[np.arange(B), n_emit - 1])


def test_accept_k1_is_greedy():
    rng = np.random.default_rng(1)
    a = rng.integers(0, 50, size=(200, 1))
    d = rng.integers(0, 50, size=(200, 1))
    _, n_emit, nxt = accept(d, a)
    assert np.all(n_emit == 1) and np.array_equal(nxt, a[:, 0])


def test_argmax_brute_force():
    x = np.random.default_rng(2).standard_normal((40, 333)).astype(np.float32)
    x[:, 100:110] = x[:, 0:10]  # plenty of exact duplicates
    ref = []
    for row in x:
        best = 0
        for v in range(1, len(row)):
            if row[v] > row[best]:
                best = v
        ref.append(best)
    assert argmax_rows(x).tolist() == ref


def test_argmax_planted_and_forced_prefix():
    c = make_consensus_case(3, 2, 32, 151936, dist="geometric")
    assert np.array_equal(argmax_rows(c.logits_a), c.a)
    assert np.array_equal(argmax_rows(c.logits_d), c.d)
    n_acc, n_emit, nxt = accept(argmax_rows(c.logits_d), argmax_rows(c.logits_a))
    assert np.array_equal(n_acc, c.n_acc)


@pytest.mark.parametrize("signed_zero", [False, True])
def test_argmax_ties_go_to_lowest_index(signed_zero):
    x, pos = make_tie_logits(4, 16, 1000, n_ties=4, signed_zero=signed_zero)
    assert np.array_equal(argmax_rows(x), pos[:, 0])


def test_commit_writes_exactly_the_emitted_rows():
    layers, B, K = 3, 4, 8
    c = make_paged_case(5, B, K, 4, 2, 16, [0, 15, 16, 37], layers=layers, fill="sentinel")
    rng = np.random.default_rng(6)
    kb = rng.integers(0, 0x7F00, size=(layers, B, K, 2, 16)).astype(np.uint16)
    vb = rng.integers(0, 0x7F00, size=(layers, B, K, 2, 16)).astype(np.uint16)
    n_emit = np.array([8, 1, 5, 3], np.int32)
    kn, vn, lens = commit_kv(c.k_pages, c.v_pages, c.block_table, c.seq_lens, kb, vb, n_emit)
    assert np.array_equal(lens, c.seq_lens + n_emit)
    written = np.zeros(kn.shape[:2] + (16,), bool)   # [layers, pages, slot]
    for b in range(B):
        L, e = int(c.seq_lens[b]), int(n_emit[b])
        for layer in range(layers):
            kc, vc = gather_context(kn[layer], vn[layer], c.block_table, b, L + e, 16)
            k0, v0 = gather_context(c.k_pages[layer], c.v_pages[layer], c.block_table, b, L, 16)
            assert np.array_equal(kc[:L], k0) and np.array_equal(vc[:L], v0)
            assert np.array_equal(kc[L:], kb[layer, b, :e]) and np.array_equal(vc[L:], vb[layer, b, :e])
            for p in range(L, L + e):
                written[layer, c.block_table[b, p // 16], p % 16] = True
    # every slot not written still holds exactly what it held before
    untouched = ~written[:, :, None, :, None].repeat(2, 2).repeat(16, 4)
    assert np.array_equal(kn[untouched], c.k_pages[untouched])
    assert np.array_equal(vn[untouched], c.v_pages[untouched])
    assert np.sum(kn == BF16_SENTINEL) == np.sum(c.k_pages == BF16_SENTINEL) - 2 * 16 * layers * int(n_emit.sum())


def test_commit_crossing_page_boundaries():
    # L = 30: 32 emitted rows cover positions 30..61, i.e. pages 1, 2 and 3
    c = make_paged_case(7, 1, 32, 2, 1, 8, [30], fill="sentinel")
    kb = np.arange(32 * 8, dtype=np.uint16).reshape(1, 1, 32, 1, 8)
    kn, vn, lens = commit_kv(c.k_pages, c.v_pages, c.block_table, c.seq_lens, kb, kb, np.array([32]))
    pages = [c.block_table[0, p // 16] for p in (30, 31, 32, 47, 48, 61)]
    assert kn[0, pages[0], 0, 14, 0] == kb[0, 0, 0, 0, 0]
    assert kn[0, pages[2], 0, 0, 0] == kb[0, 0, 2, 0, 0]
    assert kn[0, pages[4], 0, 0, 0] == kb[0, 0, 18, 0, 0]
    assert kn[0, pages[5], 0, 13, 0] == kb[0, 0, 31, 0, 0]
    assert np.all(kn[0, pages[5], 0, 14:] == BF16_SENTINEL)
    assert lens[0] == 62

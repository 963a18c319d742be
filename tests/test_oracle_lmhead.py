"""Pins for the oracle's LM-head projection and greedy argmax (CPU only)."""
import math

import numpy as np

from oracle import from_bf16
from oracle.lmhead import lm_argmax, lm_logits
from synth import f32_to_bf16_bits, make_lmhead_case


def test_logits_equal_exactly_rounded_sums():
    c = make_lmhead_case(11, 3, 24, 17, plant=False, w_std=0.5)
    h, w = from_bf16(c.hidden), from_bf16(c.weight)
    got = lm_logits(c.hidden, c.weight)
    for r in range(3):
        for v in range(17):
            exact = math.fsum(float(h[r, k]) * float(w[v, k]) for k in range(24))
            assert abs(got[r, v] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_planted_token_wins_by_a_wide_margin():
    c = make_lmhead_case(12, 8, 256, 5000)
    x = lm_logits(c.hidden, c.weight)
    assert np.array_equal(lm_argmax(c.hidden, c.weight), c.targets)
    for r in range(8):
        others = np.delete(x[r], c.targets[r])
        assert x[r, c.targets[r]] - others.max() > 10.0


def test_brute_force_argmax_on_small_case():
    c = make_lmhead_case(13, 5, 32, 41, plant=False, w_std=0.3)
    x = lm_logits(c.hidden, c.weight)
    got = lm_argmax(c.hidden, c.weight)
    for r in range(5):
        best = 0
        for v in range(1, 41):
            if x[r, v] > x[r, best]:
                best = v
        assert got[r] == best


def test_vocabulary_permutation_moves_the_argmax():
    c = make_lmhead_case(14, 6, 64, 300)
    perm = np.random.default_rng(0).permutation(300)
    got = lm_argmax(c.hidden, c.weight[perm])
    inv = np.argsort(perm)
    assert np.array_equal(got, inv[c.targets])


def test_positive_scaling_of_hidden_keeps_the_argmax():
    c = make_lmhead_case(15, 4, 64, 500, plant=False)
    h2 = f32_to_bf16_bits(from_bf16(c.hidden).astype(np.float32) * np.float32(4.0))   # exact
    assert np.array_equal(lm_argmax(h2, c.weight), lm_argmax(c.hidden, c.weight))


def test_duplicated_maximal_row_returns_the_lower_index():
    c = make_lmhead_case(16, 4, 64, 400, dup_rows=4)
    x = lm_logits(c.hidden, c.weight)
    got = lm_argmax(c.hidden, c.weight)
    assert np.array_equal(got, c.targets)
    for r in range(4):
        assert np.count_nonzero(x[r] == x[r].max()) >= 2

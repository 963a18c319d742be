"""The seeded input generators: reproducibility, bf16 rounding, layout."""
import numpy as np
import pytest
import torch

from synth import (BF16_NAN, bf16_bits_to_f32, f32_to_bf16_bits, make_consensus_case,
                   make_paged_case, make_tie_logits, draw_accept_lengths)


def test_bf16_round_to_nearest_even_known_values():
    x = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -2.5, 0.0, -0.0, 3.0e38],
                 dtype=np.float32)
    got = f32_to_bf16_bits(x)
    # 1+2^-8 is halfway between 0x3F80 and 0x3F81 -> even 0x3F80;
    # 1+3*2^-8 is halfway between 0x3F81 and 0x3F82 -> even 0x3F82
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000, 0x8000, 0x7F62]


def test_bf16_matches_torch_rounding():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    back = bf16_bits_to_f32(ref)
    assert np.array_equal(torch.from_numpy(back).numpy(),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_paged_case_reproducible():
    a = make_paged_case(5, 2, 4, 4, 2, 16, [33, 7])
    b = make_paged_case(5, 2, 4, 4, 2, 16, [33, 7])
    for f in ("q", "k_blk", "v_blk", "k_pages", "v_pages", "block_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_page_table_is_a_permutation_and_poison_is_unowned():
    c = make_paged_case(7, 3, 8, 4, 2, 16, [40, 1, 100], slack_pages=3)
    need = [-(-(L + 8) // 16) for L in (40, 1, 100)]
    owned = np.concatenate([c.block_table[b, :need[b]] for b in range(3)])
    assert len(set(owned.tolist())) == len(owned)
    assert owned.min() >= 0 and owned.max() < c.num_pages
    # unused table entries point at a page no sequence owns, filled with NaN
    for b in range(3):
        for e in c.block_table[b, need[b]:]:
            assert e not in set(owned.tolist())
            assert np.all(c.k_pages[0, e] == BF16_NAN)


def test_slots_beyond_context_hold_fill():
    c = make_paged_case(8, 1, 8, 2, 1, 16, [37])
    page = c.block_table[0, 37 // 16]
    assert np.all(c.k_pages[0, page, :, 37 % 16:, :] == BF16_NAN)
    assert not np.any(c.k_pages[0, page, :, :37 % 16, :] == BF16_NAN)


def test_consensus_planting():
    c = make_consensus_case(11, 4, 32, 5000, dist="geometric")
    assert np.array_equal(np.argmax(c.logits_a, axis=-1), c.a)
    assert np.array_equal(np.argmax(c.logits_d, axis=-1), c.d)
    for b in range(4):
        j = int(c.n_acc[b])
        assert np.array_equal(c.d[b, :j], c.a[b, :j])
        if j < 32:
            assert c.d[b, j] != c.a[b, j]


def test_geometric_accept_lengths_statistics():
    rng = np.random.default_rng(0)
    n = draw_accept_lengths(rng, 200000, 32, "geometric", 0.15)
    assert n.min() == 0 and n.max() == 32
    assert abs((n == 0).mean() - 0.15) < 0.005
    n_emit = np.where(n < 32, n + 1, 32)
    expected = sum(0.85**k for k in range(32))   # E[n_emit] = 6.63
    assert abs(n_emit.mean() - expected) < 0.05


@pytest.mark.parametrize("signed_zero", [False, True])
def test_tie_logits(signed_zero):
    x, pos = make_tie_logits(3, 5, 300, n_ties=3, signed_zero=signed_zero)
    for r in range(5):
        m = x[r].max()
        assert set(np.nonzero(x[r] == m)[0].tolist()) == set(pos[r].tolist())

"""Pins for the oracle's temperature > 0 consensus (CPU only)."""
import numpy as np
import pytest

from oracle import accept
from oracle.sampling import inverse_cdf, sample_rows, softmax_t, speculative_accept

GRID = 2000
U = (np.arange(GRID) + 0.5) / GRID          # midpoints of a uniform grid on [0, 1)


def test_inverse_cdf_hand_worked():
    w = [1.0, 2.0, 3.0, 4.0]                 # cumulative 1, 3, 6, 10
    assert [inverse_cdf(w, u) for u in (0.0, 0.05, 0.0999, 0.1, 0.3, 0.6, 0.9999)] == [0, 0, 0, 1, 2, 3, 3]
    assert inverse_cdf([0.0, 0.0, 5.0, 0.0], 0.0) == 2    # u = 0: the first token with weight
    assert inverse_cdf([0.0, 3.0, 0.0], 0.999999) == 1    # never a zero-weight token


def test_softmax_with_temperature_closed_form():
    z = np.array([0.0, np.log(2.0), np.log(4.0)])
    np.testing.assert_allclose(softmax_t(z, 1.0), [1 / 7, 2 / 7, 4 / 7], rtol=1e-14)
    np.testing.assert_allclose(softmax_t(z, 2.0), np.array([1, 2 ** 0.5, 2]) / (3 + 2 ** 0.5), rtol=1e-14)
    with pytest.raises(ValueError):
        softmax_t(z, 0.0)


def test_sampling_frequencies_follow_the_distribution():
    z = np.array([0.3, -1.0, 2.0, 0.0, 0.5])
    p = softmax_t(z, 0.7)
    freq = np.bincount([sample_rows(z[None], 0.7, [u])[0] for u in U], minlength=5) / GRID
    np.testing.assert_allclose(freq, p, atol=1.0 / GRID)


def _greedy_case(seed, B, K, V):
    rng = np.random.default_rng(seed)
    za = rng.standard_normal((B, K, V)) * 3.0
    zd = rng.standard_normal((B, K, V)) * 3.0
    a = za.argmax(-1)
    d = zd.argmax(-1)
    n = rng.integers(0, K + 1, size=B)
    for b in range(B):                        # the draft agrees with the AR view on a prefix
        zd[b, :n[b]] = za[b, :n[b]]
        d[b, :n[b]] = a[b, :n[b]]
    return za, zd, d


def test_zero_temperature_limit_is_the_greedy_rule():
    za, zd, d = _greedy_case(0, 6, 8, 50)
    rng = np.random.default_rng(1)
    u_acc, u_res = rng.random((6, 8)), rng.random((6, 8))
    tok, n_acc, n_emit, nxt = speculative_accept(zd, za, d, 1e-4, u_acc, u_res)
    g_acc, g_emit, g_nxt = accept(d, za.argmax(-1))
    assert np.array_equal(n_acc, g_acc) and np.array_equal(n_emit, g_emit) and np.array_equal(nxt, g_nxt)
    a = za.argmax(-1)
    for b in range(6):
        assert list(tok[b, :n_emit[b]]) == list(a[b, :n_emit[b]])
        assert np.all(tok[b, n_emit[b]:] == -1)


def test_a_draft_with_the_ar_distribution_is_always_accepted():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((3, 8, 40))
    d = sample_rows(z, 0.9, rng.random((3, 8)))
    tok, n_acc, n_emit, nxt = speculative_accept(z, z, d, 0.9, rng.random((3, 8)) * 0.999, rng.random((3, 8)))
    assert np.all(n_acc == 8) and np.all(n_emit == 8)
    assert np.array_equal(tok, d) and np.array_equal(nxt, d[:, -1])


def _emitted_distribution(zd, za, T, row):
    """Distribution of the token emitted at `row`, integrated over the draft
    sample, u_acc and u_res on a uniform grid (earlier rows are forced to be
    accepted by drafting the AR view's own distribution there)."""
    K, V = za.shape
    q = softmax_t(zd[row], T)
    dist = np.zeros(V)
    for d_tok in range(V):
        if q[d_tok] == 0:
            continue
        d = np.zeros((1, K), np.int64)
        d[0, row] = d_tok
        for u in U[::20]:                            # acceptance test: 100 points
            u_acc = np.zeros((1, K))
            u_acc[0, row] = u
            tok, n_acc, _, _ = speculative_accept(zd[None], za[None], d, T, u_acc, np.zeros((1, K)))
            if n_acc[0] > row:
                dist[d_tok] += q[d_tok] / 100
            else:                                    # rejected: integrate the residual draw
                for ur in U[::20]:
                    u_res = np.zeros((1, K))
                    u_res[0, row] = ur
                    t, _, _, _ = speculative_accept(zd[None], za[None], d, T, u_acc, u_res)
                    dist[t[0, row]] += q[d_tok] / 100 / 100
    return dist


@pytest.mark.parametrize("T", [0.5, 1.0, 2.5])
def test_emitted_token_follows_the_ar_distribution(T):
    rng = np.random.default_rng(3)
    K, V = 2, 5
    za = rng.standard_normal((K, V)) * 1.5
    zd = rng.standard_normal((K, V)) * 1.5
    zd[0] = za[0]                                    # row 0 always accepted (for the row-1 check)
    zd0 = zd.copy()
    zd0[0] = rng.standard_normal(V)                  # a different draft at row 0 (for the row-0 check)
    for row, zdr in ((0, zd0), (1, zd)):
        got = _emitted_distribution(zdr, za, T, row)
        np.testing.assert_allclose(got, softmax_t(za[row], T), atol=0.02)


def test_residual_excludes_the_rejected_token_when_the_draft_overweights_it():
    za = np.log(np.array([[0.5, 0.3, 0.2]]))
    zd = np.log(np.array([[0.1, 0.1, 0.8]]))
    d = np.array([[2]])
    # p(2)/q(2) = 0.25: u = 0.5 rejects; residual max(0, p - q) = [0.4, 0.2, 0]
    tok, n_acc, n_emit, nxt = speculative_accept(zd[None], za[None], d, 1.0, np.array([[0.5]]),
                                                 np.array([[0.7]]))
    assert n_acc[0] == 0 and n_emit[0] == 1 and tok[0, 0] == 1 and nxt[0] == 1   # 0.7 * 0.6 > 0.4
    tok, n_acc, _, _ = speculative_accept(zd[None], za[None], d, 1.0, np.array([[0.2]]), np.array([[0.7]]))
    assert n_acc[0] == 1 and tok[0, 0] == 2                                          # 0.2 * 0.8 < 0.2


def test_empty_residual_draws_from_the_ar_distribution():
    """The views agree exactly (p == q) and the drafted token has probability
    0 in both: exp underflows to 0 in fp64 for a logit 1000 below the row
    maximum.  The acceptance test 0 * u < 0 fails, so the row is rejected,
    and the residual max(0, p - q) is 0 everywhere.  The emitted token is
    then drawn from p itself.  Hand-worked: p = q = [1/4, 3/4, 0]."""
    z = np.array([[[0.0, np.log(3.0), -1000.0]]])
    d = np.array([[2]])
    assert softmax_t(z[0, 0], 1.0)[2] == 0.0
    for u_res, want in ((0.0, 0), (0.2, 0), (0.2499, 0), (0.2501, 1), (0.9, 1)):
        tok, n_acc, n_emit, nxt = speculative_accept(z, z, d, 1.0, np.array([[0.3]]), np.array([[u_res]]))
        assert (n_acc[0], n_emit[0], tok[0, 0], nxt[0]) == (0, 1, want, want), u_res
    # the same with two rows: row 0 is accepted (a token of positive weight,
    # equal views), row 1 has the zero-probability draft
    z2 = np.concatenate([z, z], axis=1)
    tok, n_acc, n_emit, nxt = speculative_accept(z2, z2, np.array([[1, 2]]), 1.0, np.array([[0.99, 0.5]]),
                                                 np.array([[0.0, 0.6]]))
    assert (n_acc[0], n_emit[0], list(tok[0]), nxt[0]) == (1, 2, [1, 1], 1)

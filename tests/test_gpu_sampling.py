"""GPU parity of the temperature > 0 consensus (orthrus_sample,
orthrus_accept_sampled) against the oracle, draw for draw on the same
uniforms.

Both sides evaluate the probabilities and cumulative weights in fp64 from the
same fp32 logits, so their decisions can differ only when a uniform falls
within about 1e-15 (relative) of a threshold; the seeded cases below hold no
such uniform, and every token, count and anchor must be equal."""
import numpy as np
import pytest
import torch

from gpu_helpers import i32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).cuda()


def llm_logits(rng, shape, scale=3.0, peak=8.0):
    """Logits with a heavy head: N(0, scale) plus a few lifted tokens per row."""
    z = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    V = shape[-1]
    flat = z.reshape(-1, V)
    for r in range(flat.shape[0]):
        top = rng.choice(V, size=min(4, V), replace=False)
        flat[r, top] += np.float32(peak) * rng.random(len(top), dtype=np.float32)
    return z


def uniforms(rng, shape):
    return rng.random(shape, dtype=np.float32)    # float32 in [0, 1)


# 1 x 4.2 M words: more than 1024 statistics chunks per row, so the draw reads
# the chunk weights from global memory instead of LDS
# 48 x 151936: 2048-entry statistics chunks (1024-entry ones would need more
# wavefronts than the GPU holds at once)
@pytest.mark.parametrize("rows,V,T", [(32, 151936, 1.0), (32, 151936, 0.6), (7, 1000, 2.5), (1, 1, 1.0),
                                      (65, 5000, 0.3), (3, 20000, 1.0), (1, 4200000, 0.8), (48, 151936, 0.8)])
def test_sample_matches_oracle(lib, rows, V, T):
    from oracle.sampling import sample_rows
    rng = np.random.default_rng(rows * 7 + V)
    z = llm_logits(rng, (rows, V))
    u = uniforms(rng, rows)
    u[0] = 0.0
    if rows > 1:
        u[1] = np.float32(1.0) - np.float32(2.0 ** -24)
    out = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    lib.orthrus_sample(f32_dev(z), T, f32_dev(u), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), sample_rows(z, T, u))


def test_one_workspace_serves_calls_in_a_row(lib):
    """One workspace, never cleared, serves calls of different shapes one
    after another, for both entry points (garbage from the previous call is
    never read)."""
    from oracle.sampling import sample_rows, speculative_accept
    rng = np.random.default_rng(21)
    shapes = ((32, 151936, 1.0), (5, 151936, 0.7), (64, 151936, 1.3), (3, 1000, 1.0), (32, 151936, 0.9))
    n = max(lib.orthrus_sample_workspace_bytes(r, V) for r, V, _ in shapes)
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    for rows, V, T in shapes:
        z = llm_logits(rng, (rows, V))
        u = uniforms(rng, rows)
        out = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
        lib.orthrus_sample(f32_dev(z), T, f32_dev(u), out, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), sample_rows(z, T, u)), (rows, V, T)
    cases = ((31, 4, 32, 151936, 0.8, 0.9), (32, 1, 32, 151936, 1.0, 0.95), (33, 4, 8, 3000, 1.2, 0.7))
    n = max(lib.orthrus_accept_sampled_workspace_bytes(B, K, V) for _, B, K, V, _, _ in cases)
    wa = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    for seed, B, K, V, T, agree in cases:
        zd, za, d, u_acc, u_res = _consensus_case(seed, B, K, V, T, agree)
        outs = [torch.full(s, -7, dtype=torch.int32, device="cuda") for s in ((B, K), (B,), (B,), (B,))]
        lib.orthrus_accept_sampled(f32_dev(zd), f32_dev(za), i32_dev(d), T, f32_dev(u_acc), f32_dev(u_res),
                                   *outs, workspace=wa)
        torch.cuda.synchronize()
        ref = speculative_accept(zd, za, d, T, u_acc, u_res)
        for got, want in zip(outs, ref):
            assert np.array_equal(got.cpu().numpy(), want), (seed, B, K)
    # and the consensus workspace then serves orthrus_sample too
    z = llm_logits(rng, (64, 151936))
    u = uniforms(rng, 64)
    out = torch.full((64,), -7, dtype=torch.int32, device="cuda")
    assert lib.orthrus_sample_workspace_bytes(64, 151936) <= wa.numel()
    lib.orthrus_sample(f32_dev(z), 1.0, f32_dev(u), out, workspace=wa)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), sample_rows(z, 1.0, u))


def test_sample_frequencies_on_a_uniform_grid(lib):
    """4096 draws of one 6-token row on a uniform grid reproduce softmax(z/T)."""
    from oracle.sampling import softmax_t
    z = np.array([1.0, -0.5, 2.0, 0.0, 0.3, -2.0], np.float32)
    n = 4096
    u = ((np.arange(n) + 0.5) / n).astype(np.float32)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    lib.orthrus_sample(f32_dev(np.tile(z, (n, 1))), 0.8, f32_dev(u), out)
    torch.cuda.synchronize()
    freq = np.bincount(out.cpu().numpy(), minlength=6) / n
    np.testing.assert_allclose(freq, softmax_t(z, 0.8), atol=1.0 / n)


def _consensus_case(seed, B, K, V, T, agree=0.7):
    """Draft logits, AR logits that agree with them on part of each row, and
    drafted tokens sampled from the draft view (as orthrus_sample draws them)."""
    from oracle.sampling import sample_rows
    rng = np.random.default_rng(seed)
    zd = llm_logits(rng, (B, K, V))
    za = (np.float32(agree) * zd + np.float32(1 - agree) * llm_logits(rng, (B, K, V))).astype(np.float32)
    d = sample_rows(zd, T, uniforms(rng, (B, K))).astype(np.int32)
    return zd, za, d, uniforms(rng, (B, K)), uniforms(rng, (B, K))


def run_accept(lib, zd, za, d, T, u_acc, u_res):
    B, K, _ = za.shape
    outs = [torch.full(s, -7, dtype=torch.int32, device="cuda") for s in ((B, K), (B,), (B,), (B,))]
    lib.orthrus_accept_sampled(f32_dev(zd), f32_dev(za), i32_dev(d), T, f32_dev(u_acc), f32_dev(u_res), *outs)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in outs]


@pytest.mark.parametrize("seed,B,K,V,T,agree", [
    (1, 1, 32, 151936, 1.0, 0.9),     # the 8B vocabulary
    (2, 4, 32, 151936, 0.7, 0.95),
    (3, 8, 8, 3000, 1.5, 0.8),
    (4, 3, 1, 500, 1.0, 0.5),          # K = 1: every step emits one AR-distributed token
    (5, 2, 64, 2048, 0.5, 0.98),
    (6, 1, 64, 151936, 0.9, 0.9),      # K = 64 at the 8B vocabulary: 149 chunks per row, 8 threads per row
    (7, 8, 8, 151936, 1.0, 0.6),       # 5 residual chunks per workgroup: two rounds of the 4 chunk groups
    (8, 2, 64, 151936, 0.8, 0.9),      # K = 64 with 2 residual chunks per workgroup
])
def test_accept_sampled_matches_oracle(lib, seed, B, K, V, T, agree):
    from oracle.sampling import speculative_accept
    zd, za, d, u_acc, u_res = _consensus_case(seed, B, K, V, T, agree)
    tok, n_acc, n_emit, nxt = run_accept(lib, zd, za, d, T, u_acc, u_res)
    r_tok, r_acc, r_emit, r_nxt = speculative_accept(zd, za, d, T, u_acc, u_res)
    print(f"seed {seed}: n_acc {list(r_acc)}", flush=True)
    assert np.array_equal(n_acc, r_acc) and np.array_equal(n_emit, r_emit) and np.array_equal(nxt, r_nxt)
    assert np.array_equal(tok, r_tok)


def test_equal_views_accept_every_token(lib):
    zd, _, d, u_acc, u_res = _consensus_case(6, 2, 32, 40000, 1.0)
    tok, n_acc, n_emit, nxt = run_accept(lib, zd, zd, d, 1.0, u_acc, u_res)
    assert np.all(n_acc == 32) and np.all(n_emit == 32)
    assert np.array_equal(tok, d) and np.array_equal(nxt, d[:, -1])


def test_low_temperature_is_the_greedy_consensus(lib):
    """T = 1e-3 with logit gaps >> T: the sampled consensus equals orthrus_accept."""
    rng = np.random.default_rng(7)
    B, K, V = 3, 32, 5000
    za = np.stack([rng.permutation(V) for _ in range(B * K)]).reshape(B, K, V).astype(np.float32) * np.float32(0.5)
    zd = za.copy()
    a = za.argmax(-1).astype(np.int32)
    d = a.copy()
    for b, m in enumerate((5, 0, 32)):                 # first disagreement at 5, 0, none
        if m < K:
            zd[b, m:] = rng.permutation(zd[b, m:].ravel()).reshape(K - m, V)
            d[b, m:] = zd[b, m:].argmax(-1)
            d[b, m] = (a[b, m] + 1) % V
            zd[b, m, d[b, m]] = zd[b, m].max() + 1.0
    tok, n_acc, n_emit, nxt = run_accept(lib, zd, za, d, 1e-3, uniforms(rng, (B, K)), uniforms(rng, (B, K)))
    g = [torch.full(s, -7, dtype=torch.int32, device="cuda") for s in ((B, K), (B,), (B,), (B,))]
    lib.orthrus_accept(f32_dev(za), i32_dev(d), *g)
    torch.cuda.synchronize()
    ga, g_acc, g_emit, g_nxt = (t.cpu().numpy() for t in g)
    assert list(g_acc) == [5, 0, 32]
    assert np.array_equal(n_acc, g_acc) and np.array_equal(n_emit, g_emit) and np.array_equal(nxt, g_nxt)
    for b in range(B):
        assert np.array_equal(tok[b, :n_emit[b]], ga[b, :n_emit[b]])


def test_rejects_bad_temperature_and_small_workspace(lib):
    z = torch.zeros((2, 10), dtype=torch.float32, device="cuda")
    u = torch.zeros(2, dtype=torch.float32, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(lib.OrthrusError, match="INVALID_ARG"):
        lib.orthrus_sample(z, 0.0, u, out)
    with pytest.raises(lib.OrthrusError, match="WORKSPACE_TOO_SMALL"):
        lib.orthrus_sample(z, 1.0, u, out, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))


def test_empty_residual_draws_from_the_ar_distribution(lib):
    """Equal views (p == q) and drafted tokens whose logit sits 1000 below the
    row maximum: p = q = 0 in fp64 for them, so the row is rejected and the
    residual max(0, p - q) is empty.  The emitted token must be the oracle's
    draw from p with u_res (the kernel's fallback path)."""
    from oracle.sampling import speculative_accept
    rng = np.random.default_rng(11)
    B, K, V = 3, 32, 151936
    z = llm_logits(rng, (B, K, V))
    d = z.argmax(-1).astype(np.int32)                # accepted rows: each row's most likely token
    for b, j in enumerate((0, 7, 31)):               # first zero-probability draft at row j
        tok = int(rng.integers(0, V))
        z[b, j, tok] = z[b, j].max() - np.float32(1000.0)
        d[b, j] = tok
    u_acc = uniforms(rng, (B, K)) * np.float32(0.5)  # rows with p = q > 0 are accepted
    u_res = uniforms(rng, (B, K))
    tok, n_acc, n_emit, nxt = run_accept(lib, z, z, d, 1.0, u_acc, u_res)
    r_tok, r_acc, r_emit, r_nxt = speculative_accept(z, z, d, 1.0, u_acc, u_res)
    assert list(r_acc) == [0, 7, 31]
    assert np.array_equal(n_acc, r_acc) and np.array_equal(n_emit, r_emit) and np.array_equal(nxt, r_nxt)
    assert np.array_equal(tok, r_tok)

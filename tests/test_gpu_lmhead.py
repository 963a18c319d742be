"""GPU parity of the fused LM head + argmax (orthrus_lmhead_argmax,
orthrus_lmhead_accept) against the oracle.

The tokens are integers decided by floating point: the fused kernel's own
fp32 logits (written on request by the same launch) must give exactly the
same argmax, those logits must lie within the fp32 summation bound of the
fp64 oracle logits, and the chosen token must be an oracle maximum up to that
bound (exactly the oracle's token where a planted winner leads by far)."""
import numpy as np
import pytest
import torch

from gpu_helpers import bf16_dev, i32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def run(dv, c, with_logits=True):
    h, w = bf16_dev(c.hidden), bf16_dev(c.weight)
    R, V = c.hidden.shape[0], c.weight.shape[0]
    out = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    logits = torch.full((R, V), float("nan"), dtype=torch.float32, device="cuda") if with_logits else None
    dv.orthrus_lmhead_argmax(h, w, out, logits=logits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (logits.cpu().numpy() if with_logits else None)


def check_against_oracle(c, tok, logits, exact_tokens):
    from oracle import from_bf16
    from oracle.lmhead import lm_argmax, lm_logits
    ref = lm_logits(c.hidden, c.weight)
    # |fp32 sum - exact| <= hidden * 2^-23 * sum_k |h_k w_k| for every logit
    bound = c.hidden.shape[1] * 2.0 ** -23 * (np.abs(from_bf16(c.hidden)) @ np.abs(from_bf16(c.weight)).T)
    # 1. the fused argmax is the argmax of the launch's own fp32 logits, bit for bit
    own = logits.max(axis=1, keepdims=True)
    assert np.array_equal(tok, (logits == own).argmax(axis=1).astype(np.int32))
    # 2. those logits are the oracle's within the summation bound
    err = np.abs(logits - ref)
    assert np.all(err <= bound + 1e-30), f"max err {err.max():.3e} vs bound {bound.max():.3e}"
    # 3. the chosen token is an oracle maximum up to twice the bound
    rows = np.arange(len(tok))
    assert np.all(ref[rows, tok] >= ref.max(axis=1) - 2 * bound.max(axis=1))
    if exact_tokens:
        assert np.array_equal(tok, lm_argmax(c.hidden, c.weight))


# up to 32 rows: the streaming kernel (vocabulary ranges, 32 rows staged in
# LDS with the weight tiles); 33-128 rows: one GEMM row tile over ranges
@pytest.mark.parametrize("R,Hd,V", [(32, 256, 5000), (7, 128, 777), (1, 64, 1), (40, 128, 3000),
                                    (32, 4096, 20011), (3, 64, 10), (65, 192, 300), (9, 5120, 700),
                                    (8, 8192, 3000), (5, 5184, 1000), (33, 576, 2049)])
def test_planted_winner(lib, R, Hd, V):
    from synth import make_lmhead_case
    c = make_lmhead_case(R * 31 + V, R, Hd, V)
    tok, logits = run(lib, c)
    check_against_oracle(c, tok, logits, exact_tokens=True)
    assert np.array_equal(tok, c.targets)


@pytest.mark.parametrize("R,Hd,V", [(32, 4096, 50000), (16, 512, 7777)])
def test_random_rows_without_a_winner(lib, R, Hd, V):
    from synth import make_lmhead_case
    c = make_lmhead_case(R + Hd + V, R, Hd, V, plant=False)
    tok, logits = run(lib, c)
    check_against_oracle(c, tok, logits, exact_tokens=False)


def test_duplicated_maximum_returns_lowest_index(lib):
    from synth import make_lmhead_case
    c = make_lmhead_case(5, 32, 512, 9000, dup_rows=32)
    tok, logits = run(lib, c)
    assert np.array_equal(tok, c.targets)
    rows = np.arange(32)
    assert np.all(np.count_nonzero(logits == logits[rows, tok][:, None], axis=1) >= 2)


def test_qwen3_8b_vocabulary_full_size(lib):
    """The 8B shape: 32 rows, hidden 4096, vocabulary 151936 (1.24 GB of weights)."""
    from synth import make_lmhead_case
    c = make_lmhead_case(8, 32, 4096, 151936)
    tok, logits = run(lib, c)
    check_against_oracle(c, tok, logits, exact_tokens=True)
    tok2, _ = run(lib, c, with_logits=False)          # the fast path gives the same tokens
    assert np.array_equal(tok, tok2)


@pytest.mark.parametrize("n_acc", [0, 3, 31, 32])
def test_lmhead_accept_matches_oracle(lib, n_acc):
    from oracle import accept
    from synth import make_lmhead_case
    B, K, Hd, V = 2, 32, 1024, 30000
    c = make_lmhead_case(100 + n_acc, B * K, Hd, V)
    a = c.targets.reshape(B, K)
    d = a.copy()
    for b in range(B):
        if n_acc < K:
            d[b, n_acc] = (a[b, n_acc] + 1) % V
    h = bf16_dev(c.hidden).view(B, K, Hd)
    w = bf16_dev(c.weight)
    outs = [torch.full(s, -7, dtype=torch.int32, device="cuda") for s in ((B, K), (B,), (B,), (B,))]
    lib.orthrus_lmhead_accept(h, w, i32_dev(d), *outs)
    torch.cuda.synchronize()
    ar, na, ne, nx = (t.cpu().numpy() for t in outs)
    ref_na, ref_ne, ref_nx = accept(d, a)
    assert np.array_equal(ar, a)
    assert np.array_equal(na, ref_na) and np.array_equal(ne, ref_ne) and np.array_equal(nx, ref_nx)
    assert np.all(na == n_acc)


# more than 64 rows take a GEMM-tiled kernel: up to 128 rows (one row tile)
# the narrow kernel over contiguous vocabulary ranges (one per CU; 65 rows over
# 300 words leaves most ranges one or two words long), above that 256 x 128
# tiles, or 256 x 256 tiles where those fill rounds of 256 workgroups better.
# Every shape below has ragged row and vocabulary tails; 300 rows over 25523
# words (100 vocabulary tiles) take the wide kernel (200 workgroups against
# 300); hidden 64 has fewer hidden tiles than either ring has stages in flight.
@pytest.mark.parametrize("R,Hd,V", [(65, 192, 300), (128, 320, 4099), (129, 256, 5000), (130, 64, 777),
                                    (257, 128, 1000), (300, 1024, 20011), (200, 8192, 3000),
                                    (300, 64, 25523), (300, 1024, 25523), (96, 4096, 151936)])
def test_gemm_tiled_planted_winner(lib, R, Hd, V):
    from synth import make_lmhead_case
    c = make_lmhead_case(R * 13 + V, R, Hd, V)
    tok, logits = run(lib, c)
    check_against_oracle(c, tok, logits, exact_tokens=True)
    assert np.array_equal(tok, c.targets)


def _logits_of(lib, h, w, lo, hi):
    out = torch.full((hi - lo,), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((hi - lo, w.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    lib.orthrus_lmhead_argmax(h[lo:hi].contiguous(), w, out, logits=lg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lg.cpu().numpy()


def test_gemm_kernels_agree_bit_for_bit(lib):
    """Both GEMM kernels keep one fp32 running sum per logit over the hidden
    dimension in 16-element products taken in increasing order, so the wide
    kernel (300 rows over 100 vocabulary tiles) and the narrow one (the same
    rows in calls of 129 and 171) give identical logits and tokens."""
    from synth import make_lmhead_case
    c = make_lmhead_case(31, 300, 1024, 25523, plant=False)
    tok_all, logits_all = run(lib, c)
    check_against_oracle(c, tok_all, logits_all, exact_tokens=False)
    h, w = bf16_dev(c.hidden), bf16_dev(c.weight)
    for lo, hi in ((0, 129), (129, 300)):
        tok, lg = _logits_of(lib, h, w, lo, hi)
        assert np.array_equal(lg.view(np.uint32), logits_all[lo:hi].view(np.uint32)), (lo, hi)
        assert np.array_equal(tok, tok_all[lo:hi]), (lo, hi)


@pytest.mark.parametrize("Hd", [1024, 4096, 8192])
def test_a_rows_logits_do_not_depend_on_the_call(lib, Hd):
    """Every LM-head kernel keeps one fp32 running sum per logit over 16-element
    products in increasing hidden order, so a row's logits are the same bits
    in calls of 1, 32 (the streaming kernel), 33-128 (vocabulary ranges of
    one 128-row tile) and 512 rows (wide GEMM tiles).  Greedy decoding of B
    sequences (B rows) and the Orthrus verify pass (B*K rows) therefore pick
    the same AR tokens even at near-ties."""
    from synth import make_lmhead_case
    c = make_lmhead_case(37 + Hd, 512, Hd, 3001, plant=False)
    h, w = bf16_dev(c.hidden), bf16_dev(c.weight)
    tok_all, lg_all = _logits_of(lib, h, w, 0, 512)
    for lo, hi in ((0, 1), (5, 37), (63, 64), (0, 32), (100, 196), (200, 328), (511, 512)):
        tok, lg = _logits_of(lib, h, w, lo, hi)
        assert np.array_equal(lg.view(np.uint32), lg_all[lo:hi].view(np.uint32)), (lo, hi)
        assert np.array_equal(tok, tok_all[lo:hi]), (lo, hi)


def test_gemm_tiled_random_rows(lib):
    from synth import make_lmhead_case
    c = make_lmhead_case(77, 160, 2048, 30000, plant=False)
    tok, logits = run(lib, c)
    check_against_oracle(c, tok, logits, exact_tokens=False)


def test_gemm_tiled_8b_vocabulary_batch_16(lib):
    """B*K = 512 rows (batch 16, K 32) against the 8B vocabulary; the tokens of
    the logits-free path equal those of the launch that also writes logits."""
    from synth import make_lmhead_case
    c = make_lmhead_case(9, 512, 4096, 151936)
    tok, logits = run(lib, c)
    check_against_oracle(c, tok, logits, exact_tokens=True)
    tok2, _ = run(lib, c, with_logits=False)
    assert np.array_equal(tok, tok2)


def test_gemm_tiled_accept_batch_16(lib):
    from oracle import accept
    from synth import make_lmhead_case
    B, K, Hd, V = 16, 32, 1024, 30000
    c = make_lmhead_case(101, B * K, Hd, V)
    a = c.targets.reshape(B, K)
    d = a.copy()
    rng = np.random.default_rng(4)
    for b in range(B):
        m = int(rng.integers(0, K + 1))
        if m < K:
            d[b, m] = (a[b, m] + 1) % V
    h = bf16_dev(c.hidden).view(B, K, Hd)
    outs = [torch.full(s, -7, dtype=torch.int32, device="cuda") for s in ((B, K), (B,), (B,), (B,))]
    lib.orthrus_lmhead_accept(h, bf16_dev(c.weight), i32_dev(d), *outs)
    torch.cuda.synchronize()
    ar, na, ne, nx = (t.cpu().numpy() for t in outs)
    ref_na, ref_ne, ref_nx = accept(d, a)
    assert np.array_equal(ar, a)
    assert np.array_equal(na, ref_na) and np.array_equal(ne, ref_ne) and np.array_equal(nx, ref_nx)


@pytest.mark.parametrize("R,Hd,V", [(129, 256, 5000), (256, 512, 30011), (512, 1024, 151936),
                                    (1024, 256, 7777), (700, 128, 22991)])
def test_tokens_do_not_depend_on_the_logits_output(lib, R, Hd, V):
    """A launch that also writes the logits and one that does not take the
    same products in the same order, so on rows without a planted winner the
    tokens agree exactly, near-ties included (narrow and wide GEMM tiles, one
    to four row tiles)."""
    from synth import make_lmhead_case
    c = make_lmhead_case(R + 3 * V, R, Hd, V, plant=False)
    tok, logits = run(lib, c)
    check_against_oracle(c, tok, logits, exact_tokens=False)
    tok2, _ = run(lib, c, with_logits=False)
    assert np.array_equal(tok, tok2)


def test_gemm_tiled_accept_batch_16_8b_vocabulary(lib):
    """The fused acceptance at batch 16, K 32 over the 8B vocabulary (512 rows,
    wide GEMM tiles) against the oracle's prefix rule on the planted AR
    tokens."""
    from oracle import accept
    from synth import make_lmhead_case
    B, K, Hd, V = 16, 32, 512, 151936
    c = make_lmhead_case(102, B * K, Hd, V)
    a = c.targets.reshape(B, K)
    d = a.copy()
    rng = np.random.default_rng(5)
    for b in range(B):
        m = int(rng.integers(0, K + 1))
        if m < K:
            d[b, m] = (a[b, m] + 7) % V
    h = bf16_dev(c.hidden).view(B, K, Hd)
    outs = [torch.full(s, -7, dtype=torch.int32, device="cuda") for s in ((B, K), (B,), (B,), (B,))]
    lib.orthrus_lmhead_accept(h, bf16_dev(c.weight), i32_dev(d), *outs)
    torch.cuda.synchronize()
    ar, na, ne, nx = (t.cpu().numpy() for t in outs)
    ref_na, ref_ne, ref_nx = accept(d, a)
    assert np.array_equal(ar, a)
    assert np.array_equal(na, ref_na) and np.array_equal(ne, ref_ne) and np.array_equal(nx, ref_nx)

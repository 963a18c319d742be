"""GPU parity of orthrus_argmax / orthrus_accept / orthrus_commit_kv: bit-exact
against the oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import bf16_dev, bf16_host_bits, i32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def gpu_argmax(dv, x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    out = torch.full(x.shape[:-1], -7, dtype=torch.int32, device="cuda")
    dv.orthrus_argmax(t, out)
    return out.cpu().numpy()


@pytest.mark.parametrize("rows,V", [(8, 1024), (32, 151936), (3, 32000), (5, 1001), (1, 1), (64, 7)])
def test_argmax_random_rows(lib, rows, V):
    from oracle import argmax_rows
    x = np.random.default_rng(rows * 7 + V).standard_normal((rows, V)).astype(np.float32)
    assert np.array_equal(gpu_argmax(lib, x), argmax_rows(x))


@pytest.mark.parametrize("signed_zero", [False, True])
@pytest.mark.parametrize("V", [151936, 999])
def test_argmax_ties_lowest_index(lib, signed_zero, V):
    from oracle import argmax_rows
    from synth import make_tie_logits
    x, pos = make_tie_logits(17, 12, V, n_ties=4, signed_zero=signed_zero)
    got = gpu_argmax(lib, x)
    assert np.array_equal(got, argmax_rows(x)) and np.array_equal(got, pos[:, 0])


def test_argmax_extreme_values(lib):
    from oracle import argmax_rows
    x = np.full((4, 5000), -np.inf, dtype=np.float32)
    x[0, 17] = -3.4e38
    x[1, :] = np.finfo(np.float32).max
    x[2, 4999] = np.float32(1e-45)   # smallest denormal beats zeros/-inf
    x[2, :10] = 0.0
    x[3, 123] = np.inf
    assert np.array_equal(gpu_argmax(lib, x), argmax_rows(x))


def _accept_gpu(dv, logits_a, d):
    B, K, V = logits_a.shape
    la = torch.from_numpy(logits_a).cuda()
    dd = i32_dev(d)
    a = torch.empty((B, K), dtype=torch.int32, device="cuda")
    outs = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(3)]
    dv.orthrus_accept(la, dd, a, *outs)
    return a.cpu().numpy(), *(o.cpu().numpy() for o in outs)


@pytest.mark.parametrize("name,seed,B,K,V,dist", [
    ("tiny", 1, 1, 8, 1024, "uniform"),
    ("qwen3_8b", 2, 1, 32, 151936, "geometric"),
    ("ragged16", 4, 16, 32, 151936, "geometric"),
    ("odd_vocab", 5, 3, 5, 1001, "uniform"),
    ("k64", 6, 2, 64, 4096, "uniform"),
    # 38 chunk keys per row and 48 rows: more rows than one 256-thread pass
    # holds, so the 1024-thread reduction runs
    ("k48_big_vocab", 7, 1, 48, 151936, "geometric"),
    ("k64_big_vocab", 8, 2, 64, 151936, "uniform"),
])
def test_accept_matches_oracle(lib, name, seed, B, K, V, dist):
    from oracle import accept, argmax_rows
    from synth import make_consensus_case
    c = make_consensus_case(seed, B, K, V, dist=dist)
    d_gpu = gpu_argmax(lib, c.logits_d)
    assert np.array_equal(d_gpu, argmax_rows(c.logits_d))
    a, n_acc, n_emit, nxt = _accept_gpu(lib, c.logits_a, d_gpu)
    a_ref = argmax_rows(c.logits_a)
    ref = accept(d_gpu, a_ref)
    assert np.array_equal(a, a_ref)
    assert np.array_equal(n_acc, ref[0]) and np.array_equal(n_emit, ref[1])
    assert np.array_equal(nxt, ref[2])
    assert np.array_equal(n_acc, c.n_acc)    # the drawn forced-match length


def test_accept_golden_cases(lib):
    import os
    from oracle import accept
    path = os.path.join(os.path.dirname(__file__), "golden", "accept_cases.txt")
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        name, d, a, exp = (s.strip() for s in line.split("|"))
        d = np.array([[int(t) for t in d.split()]], np.int32)
        a_tok = [int(t) for t in a.split()]
        K = d.shape[1]
        V = 64
        logits = np.zeros((1, K, V), np.float32)
        for i, t in enumerate(a_tok):
            logits[0, i, t] = 1.0
        a_gpu, n_acc, n_emit, nxt = _accept_gpu(lib, logits, d)
        assert [int(n_acc[0]), int(n_emit[0]), int(nxt[0])] == [int(t) for t in exp.split()], name
        assert list(a_gpu[0]) == a_tok


@pytest.mark.parametrize("lens,K,layers,D", [
    ([0, 15, 16, 37], 8, 3, 64),
    ([40960], 32, 2, 128),          # 40K context: two freshly allocated pages
    ([1, 1024, 30000, 77, 4095], 32, 1, 128),
    ("ragged16", 32, 2, 128),       # batch 16, L_b ~ U[1024, 32768]
])
def test_commit_matches_oracle(lib, lens, K, layers, D):
    from oracle import commit_kv
    from synth import make_paged_case, ragged_lengths
    if lens == "ragged16":
        lens = ragged_lengths(4, 16)
    B = len(lens)
    Hkv = 8 if D == 128 else 2
    c = make_paged_case(21, B, K, 4 * Hkv, Hkv, D, lens, layers=layers, fill="sentinel")
    rng = np.random.default_rng(22)
    kb = rng.integers(0, 0x7F00, size=(layers, B, K, Hkv, D)).astype(np.uint16)
    vb = rng.integers(0, 0x7F00, size=(layers, B, K, Hkv, D)).astype(np.uint16)
    n_emit = rng.integers(1, K + 1, size=B).astype(np.int32)
    n_emit[0] = K
    import dual_view_draft_amd as dv
    kp, vp = bf16_dev(c.k_pages), bf16_dev(c.v_pages)
    kv = dv.PagedKV(kp[0], vp[0], i32_dev(c.block_table), i32_dev(c.seq_lens))
    out_lens = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    dv.orthrus_commit_kv(kv, bf16_dev(kb), bf16_dev(vb), i32_dev(n_emit), out_lens,
                         pool_layer_stride=kp.stride(0))
    torch.cuda.synchronize()
    k_ref, v_ref, lens_ref = commit_kv(c.k_pages, c.v_pages, c.block_table, c.seq_lens, kb, vb, n_emit)
    assert np.array_equal(bf16_host_bits(kp), k_ref)
    assert np.array_equal(bf16_host_bits(vp), v_ref)
    assert np.array_equal(out_lens.cpu().numpy(), lens_ref)


def test_commit_rejects_aliased_seq_lens(lib):
    import dual_view_draft_amd as dv
    from synth import make_paged_case
    c = make_paged_case(23, 1, 4, 2, 1, 64, [10])
    kv = dv.PagedKV(bf16_dev(c.k_pages[0]), bf16_dev(c.v_pages[0]), i32_dev(c.block_table),
                    i32_dev(c.seq_lens))
    kb = bf16_dev(np.zeros((1, 1, 4, 1, 64), np.uint16))
    with pytest.raises(dv.OrthrusError, match="INVALID_ARG"):
        dv.orthrus_commit_kv(kv, kb, kb, i32_dev([1]), kv.seq_lens)

"""GPU parity of orthrus_attn_draft / orthrus_attn_verify against the oracle.

Tolerance (bf16 inputs, fp32 accumulation, bf16 output): elementwise
|gpu - oracle| <= 2e-2 + 1e-2 |oracle|.  Inputs are the seeded synthetic
workloads; "sharp" inputs (unscaled values plus planted needle keys) are used
beside the 1/sqrt(D)-scaled ones because the latter give near-uniform softmax
weights that even an all-zero output would match.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import bf16_host_bits, compare, oracle_inputs, upload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def run(dv, c, mode, max_ctx=None, split=0, layer=0):
    kv, q, kb, vb = upload_case(c, layer)
    out = torch.empty_like(q)
    mc = int(max(c.seq_lens)) if max_ctx is None else max_ctx
    fn = dv.orthrus_attn_draft if mode == "draft" else dv.orthrus_attn_verify
    fn(kv, q, kb, vb, out, max_ctx=mc, split_tokens=split)
    torch.cuda.synchronize()
    return out


def oracle(c, mode):
    from oracle import block_attention
    return block_attention(*oracle_inputs(c), mode)


def case(seed, B, K, Hq, Hkv, D, lens, **kw):
    from synth import make_paged_case
    return make_paged_case(seed, B, K, Hq, Hkv, D, lens, **kw)


@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_tiny_workload(lib, mode):
    # 1 layer, 2 query heads / 1 KV head, D 64, L 256, K 8, Q/K/V ~ N(0,1)
    c = case(1, 1, 8, 2, 1, 64, [256], std=1.0)
    print(f"tiny {mode}", flush=True)
    compare(run(lib, c, mode), oracle(c, mode), f"tiny {mode}")


@pytest.mark.parametrize("mode", ["draft", "verify"])
@pytest.mark.parametrize("split", [0, 64, 256])
def test_ragged_sharp_small(lib, mode, split):
    # several tiles, ragged lengths incl. empty cache, partial pages, 128 rows
    c = case(12, 4, 32, 8, 2, 128, [0, 37, 1000, 333], sharp=True)
    print(f"ragged sharp {mode} split={split}", flush=True)
    compare(run(lib, c, mode, split=split), oracle(c, mode), f"ragged {mode} split {split}")


@pytest.mark.parametrize("mode", ["draft", "verify"])
@pytest.mark.parametrize("sharp", [False, True])
def test_qwen3_8b_4k(lib, mode, sharp):
    c = case(2, 1, 32, 32, 8, 128, [4096], sharp=sharp)
    print(f"qwen3-8b 4k {mode} sharp={sharp}", flush=True)
    compare(run(lib, c, mode), oracle(c, mode), f"4k {mode} sharp={sharp}")


@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_qwen3_8b_40k_sharp(lib, mode):
    c = case(3, 1, 32, 32, 8, 128, [40960], sharp=True)
    print(f"qwen3-8b 40k {mode}", flush=True)
    compare(run(lib, c, mode), oracle(c, mode), f"40k {mode}")


def test_ragged16_all_sequences(lib):
    # batch 16, L_b ~ U[1024, 32768], K 32: every sequence, every row against the oracle
    from synth import ragged_lengths
    lens = ragged_lengths(4, 16)
    c = case(4, 16, 32, 32, 8, 128, lens, sharp=True)
    for mode in ("draft", "verify"):
        print(f"ragged16 {mode}", flush=True)
        compare(run(lib, c, mode), oracle(c, mode), f"ragged16 {mode}")


def test_k1_is_decode_and_masks_agree(lib):
    c = case(5, 2, 1, 32, 8, 128, [777, 3000], sharp=True)
    d, v = run(lib, c, "draft"), run(lib, c, "verify")
    assert torch.equal(d.view(torch.int16), v.view(torch.int16))
    compare(v, oracle(c, "verify"), "K=1")


def test_empty_cache_chunked_prefill_shape(lib):
    # L = 0, K = 64 with the toy model's heads (16 / 4, D 64): 256 rows -> 2 row chunks
    c = case(6, 2, 64, 16, 4, 64, [0, 0], sharp=True)
    for mode in ("draft", "verify"):
        compare(run(lib, c, mode), oracle(c, mode), f"prefill chunk {mode}")


def test_group_size_8_rows_over_128(lib):
    c = case(7, 1, 20, 16, 2, 64, [300], sharp=True)   # G = 8, 160 rows
    for mode in ("draft", "verify"):
        compare(run(lib, c, mode), oracle(c, mode), f"G=8 {mode}")


def _random_shape(i):
    """Seeded random attention shape: batch 1-3, K 1-64, 1-4 KV heads, group
    1-16, head_dim 64 or 128, cached lengths 0-1500 (ragged), a split size
    from the library's choice down to one tile, and sometimes a max_ctx above
    the longest sequence (splits past every sequence exit)."""
    rng = np.random.default_rng(1000 + i)
    B = int(rng.integers(1, 4))
    K = int(rng.choice([1, 2, 7, 8, 13, 32, 33, 64]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    D = int(rng.choice([64, 128]))
    lens = [int(x) for x in rng.integers(0, 1501, size=B)]
    split = int(rng.choice([0, 64, 128, 320]))
    slack = int(rng.choice([0, 0, 700]))
    return B, K, G * Hkv, Hkv, D, lens, split, slack


@pytest.mark.parametrize("i", range(16))
def test_random_shapes(lib, i):
    B, K, Hq, Hkv, D, lens, split, slack = _random_shape(i)
    c = case(2000 + i, B, K, Hq, Hkv, D, lens, sharp=bool(i % 2), extra_pages_per_seq=(slack + 15) // 16)
    print(f"random {i}: B={B} K={K} Hq={Hq} Hkv={Hkv} D={D} lens={lens} split={split} slack={slack}", flush=True)
    for mode in ("draft", "verify"):
        got = run(lib, c, mode, max_ctx=max(lens) + slack, split=split)
        compare(got, oracle(c, mode), f"random {i} {mode}")


def test_last_row_draft_equals_verify_bitwise(lib):
    c = case(8, 2, 32, 32, 8, 128, [1500, 64], sharp=True)
    d, v = run(lib, c, "draft"), run(lib, c, "verify")
    assert torch.equal(d[:, -1].view(torch.int16), v[:, -1].view(torch.int16))


def test_deterministic_and_split_independent_within_tolerance(lib):
    c = case(9, 1, 32, 32, 8, 128, [5000], sharp=True)
    a1, a2 = run(lib, c, "verify"), run(lib, c, "verify")
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    ref = oracle(c, "verify")
    for split in (64, 640, 4096):
        compare(run(lib, c, "verify", split=split), ref, f"split {split}")


def test_verify_row_is_batch_invariant(lib):
    """Row i of a K-row verify pass at L equals, bit for bit, a 1-row verify
    pass at L+i whose cache already holds block rows 0..i-1 (the property that
    makes the Orthrus loop emit exactly the greedy tokens)."""
    import synth
    L, K, Hkv, D = 901, 32, 8, 128
    c = case(10, 1, K, 32, Hkv, D, [L], sharp=True, extra_pages_per_seq=3)
    max_ctx = L + K
    full = run(lib, c, "verify", max_ctx=max_ctx)
    for i in (0, 1, 7, 22, 31):
        ci = synth.make_paged_case(10, 1, K, 32, Hkv, D, [L], sharp=True, extra_pages_per_seq=3)
        # move block rows 0..i-1 into the cache, row i becomes a 1-row block
        for r in range(i):
            p = L + r
            page = ci.block_table[0, p // 16]
            ci.k_pages[0, page, :, p % 16] = ci.k_blk[0, r]
            ci.v_pages[0, page, :, p % 16] = ci.v_blk[0, r]
        ci.seq_lens = np.array([L + i], np.int32)
        ci.q = np.ascontiguousarray(ci.q[:, i:i + 1])
        ci.k_blk = np.ascontiguousarray(ci.k_blk[:, i:i + 1])
        ci.v_blk = np.ascontiguousarray(ci.v_blk[:, i:i + 1])
        ci.K = 1
        one = run(lib, ci, "verify", max_ctx=max_ctx)
        assert torch.equal(one[:, 0].view(torch.int16), full[:, i].view(torch.int16)), f"row {i}"


def test_batch_zero_is_noop(lib):
    c = case(11, 1, 4, 4, 2, 64, [40])
    kv, q, kb, vb = upload_case(c)
    out = torch.zeros_like(q)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    lib.orthrus_attn_draft(kv, q[:0], kb[:0], vb[:0], out[:0], max_ctx=40, workspace=ws)
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any()


def test_rejects_small_workspace_before_launch(lib):
    c = case(11, 1, 4, 4, 2, 64, [40])
    kv, q, kb, vb = upload_case(c)
    out = torch.zeros_like(q)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.OrthrusError, match="WORKSPACE_TOO_SMALL"):
        lib.orthrus_attn_verify(kv, q, kb, vb, out, max_ctx=40, workspace=ws)
    assert not out.view(torch.int16).any()

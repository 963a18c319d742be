"""GPU parity of the e4m3 KV cache: orthrus_quantize_kv bit for bit against the
oracle, attention over an e4m3 cache (orthrus_attn_draft / orthrus_attn_verify
with kv_dtype ORTHRUS_KV_FP8_E4M3) against the oracle's attention over the
decoded values, and the commit of e4m3 rows.

The attention tolerance is the bf16 cache's, |gpu - oracle| <= 2e-2 +
1e-2 |oracle|: the oracle decodes the same codes exactly, and the kernel widens
them to bf16 exactly, so its remaining error sources are those of the bf16
path (bf16 P, fp32 accumulation, bf16 output).  How far the e4m3 cache's
result lies from the bf16 cache's is the quantisation's own error, which is
reported beside (and bounded loosely), not a parity criterion.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import bf16_dev, bf16_host_bits, compare, i32_dev

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


@pytest.fixture(scope="module", autouse=True)
def lib():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.uint8))).cuda()


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).cuda()


def amax_scales(pages_bits, blk_bits, fill_bits):
    """Per-KV-head fp32 scale amax / 448 over the finite cache and block values."""
    from oracle import from_bf16
    Hkv = blk_bits.shape[2]
    p = from_bf16(np.where(pages_bits == fill_bits, 0, pages_bits))     # [pages, Hkv, 16, D]
    bl = from_bf16(blk_bits)                                            # [B, K, Hkv, D]
    amax = np.maximum(np.abs(p).max(axis=(0, 2, 3)), np.abs(bl).max(axis=(0, 1, 3)))
    return (np.maximum(amax, 1e-3) / 448.0).astype(np.float32).reshape(Hkv)


def to_fp8(c, layer=0):
    """e4m3 codes of a synth.PagedCase (poisoned slots become the NaN code)."""
    from oracle.fp8 import quantize_kv
    kp, vp = c.k_pages[layer], c.v_pages[layer]
    ks = amax_scales(kp, c.k_blk, c.fill_bits)
    vs = amax_scales(vp, c.v_blk, c.fill_bits)

    def pages(bits, s):
        poison = bits == c.fill_bits
        codes = quantize_kv(np.where(poison, 0, bits), s, head_axis=1)
        return np.where(poison, NAN_CODE, codes).astype(np.uint8)

    return dict(k_pages=pages(kp, ks), v_pages=pages(vp, vs), k_blk=quantize_kv(c.k_blk, ks),
                v_blk=quantize_kv(c.v_blk, vs), k_scale=ks, v_scale=vs)


def run_fp8(dv, c, f, mode, max_ctx=None, split=0):
    kv = dv.PagedKV(u8_dev(f["k_pages"]), u8_dev(f["v_pages"]), i32_dev(c.block_table), i32_dev(c.seq_lens),
                    k_scale=f32_dev(f["k_scale"]), v_scale=f32_dev(f["v_scale"]))
    q = bf16_dev(c.q)
    out = torch.empty_like(q)
    mc = int(max(c.seq_lens)) if max_ctx is None else max_ctx
    fn = dv.orthrus_attn_draft if mode == "draft" else dv.orthrus_attn_verify
    fn(kv, q, u8_dev(f["k_blk"]), u8_dev(f["v_blk"]), out, max_ctx=mc, split_tokens=split)
    torch.cuda.synchronize()
    return out


def oracle_fp8(c, f, mode, rows=None):
    from oracle.fp8 import block_attention_fp8
    sl = slice(None) if rows is None else rows
    return block_attention_fp8(c.q[sl], f["k_blk"][sl], f["v_blk"][sl], f["k_pages"], f["v_pages"],
                               f["k_scale"], f["v_scale"], c.block_table[sl], c.seq_lens[sl], mode)


def case(seed, B, K, Hq, Hkv, lens, **kw):
    from synth import make_paged_case
    return make_paged_case(seed, B, K, Hq, Hkv, 128, lens, **kw)


# ---- quantisation --------------------------------------------------------
@pytest.mark.parametrize("scale", [1.0, 0.37, 3.0e-3, 1.0e-5, 250.0])
def test_quantize_every_finite_bf16_value(lib, scale):
    from oracle.fp8 import quantize_kv
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80].reshape(-1, 2, 128)     # finite values, Hkv 2, D 128
    s = np.array([scale, scale * 1.5], np.float32)
    k_out = torch.empty(bits.shape, dtype=torch.uint8, device="cuda")
    v_out = torch.empty_like(k_out)
    kb = bf16_dev(bits)
    vb = bf16_dev(bits[::-1].copy())
    lib.orthrus_quantize_kv(kb, vb, f32_dev(s), f32_dev(s[::-1].copy()), k_out, v_out)
    torch.cuda.synchronize()
    assert np.array_equal(k_out.cpu().numpy(), quantize_kv(bits, s))
    assert np.array_equal(v_out.cpu().numpy(), quantize_kv(bits[::-1], s[::-1].copy()))


def test_quantize_block_rows_of_the_8b_shape(lib):
    from oracle.fp8 import quantize_kv
    from synth import make_block_qkv
    _, k, v = make_block_qkv(30, 2, 32, 32, 8, 128, std=1.5)
    ks = np.linspace(0.004, 0.03, 8).astype(np.float32)
    vs = np.linspace(0.02, 0.002, 8).astype(np.float32)
    k_out = torch.empty(k.shape, dtype=torch.uint8, device="cuda")
    v_out = torch.empty_like(k_out)
    lib.orthrus_quantize_kv(bf16_dev(k), bf16_dev(v), f32_dev(ks), f32_dev(vs), k_out, v_out)
    torch.cuda.synchronize()
    assert np.array_equal(k_out.cpu().numpy(), quantize_kv(k, ks))
    assert np.array_equal(v_out.cpu().numpy(), quantize_kv(v, vs))


# ---- attention over an e4m3 cache ------------------------------------------
@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_small_one_kv_head(lib, mode):
    c = case(41, 1, 8, 2, 1, [256], std=1.0)
    f = to_fp8(c)
    print(f"fp8 small {mode}", flush=True)
    compare(run_fp8(lib, c, f, mode), oracle_fp8(c, f, mode), f"fp8 small {mode}")


@pytest.mark.parametrize("mode", ["draft", "verify"])
@pytest.mark.parametrize("split", [0, 64, 256])
def test_ragged_sharp(lib, mode, split):
    # several tiles, ragged lengths incl. an empty cache and partial pages
    c = case(42, 4, 32, 8, 2, [0, 37, 1000, 333], sharp=True)
    f = to_fp8(c)
    print(f"fp8 ragged {mode} split={split}", flush=True)
    compare(run_fp8(lib, c, f, mode, split=split), oracle_fp8(c, f, mode), f"fp8 ragged {mode} {split}")


@pytest.mark.parametrize("mode", ["draft", "verify"])
@pytest.mark.parametrize("sharp", [False, True])
def test_qwen3_8b_4k(lib, mode, sharp):
    c = case(43, 1, 32, 32, 8, [4096], sharp=sharp)
    f = to_fp8(c)
    print(f"fp8 4k {mode} sharp={sharp}", flush=True)
    compare(run_fp8(lib, c, f, mode), oracle_fp8(c, f, mode), f"fp8 4k {mode} sharp={sharp}")


@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_qwen3_8b_40k_sharp(lib, mode):
    c = case(44, 1, 32, 32, 8, [40960], sharp=True)
    f = to_fp8(c)
    print(f"fp8 40k {mode}", flush=True)
    compare(run_fp8(lib, c, f, mode), oracle_fp8(c, f, mode), f"fp8 40k {mode}")


def _random_shape(i):
    """Seeded random e4m3-cache shape: batch 1-3, K 1-64, 1-4 KV heads, group
    1-16, head_dim 128, cached lengths 0-1500 (ragged), a split size from the
    library's choice down to one tile, and sometimes a max_ctx above the
    longest sequence."""
    rng = np.random.default_rng(3000 + i)
    B = int(rng.integers(1, 4))
    K = int(rng.choice([1, 2, 7, 8, 13, 32, 33, 64]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    lens = [int(x) for x in rng.integers(0, 1501, size=B)]
    split = int(rng.choice([0, 64, 128, 320]))
    slack = int(rng.choice([0, 0, 700]))
    return B, K, G * Hkv, Hkv, lens, split, slack


@pytest.mark.parametrize("i", range(12))
def test_random_shapes(lib, i):
    B, K, Hq, Hkv, lens, split, slack = _random_shape(i)
    c = case(4000 + i, B, K, Hq, Hkv, lens, sharp=bool(i % 2), extra_pages_per_seq=(slack + 15) // 16)
    f = to_fp8(c)
    print(f"fp8 random {i}: B={B} K={K} Hq={Hq} Hkv={Hkv} lens={lens} split={split} slack={slack}", flush=True)
    for mode in ("draft", "verify"):
        got = run_fp8(lib, c, f, mode, max_ctx=max(lens) + slack, split=split)
        compare(got, oracle_fp8(c, f, mode), f"fp8 random {i} {mode}")


def test_k1_decode_and_last_row(lib):
    c = case(45, 2, 1, 32, 8, [777, 3000], sharp=True)
    f = to_fp8(c)
    d, v = run_fp8(lib, c, f, "draft"), run_fp8(lib, c, f, "verify")
    assert torch.equal(d.view(torch.int16), v.view(torch.int16))
    compare(v, oracle_fp8(c, f, "verify"), "fp8 K=1")
    c = case(46, 2, 32, 32, 8, [1500, 64], sharp=True)
    f = to_fp8(c)
    d, v = run_fp8(lib, c, f, "draft"), run_fp8(lib, c, f, "verify")
    assert torch.equal(d[:, -1].view(torch.int16), v[:, -1].view(torch.int16))


def test_ragged16_all_sequences(lib):
    from synth import ragged_lengths
    c = case(47, 16, 32, 32, 8, ragged_lengths(47, 16), sharp=True)
    f = to_fp8(c)
    for mode in ("draft", "verify"):
        print(f"fp8 ragged16 {mode}", flush=True)
        compare(run_fp8(lib, c, f, mode), oracle_fp8(c, f, mode), f"fp8 ragged16 {mode}")


def test_verify_row_is_batch_invariant(lib):
    """Row i of a K-row verify pass equals, bit for bit, a 1-row pass at L+i whose
    cache holds block rows 0..i-1 as e4m3 codes: the e4m3 cache keeps the
    property that makes the Orthrus loop emit the greedy tokens."""
    L, K = 901, 32
    c = case(48, 1, K, 32, 8, [L], sharp=True, extra_pages_per_seq=3)
    f = to_fp8(c)
    full = run_fp8(lib, c, f, "verify", max_ctx=L + K)
    for i in (0, 1, 13, 31):
        g = {k: v.copy() for k, v in f.items()}
        for r in range(i):
            p = L + r
            page = c.block_table[0, p // 16]
            g["k_pages"][page, :, p % 16] = f["k_blk"][0, r]
            g["v_pages"][page, :, p % 16] = f["v_blk"][0, r]
        g["k_blk"] = np.ascontiguousarray(f["k_blk"][:, i:i + 1])
        g["v_blk"] = np.ascontiguousarray(f["v_blk"][:, i:i + 1])
        ci = case(48, 1, K, 32, 8, [L], sharp=True, extra_pages_per_seq=3)
        ci.seq_lens = np.array([L + i], np.int32)
        ci.q = np.ascontiguousarray(c.q[:, i:i + 1])
        ci.K = 1
        one = run_fp8(lib, ci, g, "verify", max_ctx=L + K)
        assert torch.equal(one[:, 0].view(torch.int16), full[:, i].view(torch.int16)), f"row {i}"


def test_quantisation_error_against_the_bf16_cache(lib):
    """The e4m3 cache's output beside the bf16 cache's on the same data (the
    quantisation's own error, reported; bounded loosely)."""
    from gpu_helpers import oracle_inputs
    from oracle import block_attention, from_bf16
    c = case(49, 1, 32, 32, 8, [4096], std=1.0)
    f = to_fp8(c)
    ref16 = block_attention(*oracle_inputs(c), "verify")
    x = from_bf16(bf16_host_bits(run_fp8(lib, c, f, "verify")))
    err = np.abs(x - ref16)
    rms = float(np.sqrt(np.mean(ref16 ** 2)))
    print(f"e4m3 vs bf16 cache: max abs {err.max():.3e}, max / rms {err.max() / rms:.3e}, "
          f"mean abs / rms {err.mean() / rms:.3e}", flush=True)
    assert err.max() <= 0.25 * rms and err.mean() <= 0.05 * rms


# ---- commit -----------------------------------------------------------------
def test_commit_of_e4m3_rows(lib):
    from oracle import commit_kv
    from synth import make_paged_case
    lens, K, layers, Hkv = [1, 1024, 40960, 77], 32, 2, 8
    B = len(lens)
    c = make_paged_case(50, B, K, 4 * Hkv, Hkv, 128, lens, layers=layers, fill="sentinel")
    rng = np.random.default_rng(51)
    kp = rng.integers(0, 256, size=c.k_pages.shape).astype(np.uint8)
    vp = rng.integers(0, 256, size=c.v_pages.shape).astype(np.uint8)
    kb = rng.integers(0, 256, size=(layers, B, K, Hkv, 128)).astype(np.uint8)
    vb = rng.integers(0, 256, size=(layers, B, K, Hkv, 128)).astype(np.uint8)
    n_emit = rng.integers(1, K + 1, size=B).astype(np.int32)
    n_emit[2] = K
    kpd, vpd = u8_dev(kp), u8_dev(vp)
    kv = lib.PagedKV(kpd[0], vpd[0], i32_dev(c.block_table), i32_dev(c.seq_lens))
    out_lens = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lib.orthrus_commit_kv(kv, u8_dev(kb), u8_dev(vb), i32_dev(n_emit), out_lens, pool_layer_stride=kpd.stride(0))
    torch.cuda.synchronize()
    k_ref, v_ref, lens_ref = commit_kv(kp, vp, c.block_table, c.seq_lens, kb, vb, n_emit)
    assert np.array_equal(kpd.cpu().numpy(), k_ref)
    assert np.array_equal(vpd.cpu().numpy(), v_ref)
    assert np.array_equal(out_lens.cpu().numpy(), lens_ref)

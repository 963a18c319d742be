"""A whole decode step captured in one HIP graph and replayed.

Every replay must reproduce the eager calls' outputs bit for bit: the draft
and verify attention passes, the draft argmax, the acceptance, the KV commit
(into the pools, which the graph restores from a pristine copy first), the fused
LM head with its argmax, and the temperature-1 sampling and acceptance.  The
outputs are poisoned before each replay and eager work runs between replays,
so a call that kept state from one launch to the next on the host, or
depended on memory a previous call left behind, would show here.
"""
import pytest
import torch

from gpu_helpers import bf16_dev, upload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def test_step_graph_replays_match_eager(lib):
    from synth import make_lmhead_case, make_paged_case
    dv = lib
    dev = torch.device("cuda:0")
    B, K, Hq, Hkv, D, V = 2, 32, 32, 8, 128, 5000
    c = make_paged_case(61, B, K, Hq, Hkv, D, [3000, 777], extra_pages_per_seq=3)
    kv, q, kb, vb = upload_case(c)
    max_ctx = int(max(c.seq_lens)) + K
    kp0, vp0 = kv.k_pages.clone(), kv.v_pages.clone()          # pristine pools
    kvw = dv.PagedKV(kv.k_pages, kv.v_pages, kv.block_table, kv.seq_lens)
    g = torch.Generator(device=dev).manual_seed(62)
    logits_d = torch.randn((B, K, V), generator=g, device=dev) * 3
    logits_a = (0.9 * logits_d + 0.1 * torch.randn((B, K, V), generator=g, device=dev) * 3).contiguous()
    u1, u2, u3 = (torch.rand((B, K), generator=g, device=dev) for _ in range(3))
    lm = make_lmhead_case(63, B * K, 256, V, plant=False)
    lm_h, lm_w = bf16_dev(lm.hidden), bf16_dev(lm.weight)

    ws_attn = dv.attn_workspace(kv, q, max_ctx)
    ws_arg = dv.argmax_workspace(B * K, V, dev)
    ws_acc = dv.argmax_workspace(B * K, V, dev)
    ws_lm = dv.lmhead_workspace(B * K, 256, V, dev)
    ws_s = torch.empty(dv.orthrus_sample_workspace_bytes(B * K, V), dtype=torch.uint8, device=dev)
    ws_as = torch.empty(dv.orthrus_accept_sampled_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)

    out = {
        "draft_attn": torch.empty_like(q), "verify_attn": torch.empty_like(q),
        "d": torch.empty((B, K), dtype=torch.int32, device=dev),
        "a": torch.empty((B, K), dtype=torch.int32, device=dev),
        "n_acc": torch.empty(B, dtype=torch.int32, device=dev),
        "n_emit": torch.empty(B, dtype=torch.int32, device=dev),
        "next": torch.empty(B, dtype=torch.int32, device=dev),
        "seq_out": torch.empty(B, dtype=torch.int32, device=dev),
        "lm_tok": torch.empty(B * K, dtype=torch.int32, device=dev),
        "s": torch.empty((B, K), dtype=torch.int32, device=dev),
        "st": torch.empty((B, K), dtype=torch.int32, device=dev),
        "s_acc": torch.empty(B, dtype=torch.int32, device=dev),
        "s_emit": torch.empty(B, dtype=torch.int32, device=dev),
        "s_next": torch.empty(B, dtype=torch.int32, device=dev),
    }

    def restore():
        # an elementwise kernel, bit for bit (no copy or fill node in the graph)
        torch.bitwise_or(kp0.view(torch.int16), 0, out=kvw.k_pages.view(torch.int16))
        torch.bitwise_or(vp0.view(torch.int16), 0, out=kvw.v_pages.view(torch.int16))

    def step():
        restore()                                # the pools as the step starts
        dv.orthrus_attn_draft(kv, q, kb, vb, out["draft_attn"], max_ctx=max_ctx, workspace=ws_attn)
        dv.orthrus_argmax(logits_d, out["d"], workspace=ws_arg)
        dv.orthrus_attn_verify(kv, q, kb, vb, out["verify_attn"], max_ctx=max_ctx, workspace=ws_attn)
        dv.orthrus_accept(logits_a, out["d"], out["a"], out["n_acc"], out["n_emit"], out["next"], workspace=ws_acc)
        dv.orthrus_commit_kv(kvw, kb.unsqueeze(0), vb.unsqueeze(0), out["n_emit"], out["seq_out"])
        dv.orthrus_lmhead_argmax(lm_h, lm_w, out["lm_tok"], workspace=ws_lm)
        dv.orthrus_sample(logits_d, 1.0, u1, out["s"], workspace=ws_s)
        dv.orthrus_accept_sampled(logits_d, logits_a, out["s"], 1.0, u2, u3, out["st"], out["s_acc"],
                                  out["s_emit"], out["s_next"], workspace=ws_as)

    def snapshot():
        snap = {k: v.clone() for k, v in out.items()}
        snap["k_pages"], snap["v_pages"] = kvw.k_pages.clone(), kvw.v_pages.clone()
        return snap

    def poison():
        for t in out.values():
            if t.dtype == torch.int32:
                t.fill_(-7)
            else:
                t.fill_(float("nan"))
        kvw.k_pages.fill_(float("nan"))
        kvw.v_pages.fill_(float("nan"))

    def bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t

    step()
    torch.cuda.synchronize()
    eager = snapshot()
    assert int(eager["n_emit"].min()) >= 1 and bool((eager["seq_out"] > kv.seq_lens).all())

    # capture on a side stream (the bindings launch on the current stream)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.synchronize()

    filler = torch.randn((1024, 1024), device=dev)
    for rep in range(3):
        poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, v in eager.items():
            assert torch.equal(bits(got[k]), bits(v)), f"replay {rep}: {k}"
        # unrelated eager work and a synchronisation between replays
        filler = torch.tanh(filler @ filler.t() * 1e-3)
        torch.cuda.synchronize()

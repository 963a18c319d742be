#!/usr/bin/env python3
"""Benchmark of one Orthrus decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  draft attention (diffusion view, block-bidirectional mask)
  -> draft argmax over the draft logits
  -> verify attention (AR view, causal inside the block)
  -> accept (AR argmax + longest matching prefix)
  -> commit of the accepted rows' K/V into the paged cache.
Everything runs in liborthrus (HIP, gfx950) on torch's current stream; inputs
are resident in HBM before the timed region.  The KV pool is replicated into
several independently permuted copies (more bytes than the 256 MB Infinity
Cache) and the steps rotate through them, so repeated steps cannot be served
from the last-level cache.

Output: one JSON line (metric, value, roofline of the attention pass,
cpu_baseline of the CPU oracle on the same workload, per-op timings).

    python bench.py [--gpus 1] [--steps 100] [--warmup 300] [--workload qwen3_8b_40k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
METRIC = "block-attn KV-read GB/s (% HBM peak) + draft/verify steps/s, 8B shape @40K"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_split_kernel_traffic.json")
ATTN_SRC = os.path.join(ROOT, "dual_view_draft_amd", "csrc", "attn.hip")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", default="qwen3_8b_40k",
                   choices=["qwen3_8b_40k", "qwen3_8b_4k", "qwen3_8b_ragged16", "tiny"])
    p.add_argument("--pools", type=int, default=0, help="KV pool copies to rotate (0 = auto)")
    p.add_argument("--split", type=int, default=0, help="split_tokens override (0 = library choice)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra-workloads", action="store_true",
                   help="skip the 4K and 16-sequence ragged objects of the default (40K) run")
    p.add_argument("--no-graph", dest="graph", action="store_false",
                   help="launch the timed steps eagerly instead of replaying HIP graphs")
    p.add_argument("--cpu-steps", type=int, default=3)
    p.add_argument("--quick", action="store_true",
                   help="timed steps only (no per-op breakdown, no CPU baseline): for profiler runs")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--e2e", action="store_true",
                   help="only time whole decode steps of the Qwen3-8B-shaped model (greedy vs Orthrus)")
    p.add_argument("--e2e-contexts", default="4096,40960")
    p.add_argument("--lmhead-rows", type=int, default=0,
                   help="only time the fused LM head + argmax of the Qwen3-8B shape (hidden 4096, "
                        "vocabulary 151936) over this many rows, eager launches (for profiler runs)")
    return p.parse_args()


def kernel_source_hash() -> str:
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str, key: str = "hbm_bytes_per_attention_call"):
    """HBM bytes per attention call (bf16 cache, or key
    "hbm_bytes_per_fp8_attention_call") from the committed rocprofv3 counter
    summary, or None if it was taken on another workload or the attention
    kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attn_source_sha256_16") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get(key)


def setup(args, torch, dv, synth):
    w = dict(synth.WORKLOADS[args.workload])
    B, K, Hq, Hkv, D, V = w["B"], w["K"], w["Hq"], w["Hkv"], w["D"], w["V"]
    lens = w["seq_lens"] if w["seq_lens"] is not None else synth.ragged_lengths(w["seed"], B)
    case = synth.make_paged_case(w["seed"], B, K, Hq, Hkv, D, lens, fill="sentinel")
    qv, kbv, vbv = synth.make_block_qkv(w["seed"] + 100, B, K, Hq, Hkv, D)
    cons = synth.make_consensus_case(w["seed"], B, K, V, dist=w["accept"])
    return w, case, (qv, kbv, vbv), cons


def to_dev16(torch, np, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def lmhead_only(args, torch, dv, synth):
    """The fused LM head + argmax alone at the Qwen3-8B shape over
    args.lmhead_rows rows: weights N(0, 0.02) and hidden states N(0, 1), bf16,
    drawn on the device; args.warmup untimed and args.steps timed eager calls."""
    w = synth.WORKLOADS["qwen3_8b_40k"]
    V, Hd, R = w["V"], w["hidden"], args.lmhead_rows
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(w["seed"] + 7)
    lm_w = torch.randn((V, Hd), generator=gen, device=dev).mul_(0.02).to(torch.bfloat16)
    lm_h = torch.randn((R, Hd), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty(R, dtype=torch.int32, device=dev)
    ws = dv.lmhead_workspace(R, Hd, V, dev)
    for _ in range(args.warmup):
        dv.orthrus_lmhead_argmax(lm_h, lm_w, out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dv.orthrus_lmhead_argmax(lm_h, lm_w, out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / max(args.steps, 1) * 1e3
    return {"lmhead_rows": R, "hidden": Hd, "vocab": V, "us_per_call": round(us, 1),
            "tflops": round(2.0 * R * Hd * V / (us * 1e-6) / 1e12, 1),
            "weight_gbps": round(V * Hd * 2 / (us * 1e-6) / 1e9, 1)}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dual_view_draft_amd as dv
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dv.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(5):
            torch.add(a, 0.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": a.numel() * 4,
                          "copy_calibration_bytes_written": b.numel() * 4}))
        return

    if args.e2e:
        print(json.dumps(e2e(args, torch, dv, synth)), flush=True)
        return

    if args.lmhead_rows > 0:
        print(json.dumps(lmhead_only(args, torch, dv, synth)), flush=True)
        return

    w, case, (qv, kbv, vbv), cons = setup(args, torch, dv, synth)
    B, K, Hq, Hkv, D, V = w["B"], w["K"], w["Hq"], w["Hkv"], w["D"], w["V"]
    L = [int(x) for x in case.seq_lens]
    max_ctx = max(L)
    kv_bytes = 4 * Hkv * D * sum(L)                       # K and V, bf16, every cached token
    pool_bytes = 2 * case.k_pages[0].nbytes
    n_pools = args.pools or max(2, min(16, math.ceil(1.3e9 / pool_bytes)))

    # ---- device inputs --------------------------------------------------------
    kp0 = to_dev16(torch, np, case.k_pages[0])
    vp0 = to_dev16(torch, np, case.v_pages[0])
    table0 = torch.from_numpy(case.block_table).to(dev)
    seq_lens = torch.from_numpy(case.seq_lens).to(dev)
    kvs = [dv.PagedKV(kp0, vp0, table0, seq_lens)]
    g = torch.Generator(device="cpu").manual_seed(12345)
    for _ in range(1, n_pools):
        perm = torch.randperm(case.num_pages, generator=g).to(dev)
        inv = torch.empty_like(perm)
        inv[perm] = torch.arange(case.num_pages, device=dev)
        kvs.append(dv.PagedKV(kp0[perm].contiguous(), vp0[perm].contiguous(),
                              inv[table0.long()].to(torch.int32).contiguous(), seq_lens))
    q_d, kb_d, vb_d = (to_dev16(torch, np, x) for x in (case.q, case.k_blk, case.v_blk))
    q_v, kb_v, vb_v = (to_dev16(torch, np, x) for x in (qv, kbv, vbv))
    # the consensus reads rotating logits buffers (8 per view: 156 MB per view
    # at B = 1, more than the Infinity Cache holds next to the KV stream), as a
    # real step reads the LM head's fresh output; the copies hold the same
    # planted values, so every step has the drawn accepted lengths
    n_logits = 8
    logits_d0 = torch.from_numpy(cons.logits_d).to(dev)
    logits_a0 = torch.from_numpy(cons.logits_a).to(dev)
    logits_ds = [logits_d0] + [logits_d0.clone() for _ in range(n_logits - 1)]
    logits_as = [logits_a0] + [logits_a0.clone() for _ in range(n_logits - 1)]
    out_d = torch.empty_like(q_d)
    out_v = torch.empty_like(q_v)
    d_tok = torch.empty((B, K), dtype=torch.int32, device=dev)
    a_tok = torch.empty((B, K), dtype=torch.int32, device=dev)
    n_acc, n_emit, nxt, lens_out = (torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4))
    ws_attn = dv.attn_workspace(kvs[0], q_d, max_ctx, args.split)
    ws_arg = dv.argmax_workspace(B * K, V, dev)
    kb_commit, vb_commit = kb_v[None], vb_v[None]
    torch.cuda.synchronize()

    def step(i):
        kv = kvs[(2 * i) % n_pools]           # draft and verify read different pool copies,
        kv_v = kvs[(2 * i + 1) % n_pools]     # as a real model's two passes are layers apart
        s_ = torch.cuda.current_stream()      # the capture stream while a graph is recorded
        dv.orthrus_attn_draft(kv, q_d, kb_d, vb_d, out_d, max_ctx=max_ctx, split_tokens=args.split,
                              workspace=ws_attn, stream=s_)
        dv.orthrus_argmax(logits_ds[i % n_logits], d_tok, workspace=ws_arg, stream=s_)
        dv.orthrus_attn_verify(kv_v, q_v, kb_v, vb_v, out_v, max_ctx=max_ctx, split_tokens=args.split,
                               workspace=ws_attn, stream=s_)
        dv.orthrus_accept(logits_as[i % n_logits], d_tok, a_tok, n_acc, n_emit, nxt, workspace=ws_arg,
                          stream=s_)
        dv.orthrus_commit_kv(kv_v, kb_commit, vb_commit, n_emit, lens_out, stream=s_)

    # the first warmup steps run eagerly (they also initialise everything the
    # graphs capture); the rest replay the graphs, so the clocks have settled
    n_eager = min(args.warmup, 2) if args.graph else args.warmup
    for i in range(n_eager):
        step(i)
    torch.cuda.synchronize()
    # sanity: the consensus reproduces the drawn accepted lengths
    assert n_eager == 0 or torch.equal(n_acc.cpu(), torch.from_numpy(cons.n_acc)), "accept mismatch"

    def capture(fn):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        return graph

    # ---- timed region ------------------------------------------------------------
    # Each step is replayed from a HIP graph of the same five library calls, so
    # the GPU runs the kernels back to back without host gaps.  Draft and
    # verify read different pool copies; the graphs cycle through the copies.
    n_graphs = max(1, n_pools // 2, n_logits) if args.graph else 0
    graphs = [capture(lambda j=j: step(j)) for j in range(n_graphs)]
    torch.cuda.synchronize()
    for i in range(n_eager, args.warmup):          # the remaining warmup steps
        if args.graph:
            graphs[i % n_graphs].replay()
        else:
            step(i)
    # settle the clocks whatever --warmup says: at least 40 ms of untimed steps
    # (a few steps leave the shader clock ramping and read ~10 % slow)
    torch.cuda.synchronize()
    t_settle, n_settle = time.perf_counter(), 0
    while time.perf_counter() - t_settle < 0.04 or n_settle < 8:
        if args.graph:
            graphs[n_settle % n_graphs].replay()
        else:
            step(n_settle)
        n_settle += 1
        if n_settle % 8 == 0:
            torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        if args.graph:
            graphs[i % n_graphs].replay()
        else:
            step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # ---- per-op device time: graphs of REPS back-to-back calls of one op ----
    REPS = 16
    op_calls = {
        "draft_attn": lambda i: dv.orthrus_attn_draft(kvs[(2 * i) % n_pools], q_d, kb_d, vb_d, out_d,
                                                      max_ctx=max_ctx, split_tokens=args.split,
                                                      workspace=ws_attn, stream=None),
        "draft_argmax": lambda i: dv.orthrus_argmax(logits_ds[i % n_logits], d_tok, workspace=ws_arg,
                                                    stream=None),
        "verify_attn": lambda i: dv.orthrus_attn_verify(kvs[(2 * i + 1) % n_pools], q_v, kb_v, vb_v, out_v,
                                                        max_ctx=max_ctx, split_tokens=args.split,
                                                        workspace=ws_attn, stream=None),
        "accept": lambda i: dv.orthrus_accept(logits_as[i % n_logits], d_tok, a_tok, n_acc, n_emit, nxt,
                                              workspace=ws_arg, stream=None),
        "commit": lambda i: dv.orthrus_commit_kv(kvs[(2 * i + 1) % n_pools], kb_commit, vb_commit, n_emit,
                                                 lens_out, stream=None),
    }
    # fused LM head + argmax (the logits-free consensus), at the model's
    # hidden size: weights N(0, 0.02) and hidden states N(0, 1), bf16, drawn
    # on the device from a seeded generator (1.24 GB of weights at the 8B
    # shape, far more than the Infinity Cache)
    Hd = w["hidden"]
    lm_bytes = V * Hd * 2 + B * K * Hd * 2 + B * K * 4
    if not args.quick:
        gen = torch.Generator(device=dev).manual_seed(w["seed"] + 7)
        lm_w = torch.randn((V, Hd), generator=gen, device=dev).mul_(0.02).to(torch.bfloat16)
        lm_h = torch.randn((B, K, Hd), generator=gen, device=dev).to(torch.bfloat16)
        ws_lm = dv.lmhead_workspace(B * K, Hd, V, dev)
        op_calls["lmhead_argmax"] = lambda i: dv.orthrus_lmhead_argmax(lm_h, lm_w, d_tok, workspace=ws_lm,
                                                                       stream=None)
        op_calls["lmhead_accept"] = lambda i: dv.orthrus_lmhead_accept(lm_h, lm_w, d_tok, a_tok, n_acc, n_emit,
                                                                       nxt, workspace=ws_lm, stream=None)
    # the same attention over an e4m3 copy of every pool (one scale for all
    # heads, so the pages can be quantised in their own layout); the block's
    # rows are quantised with the same scales, as the model does each layer
    if not args.quick:
        scale = torch.full((Hkv,), 4.0 / math.sqrt(D) / 448.0, dtype=torch.float32, device=dev)

        def fp8_rows(k, v):
            ko = torch.empty(k.shape, dtype=torch.uint8, device=dev)
            vo = torch.empty_like(ko)
            dv.orthrus_quantize_kv(k, v, scale, scale, ko, vo)
            return ko, vo

        kvs8 = []
        for kv in kvs:
            n = kv.k_pages.shape[0]
            k8, v8 = fp8_rows(kv.k_pages.view(n * 16, Hkv, D), kv.v_pages.view(n * 16, Hkv, D))
            kvs8.append(dv.PagedKV(k8.view(kv.k_pages.shape), v8.view(kv.v_pages.shape), kv.block_table,
                                   kv.seq_lens, k_scale=scale, v_scale=scale))
        kb8_d, vb8_d = fp8_rows(kb_d, vb_d)
        kb8_v, vb8_v = fp8_rows(kb_v, vb_v)
        op_calls["draft_attn_fp8"] = lambda i: dv.orthrus_attn_draft(
            kvs8[(2 * i) % n_pools], q_d, kb8_d, vb8_d, out_d, max_ctx=max_ctx, split_tokens=args.split,
            workspace=ws_attn, stream=None)
        op_calls["verify_attn_fp8"] = lambda i: dv.orthrus_attn_verify(
            kvs8[(2 * i + 1) % n_pools], q_v, kb8_v, vb8_v, out_v, max_ctx=max_ctx, split_tokens=args.split,
            workspace=ws_attn, stream=None)
        # consensus at temperature 1: drafted tokens drawn from the draft
        # logits, speculative-sampling acceptance against the AR logits
        gen_u = torch.Generator(device=dev).manual_seed(w["seed"] + 11)
        u_draft, u_acc, u_res = (torch.rand((B, K), generator=gen_u, device=dev) for _ in range(3))
        tok_s = torch.empty((B, K), dtype=torch.int32, device=dev)
        ws_samp = torch.empty(dv.orthrus_sample_workspace_bytes(B * K, V), dtype=torch.uint8, device=dev)
        ws_accs = torch.empty(dv.orthrus_accept_sampled_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
        op_calls["draft_sample_t1"] = lambda i: dv.orthrus_sample(logits_ds[i % n_logits], 1.0, u_draft, d_tok,
                                                                  workspace=ws_samp,
                                                                  stream=None)
        op_calls["accept_sampled_t1"] = lambda i: dv.orthrus_accept_sampled(
            logits_ds[i % n_logits], logits_as[i % n_logits], d_tok, 1.0, u_acc, u_res, tok_s, n_acc, n_emit, nxt,
            workspace=ws_accs,
            stream=None)
        op_calls["quantize_block_kv"] = lambda i: dv.orthrus_quantize_kv(kb_v, vb_v, scale, scale, kb8_v, vb8_v,
                                                                         stream=None)
        torch.cuda.synchronize()
    op_ms, op_min = {}, {}
    for op, call in ([] if args.quick else op_calls.items()):
        graph = capture(lambda call=call: [call(i) for i in range(REPS)])
        # settle clocks and caches before timing: replay for at least 40 ms
        # (a few replays leave the shader clock ramping and read ~10 % slow)
        torch.cuda.synchronize()
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < 0.04:
            graph.replay()
            torch.cuda.synchronize()
        samples = []
        for _ in range(9):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            samples.append(e0.elapsed_time(e1) / REPS)
        op_ms[op] = statistics.median(samples)
        op_min[op] = min(samples)
    op_med = op_ms

    # ---- algorithmic bytes / flops per attention launch ----------------------
    pages_read = sum(-(-l // 16) for l in L)
    attn_bytes = (kv_bytes + 2 * B * K * Hq * D * 2 + 2 * 2 * B * K * Hkv * D * 2 + 4 * pages_read + 4 * B)
    attn_flops = 4.0 * Hq * K * D * sum(l + K for l in L)
    if args.quick:
        print(json.dumps({"ms_per_step": round(ms_per_step, 4), "steps": args.steps}), flush=True)
        return
    dom = max(("draft_attn", "verify_attn"), key=lambda o: op_ms[o])
    dom_s = op_ms[dom] * 1e-3
    achieved = attn_bytes / dom_s / 1e9
    traffic = measured_traffic(args.workload)

    value = 2 * kv_bytes / (ms_per_step * 1e-3) / 1e9   # KV bytes of both passes per step
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1/sqrt(D)) bf16 Q/K/V, shuffled 16-token pages; "
                "planted-argmax fp32 logits with geometric(0.15) accepted lengths)",
        "config": {"workload": args.workload, "batch": B, "context": L if B > 1 else L[0],
                   "block_k": K, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "page_size": 16,
                   "vocab": V, "split_tokens": dv.orthrus_attn_split_tokens(B, Hkv, max_ctx)
                   if args.split == 0 else args.split, "kv_pool_copies": n_pools},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "steps_per_s": round(1e3 / ms_per_step, 1),
        # emitted tokens per step: the timed step's own drawn accepted lengths,
        # and the expectation under geometric(0.15) acceptance (per sequence
        # sum_{k<K} 0.85^k = 6.63 at K = 32)
        "tokens_per_step": {
            "realised": int(sum(min(int(a) + 1, K) for a in cons.n_acc)),
            "expected": round(B * sum(0.85 ** k for k in range(K)), 2),
            # the same expectation for other per-token rejection rates p (the
            # step's time does not depend on it; tokens/s = tokens/step x steps/s)
            "expected_by_p": {str(pr): round(B * sum((1 - pr) ** k for k in range(K)), 2)
                              for pr in (0.08, 0.15, 0.3)},
        },
        "settle": {"warmup_steps": args.warmup, "settle_steps": n_settle, "settle_min_ms": 40},
        "op_ms": {k: round(v, 4) for k, v in op_ms.items()},
        "timing": "HIP graph replay" if args.graph else "eager launches",
        "attn_kv_gbps": {o: round(kv_bytes / (op_ms[o] * 1e-3) / 1e9, 1)
                         for o in ("draft_attn", "verify_attn")},
        "roofline": {
            "kernel": f"{dom}: attn_split_kernel + attn_combine_kernel (one ABI call)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": attn_bytes,
            "mfma_tflops": round(attn_flops / dom_s / 1e12, 1),
            "mfma_frac": round(attn_flops / dom_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        },
    }
    lm_s = op_ms["lmhead_argmax"] * 1e-3
    if B * K <= 32:      # weight-streaming kernel: bound by one pass over the weights
        lm_roof = {"kernel": "lmhead_kernel + argmax_final_kernel (one ABI call)", "bound": "hbm",
                   "achieved": round(lm_bytes / lm_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                   "frac": round(lm_bytes / lm_s / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                   "algorithmic_bytes_per_launch": lm_bytes}
    else:                # GEMM-tiled kernel: a dense contraction over B*K rows
        lm_flops = 2.0 * B * K * V * Hd
        lm_roof = {"kernel": "lmhead_gemm_range_kernel, lmhead_gemm_kernel or lmhead_gemm_wide_kernel (the host's pick) + argmax_final_kernel"
                             " (one ABI call)", "bound": "mfma",
                   "achieved": round(lm_flops / lm_s / 1e12, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": round(lm_flops / lm_s / 1e12 / BF16_PEAK_TFLOPS, 4), "traffic": None,
                   "algorithmic_flops_per_launch": lm_flops, "algorithmic_bytes_per_launch": lm_bytes}
    res["lmhead"] = {
        "config": {"rows": B * K, "hidden": Hd, "vocab": V},
        "op_ms": {o: round(op_ms[o], 4) for o in ("lmhead_argmax", "lmhead_accept")},
        "roofline": lm_roof,
    }
    attn8 = ("draft_attn_fp8", "verify_attn_fp8")
    dom8 = max(attn8, key=lambda o: op_ms[o])
    attn_bytes8 = (kv_bytes // 2 + 2 * B * K * Hq * D * 2 + 2 * B * K * Hkv * D + 4 * pages_read + 4 * B
                   + 2 * 4 * Hkv)
    res["fp8_kv"] = {
        "kv_dtype": "e4m3 (per-KV-head fp32 scales), attention arithmetic as the bf16 cache's",
        "op_ms": {o: round(op_ms[o], 4) for o in attn8 + ("quantize_block_kv",)},
        "attn_kv_gbps": {o: round(kv_bytes / 2 / (op_ms[o] * 1e-3) / 1e9, 1) for o in attn8},
        "speedup_vs_bf16_cache": {o: round(op_ms[o.replace("_fp8", "")] / op_ms[o], 3) for o in attn8},
        "roofline": {"kernel": f"{dom8}: attn_split_kernel<e4m3> + attn_combine_kernel (one ABI call)",
                     "bound": "hbm", "achieved": round(attn_bytes8 / (op_ms[dom8] * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_bytes8 / (op_ms[dom8] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.workload, "hbm_bytes_per_fp8_attention_call"),
                     "algorithmic_bytes_per_launch": attn_bytes8,
                     "mfma_tflops": round(attn_flops / (op_ms[dom8] * 1e-3) / 1e12, 1)},
    }
    logit_bytes = B * K * V * 4
    samp_gbps = logit_bytes / (op_ms["draft_sample_t1"] * 1e-3) / 1e9
    res["sampling_t1"] = {
        "op_ms": {o: round(op_ms[o], 4) for o in ("draft_sample_t1", "accept_sampled_t1")},
        "logits_gbps": {"draft_sample_t1": round(samp_gbps, 1),
                        "accept_sampled_t1": round(2 * logit_bytes / (op_ms["accept_sampled_t1"] * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": "draft_sample_t1: sample_stats_kernel + sample_draw_kernel (one ABI call)",
                     "bound": "hbm", "achieved": round(samp_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(samp_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": logit_bytes},
        "note": "fp32 logits read once per statistics pass (the draw rereads one chunk per row); "
                "fp64 exponentials",
    }
    # the consensus ops of the timed step, each one pass over one view's fp32 logits
    res["consensus_roofline"] = {
        o: {"bound": "hbm", "achieved": round(logit_bytes / (op_ms[o] * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(logit_bytes / (op_ms[o] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes_per_launch": logit_bytes}
        for o in ("draft_argmax", "accept")}
    if args.workload == "qwen3_8b_40k" and not args.no_extra_workloads:
        res["qwen3_8b_4k"] = workload_object(args, torch, dv, synth, "qwen3_8b_4k")
        res["qwen3_8b_ragged16"] = workload_object(args, torch, dv, synth, "qwen3_8b_ragged16")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, case, (qv, kbv, vbv), cons, kv_bytes)
    print(json.dumps(res), flush=True)


def time_graph(torch, graph, reps):
    """Replay a captured graph for at least 40 ms (settled clocks), then
    return the median of 9 timed replays, in ms per call (reps calls each)."""
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.04:
        graph.replay()
        torch.cuda.synchronize()
    samples = []
    stream = torch.cuda.current_stream()
    for _ in range(9):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        samples.append(e0.elapsed_time(e1) / reps)
    return statistics.median(samples)


def workload_object(args, torch, dv, synth, name):
    """Draft and verify attention, the consensus and the commit of another
    workload (the 4K single sequence or the 16-sequence ragged batch), with
    inputs drawn on the device from a seeded generator: K/V N(0, 1/sqrt(D))
    in independently permuted pool copies (at least 1.3 GB in all), planted
    argmax logits with geometric(0.15) accepted lengths in 8 rotating buffers
    per view.  Per-op times are graph replays of 16 calls; the step time is
    graph replays of whole steps."""
    import numpy as np
    w = synth.WORKLOADS[name]
    B, K, Hq, Hkv, D, V = w["B"], w["K"], w["Hq"], w["Hkv"], w["D"], w["V"]
    lens = np.asarray(w["seq_lens"] if w["seq_lens"] is not None else synth.ragged_lengths(w["seed"], B),
                      dtype=np.int64)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(w["seed"] + 31)
    per_seq = [-(-(int(l) + K) // 16) for l in lens]
    maxp = max(per_seq) + 1
    npages = sum(per_seq) + 8
    sd = 1.0 / math.sqrt(D)
    kp = (torch.randn((npages, Hkv, 16, D), generator=g, device=dev) * sd).to(torch.bfloat16)
    vp = (torch.randn((npages, Hkv, 16, D), generator=g, device=dev) * sd).to(torch.bfloat16)
    n_pools = max(2, min(128, math.ceil(1.3e9 / (2 * kp.numel() * 2))))
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    kvs = []
    for c in range(n_pools):
        perm = torch.randperm(npages, generator=g, device=dev).to(torch.int32)
        table = torch.full((B, maxp), int(perm[-1]), dtype=torch.int32, device=dev)
        o = 0
        for b, n in enumerate(per_seq):
            table[b, :n] = perm[o:o + n]
            o += n
        kvs.append(dv.PagedKV(kp if c == 0 else kp.clone(), vp if c == 0 else vp.clone(), table, seq))
    q = [(torch.randn((B, K, Hq, D), generator=g, device=dev) * sd).to(torch.bfloat16) for _ in range(2)]
    kb = [(torch.randn((B, K, Hkv, D), generator=g, device=dev) * sd).to(torch.bfloat16) for _ in range(2)]
    vb = [(torch.randn((B, K, Hkv, D), generator=g, device=dev) * sd).to(torch.bfloat16) for _ in range(2)]
    out = [torch.empty_like(q[0]) for _ in range(2)]
    # planted consensus: the draft agrees with the AR view on the drawn n_acc
    # positions of every sequence, the next position differs
    rng = np.random.default_rng(w["seed"] + 32)
    n_acc_drawn = synth.draw_accept_lengths(rng, B, K, "geometric", 0.15)
    a_idx = rng.integers(0, V, size=(B, K))
    d_idx = rng.integers(0, V, size=(B, K))
    for b in range(B):
        j = int(n_acc_drawn[b])
        d_idx[b, :j] = a_idx[b, :j]
        if j < K:
            d_idx[b, j] = (a_idx[b, j] + 1 + rng.integers(0, V - 1)) % V
    bi = torch.arange(B, device=dev)[:, None].expand(B, K)
    ki = torch.arange(K, device=dev)[None, :].expand(B, K)

    def planted(idx):
        x = torch.randn((B, K, V), generator=g, device=dev).clamp_(-8.0, 8.0)
        x[bi, ki, torch.from_numpy(idx).to(dev)] = 9.0 + torch.rand((B, K), generator=g, device=dev)
        return x
    n_logits = 8
    lds = [planted(d_idx) for _ in range(n_logits)]
    las = [planted(a_idx) for _ in range(n_logits)]
    max_ctx = int(lens.max())
    ws_attn = dv.attn_workspace(kvs[0], q[0], max_ctx, 0)
    ws_arg = dv.argmax_workspace(B * K, V, dev)
    d_tok, a_tok = (torch.empty((B, K), dtype=torch.int32, device=dev) for _ in range(2))
    n_acc, n_emit, nxt, lens_out = (torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4))
    ops = {
        "draft_attn": lambda i: dv.orthrus_attn_draft(kvs[(2 * i) % n_pools], q[0], kb[0], vb[0], out[0],
                                                      max_ctx=max_ctx, workspace=ws_attn, stream=None),
        "draft_argmax": lambda i: dv.orthrus_argmax(lds[i % n_logits], d_tok, workspace=ws_arg, stream=None),
        "verify_attn": lambda i: dv.orthrus_attn_verify(kvs[(2 * i + 1) % n_pools], q[1], kb[1], vb[1], out[1],
                                                        max_ctx=max_ctx, workspace=ws_attn, stream=None),
        "accept": lambda i: dv.orthrus_accept(las[i % n_logits], d_tok, a_tok, n_acc, n_emit, nxt,
                                              workspace=ws_arg, stream=None),
        "commit": lambda i: dv.orthrus_commit_kv(kvs[(2 * i + 1) % n_pools], kb[1][None], vb[1][None], n_emit,
                                                 lens_out, stream=None),
    }
    for i in range(2):                      # eager: initialises everything the graphs capture
        for op in ops.values():
            op(i)
    torch.cuda.synchronize()
    assert torch.equal(n_acc.cpu(), torch.from_numpy(np.asarray(n_acc_drawn, dtype=np.int32))), "accept mismatch"

    def capture(fn):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        return graph
    REPS = 16
    op_ms = {op: time_graph(torch, capture(lambda call=call: [call(i) for i in range(REPS)]), REPS)
             for op, call in ops.items()}
    n_steps = 8                              # one graph of 8 whole steps (rotating copies)
    ms_per_step = time_graph(torch, capture(lambda: [ops[o](j) for j in range(n_steps) for o in ops]), n_steps)
    kv_bytes = 4 * Hkv * D * int(lens.sum())
    pages_read = int(sum(-(-int(l) // 16) for l in lens))
    attn_bytes = kv_bytes + 2 * B * K * Hq * D * 2 + 2 * 2 * B * K * Hkv * D * 2 + 4 * pages_read + 4 * B
    attn_flops = 4.0 * Hq * K * D * float(sum(int(l) + K for l in lens))
    dom = max(("draft_attn", "verify_attn"), key=lambda o: op_ms[o])
    dom_s = op_ms[dom] * 1e-3
    res = {
        "config": {"workload": name, "batch": B, "context": [int(x) for x in lens] if B > 1 else int(lens[0]),
                   "block_k": K, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "vocab": V,
                   "split_tokens": dv.orthrus_attn_split_tokens(B, Hkv, max_ctx), "kv_pool_copies": n_pools},
        "data": "synthetic, drawn on the device (seeded): K/V N(0,1/sqrt(D)), planted-argmax logits with "
                "geometric(0.15) accepted lengths",
        "op_ms": {k: round(v, 4) for k, v in op_ms.items()},
        "ms_per_step": round(ms_per_step, 4),
        "steps_per_s": round(1e3 / ms_per_step, 1),
        "kv_gbps_per_step": round(2 * kv_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "tokens_per_step": {"realised": int(sum(min(int(a) + 1, K) for a in n_acc_drawn)),
                            "expected": round(B * sum(0.85 ** k for k in range(K)), 2)},
        "attn_kv_gbps": {o: round(kv_bytes / (op_ms[o] * 1e-3) / 1e9, 1) for o in ("draft_attn", "verify_attn")},
        "roofline": {"kernel": f"{dom}: attn_split_kernel + attn_combine_kernel (one ABI call)", "bound": "hbm",
                     "achieved": round(attn_bytes / dom_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_bytes / dom_s / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": attn_bytes,
                     "mfma_tflops": round(attn_flops / dom_s / 1e12, 1)},
    }
    del kvs, kp, vp, lds, las
    torch.cuda.empty_cache()
    return res


def e2e(args, torch, dv, synth):
    """Whole decode steps of the Qwen3-8B-shaped model (36 layers, random bf16
    weights, all layers' KV cache filled with N(0,1) values to the given
    context): one greedy step (1 row) against one Orthrus step (draft pass of K
    rows, fused LM-head argmax, verify pass, fused LM-head acceptance, commit),
    each replayed from a HIP graph.  Tokens per second of the Orthrus loop are
    given for mean emitted lengths 5.39 (the pages' reported mean) and 6.63
    (geometric(0.15) acceptance); acceptance changes only the commit size."""
    from dual_view_draft_amd.model import DualViewModel, ModelCache
    cfg, K = synth.QWEN3_8B, 32
    dev = torch.device("cuda:0")
    model = DualViewModel(cfg, synth.make_model_weights_device(8, cfg, dev), max_block=K)
    res = {"e2e": "qwen3_8b_shape", "layers": cfg.layers, "hidden": cfg.hidden, "vocab": cfg.vocab,
           "block_k": K, "timing": "HIP graph replay", "contexts": []}
    reps = 10
    # an e4m3 cache uses one scale (1/32) for every layer and head here: the
    # timing does not depend on the values
    scale8 = torch.full((cfg.layers, cfg.Hkv), 1.0 / 32, dtype=torch.float32, device=dev)
    runs = [(int(x), kv) for x in args.e2e_contexts.split(",") for kv in ("bf16", "e4m3")]
    for L, kv in runs:
        cache = ModelCache(cfg, L + (4 * reps + 8) * K + 256, dev,
                           kv_scales=(scale8, scale8) if kv == "e4m3" else None)
        cache.fill_random(L)
        tok = torch.zeros(1, dtype=torch.int64, device=dev)
        out = torch.zeros(1, dtype=torch.int32, device=dev)
        anchor = torch.zeros(1, dtype=torch.int64, device=dev)
        d, a = (torch.zeros((1, K), dtype=torch.int32, device=dev) for _ in range(2))
        n_acc, n_emit, nxt = (torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(3))

        def greedy2():
            for _ in range(2):                 # two steps: the length buffers return to their roles
                model.greedy_step(cache, tok, out)

        def orthrus2():
            for _ in range(2):
                model.orthrus_step(cache, anchor, K, d, a, n_acc, n_emit, nxt)

        times = {}
        for name, fn in (("greedy_step_ms", greedy2), ("orthrus_step_ms", orthrus2)):
            fn()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            times[name] = e0.elapsed_time(e1) / (2 * reps)
        tg, to = times["greedy_step_ms"], times["orthrus_step_ms"]
        res["contexts"].append({
            "context": L, "kv_cache": kv, "greedy_step_ms": round(tg, 3), "orthrus_step_ms": round(to, 3),
            "greedy_tokens_per_s": round(1e3 / tg, 1),
            "orthrus_tokens_per_s": {str(e): round(e * 1e3 / to, 1) for e in (5.39, 6.63)},
            "speedup_vs_greedy": {str(e): round(e * tg / to, 2) for e in (5.39, 6.63)},
            "break_even_tokens_per_step": round(to / tg, 2)})
        del cache
        torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, case, vqkv, cons, kv_bytes):
    """The CPU oracle (fp64 numpy) timed on this host over the same workload:
    a bounded sample of whole steps (draft + verify attention over every head,
    both argmaxes, acceptance, commit), with every BLAS thread the process may
    use, then one step on a single thread."""
    import numpy as np
    import threadpoolctl

    import oracle
    qv, kbv, vbv = vqkv
    f = oracle.from_bf16
    kp, vp = f(case.k_pages[0]), f(case.v_pages[0])

    def one_step():
        t = time.perf_counter()
        oracle.block_attention(f(case.q), f(case.k_blk), f(case.v_blk), kp, vp, case.block_table,
                               case.seq_lens, "draft")
        d = oracle.argmax_rows(cons.logits_d)
        oracle.block_attention(f(qv), f(kbv), f(vbv), kp, vp, case.block_table, case.seq_lens, "verify")
        a = oracle.argmax_rows(cons.logits_a)
        _, n_emit, _ = oracle.accept(d, a)
        oracle.commit_kv(case.k_pages[:1], case.v_pages[:1], case.block_table, case.seq_lens,
                         kbv[None], vbv[None], n_emit)
        return time.perf_counter() - t

    times = [one_step() for _ in range(max(1, args.cpu_steps))]
    sec = statistics.median(times)
    threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    with threadpoolctl.threadpool_limits(limits=1):
        sec1 = one_step()
    try:
        affinity = sorted(os.sched_getaffinity(0))
    except AttributeError:
        affinity = list(range(os.cpu_count() or 1))
    return {"value": round(2 * kv_bytes / sec / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "seconds_per_step": round(sec, 3),
            "steps_per_s": round(1.0 / sec, 4),
            "single_thread": {"seconds_per_step": round(sec1, 3), "value": round(2 * kv_bytes / sec1 / 1e9, 3),
                              "unit": "GB/s"},
            "cpu_model": cpu_model(), "affinity": f"{len(affinity)} CPUs: {affinity[0]}-{affinity[-1]}"
            if affinity and affinity[-1] - affinity[0] + 1 == len(affinity) else str(affinity),
            "sample": f"{len(times)} whole steps of the {args.workload} workload (median) with {threads} "
                      f"BLAS threads on {len(affinity)} CPUs the process may use, then 1 step on 1 thread; "
                      f"numpy fp64"}


if __name__ == "__main__":
    main()

"""The GPU models' dense-layer code against the fp64 oracle decoder
(oracle/toy.py) on one small shared config, TOY_CHECK (2 layers, hidden 256,
8/2 heads of 64, SwiGLU 512, vocabulary 2048, RoPE base 1e6), with the same
bf16 weights.  Orthrus == greedy alone cannot catch a mistake that both
loops share (a wrong RoPE base, QK-norm or <mask> embedding); this does.

Checked: the logits of every prompt position (a 200-token prompt, four
64-row prefill blocks through the paged cache) and of the diffusion view's
draft block [anchor, <mask> x 31] after it.  Bound: |gpu - oracle| <=
2^-4 * rms(row), from the bf16 roundings both GPU models make.
* The attention kernel takes q, k, v in bf16 (relative error 2^-9 each).
  After the QK RMSNorm |q| and |k| are at most sqrt(D), so a score
  q.k / sqrt(D) has magnitude at most sqrt(D) = 8 and moves by at most
  2 * 2^-9 * 8 = 2^-5: every softmax weight by a factor within e^(+-2^-5).
  Over the two layers the hidden state, and with it every logit, can move
  by about 2 * 2^-5 = 2^-4 of its scale.
* DualViewModel (the full-size model's code) also rounds every matrix
  product's inputs and outputs to bf16: about 20 more roundings of 2^-9
  whose signs are independent, so together about sqrt(20) * 2^-9 = 2^-6.8
  of the scale, inside the same bound; ToyOrthrus keeps its dense layers
  in fp64.
Greedy tokens: where the oracle's top-2 gap exceeds twice the bound, the
GPU's argmax must be the oracle's token (at least half of the positions
qualify at these seeds).

Planted mistakes in the oracle (RoPE base 1e4, a doubled QK-norm gain, a
wrong <mask> row) move the logits by 3-5 times the row's rms, far beyond
either bound (checked on the CPU in tests/test_oracle_toy.py)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

P, K, SEED = 200, 32, 21


@pytest.fixture(scope="module")
def ref():
    from oracle.toy import ToyModel
    from synth import TOY_CHECK, make_prompt, make_toy_weights
    cfg = TOY_CHECK
    bits = make_toy_weights(SEED, cfg)
    prompt = make_prompt(SEED, P, cfg.vocab)
    m = ToyModel(cfg, bits)
    cache = m.new_cache(P + 2 * K + 64)
    lz, k, v = m.forward(prompt, cache, "ar", "verify")
    m.commit(cache, k, v, P)
    ld, _, _ = m.forward([int(prompt[-1])] + [cfg.mask_id] * (K - 1), cache, "diff", "draft")
    return cfg, bits, prompt, lz, ld


def _check(name, got, want, tol_frac, min_checked=0.5):
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    tol = tol_frac * rms
    err = np.abs(got - want)
    worst = float((err / rms).max())
    assert np.all(err <= tol), f"{name}: max |gpu - oracle| / rms = {worst:.3e} > {tol_frac:.3e}"
    srt = np.sort(want, axis=-1)
    gap = srt[:, -1] - srt[:, -2]
    sure = gap > 2 * tol[:, 0]
    assert sure.mean() >= min_checked, f"{name}: only {sure.mean():.2f} of rows have a clear winner"
    assert np.array_equal(got[sure].argmax(-1), want[sure].argmax(-1)), f"{name}: greedy token differs"
    print(f"{name}: max err / rms {worst:.2e}, tokens compared at {int(sure.sum())}/{len(sure)} rows",
          flush=True)


def _prompt_and_draft_logits(model, cache, prompt, cfg, block_fn):
    rows = []
    for s0 in range(0, P, 64):
        rows.append(block_fn(prompt[s0:s0 + 64], cache, "ar", "verify", True))
    blk = torch.cat([prompt[-1:], torch.full((K - 1,), cfg.mask_id, dtype=torch.int64, device="cuda")])
    ld = block_fn(blk, cache, "diff", "draft", False)
    return torch.cat(rows).double().cpu().numpy(), ld.double().cpu().numpy()


def test_dual_view_model_matches_oracle(ref):
    import dual_view_draft_amd as dv
    from dual_view_draft_amd.model import DualViewModel
    cfg, bits, prompt_np, lz, ld = ref
    dv.load_library()

    def dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)
    w = {"embed": dev(bits["embed"]), "final_norm": dev(bits["final_norm"]),
         "lm_head": dev(bits["lm_head"]).t().contiguous()}
    for i in range(cfg.layers):
        p = f"l{i}."
        for n in ("attn_norm", "ffn_norm", "q_norm", "k_norm", "wo", "wo_diff", "w_down"):
            w[p + n] = dev(bits[p + n])
        for sfx in ("", "_diff"):
            w[p + "wqkv" + sfx] = torch.cat([dev(bits[p + x + sfx]) for x in ("wq", "wk", "wv")], 1).contiguous()
        w[p + "w_gate_up"] = torch.cat([dev(bits[p + "w_gate"]), dev(bits[p + "w_up"])], 1).contiguous()
    model = DualViewModel(cfg, w, max_block=K)
    cache = model.new_cache(P, 2 * K)
    prompt = torch.from_numpy(prompt_np).cuda()
    gz, gd = _prompt_and_draft_logits(model, cache, prompt, cfg,
                                      lambda t, c, view, mode, commit: model.block_logits(t, c, view, mode, commit))
    _check("DualViewModel prefill", gz, lz, 2.0 ** -4)
    _check("DualViewModel draft block", gd, ld, 2.0 ** -4)


def test_toy_orthrus_matches_oracle(ref):
    import dual_view_draft_amd as dv
    from dual_view_draft_amd.toy import ToyOrthrus
    cfg, bits, prompt_np, lz, ld = ref
    dv.load_library()
    model = ToyOrthrus(cfg, bits, max_block=K)
    cache = model.new_cache(P, 2 * K)
    prompt = torch.from_numpy(prompt_np).cuda()

    def block(t, c, view, mode, commit):
        logits, k, v = model.forward(t, c, view, mode)
        if commit:
            n = t.shape[0]
            c.commit(k, v, torch.full((1,), n, dtype=torch.int32, device="cuda"), n)
        return logits
    gz, gd = _prompt_and_draft_logits(model, cache, prompt, cfg, block)
    _check("ToyOrthrus prefill", gz, lz, 2.0 ** -4)
    _check("ToyOrthrus draft block", gd, ld, 2.0 ** -4)

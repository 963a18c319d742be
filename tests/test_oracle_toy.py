"""Pins for the oracle's decode loop: the Orthrus loop must emit exactly the
tokens of plain greedy decoding of the same model (CPU only, fp64)."""
import numpy as np
import pytest

from oracle import argmax_rows
from oracle.toy import (DiffusionDrafter, TeacherDrafter, ToyModel, WrongDrafter,
                        greedy_generate, orthrus_generate)
from synth import TOY_TINY, make_prompt, make_toy_weights

N, K = 40, 8


@pytest.fixture(scope="module")
def model():
    return ToyModel(TOY_TINY, make_toy_weights(21, TOY_TINY), page_size=4)


@pytest.fixture(scope="module")
def prompt():
    return make_prompt(22, 20, TOY_TINY.vocab)


@pytest.fixture(scope="module")
def greedy_ref(model, prompt):
    return greedy_generate(model, prompt, N + K)


def test_cached_greedy_equals_cache_free_recompute(model, prompt, greedy_ref):
    # greedy decoding by definition: rerun the whole sequence through the causal
    # AR view (no cache reuse) and take the last row's argmax
    seq = list(prompt)
    for t in range(12):
        cache = model.new_cache(len(seq) + 1)
        logits, _, _ = model.forward(seq, cache, "ar", "verify")
        nxt = int(argmax_rows(logits[-1:])[0])
        assert nxt == greedy_ref[t]
        seq.append(nxt)


def test_greedy_is_not_degenerate(greedy_ref):
    assert len(set(greedy_ref)) > 10


def test_orthrus_with_diffusion_drafter_is_lossless(model, prompt, greedy_ref):
    toks, emits = orthrus_generate(model, prompt, N, K, DiffusionDrafter())
    assert toks == greedy_ref[:N]
    assert all(1 <= e <= K for e in emits)


def test_orthrus_with_teacher_drafter_is_lossless(model, prompt, greedy_ref):
    toks, emits = orthrus_generate(model, prompt, N, K,
                                   TeacherDrafter(greedy_ref, 0.15, 5, TOY_TINY.vocab))
    assert toks == greedy_ref[:N]
    assert max(emits) == K and min(emits) >= 1
    assert len(emits) < N // 2  # several tokens per step on average


def test_orthrus_with_wrong_drafter_emits_one_per_step(model, prompt, greedy_ref):
    toks, emits = orthrus_generate(model, prompt, N, K, WrongDrafter(greedy_ref, TOY_TINY.vocab))
    assert toks == greedy_ref[:N]
    assert emits == [1] * (N - 1)


def test_orthrus_k1_is_greedy(model, prompt, greedy_ref):
    toks, emits = orthrus_generate(model, prompt, 15, 1, DiffusionDrafter())
    assert toks == greedy_ref[:15] and emits == [1] * 14


def test_sensitivity_wrong_commit_breaks_losslessness(model, prompt, greedy_ref):
    # planted mistake (in a copy of the oracle loop): commit one row too many
    # on a mismatch, i.e. keep the K/V of the rejected draft token
    class Bad(ToyModel):
        def new_cache(self, capacity, seed=0):
            return super().new_cache(2 * capacity, seed)

        def commit(self, cache, k, v, n_emit):
            super().commit(cache, k, v, min(n_emit + 1, k.shape[1]))
    bad = Bad(TOY_TINY, make_toy_weights(21, TOY_TINY), page_size=4)
    toks, _ = orthrus_generate(bad, prompt, N, K, TeacherDrafter(greedy_ref, 0.15, 5, TOY_TINY.vocab))
    assert toks != greedy_ref[:N]


def test_planted_model_mistakes_exceed_the_gpu_bounds():
    """The GPU models are compared with this oracle on TOY_CHECK at
    |gpu - oracle| <= 2^-4 rms(row) (tests/test_gpu_model_oracle.py).  A
    mistake the Orthrus == greedy checks cannot see, because both loops
    would share it, must move the logits far past that bound: a RoPE base of
    1e4 instead of 1e6, a doubled QK-norm gain, the wrong <mask> row."""
    import dataclasses
    from oracle.toy import ToyModel
    from synth import TOY_CHECK, f32_to_bf16_bits, make_prompt, make_toy_weights
    cfg = TOY_CHECK
    bits = make_toy_weights(21, cfg)
    prompt = make_prompt(21, 200, cfg.vocab)

    def logits(c, b, mask_tok):
        m = ToyModel(c, b)
        cache = m.new_cache(200 + 96)
        lz, k, v = m.forward(prompt, cache, "ar", "verify")
        m.commit(cache, k, v, 200)
        ld, _, _ = m.forward([int(prompt[-1])] + [mask_tok] * 31, cache, "diff", "draft")
        return lz, ld

    lz, ld = logits(cfg, bits, cfg.mask_id)
    doubled = {f"l{i}.q_norm": f32_to_bf16_bits(np.full(cfg.D, 2.0, np.float32)) for i in range(cfg.layers)}
    for name, c2, b2, mt in [("rope base", dataclasses.replace(cfg, rope_base=1e4), bits, cfg.mask_id),
                             ("qk norm", cfg, {**bits, **doubled}, cfg.mask_id),
                             ("mask row", cfg, bits, 5)]:
        z2, d2 = logits(c2, b2, mt)
        worst = max(float((np.abs(z2 - lz) / np.sqrt((lz * lz).mean(-1, keepdims=True))).max()),
                    float((np.abs(d2 - ld) / np.sqrt((ld * ld).mean(-1, keepdims=True))).max()))
        assert worst > 8 * 2.0 ** -4, (name, worst)

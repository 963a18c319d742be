"""End-to-end losslessness at the Qwen3-8B shape on the GPU: 36 layers, hidden
4096, 32/8 heads of 128, SwiGLU 12288, vocabulary 151936, random bf16 weights
N(0, 0.02) with a random diffusion module per layer (about 19 GB), bf16
matrix products with fp32 accumulation.  The Orthrus loop must emit exactly
the tokens of plain greedy decoding of the same model: with its own
(untrained) drafter, with a teacher drafter that proposes the greedy
continuation corrupted at a geometric position, and with a drafter that is
always wrong; and the same with an e4m3 KV cache (scales calibrated on the
prompt), whose block rows are quantised before both passes."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

PROMPT, N_NEW, K = 80, 48, 32


@pytest.fixture(scope="module")
def setup():
    import dual_view_draft_amd as dv
    from dual_view_draft_amd.model import DualViewModel
    from synth import QWEN3_8B, make_model_weights_device, make_prompt
    dv.load_library()
    cfg = QWEN3_8B
    model = DualViewModel(cfg, make_model_weights_device(8, cfg, "cuda"), max_block=K)
    prompt = torch.from_numpy(make_prompt(8, PROMPT, cfg.vocab)).cuda()
    ref, secs = model.greedy(prompt, N_NEW + K)          # extra tokens for the teacher drafter
    print(f"greedy: {len(ref)} tokens, {secs:.2f} s (eager launches)", flush=True)
    return model, prompt, ref


def test_greedy_is_not_degenerate(setup):
    _, _, ref = setup
    assert len(set(ref[:N_NEW])) > 10


def test_orthrus_own_drafter_matches_greedy(setup):
    model, prompt, ref = setup
    toks, emits, _ = model.orthrus(prompt, 16, K)
    assert toks == ref[:16]
    assert min(emits) >= 1


def test_orthrus_teacher_drafter_matches_greedy(setup):
    model, prompt, ref = setup
    rng = np.random.default_rng(3)
    V = model.cfg.vocab

    def teacher(out, k):
        e = len(out)
        d = np.array(ref[e:e + k], dtype=np.int32)
        m = min(int(rng.geometric(0.15)) - 1, k)
        if m < k:
            d[m] = (d[m] + 1) % V
        return d

    toks, emits, _ = model.orthrus(prompt, N_NEW, K, drafter=teacher)
    print(f"teacher drafter: {len(emits)} steps, mean emitted {np.mean(emits):.2f}", flush=True)
    assert toks == ref[:N_NEW]
    assert len(emits) < N_NEW // 2


def test_orthrus_wrong_drafter_matches_greedy(setup):
    model, prompt, ref = setup
    V = model.cfg.vocab
    toks, emits, _ = model.orthrus(prompt, 12, K,
                                   drafter=lambda out, k: (np.array(ref[len(out):len(out) + k]) + 1) % V)
    assert toks == ref[:12]
    assert emits == [1] * 11


@pytest.fixture(scope="module")
def fp8_ref(setup):
    model, prompt, _ = setup
    scales = model.calibrate_kv_scales(prompt)
    ref, _ = model.greedy(prompt, 32 + K, kv_scales=scales)
    print(f"greedy with the e4m3 cache: {ref[:12]} ...", flush=True)
    return scales, ref


def test_fp8_cache_teacher_drafter_matches_greedy(setup, fp8_ref):
    model, prompt, _ = setup
    scales, ref = fp8_ref
    assert len(set(ref[:32])) > 8
    rng = np.random.default_rng(5)
    V = model.cfg.vocab

    def teacher(out, k):
        e = len(out)
        d = np.array(ref[e:e + k], dtype=np.int32)
        m = min(int(rng.geometric(0.15)) - 1, k)
        if m < k:
            d[m] = (d[m] + 1) % V
        return d

    toks, emits, _ = model.orthrus(prompt, 32, K, drafter=teacher, kv_scales=scales)
    print(f"e4m3 teacher drafter: {len(emits)} steps, mean emitted {np.mean(emits):.2f}", flush=True)
    assert toks == ref[:32]
    assert len(emits) < 16


def test_fp8_cache_own_drafter_matches_greedy(setup, fp8_ref):
    model, prompt, _ = setup
    scales, ref = fp8_ref
    toks, emits, _ = model.orthrus(prompt, 12, K, kv_scales=scales)
    assert toks == ref[:12]


# ---- long context: the pages' 4K-40K regime, many splits and the merge ----
LONG_L, LONG_N = 40960, 48


def _teacher(ref, V, seed):
    rng = np.random.default_rng(seed)

    def teacher(out, k):
        e = len(out)
        d = np.array(ref[e:e + k], dtype=np.int32)
        m = min(int(rng.geometric(0.15)) - 1, k)
        if m < k:
            d[m] = (d[m] + 1) % V
        return d
    return teacher


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_orthrus_matches_greedy_at_40k_context(setup, kv):
    """Both loops start from the same 40960-token cache state (every layer's
    cache filled with the same seeded values) and the same anchor: the
    attention calls take 31 context splits and the combine, and the Orthrus
    loop must still emit greedy decoding's tokens, with the teacher drafter
    (every accepted length) and with the model's own drafter."""
    from dual_view_draft_amd.model import ModelCache
    model = setup[0]
    cfg = model.cfg
    scales = None
    if kv == "e4m3":
        s = torch.full((cfg.layers, cfg.Hkv), 1.0 / 32, dtype=torch.float32, device="cuda")
        scales = (s, s)
    import dual_view_draft_amd as dv
    dv.device_errors(clear=True)
    cache = ModelCache(cfg, LONG_L + LONG_N + 3 * K + 128, "cuda", seed=4, kv_scales=scales)
    first = 1234
    cache.fill_random(LONG_L, seed=9)
    ref, secs = model.decode_greedy(cache, first, LONG_N + K)
    print(f"{kv} 40K greedy: {len(ref)} tokens in {secs:.2f} s", flush=True)
    assert len(set(ref[:LONG_N])) > 10
    cache.fill_random(LONG_L, seed=9)
    toks, emits, _ = model.decode_orthrus(cache, first, LONG_N, K, drafter=_teacher(ref, cfg.vocab, 11))
    print(f"{kv} 40K teacher drafter: {len(emits)} steps, mean emitted {np.mean(emits):.2f}", flush=True)
    assert toks == ref[:LONG_N]
    assert len(emits) < LONG_N // 2
    cache.fill_random(LONG_L, seed=9)
    toks, emits, _ = model.decode_orthrus(cache, first, 12, K)
    assert toks == ref[:12]
    assert dv.device_errors(clear=True) == 0     # every length, page id and count the loops passed held

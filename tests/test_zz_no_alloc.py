"""orthrus_attn_verify_noalloc (no workspace: the library's static scratch)
against orthrus_attn_verify with a caller workspace: the same kernels, so
the outputs must be equal bit for bit.  Two calls in a row, the second on a
smaller input; then a call whose partials would not fit the scratch is
refused with ORTHRUS_ERR_WORKSPACE_TOO_SMALL and enqueues nothing."""
import pytest
import torch

from gpu_helpers import upload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def _both(dv, c, max_ctx):
    kv, q, kb, vb = upload_case(c)
    ref = torch.empty_like(q)
    dv.orthrus_attn_verify(kv, q, kb, vb, ref, max_ctx=max_ctx)
    got = torch.full_like(q, float("nan"))
    dv.orthrus_attn_verify_noalloc(kv, q, kb, vb, got, max_ctx=max_ctx)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_call_twice(lib):
    from synth import make_paged_case
    # the 40K workload's shape first (31 splits of 8 KV heads: 8.6 MB of
    # partials), then a smaller ragged batch that reuses the scratch
    big = make_paged_case(3, 1, 32, 32, 8, 128, [40960], sharp=True)
    print("noalloc 40K", flush=True)
    ref, got = _both(lib, big, 40960)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    small = make_paged_case(12, 3, 32, 8, 2, 128, [0, 37, 1000], sharp=True)
    print("noalloc small", flush=True)
    ref, got = _both(lib, small, 1000)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


def test_noalloc_refuses_calls_beyond_the_scratch(lib):
    from synth import make_paged_case
    c = make_paged_case(13, 1, 32, 32, 8, 128, [100])
    kv, q, kb, vb = upload_case(c)
    out = torch.zeros_like(q)
    # a max_ctx of 2^20 with 64-token splits asks for far more than 16 MiB
    # of partials; the host check refuses before anything is enqueued
    assert lib.orthrus_attn_workspace_bytes(1, 32, 32, 8, 128, 1 << 20, 64) > 16 << 20
    with pytest.raises(lib.OrthrusError, match="WORKSPACE_TOO_SMALL"):
        lib.orthrus_attn_verify_noalloc(kv, q, kb, vb, out, max_ctx=1 << 20, split_tokens=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)) == 0

"""The device error word: kernels that meet a violated device-side
precondition (a sequence length, a page id, an emitted count: values the
host checks cannot see) clamp it, stay in bounds, and set a bit that
orthrus_device_errors reads.  Valid inputs, including garbage in block-table
entries that no cached position uses, set nothing.  Every case here runs the
kernels' own bounds clamps; no access leaves the buffers."""
import numpy as np
import pytest
import torch

from gpu_helpers import bf16_dev, i32_dev, upload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dv():
    import dual_view_draft_amd as dv
    dv.load_library()
    return dv


def attend(dv, kv, q, kb, vb, max_ctx):
    out = torch.empty_like(q)
    dv.orthrus_attn_verify(kv, q, kb, vb, out, max_ctx=max_ctx)
    torch.cuda.synchronize()


def paged(seed, lens, K=8):
    from synth import make_paged_case
    return make_paged_case(seed, len(lens), K, 8, 2, 128, lens, fill="sentinel", extra_pages_per_seq=2)


def test_valid_calls_set_nothing(dv):
    dv.device_errors(clear=True)
    c = paged(1, [300, 0, 1000])
    kv, q, kb, vb = upload_case(c)
    # block-table entries past every sequence's cached positions may hold anything
    bt = kv.block_table.clone()
    for b, L in enumerate(c.seq_lens):
        first_unused = (int(L) + 15) // 16 + 1
        bt[b, first_unused:] = 10 ** 6
    kv.block_table = bt
    attend(dv, kv, q, kb, vb, int(max(c.seq_lens)))
    assert dv.device_errors(clear=True) == 0


def test_attention_flags_length_and_page(dv):
    dv.device_errors(clear=True)
    c = paged(2, [700, 90])
    kv, q, kb, vb = upload_case(c)
    kv.seq_lens = i32_dev([700 + 64, 90])             # beyond max_ctx = 700: clamped, flagged
    attend(dv, kv, q, kb, vb, 700)
    flags = dv.device_errors(clear=False)
    assert flags == dv.DEVERR_SEQ_LEN
    assert dv.device_errors(clear=True) == flags     # clear=False left it
    assert dv.device_errors(clear=True) == 0
    kv.seq_lens = i32_dev([700, 90])
    bt = kv.block_table.clone()
    bt[0, 20] = c.k_pages.shape[1] + 7                # a page of cached positions 320..335
    kv.block_table = bt
    attend(dv, kv, q, kb, vb, 700)
    assert dv.device_errors(clear=True) == dv.DEVERR_PAGE_ID
    bt[0, 20] = -3
    attend(dv, kv, q, kb, vb, 700)
    assert dv.device_errors(clear=True) == dv.DEVERR_PAGE_ID


def test_commit_flags_count_length_and_page(dv):
    K = 8
    c = paged(3, [40, 17], K)
    layers, B, Hkv, D = 1, 2, 2, 128
    kp, vp = bf16_dev(c.k_pages), bf16_dev(c.v_pages)
    kb = bf16_dev(np.zeros((layers, B, K, Hkv, D), np.uint16))
    out = torch.empty(B, dtype=torch.int32, device="cuda")

    def commit(seq_lens, n_emit, bt=None):
        kv = dv.PagedKV(kp[0], vp[0], bt if bt is not None else i32_dev(c.block_table), i32_dev(seq_lens))
        dv.device_errors(clear=True)
        dv.orthrus_commit_kv(kv, kb, kb, i32_dev(n_emit), out, pool_layer_stride=kp.stride(0))
        torch.cuda.synchronize()
        return dv.device_errors(clear=True)

    assert commit([40, 17], [K, 3]) == 0
    assert commit([40, 17], [K + 3, 3]) == dv.DEVERR_N_EMIT
    assert out.cpu().tolist() == [40 + K, 17 + 3]
    assert commit([40, 17], [-2, 3]) == dv.DEVERR_N_EMIT
    assert out.cpu().tolist() == [40, 20]
    maxp = c.block_table.shape[1]
    assert commit([2 ** 31 - 5, 17], [0, 3]) == dv.DEVERR_SEQ_LEN
    assert out.cpu().tolist()[0] == maxp * 16
    bt = i32_dev(c.block_table).clone()
    bt[1, 17 // 16] = -1                              # the page of row 0 of sequence 1
    assert commit([40, 17], [K, 3], bt) == dv.DEVERR_PAGE_ID
    assert commit([maxp * 16 - 2, 17], [K, 0]) == dv.DEVERR_PAGE_ID   # rows past the block table

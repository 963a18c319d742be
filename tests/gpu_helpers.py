"""Helpers shared by the GPU parity tests: upload synthetic cases, compare."""
import numpy as np
import torch

ATOL, RTOL = 2e-2, 1e-2   # |gpu - ref| <= ATOL + RTOL * |ref| for bf16 attention outputs


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def upload_case(c, layer: int = 0):
    """Device tensors of a synth.PagedCase (one layer's pools unless layer is None)."""
    from dual_view_draft_amd import PagedKV
    kp = bf16_dev(c.k_pages if layer is None else c.k_pages[layer])
    vp = bf16_dev(c.v_pages if layer is None else c.v_pages[layer])
    kv = PagedKV(kp, vp, i32_dev(c.block_table), i32_dev(c.seq_lens))
    return kv, bf16_dev(c.q), bf16_dev(c.k_blk), bf16_dev(c.v_blk)


def oracle_inputs(c):
    from oracle import from_bf16
    return (from_bf16(c.q), from_bf16(c.k_blk), from_bf16(c.v_blk), from_bf16(c.k_pages[0]),
            from_bf16(c.v_pages[0]), c.block_table, c.seq_lens)


def compare(gpu_bf16: torch.Tensor, ref: np.ndarray, what: str = ""):
    from oracle import from_bf16
    x = from_bf16(bf16_host_bits(gpu_bf16))
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), f"{what}: non-finite output"
    err = np.abs(x - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    msg = (f"{what}: {int(bad.sum())}/{bad.size} outside |d| <= {ATOL} + {RTOL}|ref|; "
           f"max abs err {err.max():.3e}, max err / rms(ref) {err.max() / rms:.3e}")
    assert not bad.any(), msg
    return float(err.max()), float(err.max() / rms)

"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and rejects invalid arguments before any GPU work (host
checks only; no kernel is launched here)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orthrus.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ORTHRUS_API\s+[\w\s\*]+?\b(orthrus_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import dual_view_draft_amd as dv
    return dv.load_library()


def test_header_declares_the_method_entry_points():
    names = declared_functions()
    for n in ("orthrus_attn_draft", "orthrus_attn_verify", "orthrus_accept", "orthrus_commit_kv",
              "orthrus_argmax"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (orthrus_\w+)", out))
    assert set(declared_functions()) == exported
    for n in declared_functions():
        assert hasattr(lib, n)


def test_binding_covers_every_export():
    import dual_view_draft_amd.binding as b
    assert set(b.EXPORTS) == set(declared_functions())
    for n in declared_functions():
        assert callable(getattr(b, n))


def test_version_and_status_strings(lib):
    assert lib.orthrus_abi_version() == 2
    assert lib.orthrus_status_string(-3) == b"ORTHRUS_ERR_WORKSPACE_TOO_SMALL"
    assert lib.orthrus_status_string(0) == b"ORTHRUS_OK"


def test_workspace_queries(lib):
    n = lib.orthrus_attn_workspace_bytes(1, 32, 32, 8, 128, 40960, 0)
    split = lib.orthrus_attn_split_tokens(1, 8, 40960)
    assert split % 64 == 0 and split > 0
    nsplit = -(-(40960 + 32) // split)
    assert n >= nsplit * 8 * 128 * (128 * 2 + 2 * 4)
    assert lib.orthrus_attn_workspace_bytes(1, 65, 32, 8, 128, 100, 0) == 0
    assert lib.orthrus_attn_workspace_bytes(1, 32, 32, 8, 96, 100, 0) == 0
    assert lib.orthrus_argmax_workspace_bytes(32, 151936) >= 32 * 8


def _kv(b, **kw):
    f = dict(k_pages=0x10000, v_pages=0x10000, block_table=0x20000, seq_lens=0x20000,
             num_pages=4096, page_size=16, num_kv_heads=8, head_dim=128, max_pages_per_seq=2600)
    f.update(kw)
    return b.orthrus_kv(**f)


@pytest.mark.parametrize("change,status", [
    (dict(page_size=8), -2), (dict(head_dim=80), -2), (dict(k_pages=0), -1),
    (dict(max_pages_per_seq=10), -4), (dict(v_pages=0x10004), -1),
])
def test_attention_rejects_bad_cache_descriptor(lib, change, status):
    import dual_view_draft_amd.binding as b
    kv = _kv(b, **change)
    P = ctypes.c_void_p(0x10000)
    for fn in (lib.orthrus_attn_draft, lib.orthrus_attn_verify):
        rc = fn(ctypes.byref(kv), P, P, P, P, 1, 32, 32, 0.088, 1000, 0, P, 1 << 40, None)
        assert rc == status, lib.orthrus_last_error()
        assert lib.orthrus_last_error() != b""


def test_attention_rejects_small_workspace_before_any_launch(lib):
    import dual_view_draft_amd.binding as b
    kv = _kv(b)
    P = ctypes.c_void_p(0x10000)
    need = lib.orthrus_attn_workspace_bytes(1, 32, 32, 8, 128, 1000, 0)
    rc = lib.orthrus_attn_verify(ctypes.byref(kv), P, P, P, P, 1, 32, 32, 0.088, 1000, 0, P, need - 16, None)
    assert rc == -3 and b"workspace" in lib.orthrus_last_error()


def test_batch_zero_calls_succeed_without_gpu(lib):
    import dual_view_draft_amd.binding as b
    kv = _kv(b)
    assert lib.orthrus_attn_draft(ctypes.byref(kv), None, None, None, None, 0, 32, 32, 0.088, 1000,
                                  0, None, 0, None) == 0
    assert lib.orthrus_argmax(None, 0, 151936, None, None, 0, None) == 0
    assert lib.orthrus_accept(None, None, 0, 32, 151936, None, None, None, None, None, 0, None) == 0
    assert lib.orthrus_commit_kv(ctypes.byref(kv), 1, 0, None, None, 0, None, 0, 32, None, None) == 0


def test_consensus_and_commit_argument_checks(lib):
    import dual_view_draft_amd.binding as b
    P = ctypes.c_void_p(0x10000)
    assert lib.orthrus_argmax(P, 4, 0, P, P, 1 << 20, None) == -1
    assert lib.orthrus_argmax(P, 4, 1000, P, P, 8, None) == -3
    assert lib.orthrus_accept(P, P, 1, 65, 1000, P, P, P, P, P, 1 << 20, None) == -2
    kv = _kv(b)
    assert lib.orthrus_commit_kv(ctypes.byref(kv), 1, 0, P, P, 0, P, 1, 32,
                                 ctypes.c_void_p(0x20000), None) == -1   # aliases seq_lens
    assert lib.orthrus_commit_kv(ctypes.byref(kv), 0, 0, P, P, 0, P, 1, 32, P, None) == -1


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "check_driver")
    csrc = os.path.join(ROOT, "dual_view_draft_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{csrc}", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "host", "check_driver.cpp"), os.path.join(csrc, "check.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK (0 failures)" in r.stdout


def test_device_errors_argument_checks(lib):
    lib.orthrus_device_errors.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert lib.orthrus_device_errors(None, 1, None) == -1          # null flags pointer
    assert lib.orthrus_device_errors(ctypes.c_void_p(0x10002), 0, None) == -1   # misaligned


def test_lmhead_workspace_and_argument_checks(lib):
    P = ctypes.c_void_p(0x10000)
    n = lib.orthrus_lmhead_workspace_bytes(32, 4096, 151936)
    assert n >= 32 * 256 * 8
    assert lib.orthrus_lmhead_workspace_bytes(32, 100, 151936) == 0      # hidden not a multiple of 64
    assert lib.orthrus_lmhead_workspace_bytes(32, 4096, 0) == 0
    assert lib.orthrus_lmhead_workspace_bytes(3, 64, 10) >= 3 * 10 * 8    # one workgroup per token
    assert lib.orthrus_lmhead_argmax(None, None, 0, 4096, 151936, None, None, None, 0, None) == 0
    assert lib.orthrus_lmhead_argmax(P, P, 4, 100, 1000, P, None, P, 1 << 20, None) == -2
    assert lib.orthrus_lmhead_argmax(P, P, 4, 128, 0, P, None, P, 1 << 20, None) == -1
    assert lib.orthrus_lmhead_argmax(P, P, 4, 128, 1000, P, None, P, 8, None) == -3
    assert lib.orthrus_lmhead_argmax(ctypes.c_void_p(0x10008), P, 4, 128, 1000, P, None, P, 1 << 20,
                                     None) == -1                            # misaligned hidden
    assert lib.orthrus_lmhead_accept(P, P, P, 1, 65, 128, 1000, P, P, P, P, P, 1 << 20, None) == -2
    assert lib.orthrus_lmhead_accept(None, None, None, 0, 32, 128, 1000, None, None, None, None, None, 0,
                                     None) == 0


@pytest.mark.parametrize("change,status", [
    (dict(kv_dtype=2), -1),                                   # unknown element type
    (dict(kv_dtype=1, head_dim=64), -2),                      # e4m3 needs head_dim 128
    (dict(kv_dtype=1, k_scale=0x30000, v_scale=0), -1),       # missing scale
    (dict(kv_dtype=1, k_scale=0x30002, v_scale=0x30000), -1), # misaligned scale
])
def test_attention_checks_the_e4m3_cache_descriptor(lib, change, status):
    import dual_view_draft_amd.binding as b
    kv = _kv(b, **change)
    P = ctypes.c_void_p(0x10000)
    for fn in (lib.orthrus_attn_draft, lib.orthrus_attn_verify):
        rc = fn(ctypes.byref(kv), P, P, P, P, 1, 32, 32, 0.088, 1000, 0, P, 1 << 40, None)
        assert rc == status, lib.orthrus_last_error()


def test_commit_of_an_e4m3_cache_needs_no_scales(lib):
    import dual_view_draft_amd.binding as b
    kv = _kv(b, kv_dtype=1)
    P = ctypes.c_void_p(0x10000)
    # a bad layer stride is the first failure, so the scales were not asked for
    assert lib.orthrus_commit_kv(ctypes.byref(kv), 2, 8, P, P, 0, P, 1, 32, P, None) == -1
    assert b"stride" in lib.orthrus_last_error()
    pool = 4096 * 8 * 16 * 128
    # strides in elements: a 1-byte element needs a multiple of 16 elements
    assert lib.orthrus_commit_kv(ctypes.byref(kv), 2, pool + 8, P, P, 32 * 8 * 128, P, 1, 32, P, None) == -1
    assert b"alignment" in lib.orthrus_last_error()


def test_quantize_argument_checks(lib):
    P = ctypes.c_void_p(0x10000)
    S = ctypes.c_void_p(0x20004)
    assert lib.orthrus_quantize_kv(None, None, None, None, 0, 8, 128, None, None, None) == 0
    assert lib.orthrus_quantize_kv(P, P, S, S, 32, 8, 120, P, P, None) == -1     # head_dim % 16
    assert lib.orthrus_quantize_kv(P, P, S, S, -1, 8, 128, P, P, None) == -1
    assert lib.orthrus_quantize_kv(P, P, None, S, 32, 8, 128, P, P, None) == -1
    assert lib.orthrus_quantize_kv(P, P, ctypes.c_void_p(0x20002), S, 32, 8, 128, P, P, None) == -1
    assert lib.orthrus_quantize_kv(P, ctypes.c_void_p(0x10008), S, S, 32, 8, 128, P, P, None) == -1


def test_sampling_workspace_and_argument_checks(lib):
    P = ctypes.c_void_p(0x10000)
    n = lib.orthrus_sample_workspace_bytes(32, 151936)
    assert n >= 32 * 12 * (4 + 8)                       # chunk statistics of every row
    assert lib.orthrus_sample_workspace_bytes(-1, 10) == 0
    assert lib.orthrus_sample(None, 0, 151936, ctypes.c_float(1.0), None, None, None, 0, None) == 0
    assert lib.orthrus_sample(P, 4, 1000, ctypes.c_float(0.0), P, P, P, 1 << 20, None) == -1
    assert lib.orthrus_sample(P, 4, 1000, ctypes.c_float(float("inf")), P, P, P, 1 << 20, None) == -1
    assert lib.orthrus_sample(P, 4, 1000, ctypes.c_float(1.0), None, P, P, 1 << 20, None) == -1
    assert lib.orthrus_sample(P, 4, 1000, ctypes.c_float(1.0), P, P, P, 8, None) == -3
    m = lib.orthrus_accept_sampled_workspace_bytes(4, 32, 151936)
    assert m > lib.orthrus_sample_workspace_bytes(2 * 4 * 32, 151936)   # plus the per-sequence state
    assert lib.orthrus_accept_sampled_workspace_bytes(1024, 64, 1000) == 0   # 2*B*K > 65535
    F = ctypes.c_float(1.0)
    assert lib.orthrus_accept_sampled(P, P, P, 1, 65, 1000, F, P, P, P, P, P, P, P, 1 << 20, None) == -2
    assert lib.orthrus_accept_sampled(P, P, P, 1, 32, 1000, ctypes.c_float(-1.0), P, P, P, P, P, P, P,
                                      1 << 20, None) == -1
    assert lib.orthrus_accept_sampled(P, P, P, 1, 32, 1000, F, P, None, P, P, P, P, P, 1 << 20, None) == -1
    assert lib.orthrus_accept_sampled(P, P, P, 1, 32, 1000, F, P, P, P, P, P, P, P, 64, None) == -3
    assert lib.orthrus_accept_sampled(None, None, None, 0, 32, 1000, F, None, None, None, None, None, None,
                                      None, 0, None) == 0

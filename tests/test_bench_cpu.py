"""bench.py's host-side bookkeeping (no GPU): the measured HBM traffic of the
attention call is reported only for the workload and kernel source it was
measured on."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_only_for_its_workload_and_source():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert bench.measured_traffic("qwen3_8b_ragged16") is None
    assert bench.measured_traffic("tiny") is None
    if t["attn_source_sha256_16"] == bench.kernel_source_hash():
        assert bench.measured_traffic(t["workload"]) == t["hbm_bytes_per_attention_call"]
        assert bench.measured_traffic(t["workload"], "hbm_bytes_per_fp8_attention_call") == \
            t["hbm_bytes_per_fp8_attention_call"]
    else:
        assert bench.measured_traffic(t["workload"]) is None


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    try:
        bench.main()
    except SystemExit as e:
        assert e.code == 2
    else:
        raise AssertionError("bench.py accepted --gpus 2")
    assert "one GPU only" in capsys.readouterr().err

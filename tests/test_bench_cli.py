"""bench.py's host-side contract (no GPU): a run on more than one GPU is
refused with a message, and a stored HBM traffic record is reported only
while it was taken on the current kernel source."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode != 0
    assert "one GPU" in (out.stdout + out.stderr)


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// version 1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_source_sha256": bench.kernel_source_digest(str(src)),
           "hbm_bytes_per_launch": 1234.0}
    (prof / "traffic_attn_fwd_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", "attn_fwd", str(src)) == pytest.approx(1234.0)
    assert bench.measured_traffic("other", "attn_fwd", str(src)) is None
    src.write_text("// version 2\n")  # the kernel changed since the counters were taken
    assert bench.measured_traffic("w", "attn_fwd", str(src)) is None


def test_committed_traffic_records_name_their_kernel_and_workload():
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not (name.startswith("traffic_") and name.endswith(".json")):
            continue
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
        assert name.endswith(f"_{rec['workload']}.json"), name
        assert rec["hbm_bytes_per_launch"] == pytest.approx(
            rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"])
        assert len(rec["kernel_source_sha256"]) == 64


def test_committed_traffic_records_match_the_current_kernel_sources():
    """Every committed traffic record was taken on the kernel source as it
    stands, so each bench line reports it (a kernel change since the counters
    were taken would turn the line's traffic into null)."""
    csrc = os.path.join(ROOT, "exact_attention_forward_02_amd", "csrc")
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not (name.startswith("traffic_") and name.endswith(".json")):
            continue
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
        src = os.path.join(csrc, rec["kernel_source"])
        assert rec["kernel_source_sha256"] == bench.kernel_source_digest(src), name

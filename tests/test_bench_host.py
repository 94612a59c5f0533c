"""Host-side parts of bench.py: the one-GPU contract and the counter-traffic
lookup (no GPU needed; nothing here launches a kernel)."""

import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_traffic_is_reported_only_for_the_counted_source_and_workload(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_FILE))
    sha = hashlib.sha256(open(bench.SCORE_SRC, "rb").read()).hexdigest()
    want = rec["hbm_bytes_per_launch"] if rec["score_hip_sha256"] == sha else None
    assert bench.traffic_if_current("llama8b-1m") == want
    assert bench.traffic_if_current("llama8b-32k") is None
    # a changed scorer source voids the stored counters
    src = tmp_path / "score.hip"
    src.write_bytes(open(bench.SCORE_SRC, "rb").read() + b"\n// changed\n")
    monkeypatch.setattr(bench, "SCORE_SRC", str(src))
    assert bench.traffic_if_current("llama8b-1m") is None
    # a missing counter file gives no traffic figure
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.traffic_if_current("llama8b-1m") is None


def test_algorithmic_units():
    # K2 page-head: 832-byte record read + 4 fp32 page scores written; K4: 16 x 128 bf16 of K and V
    assert bench.SCORE_BYTES_PER_PAGE_HEAD == 848
    assert bench.ATTEND_BYTES_PER_PAGE_HEAD == 2 * 16 * 128 * 2
    assert bench.PEAK_HBM_GBS == 8000.0

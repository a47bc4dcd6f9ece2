"""Host-side logic of bench.py (no GPU): the one-GPU guard and the rule that HBM
traffic is reported only from counters taken on the current kernel source."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr


def test_traffic_only_from_counters_of_the_current_source(tmp_path, monkeypatch):
    sha = bench.source_sha(bench.PREFILL_SOURCES)
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile(sha, 1.0) is None  # no counters at all
    path = prof / "prefill_swa_T32768_counters.json"
    path.write_text(json.dumps({"kernel_source_sha": sha, "hbm_bytes_per_launch": 1.6e9}))
    assert bench.traffic_from_profile(sha, 1.0) == 1.6e9
    path.write_text(json.dumps({"kernel_source_sha": "0" * 16, "hbm_bytes_per_launch": 1.6e9}))
    assert bench.traffic_from_profile(sha, 1.0) is None  # taken on another source
    path.write_text("not json")
    assert bench.traffic_from_profile(sha, 1.0) is None


def test_source_sha_covers_the_headline_kernel_files():
    assert "sliding_window_sink_amd/csrc/prefill_swa.hip" in bench.PREFILL_SOURCES
    assert "sliding_window_sink_amd/csrc/common.h" in bench.PREFILL_SOURCES
    assert len(bench.source_sha(bench.PREFILL_SOURCES)) == 16

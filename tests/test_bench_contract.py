"""Host-side pieces of bench.py's output contract: a recorded HBM-traffic figure is reported only for
the exact kernel sources and weight layout it was measured with, the algorithmic-byte count of the
decode step adds up, and asking for more than one GPU exits with a message."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_recorded_traffic_matches_sources_and_layout(tmp_path, monkeypatch):
    sha = bench.sources_sha("config3")
    rec = {"config3": {"layout": "swizzled", "gemm_sources_sha": sha, "hbm_bytes_per_launch": 123}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("config3", "swizzled") == 123
    assert bench.recorded_traffic("config3", "plain") is None          # other layout
    assert bench.recorded_traffic("config4", "swizzled") is None       # no record
    rec["config3"]["gemm_sources_sha"] = "0" * 16                      # sources changed since
    f.write_text(json.dumps(rec))
    assert bench.recorded_traffic("config3", "swizzled") is None


def test_decode_step_algorithmic_bytes():
    wl = workloads.config3()
    alg = bench.algorithmic_bytes(wl)
    assert alg["weights"] == 256 * (2048 * 7168 // 2 + 2048 * 7168 // 16 + 4) == 2_113_930_240
    assert alg["acts"] == 512 * 7168 + 512 * 56 * 4
    assert alg["out"] == 4096 * 2048 * 4
    assert alg["total"] == 2_151_292_932


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

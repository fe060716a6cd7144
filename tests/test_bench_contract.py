"""bench.py's contract on the host: one GPU only (a clear error for --gpus N
above 1, before any GPU is touched), and the measured-traffic figure taken
from the committed counter summary only while it matches the kernel
sources."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_summary_parses_and_is_tied_to_the_sources(tmp_path, monkeypatch):
    text = open(bench.TRAFFIC_FILE).read()
    assert "hbm_bytes_per_launch:" in text and "sources_sha256:" in text
    t = bench.measured_traffic()
    # either the committed counters belong to these sources, or the bench
    # reports no traffic
    assert t is None or 1e9 < t < 1e11
    # a summary with the current sources' hash is read; another hash is not
    good = tmp_path / "good.md"
    good.write_text(f"hbm_bytes_per_launch: 1.5e9\nsources_sha256: "
                    f"{bench.kernel_sources_sha256()}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.measured_traffic() == 1.5e9
    bad = tmp_path / "bad.md"
    bad.write_text("hbm_bytes_per_launch: 1.5e9\nsources_sha256: " + "0" * 64 + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(bad))
    assert bench.measured_traffic() is None

"""Host-side parts of bench.py (no GPU): more than one GPU is refused with a
message, and the counter-based traffic figure is reported only while the
committed summary was taken on the current kernel source."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    fresh = tmp_path / "fresh.md"
    fresh.write_text(f"kernel_source_sha256_16: {bench.kernel_sha()}\ntraffic_bytes_per_launch: 123456789\n")
    monkeypatch.setattr(bench, "TRAFFIC", str(fresh))
    assert bench.read_traffic() == (123456789.0, "fresh")

    stale = tmp_path / "stale.md"
    stale.write_text("kernel_source_sha256_16: 0123456789abcdef\ntraffic_bytes_per_launch: 123456789\n")
    monkeypatch.setattr(bench, "TRAFFIC", str(stale))
    assert bench.read_traffic() == (None, "stale")

    monkeypatch.setattr(bench, "TRAFFIC", str(tmp_path / "missing.md"))
    assert bench.read_traffic() == (None, None)


def test_committed_summary_is_readable():
    """The committed summary parses; whether it is fresh depends on whether
    the kernel changed after the counters were taken."""
    val, state = bench.read_traffic()
    assert state in ("fresh", "stale")
    if state == "fresh":
        assert val > 0

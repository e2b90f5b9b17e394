"""Host-side behaviour of bench.py that needs no GPU: a run on more than one GPU
is refused with a message (the path has no collectives), and the embedded HBM
counters of a kernel are reported only while its sources match the hash they
were taken with."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_needs_matching_sources(monkeypatch):
    files = bench._GEMM_SRC
    digest = bench._src_hash(files)
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, ("probe", "k"), (files, digest, 1000.0, 500.0))
    expect = int(round((1000.0 * bench.FETCH_SCALE + 500.0 * bench.WRITE_SCALE) * 1024))
    assert bench.measured_traffic("probe", "k") == expect
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, ("probe", "k"), (files, "0" * 16, 1000.0, 500.0))
    assert bench.measured_traffic("probe", "k") is None
    assert bench.measured_traffic("probe", "absent") is None

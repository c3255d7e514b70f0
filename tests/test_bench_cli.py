"""bench.py's command line on the host: more than one GPU is refused before any GPU work,
and the headline's HBM traffic is read from the committed counter summary."""
import os
import subprocess
import sys

from conftest import ROOT


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summary_is_readable():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.measured_traffic()
    # None only once the forward's sources change after the counters were taken
    assert t is None or 16 * 2 ** 20 <= t <= 20 * 2 ** 20

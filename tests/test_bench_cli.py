"""bench.py's command line on the CPU: more than one GPU is refused with a
message (the benchmark measures one GPU), and the traffic figures are read only
while the kernel source matches the one the counters were taken on."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_follows_the_kernel_source_hash(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    t = bench.measured_traffic("gemm_fwd_nt")
    assert t is None or t > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "not-the-source")
    assert bench.measured_traffic("gemm_fwd_nt") is None

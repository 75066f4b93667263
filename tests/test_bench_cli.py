"""bench.py's command line on the CPU: more than one GPU is refused with a
message (the benchmark measures one GPU), and the traffic figures are read only
while the kernel's code (its comments aside) matches the code the counters were
taken on."""

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


def test_kernel_hash_sees_code_not_comments():
    sys.path.insert(0, ROOT)
    import bench

    src = "int f(int x) {  // doubles x\n  /* body */\n  return 2 * x;\n}\n"
    reworded = "// f: twice its argument\nint f(int x) {  // x times two\n\n  return 2 * x;   \n}\n"
    changed = "int f(int x) {  // doubles x\n  return 3 * x;\n}\n"
    assert bench._code_only(src) == bench._code_only(reworded)
    assert bench._code_only(src) != bench._code_only(changed)

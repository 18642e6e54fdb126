"""bench.py's command line on the CPU: a GPU count other than one is refused
with a message (the benchmark runs on one GPU), before any device is touched;
the workload list and the byte accounting helpers are importable."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_workloads_listed():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.WORKLOADS[0] == "fp8_decode"
    assert len(set(bench.WORKLOADS)) == len(bench.WORKLOADS)

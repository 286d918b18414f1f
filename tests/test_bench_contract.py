"""bench.py's command-line contract, on the CPU: more than one GPU is refused with exit code 2
before anything touches a device, and the traffic summary it reports is plausible or withheld."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2, r.stderr[-500:]
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_summary_is_plausible_or_withheld():
    """The committed counter summary gives HBM bytes per attention call near the algorithmic
    277.4 MB of the loop workload, or nothing (None) once the kernel or its flags have changed."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.measured_traffic()
    assert t is None or 0.9 * 277413888 < t < 1.5 * 277413888

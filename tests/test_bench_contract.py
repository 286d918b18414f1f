"""bench.py's command-line contract, on the CPU: more than one GPU is refused with exit code 2
before anything touches a device, the traffic summary it reports is plausible or withheld, and the
board power readout is parsed from the tools' text or withheld when they fail."""
import os
import subprocess
import sys
import time

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


def test_power_clock_parsing():
    """The board power readout takes SOCKET_POWER and the CLK of each GFX_n domain, not the
    MIN/MAX limits nor the memory clock (text laid out as amd-smi prints it for one GPU)."""
    sys.path.insert(0, ROOT)
    import bench
    text = ("GPU: 0\n    POWER:\n        SOCKET_POWER: 1385 W\n        GFX_VOLTAGE: N/A\n    CLOCK:\n"
            "        GFX_0:\n            CLK: 1975 MHz\n            MIN_CLK: 500 MHz\n            MAX_CLK: 2400 MHz\n"
            "        GFX_1:\n            CLK: 1918 MHz\n            MIN_CLK: 500 MHz\n"
            "        MEM_0:\n            CLK: 2000 MHz\n            MIN_CLK: 2000 MHz\n")
    assert bench.parse_power_clock(text) == (1385, [1975, 1918])
    assert bench.parse_power_clock("no readings") == (None, [])


def test_power_readout_withheld_when_the_tool_fails(monkeypatch):
    """No amd-smi, or an amd-smi that fails or hangs, leaves the readout None instead of ending the
    bench; the busy-work thread is stopped either way."""
    sys.path.insert(0, ROOT)
    import bench
    calls = []
    monkeypatch.setattr(bench.shutil, "which", lambda name: None)
    assert bench.board_power(lambda: calls.append(1), settle_s=0.0) is None

    def hang(*a, **k):
        raise subprocess.TimeoutExpired(cmd="amd-smi", timeout=30)

    monkeypatch.setattr(bench.shutil, "which", lambda name: "/usr/bin/" + name)
    monkeypatch.setattr(bench.subprocess, "run", hang)
    assert bench.board_power(lambda: time.sleep(0.001), settle_s=0.0) is None


def test_power_readout_from_tool_text(monkeypatch):
    """Readings parsed from the tools' text, the cap from rocm-smi."""
    sys.path.insert(0, ROOT)
    import bench
    smi = ("GPU: 0\n    POWER:\n        SOCKET_POWER: 1399 W\n    CLOCK:\n        GFX_0:\n            CLK: 1990 MHz\n"
           "        GFX_1:\n            CLK: 2010 MHz\n")
    cap = "GPU[0]\t\t: Max Graphics Package Power (W): 1400.0\n"

    def run(cmd, **k):
        return subprocess.CompletedProcess(cmd, 0, stdout=cap if "--showmaxpower" in cmd else smi, stderr="")

    monkeypatch.setattr(bench.shutil, "which", lambda name: "/usr/bin/" + name)
    monkeypatch.setattr(bench.subprocess, "run", run)
    r = bench.board_power(lambda: time.sleep(0.001), settle_s=0.0, samples=2)
    assert r["board_w"] == [1399, 1399] and r["cap_w"] == 1400.0
    assert r["shader_mhz"] == {"min": 1990, "mean": 2000.0, "max": 2010}

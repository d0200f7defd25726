"""bench.py's contract on the host: one GPU only, and the counter-derived
traffic figure belongs to the committed source of the kernel it describes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_measured_traffic_matches_source():
    import bench
    # the byte counters were taken on this exact source of the headline kernel
    assert bench.measured_traffic("rb_gemv.hip", 1) == bench.MEASURED_TRAFFIC["rb_gemv.hip"][1]
    # only the measured configuration carries a figure
    assert bench.measured_traffic("rb_gemv.hip", 4) is None
    assert bench.measured_traffic("tq_wave.hip", 1) is None

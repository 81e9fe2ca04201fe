"""CPU checks of bench.py's command-line contract: one JSON line per run is a
GPU matter, but the defaults and the refusal of several GPUs are host logic."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_bench_defaults(monkeypatch):
    sys.path.insert(0, ROOT)
    try:
        import bench
    finally:
        sys.path.remove(ROOT)
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.algo) == (1, 50, 5, "lookback")
    assert not a.eager and not a.no_rows and a.rows == ""
    assert bench.N == 10 ** 8 and bench.HBM_PEAK_GBS == 8000.0

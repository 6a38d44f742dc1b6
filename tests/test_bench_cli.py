"""The bench's command-line contract on the host: more than one GPU is
declined with a message (this path is measured on one GPU only) and no
measurement line is printed; the fixed constants of the line.  No GPU is
touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_declined():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode != 0
    assert "one GPU only" in out and "--gpus 2" in out
    assert not any(l.startswith("{") for l in r.stdout.splitlines())


def test_bench_constants():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.HBM_PEAK_GBPS == 8000.0   # MI355X HBM3E datasheet peak
    assert bench.SMALL_M_LIST == (1, 2, 4, 8, 16, 24, 32, 48, 64)

"""CPU checks of bench.py's command-line contract (no GPU needed): more than
one GPU is refused with exit status 2 and a message, before anything touches
a device; the defaults finish within minutes (20 timed steps, 3 warm-up)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr and r.stdout == ""


def test_defaults():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert (a.gpus, a.steps, a.warmup) == (1, 20, 3)
    assert not a.no_cpu_baseline and not a.headline_only

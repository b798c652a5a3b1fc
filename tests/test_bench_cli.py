"""Host-side checks of bench.py's command line: refusals happen before any
GPU work (no device is needed to run these)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "single MI355X" in r.stderr and r.stdout == ""


def test_stack_batch_outside_range_is_refused():
    for b in ("0", "17"):
        r = _run("--stack-batch", b)
        assert r.returncode == 2 and "--stack-batch" in r.stderr and r.stdout == ""

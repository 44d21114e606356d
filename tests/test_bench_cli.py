"""bench.py's command line on a machine without a GPU: a run on more than one
GPU is refused with a message (the library has no multi-GPU path), before any
GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_names_the_timing_contract():
    r = _run("--help")
    assert r.returncode == 0
    assert "exactly K calls" in r.stdout

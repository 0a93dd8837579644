"""bench.py's command line on a machine without a GPU (no kernels run)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_modes():
    r = _run("--help")
    assert r.returncode == 0
    for mode in ("bench", "profile", "power", "selection", "workloads"):
        assert mode in r.stdout

"""Host-side checks of the benchmark script's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "ONE GPU" in (r.stdout + r.stderr)


def test_unknown_workload_is_rejected():
    r = _run("--workload", "cfg9")
    assert r.returncode != 0

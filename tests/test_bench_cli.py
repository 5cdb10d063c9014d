"""bench.py's command-line checks (host only: both exit before any GPU work)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_negative_seqs_is_refused():
    r = run("--workload", "1", "--seqs", "-1")
    assert r.returncode == 2
    assert "--seqs" in r.stderr

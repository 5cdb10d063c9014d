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


def test_acceptance_summary():
    """Per-position acceptance from counts, and the pages' E[N] formula at the
    measured rate (host arithmetic only)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    a = bench.acceptance_summary(np.array([0, 1, 1]), np.array([1, 1, 2]), 2)
    assert a["tested"] == [3, 1] and a["per_position"] == [0.6667, 0.0] and a["beta"] == 0.5
    assert abs(a["tokens_per_round"] - 5 / 3) < 1e-12 and a["tokens_per_round_predicted_iid"] == 1.75
    full = bench.acceptance_summary(np.array([3, 3]), np.array([3, 3]), 3)
    assert full["beta"] == 1.0 and full["tokens_per_round_predicted_iid"] == 4.0
    assert full["per_position"] == [1.0, 1.0, 1.0]


def test_tree_rows_read():
    """Rows a chain of five nodes needs in rounds by depth: the root, depths
    1-2 under an accepted depth-1 node, deeper nodes under an accepted depth-3
    node."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    lg = np.zeros((1, 5, 4), np.float32)
    lg[:, :, 0] = 1.0  # every row's arg-max is token 0
    par = np.array([[-1, 0, 1, 2, 3]], np.int32)
    assert bench.tree_rows_read(lg, np.array([[9, 0, 0, 1, 0]], np.int32), par, "fp32", True) == 3
    assert bench.tree_rows_read(lg, np.array([[9, 0, 0, 0, 0]], np.int32), par, "fp32", True) == 5
    assert bench.tree_rows_read(lg, np.array([[9, 2, 0, 0, 0]], np.int32), par, "fp32", True) == 1
    assert bench.tree_rows_read(lg, np.array([[9, 2, 0, 0, 0]], np.int32), par, "fp32", False) == 5

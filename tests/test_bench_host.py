"""Host-side logic of bench.py (no GPU): FLOP accounting of the widened rows."""

import numpy as np
import pytest

import bench
from oracle import attention as A


@pytest.mark.parametrize("n_q,n_k,causal,window", [
    (5, 5, True, (-1, -1)), (4, 6, False, (1, 1)), (6, 3, True, (-1, -1)), (5, 2, False, (0, 1)),
    (300, 300, True, (64, 0)), (100, 333, True, (-1, -1)), (333, 100, False, (10, 5)), (64, 640, True, (100, 0)),
])
def test_visible_pairs_match_the_mask(n_q, n_k, causal, window):
    assert bench.visible_pairs(n_q, n_k, causal, window) == int(A.visible(n_q, n_k, causal, window).sum())


def test_visible_pairs_headline_shapes():
    n = 8192
    assert bench.visible_pairs(n, n, True) == n * (n + 1) // 2
    w = 1024  # a causal window 1024 keys back: rows 0..1023 see i + 1 keys, the rest 1025
    assert bench.visible_pairs(n, n, True, (w, 0)) == w * (w + 1) // 2 + (n - w) * (w + 1)
    assert bench.visible_pairs(2048, n, True) == sum(i + n - 2048 + 1 for i in range(2048))


@pytest.mark.parametrize("args", [["--seq", "512"], ["--seq", "512", "--only", "copy64"], ["--gpus", "2"]])
def test_bench_refuses_unsupported_runs(args):
    """--seq profiles one attention kernel (it needs --only with a kernel name), and
    more than one GPU is refused: both before any GPU work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + args, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])

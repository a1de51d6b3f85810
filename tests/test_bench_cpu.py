"""CPU checks of bench.py: the algorithmic work it divides by, against a brute
count from the attention mask, and its refusal of more than one GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports no GPU code at module level)


def brute_pairs(n, block, topk, q_offset=0, full=False, rows=None):
    """(row, key) pairs of the causal mask restricted to each query block's
    selected blocks: the diagonal block plus the topk-1 blocks before it (any
    choice gives the same count when every block before the diagonal is full)."""
    r = np.arange(n)[:, None] + q_offset
    c = np.arange(n + q_offset)[None, :]
    allowed = c <= r
    if not full:
        qblk = r // block
        kblk = c // block
        allowed &= (kblk == qblk) | ((kblk < qblk) & (kblk >= qblk - (topk - 1)))
    if rows is not None:
        allowed = allowed[rows[0]:rows[1]]
    return int(allowed.sum())


def test_sparse_pairs_match_the_mask():
    for n, topk in ((512, 4), (1024, 1), (768, 12), (64 * 9, 16)):
        assert bench.sparse_useful_pairs(n // 64, topk, 64) == brute_pairs(n, 64, topk), (n, topk)


def test_full_pairs_match_the_mask():
    assert bench.full_useful_pairs(0, 1000) == brute_pairs(1000, 64, 0, full=True)
    assert bench.full_useful_pairs(300, 700) == brute_pairs(1000, 64, 0, full=True, rows=(300, 700))


def test_prefill_8k_work_figures():
    # 4 d flops per attended pair (two products of 2 d), 32 heads
    sparse = 4 * 64 * 32 * bench.sparse_useful_pairs(128, 16, 64)
    full = 4 * 64 * 32 * bench.full_useful_pairs(0, 8192)
    assert round(sparse / 1e9, 2) == 62.58
    assert round(full / 1e9, 1) == 274.9


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""

"""The bench's work units and contract on the CPU (no GPU, no timing).

The reported TFLOP/s are 4 d (forward) or 10 d (backward) flops per allowed (query, key)
pair summed over query heads, so the pair count must be the mask's: it is checked against
the oracle's explicit mask built from sequence ids and positions ("Causal Mask and Ragged
Sequence Layouts", sections 1-4) and, at the named workloads' full sizes, against closed
forms of the triangular, bottom-right and windowed counts.
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _w(lq, lk, hq, mode, window=0):
    return SimpleNamespace(num_seqs=len(lq), cu_q=wl.cu_from_lengths(lq),
                           cu_k=wl.cu_from_lengths(lk), hq=hq, mask_mode=mode, window=window)


@pytest.mark.parametrize("lq,lk", [
    ([63, 64, 65], [63, 64, 65]),
    ([127, 128, 129, 1, 0, 5], [127, 128, 129, 1, 3, 0]),
    ([40, 300], [200, 100]),
    ([1, 2, 3], [300, 64, 129]),
])
@pytest.mark.parametrize("mode,window", [(0, 0), (1, 0), (2, 0), (1, 1), (1, 64), (2, 7),
                                         (2, 130)])
def test_pair_count_is_the_explicit_mask(lq, lk, mode, window):
    w = _w(lq, lk, 3, mode, window)
    m = oracle.explicit_mask(w.cu_q, w.cu_k, mode, window)
    assert bench.allowed_pairs(w) == 3 * int(m.sum())


def test_pair_counts_of_the_named_workloads():
    """Closed forms: causal top-left over N keys gives N (N + 1) / 2 pairs per (sequence,
    head); bottom-right with Nq queries over Nk >= Nq keys gives Nq (Nk - Nq) + Nq (Nq + 1)
    / 2; a window of W on top-left gives sum_i min(i + 1, W); bottom-right with Nq > Nk
    leaves the first Nq - Nk rows empty and the rest a triangle over Nk keys."""
    tri = lambda n: n * (n + 1) // 2  # noqa: E731
    # dense: B = 4, H = 16, N = 2048, top-left
    assert bench.allowed_pairs(_w([2048] * 4, [2048] * 4, 16, 1)) == 4 * 16 * tri(2048)
    # decode: B = 16, Hq = 32, Nk = 32768, bottom-right
    for nq in (1, 4, 16):
        per = nq * (32768 - nq) + tri(nq)
        assert bench.allowed_pairs(_w([nq] * 16, [32768] * 16, 32, 2)) == 16 * 32 * per
    # decode edge: Nq = 64 > Nk = 32
    assert bench.allowed_pairs(_w([64] * 16, [32] * 16, 32, 2)) == 16 * 32 * tri(32)
    # training: B = 2, Hq = 32, N = 8192, top-left, without and with a 1024-key window
    assert bench.allowed_pairs(_w([8192] * 2, [8192] * 2, 32, 1)) == 2 * 32 * tri(8192)
    win = sum(min(i + 1, 1024) for i in range(8192))
    assert win == tri(1024) + (8192 - 1024) * 1024
    assert bench.allowed_pairs(_w([8192] * 2, [8192] * 2, 32, 1, 1024)) == 2 * 32 * win
    # ragged GQA packing: every sequence causal over itself
    lens = wl.ragged_lengths(3)
    assert bench.allowed_pairs(_w(lens, lens, 32, 1)) == 32 * sum(tri(n) for n in lens)


def test_more_than_one_gpu_is_refused():
    """The bench measures one GPU: --gpus above 1 exits before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()

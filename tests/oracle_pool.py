"""Oracle slices of the large seeded workloads, computed in a pool of CPU worker processes.

Test infrastructure for the full-size GPU parity tests. Each worker is a fresh (spawned)
Python process that imports only numpy, the oracle and the workload generators - never
torch or the HIP library - regenerates the seeded workload once, and returns only the slices
it is asked for (a few MB), so nothing large crosses the process boundary.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

_W = None


def _init(factory, kwargs):
    global _W
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)      # one BLAS thread per worker: the pool is the parallelism
    except Exception:
        pass
    import workloads as wl
    _W = getattr(wl, factory)(**kwargs)


def _rows(cu, s):
    return slice(int(cu[s]), int(cu[s + 1]))


def fwd_slice(s, heads):
    """O [rows, heads, d] and LSE [heads, rows] of sequence s for the given query heads."""
    import oracle
    w = _W
    o, l = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                            seqs=[s], heads=list(heads))
    r = _rows(w.cu_q, s)
    return o[r][:, list(heads)], l[list(heads)][:, r]


def bwd_slice(s, g):
    """dQ [rows, heads of group g, d], dK and dV [key rows, d] of sequence s, K/V head g."""
    import oracle
    w = _W
    grp = w.hq // w.hkv
    heads = list(range(g * grp, (g + 1) * grp))
    dq, dk, dv = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale,
                                      w.mask_mode, w.window, seqs=[s], kv_heads=[g])
    r, kr = _rows(w.cu_q, s), _rows(w.cu_k, s)
    return dq[r][:, heads], dk[kr][:, g], dv[kr][:, g]


def run(factory, kwargs, tasks, procs=None):
    """Evaluate tasks [(fn, args), ...] (fn: fwd_slice or bwd_slice) on the workload
    workloads.<factory>(**kwargs); results in task order."""
    if procs is None:
        procs = max(1, min(12, len(tasks), (len(os.sched_getaffinity(0)) or 2) - 2))
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(procs, mp_context=ctx, initializer=_init,
                             initargs=(factory, kwargs)) as ex:
        futs = [ex.submit(fn, *args) for fn, args in tasks]
        return [f.result() for f in futs]

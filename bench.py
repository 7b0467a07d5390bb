"""Benchmark of the exact tiled attention kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense|tiny_f32_br|
                    tiny_f32_none|ragged|decode1|decode4|decode16|decode_edge|train|
                    train_w1024|train_drop] [--no-secondary] [--cpu-seconds S]
    python bench.py --sweep [--steps K] [--warmup W]    (sequence-length scaling and memory)

Headline (one JSON line on stdout): the dense bf16 causal forward workload (B=4, Hq=Hkv=16,
N=2048, d=128, causal top-left), reported as causal-adjusted TFLOP/s: 4 * d * (allowed
query-key pairs over all heads) per forward, with inputs resident in HBM before timing.
A "step" is one attn_fwd call (the whole forward path: tile scheduling, mask, QK^T, online
softmax, PV, LSE). Every other named workload is measured the same way and reported under
"secondary": the tiny fp32 forward (bottom-right and noncausal), the packed ragged GQA
forward, cached decode at Nq = 1, 4, 16 and the Nq = 64 > Nk = 32 edge (GB/s), and the
training forward + backward, causal, with a 1024-key window, and with dropout p = 0.1.

Protocol ("Attention Kernel Portability and Benchmarking", fourth and fifth sections):
outputs are validated against the fp64 oracle on a sample before timing; at least 0.25 s of
untimed calls (the device's clocks rise from idle over about 0.1 s of work) and the W
warm-up calls;
the K timed steps are bracketed by device synchronisation and by two HIP events on the
launch stream (their mean gives ms per launch for the roofline); a second pass of K steps
with per-step events gives median / p10 / p90 / max. The oracle is timed on the host cores
on a bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "exact_attention_tiled_amd/csrc/"
# Sources that determine each kernel's machine code (a stored counter reading is only
# reported while these are unchanged).
KERNEL_SOURCES = {
    "fwd_prefill_bf16_kernel": [_CSRC + "attn_device.hpp", _CSRC + "attn_fwd.hip", _CSRC + "attn_internal.h"],
    "fwd_prefill_kernel": [_CSRC + "attn_device.hpp", _CSRC + "attn_fwd.hip", _CSRC + "attn_internal.h"],
    "fwd_splitk_kernel": [_CSRC + "attn_device.hpp", _CSRC + "attn_fwd.hip", _CSRC + "attn_internal.h"],
    "bwd_main_kernel": [_CSRC + "attn_device.hpp", _CSRC + "attn_bwd.hip", _CSRC + "attn_internal.h"],
}


# ----------------------------------------------------------------------------------------
# work accounting
# ----------------------------------------------------------------------------------------

def row_counts(len_q, len_k, mode, window):
    """Allowed keys per query position of one sequence (closed form, in-sequence positions)."""
    i = np.arange(len_q, dtype=np.int64)
    if mode == wl.MASK_NONE:
        return np.full(len_q, len_k, dtype=np.int64)
    end = i if mode == wl.MASK_CAUSAL_TOP_LEFT else i + (len_k - len_q)
    hi = np.minimum(end, len_k - 1)
    lo = np.zeros_like(end) if window <= 0 else np.maximum(end - window + 1, 0)
    return np.maximum(hi - lo + 1, 0)


def allowed_pairs(w) -> int:
    """Allowed (query, key) pairs summed over sequences and query heads."""
    total = 0
    for s in range(w.num_seqs):
        lq = int(w.cu_q[s + 1] - w.cu_q[s])
        lk = int(w.cu_k[s + 1] - w.cu_k[s])
        total += int(row_counts(lq, lk, w.mask_mode, w.window).sum())
    return total * w.hq


def fwd_bytes(w) -> int:
    el = 2 if w.dtype == "bf16" else 4
    return el * (w.q.size * 2 + w.k.size + w.v.size) + 4 * w.hq * w.total_q


def bwd_bytes(w) -> int:
    el = 2 if w.dtype == "bf16" else 4
    # reads q, k, v, out, dout, lse; writes dq, dk, dv
    return el * (w.q.size * 4 + w.k.size * 2 + w.v.size * 2) + 4 * w.hq * w.total_q


def kernel_source_hash(kernel: str = "fwd_prefill_bf16_kernel") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources; None otherwise."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get("entries", {}).get(f"{kernel}@{workload}")
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


# ----------------------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------------------

# Untimed steps before the warm-up steps: after the host-side validation the device has
# been idle, and its clocks take about 0.1 s of sustained work to rise. Measured on the
# dense forward (50 timed steps): 10 warm-up steps gave 677-706 TFLOP/s, 100 gave 768 and
# 1000 (80 ms of work) 864; the timed region itself is unchanged (exactly K steps).
SETTLE_SECONDS = 0.25


def settle(fn, seconds: float = SETTLE_SECONDS) -> int:
    """Run fn untimed until `seconds` of wall time have passed (synchronising every few
    calls so the time is device time, not queueing); returns the number of calls."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n


def time_steps(fn, steps: int, warmup: int):
    """Settle, W warm-up steps, then K timed steps between two HIP events on the launch
    stream (bracketed by device synchronisation): returns wall seconds, the mean event time
    per step, and the per-step event times of a second, separate pass of K steps
    (distribution only: the per-step event pairs add their own gaps, so they are kept out of
    the timed region)."""
    import torch
    stream = torch.cuda.current_stream()
    settle(fn)
    for _ in range(warmup):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = e0.elapsed_time(e1) / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return wall, mean_ms, ms


def stats(ms):
    return {"median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
            "p90_ms": float(np.percentile(ms, 90)), "max_ms": float(ms.max()),
            "mean_ms": float(ms.mean())}


# ----------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------

def make_workload(name: str):
    if name == "dense":
        return wl.dense_bf16()
    if name == "tiny_f32_br":
        return wl.tiny_f32(wl.MASK_CAUSAL_BOTTOM_RIGHT)
    if name == "tiny_f32_none":
        return wl.tiny_f32(wl.MASK_NONE)
    if name == "ragged":
        return wl.ragged_gqa()
    if name == "decode_edge":
        return wl.decode(64, nk=32)
    if name.startswith("decode"):
        return wl.decode(int(name[len("decode"):]))
    if name == "train":
        return wl.train_bf16()
    if name == "train_w1024":
        return wl.train_bf16(window=1024)
    if name == "train_drop":
        return wl.train_bf16()
    raise ValueError(name)


def validate_sample(w, out, lse, grads=None, dropout=None):
    """Outputs checked against the oracle on one (sequence, head group) slice before any
    timing is interpreted ("Attention Kernel Portability and Benchmarking", fifth section)."""
    import oracle
    s = 0
    grp = w.hq // w.hkv
    heads = list(range(grp))
    rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
    dkw = {} if dropout is None else {"dropout_p": dropout[0], "seed": dropout[1]}
    ro, rl = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                              seqs=[s], heads=heads, **dkw)
    o = out.double().cpu().numpy()[rows][:, heads]
    l = lse.double().cpu().numpy()[heads][:, rows]
    tol = 2e-2 if w.dtype == "bf16" else 1e-5
    ok = np.all(np.abs(o - ro[rows][:, heads]) <= tol + tol * np.abs(ro[rows][:, heads]))
    fin = np.isfinite(rl[heads][:, rows])
    ok &= np.all(np.abs(l[fin] - rl[heads][:, rows][fin]) <= 1e-3)
    if grads is not None:
        rq, rk, rv = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale,
                                          w.mask_mode, w.window, seqs=[s], kv_heads=[0], **dkw)
        krows = slice(int(w.cu_k[s]), int(w.cu_k[s + 1]))
        for g, r, sl, hs in ((grads[0], rq, rows, heads), (grads[1], rk, krows, [0]),
                             (grads[2], rv, krows, [0])):
            gg = g.double().cpu().numpy()[sl][:, hs]
            rr = r[sl][:, hs]
            ok &= np.all(np.abs(gg - rr) <= 2e-2 + 2e-2 * np.abs(rr))
    return bool(ok)


def bench_forward(w, steps, warmup, validate=True):
    import torch
    import exact_attention_tiled_amd as eat
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.from_numpy(w.q).to(dev).to(dt)
    k = torch.from_numpy(w.k).to(dev).to(dt)
    v = torch.from_numpy(w.v).to(dev).to(dt)
    cu_q = torch.from_numpy(w.cu_q).to(dev)
    cu_k = torch.from_numpy(w.cu_k).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.hq, w.total_q), dtype=torch.float32, device=dev)
    wsb = eat.attn_fwd_workspace_size(q, k, cu_q, w.max_seqlen_q, w.max_seqlen_k, w.mask_mode,
                                      w.window)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    plan = eat.attn_describe_plan(q, k, cu_q, w.max_seqlen_q, w.max_seqlen_k, w.mask_mode, w.window)

    def step():
        eat.attn_fwd(q, k, v, cu_q, cu_k, w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
                     w.window, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    valid = validate_sample(w, out, lse) if validate else None
    if validate and not valid:
        raise SystemExit(f"validation against the oracle failed for {w.name}; not timing it")
    wall, mean_ms, ms = time_steps(step, steps, warmup)
    return {"wall_s": wall, "mean_ms": mean_ms, "ms": ms, "plan": plan, "validated": valid}


# Dropout leg: probability and seed of the realisation (inverted dropout on the weights).
TRAIN_DROPOUT = (0.1, 20261202)


def bench_train(w, steps, warmup, validate=True, dropout=None):
    import torch
    import exact_attention_tiled_amd as eat
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (w.q, w.k, w.v, w.dout))
    cu_q = torch.from_numpy(w.cu_q).to(dev)
    cu_k = torch.from_numpy(w.cu_k).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.hq, w.total_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = eat.attn_bwd_workspace_size(q, k, cu_q, w.max_seqlen_q, w.max_seqlen_k, w.mask_mode,
                                      w.window)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    fwsb = (eat.attn_fwd_workspace_size(q, k, cu_q, w.max_seqlen_q, w.max_seqlen_k, w.mask_mode,
                                        w.window) if dropout is None else
            eat.attn_fwd_dropout_workspace_size(q, k, cu_q, w.max_seqlen_q, w.max_seqlen_k,
                                                w.mask_mode, w.window))
    fws = torch.empty(max(fwsb, 1), dtype=torch.uint8, device=dev)
    # With dropout the forward also hands the backward its output's rounding residual, so
    # the backward forms D from it instead of recomputing S and dP for D.
    res = torch.empty_like(q) if dropout is not None else None

    def fwd():
        if dropout is None:
            eat.attn_fwd(q, k, v, cu_q, cu_k, w.max_seqlen_q, w.max_seqlen_k, w.scale,
                         w.mask_mode, w.window, out=out, lse=lse, workspace=fws)
        else:
            eat.attn_fwd_dropout(q, k, v, cu_q, cu_k, w.max_seqlen_q, w.max_seqlen_k, w.scale,
                                 w.mask_mode, w.window, dropout[0], dropout[1], out=out,
                                 lse=lse, workspace=fws, out_residual=res)

    def bwd():
        if dropout is None:
            eat.attn_bwd(q, k, v, out, lse, do, cu_q, cu_k, w.max_seqlen_q, w.max_seqlen_k,
                         w.scale, w.mask_mode, w.window, dq=dq, dk=dk, dv=dv, workspace=ws)
        else:
            eat.attn_bwd_dropout(q, k, v, out, lse, do, cu_q, cu_k, w.max_seqlen_q,
                                 w.max_seqlen_k, w.scale, w.mask_mode, w.window, dropout[0],
                                 dropout[1], dq=dq, dk=dk, dv=dv, workspace=ws,
                                 out_residual=res)

    def step():
        fwd()
        bwd()

    step()
    torch.cuda.synchronize()
    if validate and not validate_sample(w, out, lse, grads=(dq, dk, dv), dropout=dropout):
        raise SystemExit(f"validation against the oracle failed for {w.name}; not timing it")
    # Peak memory of the timed calls only (validation makes float64 copies).
    torch.cuda.reset_peak_memory_stats()
    wall, mean_ms, ms = time_steps(step, steps, warmup)
    _, mean_f, ms_f = time_steps(fwd, steps, 2)
    _, mean_b, ms_b = time_steps(bwd, steps, 2)
    return {"wall_s": wall, "mean_ms": mean_ms, "ms": ms, "mean_fwd": mean_f, "ms_fwd": ms_f,
            "mean_bwd": mean_b, "ms_bwd": ms_b}


# ----------------------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ----------------------------------------------------------------------------------------

def cpu_baseline(w, target_s: float):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity core count
        threads = len(os.sched_getaffinity(0))
    grp = w.hq // w.hkv
    slices = [(s, h) for s in range(w.num_seqs) for h in range(w.hq)]
    done_pairs = 0
    t0 = time.perf_counter()
    n = 0
    # Slices in order, cycling through the workload again if one pass is shorter than the
    # target, until about target_s seconds of CPU work are done.
    while time.perf_counter() - t0 < target_s:
        s, h = slices[n % len(slices)]
        oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                         seqs=[s], heads=[h])
        lq = int(w.cu_q[s + 1] - w.cu_q[s])
        lk = int(w.cu_k[s + 1] - w.cu_k[s])
        done_pairs += int(row_counts(lq, lk, w.mask_mode, w.window).sum())
        n += 1
    el = time.perf_counter() - t0
    flops = 4.0 * w.d * done_pairs
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "host_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)),
            "cores_meaning": "BLAS threads of the one oracle process (numpy float64)",
            "sample": f"{n} (sequence, query head) slices of the {len(slices)} of {w.name} "
                      f"({done_pairs} allowed pairs, {el:.1f} s, float64 numpy, dense-then-mask "
                      f"per sequence; group size {grp})"}


# ----------------------------------------------------------------------------------------
# Sequence-length scaling and memory ("Attention Algorithm Error and Complexity Tests",
# fifth and sixth sections: pair work, fitted exponents, saved state and workspace).
# ----------------------------------------------------------------------------------------

def fit_power(ns, ts):
    """Least-squares fit of t = a * N^k on log-log axes; returns (k, a, max relative residual)."""
    x = np.log(np.asarray(ns, dtype=np.float64))
    y = np.log(np.asarray(ts, dtype=np.float64))
    k, loga = np.polyfit(x, y, 1)
    resid = np.exp(y - (k * x + loga)) - 1.0
    return float(k), float(np.exp(loga)), float(np.abs(resid).max())


def sweep(steps: int, warmup: int, validate_max_n: int = 4096):
    """Training step (forward and backward timed separately) of one sequence of N tokens with
    Hq=32, Hkv=8, d=128, bf16, causal top-left, without and with a 1024-key window, for N from
    1k to 32k; everything else fixed. Outputs are checked against the oracle for N <= 4096."""
    import torch
    import exact_attention_tiled_amd as eat
    ns = [1024, 2048, 4096, 8192, 16384, 32768]
    rows = []
    for window in (0, 1024):
        for n in ns:
            w = wl.train_bf16(window=window, seqlen=n, batch=1)
            pairs = allowed_pairs(w)
            torch.cuda.empty_cache()
            r = bench_train(w, steps, warmup, validate=n <= validate_max_n)
            ws_bwd = eat.attn_bwd_workspace_size(
                torch.empty((w.total_q, w.hq, w.d), dtype=torch.bfloat16, device="meta"),
                torch.empty((w.total_k, w.hkv, w.d), dtype=torch.bfloat16, device="meta"),
                torch.empty((w.num_seqs + 1,), dtype=torch.int32, device="meta"),
                w.max_seqlen_q, w.max_seqlen_k, w.mask_mode, w.window)
            el = 2
            io_bytes = el * (w.q.size * 2 + w.k.size + w.v.size) + 4 * w.hq * w.total_q
            rows.append({
                "n": n, "window": window, "allowed_pairs": pairs,
                "fwd_ms": float(np.median(r["ms_fwd"])), "bwd_ms": float(np.median(r["ms_bwd"])),
                "fwd_tflops": 4.0 * w.d * pairs / (np.median(r["ms_fwd"]) * 1e-3) / 1e12,
                "bwd_tflops": 10.0 * w.d * pairs / (np.median(r["ms_bwd"]) * 1e-3) / 1e12,
                "fwd_io_bytes": io_bytes, "bwd_workspace_bytes": int(ws_bwd),
                # q, k, v, out, lse, dout, dq, dk, dv and the backward workspace
                "train_tensor_bytes": int(el * (w.q.size * 4 + w.k.size * 4) + 4 * w.hq * w.total_q
                                          + ws_bwd),
                "fwd_workspace_bytes": 0,
                "torch_peak_allocated_bytes": int(torch.cuda.max_memory_allocated()),
                "torch_peak_reserved_bytes": int(torch.cuda.max_memory_reserved()),
                "validated": n <= validate_max_n})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
            del w
    fits = {}
    for window in (0, 1024):
        sel = [r for r in rows if r["window"] == window]
        for key in ("fwd_ms", "bwd_ms", "allowed_pairs", "torch_peak_allocated_bytes"):
            k, a, res = fit_power([r["n"] for r in sel], [r[key] for r in sel])
            fits[f"window{window}_{key}"] = {"exponent": k, "coefficient": a, "max_rel_residual": res}
        # the window's pair count is linear only once N >> window: fit the upper half too
        hi = [r for r in sel if r["n"] >= 8192]
        k, a, res = fit_power([r["n"] for r in hi], [r["fwd_ms"] for r in hi])
        fits[f"window{window}_fwd_ms_n_ge_8192"] = {"exponent": k, "coefficient": a, "max_rel_residual": res}
    print(json.dumps({"sweep": "sequence-length scaling, B=1 Hq=32 Hkv=8 d=128 bf16 causal top-left",
                      "steps": steps, "warmup": warmup, "rows": rows, "fits": fits}))


# ----------------------------------------------------------------------------------------
# Secondary legs: every named workload, measured like the headline. For each: the burst
# figure (mean over K back-to-back launches between two events) and the median figure (per
# launch, events around each launch), both as a fraction of the roofline that bounds it.
# ----------------------------------------------------------------------------------------

SECONDARY = ["tiny_f32_br", "tiny_f32_none", "ragged", "decode1", "decode4", "decode16",
             "decode_edge", "train", "train_w1024", "train_drop"]


def _rates(work, mean_ms, ms, peak):
    med = float(np.median(ms))
    return {"burst": work / (mean_ms * 1e-3), "median": work / (med * 1e-3),
            "burst_frac": work / (mean_ms * 1e-3) / peak, "median_frac": work / (med * 1e-3) / peak}


def secondary_leg(name: str, steps: int = 20, warmup: int = 5):
    sw = make_workload(name)
    sp = allowed_pairs(sw)
    wname = {"tiny_f32_br": sw.name + "_bottom_right", "tiny_f32_none": sw.name + "_noncausal",
             "train_drop": f"{sw.name}_dropout{TRAIN_DROPOUT[0]}"}.get(name, sw.name)
    leg = {"workload": wname, "allowed_pairs": sp}
    if name.startswith("train"):
        drop = TRAIN_DROPOUT if name == "train_drop" else None
        rr = bench_train(sw, 5, 2, dropout=drop)
        f = _rates(4.0 * sw.d * sp / 1e12, rr["mean_fwd"], rr["ms_fwd"], PEAK_BF16_TFLOPS)
        b = _rates(10.0 * sw.d * sp / 1e12, rr["mean_bwd"], rr["ms_bwd"], PEAK_BF16_TFLOPS)
        t = _rates(14.0 * sw.d * sp / 1e12, rr["mean_ms"], rr["ms"], PEAK_BF16_TFLOPS)
        leg.update({"metric": "fwd+bwd TFLOP/s (causal-adjusted)", "unit": "TFLOP/s",
                    "value": t["burst"], "value_median": t["median"],
                    "frac_of_bf16_peak": t["burst_frac"], "median_frac": t["median_frac"],
                    "fwd_tflops": f["burst"], "fwd_tflops_median": f["median"],
                    "fwd_frac": f["burst_frac"],
                    "bwd_tflops": b["burst"], "bwd_tflops_median": b["median"],
                    "bwd_frac": b["burst_frac"],
                    "step_stats": stats(rr["ms"]), "fwd_stats": stats(rr["ms_fwd"]),
                    "bwd_stats": stats(rr["ms_bwd"]), "validated": True})
    elif name.startswith("decode"):
        rr = bench_forward(sw, steps, warmup)
        g = _rates(fwd_bytes(sw) / 1e9, rr["mean_ms"], rr["ms"], PEAK_HBM_GBS)
        leg.update({"metric": "decode GB/s", "unit": "GB/s", "value": g["burst"],
                    "value_median": g["median"], "frac_of_hbm_peak": g["burst_frac"],
                    "median_frac": g["median_frac"], "plan": rr["plan"],
                    "step_stats": stats(rr["ms"]), "validated": rr["validated"]})
        if name == "decode_edge":
            leg["note"] = ("64 query rows over 32 keys: rows 0-31 of every sequence see no key "
                           "(output +0.0, LSE -inf); launch-bound")
    else:
        rr = bench_forward(sw, steps, warmup)
        peak = PEAK_BF16_TFLOPS if sw.dtype == "bf16" else PEAK_F32_TFLOPS
        t = _rates(4.0 * sw.d * sp / 1e12, rr["mean_ms"], rr["ms"], peak)
        leg.update({"metric": "fwd TFLOP/s (causal-adjusted)", "unit": "TFLOP/s",
                    "value": t["burst"], "value_median": t["median"],
                    "frac_of_peak": t["burst_frac"], "median_frac": t["median_frac"],
                    "peak": peak, "plan": rr["plan"], "step_stats": stats(rr["ms"]),
                    "validated": rr["validated"]})
    print(json.dumps({"leg": wname, "value": leg["value"], "unit": leg["unit"]}),
          file=sys.stderr, flush=True)
    del sw
    return leg


# ----------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="sequence-length scaling and memory sweep (prints its own JSON)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_tiled_amd as eat
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    eat.load()

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": args.steps}))
        return

    if args.sweep:
        sweep(args.steps, args.warmup)
        return

    w = make_workload(args.workload)
    pairs = allowed_pairs(w)
    if args.workload.startswith("decode"):
        r = bench_forward(w, args.steps, args.warmup)
        byts = fwd_bytes(w)
        ms_avg = r["mean_ms"]
        value = byts * args.steps / r["wall_s"] / 1e9
        metric, unit = "attention decode GB/s (split-K forward)", "GB/s"
        roof = {"bound": "hbm", "achieved": byts / (ms_avg * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
        kernel = "fwd_splitk_kernel"
    elif args.workload.startswith("train"):
        r = bench_train(w, args.steps, args.warmup,
                        dropout=TRAIN_DROPOUT if args.workload == "train_drop" else None)
        flops = 14.0 * w.d * pairs
        ms_avg = r["mean_ms"]
        value = flops * args.steps / r["wall_s"] / 1e12
        metric, unit = "attention fwd+bwd TFLOP/s (causal-adjusted)", "TFLOP/s"
        roof = {"bound": "mfma", "achieved": 10.0 * w.d * pairs / (r["mean_bwd"] * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        kernel = "bwd_main_kernel"
    else:
        r = bench_forward(w, args.steps, args.warmup)
        flops = 4.0 * w.d * pairs
        ms_avg = r["mean_ms"]
        value = flops * args.steps / r["wall_s"] / 1e12
        metric, unit = "attention fwd TFLOP/s (causal-adjusted)", "TFLOP/s"
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma", "achieved": flops / (ms_avg * 1e-3) / 1e12, "peak": peak,
                "unit": "TFLOP/s"}
        kernel = "fwd_prefill_bf16_kernel" if w.dtype == "bf16" else "fwd_prefill_kernel"
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(kernel, args.workload)
    roof["kernel"] = kernel

    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["wall_s"] * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded numpy draws, N(0,1), bf16 round-to-nearest-even)",
        "config": dict(w.describe(), allowed_pairs=pairs, parallelism="single GPU"),
        "step_stats": stats(r["ms"]), "plan": r.get("plan"), "roofline": roof,
    }
    # The same work over the median of per-launch event times (each launch bracketed by its
    # own events, so no overlap with the neighbouring launches): a conservative companion to
    # the back-to-back figures above.
    work = value * r["wall_s"] / args.steps
    med = float(np.median(r["ms"])) * 1e-3
    line["value_median"] = work / med
    line["median_frac"] = line["value_median"] / roof["peak"] if not \
        args.workload.startswith("train") else None
    line["timing"] = {
        "value": "work per step x K / wall time of the K back-to-back steps (synchronised)",
        "roofline.achieved": "work per launch / mean launch time from two HIP events around "
                             "the same K steps on the launch stream",
        "value_median": "work per step / median of K separately bracketed steps",
        "warmup": f"untimed steps for at least {SETTLE_SECONDS} s (device clocks rise from "
                  "idle), then W warm-up steps, before each timed pass"}
    line["config"]["workload"] = w.name
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    if not args.no_secondary and args.workload == "dense":
        line["secondary"] = [secondary_leg(name) for name in SECONDARY]
    line["env"] = {"device": torch.cuda.get_device_name(0), "torch": torch.__version__,
                   "hip": getattr(torch.version, "hip", None), "host": platform.node(),
                   "library_version": eat.attn_version(),
                   "kernel_source_hash": kernel_source_hash(kernel)}
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""GPU backward parity against the fp64 oracle, GQA group sums, canaries (bf16 and fp32)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import BF16_TOL, assert_close, run_fwd, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import exact_attention_tiled_amd as eat
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    eat.load()


def run_bwd(w, t, out, lse, **kw):
    import exact_attention_tiled_amd as eat
    return eat.attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], t["cu_q"], t["cu_k"],
                        w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window, **kw)


def _oracle_bwd(w, seqs=None, kv_heads=None):
    return oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                                w.window, seqs=seqs, kv_heads=kv_heads)


def check_grads(w, got, ref, what):
    worst = {}
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        worst[name] = assert_close(to_np(g), r, *BF16_TOL, f"{what} {name}")
    print(f"{what}: max abs errors {worst}", flush=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (1, 70), (2, 33)])
def test_bwd_ragged_edges(d, mode, window):
    """Ragged lengths around tile edges (incl. 0, 1, Nq > Nk and Nq < Nk), GQA 4:2."""
    lq = [0, 1, 63, 64, 65, 127, 128, 129, 200, 7]
    lk = [5, 129, 128, 64, 63, 1, 300, 129, 0, 70]
    # N(0,1) values as in the training workload. Large per-sequence value offsets (used by
    # the forward tests to expose leaks) do not suit the backward: D = rowsum(dO * O) is
    # formed from the stored bf16 output, whose spacing near |O| = 90 is 0.5.
    w = wl.random_workload((21, d, mode), lq, lk, 4, 2, d, "bf16", mode, window,
                           with_dout=True, name="bwd-edge")
    print(f"bwd edges d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    out, lse = run_fwd(w, t)
    got = run_bwd(w, t, out, lse)
    check_grads(w, got, _oracle_bwd(w), f"edges d={d} mode={mode} w={window}")


def test_bwd_gqa_groups_are_summed():
    """Hq=8 over Hkv=2: dK/dV of each K/V head equal the sum over its 4 query heads, checked
    against the oracle's repeated-head (MHA) gradients summed per group."""
    lens = [150, 77]
    w = wl.random_workload(22, lens, lens, 8, 2, 128, "bf16", wl.MASK_CAUSAL_TOP_LEFT,
                           with_dout=True, name="bwd-gqa")
    t = to_device(w)
    out, lse = run_fwd(w, t)
    dq, dk, dv = run_bwd(w, t, out, lse)
    rq, rk, rv = oracle.attention_bwd(w.q, np.repeat(w.k, 4, axis=1), np.repeat(w.v, 4, axis=1),
                                      w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode, 0)
    assert_close(to_np(dk), rk.reshape(rk.shape[0], 2, 4, -1).sum(axis=2), *BF16_TOL, "gqa dK")
    assert_close(to_np(dv), rv.reshape(rv.shape[0], 2, 4, -1).sum(axis=2), *BF16_TOL, "gqa dV")
    assert_close(to_np(dq), rq, *BF16_TOL, "gqa dQ")


def test_bwd_canaries_no_out_of_bounds_writes():
    """Gradients land inside larger buffers whose slack holds sentinels: every sentinel
    survives, and keys no query can see get exactly zero dK/dV ("Causal Mask and Ragged
    Sequence Layouts", sixth section: a gradient written into a neighbouring packed
    sequence goes unnoticed by forward-only tests)."""
    import torch
    import exact_attention_tiled_amd as eat
    lq, lk = [40, 3, 90], [10, 200, 90]
    w = wl.random_workload(23, lq, lk, 4, 1, 64, "bf16", wl.MASK_CAUSAL_BOTTOM_RIGHT, 16,
                           with_dout=True, name="canary")
    t = to_device(w)
    out, lse = run_fwd(w, t)
    pad = 4096
    sentinel = -12345.0

    def padded(like):
        buf = torch.full((like.numel() + 2 * pad,), sentinel, dtype=like.dtype, device=like.device)
        return buf, buf[pad:pad + like.numel()].view(like.shape)

    bq, dq = padded(t["q"])
    bk, dk = padded(t["k"])
    bv, dv = padded(t["v"])
    eat.attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], t["cu_q"], t["cu_k"],
                 w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window, dq=dq, dk=dk,
                 dv=dv)
    torch.cuda.synchronize()
    for buf in (bq, bk, bv):
        assert torch.all(buf[:pad] == sentinel) and torch.all(buf[-pad:] == sentinel)
    m = oracle.explicit_mask(w.cu_q, w.cu_k, w.mask_mode, w.window)
    unseen = np.nonzero(~m.any(axis=0))[0]
    assert len(unseen) > 50
    assert torch.all(dk[torch.from_numpy(unseen).cuda()].float() == 0)
    assert torch.all(dv[torch.from_numpy(unseen).cuda()].float() == 0)
    check_grads(w, (dq, dk, dv), _oracle_bwd(w), "canary")


@pytest.mark.parametrize("window", [0, 1024])
def test_train_full_size(window):
    """B=2, Hq=32, Hkv=8, N=8192, d=128, causal top-left (and window 1024): full GPU
    forward + backward; against the oracle on both sequences x two K/V head groups: O, LSE of
    the groups' query heads and dQ, dK, dV of the whole groups (slices evaluated in parallel
    CPU workers)."""
    import oracle_pool as op
    w = wl.train_bf16(window=window)
    t = to_device(w)
    out, lse = run_fwd(w, t)
    dq, dk, dv = run_bwd(w, t, out, lse)
    o, l = to_np(out), to_np(lse)
    gq, gk, gv = to_np(dq), to_np(dk), to_np(dv)
    del t, out, lse, dq, dk, dv
    for x in (o, l, gq, gk, gv):
        assert np.all(np.isfinite(x))
    slices = [(s, g) for s in (0, 1) for g in (0, 5)]
    tasks = [(op.fwd_slice, (s, list(range(4 * g, 4 * g + 4)))) for s, g in slices]
    tasks += [(op.bwd_slice, (s, g)) for s, g in slices]
    print(f"train full size window={window}: {len(tasks)} oracle tasks", flush=True)
    res = op.run("train_bf16", {"window": window}, tasks)
    for (s, g), (ro, rl), (rq, rk, rv) in zip(slices, res[:4], res[4:]):
        heads = list(range(4 * g, 4 * g + 4))
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        krows = slice(int(w.cu_k[s]), int(w.cu_k[s + 1]))
        assert_close(o[rows][:, heads], ro, *BF16_TOL, f"train O s{s} g{g}")
        assert_close(l[heads][:, rows], rl, 1e-3, 0.0, f"train LSE s{s} g{g}")
        assert_close(gq[rows][:, heads], rq, *BF16_TOL, f"train dQ s{s} g{g}")
        assert_close(gk[krows][:, g], rk, *BF16_TOL, f"train dK s{s} g{g}")
        assert_close(gv[krows][:, g], rv, *BF16_TOL, f"train dV s{s} g{g}")


@pytest.mark.parametrize("window", [0, 300])
def test_head_dim_64_full_size(window):
    """head_dim 64 across many tiles: B=2, N=2048, Hq=16 over Hkv=4, causal top-left (and a
    window of 300), the pipelined bf16 forward and the backward: O and LSE of every query
    head and dQ, dK, dV of every K/V group of both sequences against the oracle at the
    standard bounds."""
    import oracle_pool as op
    kw = {"window": window, "seqlen": 2048, "hq": 16, "hkv": 4, "d": 64}
    w = wl.train_bf16(**kw)
    t = to_device(w)
    out, lse = run_fwd(w, t)
    dq, dk, dv = run_bwd(w, t, out, lse)
    o, l = to_np(out), to_np(lse)
    gq, gk, gv = to_np(dq), to_np(dk), to_np(dv)
    del t, out, lse, dq, dk, dv
    slices = [(s, g) for s in (0, 1) for g in range(4)]
    tasks = [(op.fwd_slice, (s, list(range(4 * g, 4 * g + 4)))) for s, g in slices]
    tasks += [(op.bwd_slice, (s, g)) for s, g in slices]
    res = op.run("train_bf16", kw, tasks)
    for (s, g), (ro, rl), (rq, rk, rv) in zip(slices, res[:len(slices)], res[len(slices):]):
        heads = list(range(4 * g, 4 * g + 4))
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        krows = slice(int(w.cu_k[s]), int(w.cu_k[s + 1]))
        assert_close(o[rows][:, heads], ro, *BF16_TOL, f"d64 O s{s} g{g}")
        assert_close(l[heads][:, rows], rl, 1e-3, 0.0, f"d64 LSE s{s} g{g}")
        assert_close(gq[rows][:, heads], rq, *BF16_TOL, f"d64 dQ s{s} g{g}")
        assert_close(gk[krows][:, g], rk, *BF16_TOL, f"d64 dK s{s} g{g}")
        assert_close(gv[krows][:, g], rv, *BF16_TOL, f"d64 dV s{s} g{g}")


UNEQUAL_CASES = [  # (dtype, lq, lk, mode, d)
    ("bf16", 1024, 4096, wl.MASK_CAUSAL_BOTTOM_RIGHT, 128),
    ("bf16", 4096, 1024, wl.MASK_CAUSAL_BOTTOM_RIGHT, 128),
    ("bf16", 3000, 2000, wl.MASK_CAUSAL_TOP_LEFT, 128),
    ("f32", 1024, 1024, wl.MASK_CAUSAL_TOP_LEFT, 128),
    ("f32", 700, 2100, wl.MASK_CAUSAL_BOTTOM_RIGHT, 64),
    ("bf16", 16, 8192, wl.MASK_CAUSAL_BOTTOM_RIGHT, 128),   # split-K forward
    ("f32", 4, 16384, wl.MASK_CAUSAL_BOTTOM_RIGHT, 64),     # split-K forward, fp32
]


@pytest.mark.parametrize("case", range(len(UNEQUAL_CASES)))
def test_unequal_lengths_full_size(case):
    """Query and key lengths that differ, across many tiles (two sequences, Hq=8 over
    Hkv=2): bottom-right with fewer queries than keys (a prefill against a cache) and with
    more (the first Nq - Nk rows of each sequence see no key: exact zeros), top-left with
    more queries than keys, decode shapes (the forward takes the split-K path), and fp32 at
    its 1e-5 bound. Forward and backward of every head
    against the oracle ("Causal Mask and Ragged Sequence Layouts", third and fourth
    sections: explicit alignment, empty rows)."""
    import oracle_pool as op
    from gpu_util import F32_TOL
    dtype, lq, lk, mode, d = UNEQUAL_CASES[case]
    kw = dict(seed=(61, case), lengths_q=[lq, lq // 2], lengths_k=[lk, lk // 2], hq=8, hkv=2,
              d=d, dtype=dtype, mask_mode=mode, with_dout=True, name="unequal")
    w = wl.random_workload(**kw)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    t = to_device(w)
    out, lse = run_fwd(w, t)
    if lq <= 16:
        import exact_attention_tiled_amd as eat
        plan = eat.attn_describe_plan(t["q"], t["k"], t["cu_q"], w.max_seqlen_q, w.max_seqlen_k,
                                      w.mask_mode)
        assert "path=splitk" in plan, plan
    dq, dk, dv = run_bwd(w, t, out, lse)
    o, l = to_np(out), to_np(lse)
    gq, gk, gv = to_np(dq), to_np(dk), to_np(dv)
    del t, out, lse, dq, dk, dv
    slices = [(s, g) for s in (0, 1) for g in range(2)]
    tasks = [(op.fwd_slice, (s, list(range(4 * g, 4 * g + 4)))) for s, g in slices]
    tasks += [(op.bwd_slice, (s, g)) for s, g in slices]
    res = op.run("random_workload", kw, tasks)
    for (s, g), (ro, rl), (rq, rk, rv) in zip(slices, res[:len(slices)], res[len(slices):]):
        heads = list(range(4 * g, 4 * g + 4))
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        krows = slice(int(w.cu_k[s]), int(w.cu_k[s + 1]))
        tag = f"{dtype} {lq}x{lk} mode {mode} s{s} g{g}"
        assert_close(o[rows][:, heads], ro, *tol, f"O {tag}")
        empty = ~np.isfinite(rl)
        assert np.array_equal(~np.isfinite(l[heads][:, rows]), empty), f"empty rows {tag}"
        assert np.all(o[rows][:, heads][empty.T] == 0), f"empty-row O {tag}"
        assert_close(np.where(empty, 0.0, l[heads][:, rows]), np.where(empty, 0.0, rl), 1e-3,
                     0.0, f"LSE {tag}")
        assert_close(gq[rows][:, heads], rq, *tol, f"dQ {tag}")
        assert_close(gk[krows][:, g], rk, *tol, f"dK {tag}")
        assert_close(gv[krows][:, g], rv, *tol, f"dV {tag}")


def scale_workload(scale, d=128):
    """GQA 4:2, bottom-right, ragged lengths (300/300, 129/500, 70/64) at a given scale."""
    seed = (66, int(abs(scale) * 1000)) if d == 128 else (66, int(abs(scale) * 1000), d)
    return wl.random_workload(seed, [300, 129, 70], [300, 500, 64], 4, 2, d, "bf16",
                              wl.MASK_CAUSAL_BOTTOM_RIGHT, with_dout=True, name="scale-bf16",
                              scale=scale)


def check_grads_derived(w, got, ref, what, residual, noise_draws=0):
    """Gradients against the oracle at atol = max(2e-2, 1.1 x what the CPU rounding model of
    the same route needs on these inputs), rtol 2e-2; prints the kernel's own need. With
    noise_draws the model's need is the largest over its exact-logit run and that many draws
    of the fp32 logit error (rounding_model.model_backward, logit_noise)."""
    from rounding_model import model_backward, required_atol
    need = [0.0, 0.0, 0.0]
    for draw in [None] + list(range(1, noise_draws + 1)):
        with np.errstate(over="ignore"):
            model = model_backward(w, residual=residual, logit_noise=draw)
        need = [max(n, required_atol(m, r)) for n, m, r in zip(need, model, ref)]
    for name, g, n, r in zip(("dQ", "dK", "dV"), got, need, ref):
        g = to_np(g)
        atol = max(BF16_TOL[0], 1.1 * n)
        print(f"{what} {name}: kernel needs atol {required_atol(g, r):.4f}, model "
              f"{n:.4f}, bound {atol:.4f}", flush=True)
        assert_close(g, r, atol, BF16_TOL[1], f"{what} {name}")


# Draws of the fp32 logit error behind the extreme-scale bounds: at scale 50 the rows whose
# dominant weight rounds differently change from draw to draw (d = 64: dQ needs 3.65 to 5.72
# over 16 draws, the kernel 5.42).
NOISE_DRAWS = 6


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [50.0, 1e-3, -2.0])
def test_unusual_scales_bf16(scale, d):
    """The bf16 forward and backward at extreme scales: 50 makes each row's weights nearly
    one-hot (logit gaps of hundreds, so the running offset moves at almost every stage), 1e-3
    nearly uniform, and a negative scale folds its sign into Q. Forward against the oracle at
    the standard bounds. Gradients grow with |scale| while the bf16 rounding of the stored
    output, from which D = rowsum(dO * O) is formed, does not cancel in dS = P (dP - D): at
    scale 50 the rounding model needs atol ~6 for dQ. So each route is held to the bound its
    model derives: attn_bwd (D from the stored output), and the output-residual route
    (attn_fwd_dropout / attn_bwd_dropout at p = 0 with out_residual: D from the unrounded
    output), whose need at scale 50 is far smaller. At scale 50 the fp32 rounding of the
    logits, multiplied by the scale, moves some weights across a bf16 rounding boundary, so
    each bound takes the model's worst case over draws of that error."""
    import torch
    import exact_attention_tiled_amd as eat
    w = scale_workload(scale, d)
    print(f"unusual scale {scale} d={d}", flush=True)
    t = to_device(w)
    with np.errstate(over="ignore"):
        ref_o, ref_l = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode)
        ref_g = _oracle_bwd(w)
    out, lse = run_fwd(w, t)
    assert_close(to_np(out), ref_o, *BF16_TOL, f"scale {scale} O")
    assert_close(to_np(lse), ref_l, 1e-3, 0.0, f"scale {scale} LSE")
    check_grads_derived(w, run_bwd(w, t, out, lse), ref_g, f"scale {scale}", False,
                        NOISE_DRAWS)
    args = (t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
            w.window, 0.0, 9)
    res = torch.full_like(t["q"], float("nan"))
    out_r, lse_r = eat.attn_fwd_dropout(t["q"], t["k"], t["v"], *args, out_residual=res)
    assert_close(to_np(out_r), ref_o, *BF16_TOL, f"scale {scale} residual-route O")
    assert_close(to_np(lse_r), ref_l, 1e-3, 0.0, f"scale {scale} residual-route LSE")
    # The residual is at most half a bf16 spacing of out, and out + residual is the kernel's
    # unrounded output: its mean error is far below that of out alone. (Its largest error
    # grows with |scale|, which multiplies the fp32 rounding of the logits: 1.7e-4 at 50.)
    mag = out_r.view(torch.int16) & 0x7FFF
    up = (mag + 1).view(torch.bfloat16).float() - mag.view(torch.bfloat16).float()
    assert torch.all(res.float().abs() <= 0.5 * up)
    o64 = to_np(out_r).astype(np.float64)
    err_o, err_or = np.abs(o64 - ref_o).mean(), np.abs(o64 + to_np(res) - ref_o).mean()
    print(f"scale {scale}: mean abs error of out {err_o:.3e}, of out + residual {err_or:.3e}")
    assert err_or < err_o / 16
    g = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out_r, lse_r, t["dout"], *args,
                             out_residual=res)
    check_grads_derived(w, g, ref_g, f"scale {scale} residual route", True, NOISE_DRAWS)


def test_value_offsets_residual_route():
    """16 short causal sequences (GQA 8:2) whose values carry the ragged workload's
    per-sequence offsets v (s + 1) + 10 s (outputs up to ~200): through attn_bwd the stored
    output's rounding moves dQ and dK by ~2 (the model's derived need); through the
    output-residual route (p = 0 with out_residual) D comes from the unrounded output and the
    need drops below 0.1. Both against the oracle at their routes' derived bounds."""
    import torch
    import exact_attention_tiled_amd as eat
    from test_tolerance_derivation import offset_pack_workload
    w = offset_pack_workload(True)
    t = to_device(w)
    ref_g = _oracle_bwd(w)
    out, lse = run_fwd(w, t)
    check_grads_derived(w, run_bwd(w, t, out, lse), ref_g, "offsets attn_bwd", False)
    args = (t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
            w.window, 0.0, 9)
    res = torch.full_like(t["q"], float("nan"))
    out_r, lse_r = eat.attn_fwd_dropout(t["q"], t["k"], t["v"], *args, out_residual=res)
    g = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out_r, lse_r, t["dout"], *args,
                             out_residual=res)
    check_grads_derived(w, g, ref_g, "offsets residual route", True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (1, 70), (2, 33)])
def test_residual_route_edges(d, mode, window):
    """The output-residual route at p = 0 (attn_fwd_dropout / attn_bwd_dropout with
    out_residual) on the backward's ragged edge lengths, GQA 4:2, every alignment and two
    windows: O and LSE at the standard bounds, out + residual far closer to the oracle than
    out, rows with no allowed key +0.0 in out and residual, and the gradients against the
    oracle at the model-derived bound of this route."""
    import torch
    import exact_attention_tiled_amd as eat
    lq = [0, 1, 63, 64, 65, 127, 128, 129, 200, 7]
    lk = [5, 129, 128, 64, 63, 1, 300, 129, 0, 70]
    w = wl.random_workload((21, d, mode), lq, lk, 4, 2, d, "bf16", mode, window,
                           with_dout=True, name="bwd-edge")
    print(f"residual route edges d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    ref_o, ref_l = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                                    w.window)
    args = (t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
            w.window, 0.0, 3)
    res = torch.full_like(t["q"], float("nan"))
    out, lse = eat.attn_fwd_dropout(t["q"], t["k"], t["v"], *args, out_residual=res)
    assert_close(to_np(out), ref_o, *BF16_TOL, "residual route O")
    assert_close(to_np(lse), ref_l, 1e-3, 0.0, "residual route LSE")
    o64 = to_np(out).astype(np.float64)
    err_o, err_or = np.abs(o64 - ref_o).mean(), np.abs(o64 + to_np(res) - ref_o).mean()
    assert err_or < err_o / 16, (err_o, err_or)
    empty = ~oracle.explicit_mask(w.cu_q, w.cu_k, w.mask_mode, w.window).any(axis=1)
    if empty.any():
        rows = torch.from_numpy(np.nonzero(empty)[0]).cuda()
        assert torch.all(out[rows].view(torch.int16) == 0)
        assert torch.all(res[rows].view(torch.int16) == 0)
    g = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out, lse, t["dout"], *args,
                             out_residual=res)
    check_grads_derived(w, g, _oracle_bwd(w), f"residual route d={d} mode={mode} w={window}",
                        True)


def test_residual_route_train_full_size():
    """The output-residual route at p = 0 on the training workload (B=2, Hq=32, Hkv=8,
    N=8192, d=128, top-left): the unpipelined forward writing the residual over 65-stage
    loops, and the backward forming D from it. Two (sequence, K/V group) slices (O, LSE of
    the group's 4 query heads; dQ, dK, dV) against the oracle at the standard bounds."""
    import torch
    import exact_attention_tiled_amd as eat
    import oracle_pool as op
    w = wl.train_bf16()
    t = to_device(w)
    print("residual route train full size", flush=True)
    args = (t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
            w.window, 0.0, 5)
    res = torch.full_like(t["q"], float("nan"))
    out, lse = eat.attn_fwd_dropout(t["q"], t["k"], t["v"], *args, out_residual=res)
    dq, dk, dv = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out, lse, t["dout"], *args,
                                      out_residual=res)
    o, l, gq, gk, gv = (to_np(x) for x in (out, lse, dq, dk, dv))
    del t, res, out, lse, dq, dk, dv
    torch.cuda.empty_cache()
    slices = [(0, 6), (1, 1)]
    grp = w.hq // w.hkv
    tasks = []
    for s, g in slices:
        heads = list(range(g * grp, (g + 1) * grp))
        tasks += [(op.fwd_slice, (s, heads)), (op.bwd_slice, (s, g))]
    refs = op.run("train_bf16", {}, tasks)
    for i, (s, g) in enumerate(slices):
        heads = list(range(g * grp, (g + 1) * grp))
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        (ro, rl), (rq, rk, rv) = refs[2 * i], refs[2 * i + 1]
        assert_close(o[rows][:, heads], ro, *BF16_TOL, f"residual route O s{s} g{g}")
        assert_close(l[heads][:, rows], rl, 1e-3, 0.0, f"residual route LSE s{s} g{g}")
        assert_close(gq[rows][:, heads], rq, *BF16_TOL, f"residual route dQ s{s} g{g}")
        assert_close(gk[rows][:, g], rk, *BF16_TOL, f"residual route dK s{s} g{g}")
        assert_close(gv[rows][:, g], rv, *BF16_TOL, f"residual route dV s{s} g{g}")


def test_ragged_gqa_bwd_full_size():
    """The packed ragged GQA workload's packing (16384 tokens, lengths U[1,4096] plus 63, 64,
    65, 127, 128, 129; Hq=32, Hkv=8, d=128, causal) with a loss gradient: GPU forward and
    backward, then every sequence on one K/V group (the groups rotate over the sequences) and
    all 8 groups of the longest sequence against the oracle at the standard bound: the
    gradients of a packed sequence must not take anything from its neighbours ("Causal Mask
    and Ragged Sequence Layouts", sixth section). Values are standard normal here. With the
    forward test's per-sequence value offsets (values up to ~200) the bf16 rounding of the
    stored output, from which D = rowsum(dO * O) is formed, no longer cancels in
    dS = P (dP - D): the CPU rounding model then needs atol ~2 for dQ and dK."""
    import torch
    import oracle_pool as op
    w = wl.ragged_gqa(with_dout=True, v_offsets=False)
    t = to_device(w)
    out, lse = run_fwd(w, t)
    dq, dk, dv = run_bwd(w, t, out, lse)
    gq, gk, gv = to_np(dq), to_np(dk), to_np(dv)
    del t, out, lse, dq, dk, dv
    torch.cuda.empty_cache()
    for x in (gq, gk, gv):
        assert np.all(np.isfinite(x))
    lens = np.diff(w.cu_q)
    longest = int(np.argmax(lens))
    slices = [(s, s % w.hkv) for s in range(w.num_seqs)]
    slices += [(longest, g) for g in range(w.hkv) if g != longest % w.hkv]
    print(f"ragged bwd full size: {w.num_seqs} sequences, {len(slices)} oracle tasks",
          flush=True)
    res = op.run("ragged_gqa", {"with_dout": True, "v_offsets": False},
                 [(op.bwd_slice, (s, g)) for s, g in slices])
    grp = w.hq // w.hkv
    for (s, g), (rq, rk, rv) in zip(slices, res):
        heads = list(range(g * grp, (g + 1) * grp))
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        krows = slice(int(w.cu_k[s]), int(w.cu_k[s + 1]))
        assert_close(gq[rows][:, heads], rq, *BF16_TOL, f"ragged dQ s{s} g{g}")
        assert_close(gk[krows][:, g], rk, *BF16_TOL, f"ragged dK s{s} g{g}")
        assert_close(gv[krows][:, g], rv, *BF16_TOL, f"ragged dV s{s} g{g}")


# ----------------------------------------------------------------------------------------
# fp32 backward (exact products, fp32 accumulation): the fp32 bound 1e-5 + 1e-5 |ref|
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [wl.MASK_CAUSAL_BOTTOM_RIGHT, wl.MASK_NONE])
def test_bwd_tiny_f32(mode):
    """The tiny fp32 workload (B=2, H=2, N=128, d=64; bottom-right and noncausal): forward
    and backward against the oracle at the fp32 bound."""
    import dataclasses
    from gpu_util import F32_TOL
    w = wl.tiny_f32(mode)
    w = dataclasses.replace(w, dout=np.random.default_rng((1, mode)).standard_normal(
        w.q.shape, dtype=np.float32))
    print(f"fp32 tiny backward mode={mode}", flush=True)
    t = to_device(w)
    out, lse = run_fwd(w, t)
    got = run_bwd(w, t, out, lse)
    for name, g, r in zip(("dQ", "dK", "dV"), got, _oracle_bwd(w)):
        assert g.dtype == t["q"].dtype
        worst = assert_close(to_np(g), r, *F32_TOL, f"fp32 tiny {name}")
        print(f"fp32 tiny {name}: max abs err {worst:.2e}", flush=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (1, 70), (2, 33)])
def test_bwd_ragged_edges_f32(d, mode, window):
    """fp32 backward on the ragged edge lengths with GQA 4:2 (dK, dV group sums), every
    alignment and two windows, at the fp32 bound; keys no query sees get exact zeros."""
    import torch
    from gpu_util import F32_TOL
    lq = [0, 1, 63, 64, 65, 127, 128, 129, 200, 7]
    lk = [5, 129, 128, 64, 63, 1, 300, 129, 0, 70]
    w = wl.random_workload((22, d, mode), lq, lk, 4, 2, d, "f32", mode, window,
                           with_dout=True, name="bwd-edge-f32")
    print(f"fp32 backward d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    out, lse = run_fwd(w, t)
    dq, dk, dv = run_bwd(w, t, out, lse)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), _oracle_bwd(w)):
        assert_close(to_np(g), r, *F32_TOL, f"fp32 edge {name}")
    m = oracle.explicit_mask(w.cu_q, w.cu_k, w.mask_mode, w.window)
    unseen = torch.from_numpy(np.nonzero(~m.any(axis=0))[0]).cuda()
    assert torch.all(dk[unseen] == 0) and torch.all(dv[unseen] == 0)


@pytest.mark.parametrize("d,mode,window", [(64, 1, 0), (128, 2, 0), (64, 0, 0), (128, 1, 70)])
def test_bwd_dropout_edges_f32(d, mode, window):
    """fp32 dropout backward against the oracle replaying the same realisation, at the fp32
    bound."""
    import exact_attention_tiled_amd as eat
    from gpu_util import F32_TOL
    edge = [0, 1, 63, 64, 65, 127, 128, 129]
    w = wl.random_workload((43, d, mode), edge + [5, 200], edge[::-1] + [300, 3], 4, 2, d,
                           "f32", mode, window, with_dout=True, name="drop-bwd-f32")
    print(f"fp32 dropout backward d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    p, seed = 0.2, 99
    args = (t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
            w.scale, w.mask_mode, w.window)
    out, lse = eat.attn_fwd_dropout(*args, p, seed)
    got = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out, lse, t["dout"], *args[3:], p, seed)
    ref = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                               w.window, dropout_p=p, seed=seed)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(to_np(g), r, *F32_TOL, f"fp32 dropout {name}")

"""Every kernel reads only inside its inputs: q, k, v (and dout, out, lse, the output residual
for the backward) are placed inside larger buffers whose slack before and after holds NaN.
A read past a tensor's end or before its start that reached any result would turn it into
NaN (even an excluded pair: its weight is 0, and 0 x NaN is NaN in the PV contraction), so
every output must be bitwise what the same call gives on plain tensors. Ragged lengths put
sequence ends at every tile and wave edge, where out-of-range rows are read as zeros by the
range-checked loads ("Causal Mask and Ragged Sequence Layouts", sections 2 and 5: padding
and out-of-range lanes are exclusions, never values).
"""
import pytest

import workloads as wl
from gpu_util import to_device

pytestmark = pytest.mark.gpu

PAD = 8192  # elements of NaN slack on each side


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import exact_attention_tiled_amd as eat
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    eat.load()


def slacked(x):
    """A copy of x in the middle of a NaN-filled buffer (same dtype, contiguous view)."""
    import torch
    buf = torch.full((x.numel() + 2 * PAD,), float("nan"), dtype=x.dtype, device=x.device)
    view = buf[PAD:PAD + x.numel()].view(x.shape)
    view.copy_(x)
    return view


def bitwise(a, b):
    import torch
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


EDGE_Q = [0, 1, 63, 64, 65, 127, 128, 129, 200, 7]
EDGE_K = [5, 129, 128, 64, 63, 1, 300, 129, 0, 70]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (2, 70)])
def test_prefill_and_backward_read_only_inside_inputs(dtype, d, mode, window):
    import torch
    import exact_attention_tiled_amd as eat
    w = wl.random_workload((61, d, mode), EDGE_Q, EDGE_K, 4, 2, d, dtype, mode, window,
                           with_dout=True, name="guard")
    print(f"guards prefill+bwd dtype={dtype} d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    args = (w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window)
    o1, l1 = eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args,
                          path=eat.ATTN_PATH_PREFILL)
    g1 = eat.attn_bwd(t["q"], t["k"], t["v"], o1, l1, t["dout"], t["cu_q"], t["cu_k"], *args)
    q, k, v, do = (slacked(t[n]) for n in ("q", "k", "v", "dout"))
    o2, l2 = eat.attn_fwd(q, k, v, t["cu_q"], t["cu_k"], *args, path=eat.ATTN_PATH_PREFILL)
    g2 = eat.attn_bwd(q, k, v, slacked(o1), slacked(l1), do, t["cu_q"], t["cu_k"], *args)
    torch.cuda.synchronize()
    assert bitwise(o1, o2) and bitwise(l1, l2)
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        assert bitwise(a, b), name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [0, 3])
def test_splitk_reads_only_inside_inputs(dtype, splits):
    import torch
    import exact_attention_tiled_amd as eat
    lq, lk = [1, 4, 16, 0, 3], [300, 129, 1000, 5, 2]
    d = 128 if dtype == "bf16" else 64  # the fp32 split-K path takes head_dim 64
    w = wl.random_workload((62, splits), lq, lk, 8, 2, d, dtype, wl.MASK_CAUSAL_BOTTOM_RIGHT,
                           name="guard-decode")
    print(f"guards split-K dtype={dtype} splits={splits}", flush=True)
    t = to_device(w)
    args = (w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window)
    o1, l1 = eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args,
                          path=eat.ATTN_PATH_SPLITK, num_splits=splits)
    q, k, v = (slacked(t[n]) for n in ("q", "k", "v"))
    o2, l2 = eat.attn_fwd(q, k, v, t["cu_q"], t["cu_k"], *args, path=eat.ATTN_PATH_SPLITK,
                          num_splits=splits)
    torch.cuda.synchronize()
    assert bitwise(o1, o2) and bitwise(l1, l2)


@pytest.mark.parametrize("residual", [False, True], ids=["exact_d_pass", "residual"])
def test_dropout_reads_only_inside_inputs(residual):
    import torch
    import exact_attention_tiled_amd as eat
    w = wl.random_workload(63, EDGE_Q, EDGE_K, 4, 2, 128, "bf16", wl.MASK_CAUSAL_TOP_LEFT, 0,
                           with_dout=True, name="guard-dropout")
    print(f"guards dropout residual={residual}", flush=True)
    t = to_device(w)
    args = (w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window, 0.2, 77)
    r1 = torch.empty_like(t["q"]) if residual else None
    o1, l1 = eat.attn_fwd_dropout(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args,
                                  out_residual=r1)
    g1 = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], o1, l1, t["dout"], t["cu_q"], t["cu_k"],
                              *args, out_residual=r1)
    q, k, v, do = (slacked(t[n]) for n in ("q", "k", "v", "dout"))
    r2 = torch.empty_like(t["q"]) if residual else None
    o2, l2 = eat.attn_fwd_dropout(q, k, v, t["cu_q"], t["cu_k"], *args, out_residual=r2)
    g2 = eat.attn_bwd_dropout(q, k, v, slacked(o2), slacked(l2), do, t["cu_q"], t["cu_k"], *args,
                              out_residual=slacked(r2) if residual else None)
    torch.cuda.synchronize()
    assert bitwise(o1, o2) and bitwise(l1, l2)
    if residual:
        assert bitwise(r1, r2)
    for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
        assert bitwise(a, b), name
    assert all(bool(torch.isfinite(x.float()).all()) for x in (o2, *g2))


def test_repeat_runs_are_bitwise_identical():
    """No atomics and a fixed reduction order on every path: the split-K decode, the backward
    and the dropout backward (with the output residual) give bitwise the same results when
    run twice on the same inputs (the prefill's own check is in test_gpu_fwd.py)."""
    import torch
    import exact_attention_tiled_amd as eat
    w = wl.random_workload(64, EDGE_Q, EDGE_K, 8, 2, 128, "bf16", wl.MASK_CAUSAL_BOTTOM_RIGHT,
                           0, with_dout=True, name="repeat")
    t = to_device(w)
    args = (w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window)
    runs = []
    for _ in range(2):
        o, l = eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args)
        g = eat.attn_bwd(t["q"], t["k"], t["v"], o, l, t["dout"], t["cu_q"], t["cu_k"], *args)
        r = torch.empty_like(t["q"])
        od, ld = eat.attn_fwd_dropout(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args, 0.3,
                                      5, out_residual=r)
        gd = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], od, ld, t["dout"], t["cu_q"],
                                  t["cu_k"], *args, 0.3, 5, out_residual=r)
        dec = wl.random_workload(65, [1, 4, 16, 3], [3000, 129, 1000, 2], 8, 2, 128, "bf16",
                                 wl.MASK_CAUSAL_BOTTOM_RIGHT, name="repeat-decode")
        td = to_device(dec)
        os_, ls = eat.attn_fwd(td["q"], td["k"], td["v"], td["cu_q"], td["cu_k"],
                               dec.max_seqlen_q, dec.max_seqlen_k, dec.scale, dec.mask_mode,
                               path=eat.ATTN_PATH_SPLITK)
        runs.append((o, l, *g, od, ld, r, *gd, os_, ls))
    torch.cuda.synchronize()
    names = ("O", "LSE", "dQ", "dK", "dV", "dropout O", "dropout LSE", "residual",
             "dropout dQ", "dropout dK", "dropout dV", "split-K O", "split-K LSE")
    for name, a, b in zip(names, *runs):
        assert bitwise(a, b), name

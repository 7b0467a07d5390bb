"""The hot path captured in a HIP graph (torch.cuda.graph) and replayed.

The entry points launch kernels only: no allocation, memset or host synchronisation happens
inside them, so a caller can capture a forward or backward call once and replay it on new
inputs written into the same buffers. Each test captures calls with every output and
workspace allocated beforehand, then replays the graph several times. Between replays it
writes new values into the inputs, poisons the outputs with NaN and runs eager calls of the
library on other tensors. After each replay it compares the outputs bitwise with an eager
call on the same inputs; the kernels use no atomics and a fixed reduction order, so the two
must agree bit for bit.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_util import to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import exact_attention_tiled_amd as eat
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    eat.load()


def _bitwise(a, b):
    import torch
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _replay_and_check(graph, inputs, outputs, eager, fresh, disturb):
    """Replay `graph` REPLAYS times. Before each: copy fresh(i) (tensors shaped like
    `inputs`) into `inputs`, fill `outputs` with NaN, call disturb(). After each: the outputs
    equal eager() on the same inputs, bit for bit."""
    import torch
    for i in range(REPLAYS):
        for dst, src in zip(inputs, fresh(i)):
            dst.copy_(src)
        for o in outputs:
            o.fill_(float("nan"))
        disturb()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        ref = eager()
        torch.cuda.synchronize()
        for j, (g, r) in enumerate(zip(got, ref)):
            assert _bitwise(g, r), f"replay {i}: output {j} differs from the eager call"
        print(f"replay {i}: {len(got)} outputs bitwise equal to the eager call", flush=True)


def _fresh_like(t, seed, names):
    """New seeded values (standard normal, bf16-rounded) shaped like t[name] for each name."""
    import torch
    rng = np.random.default_rng(seed)
    out = []
    for n in names:
        x = wl.round_to_bf16(rng.standard_normal(tuple(t[n].shape), dtype=np.float32))
        out.append(torch.from_numpy(x).to(t[n].device).to(t[n].dtype))
    return out


def _disturb(other):
    """Eager library work on other tensors between replays."""
    import exact_attention_tiled_amd as eat
    w, t = other

    def run():
        eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                     w.max_seqlen_k, w.scale, w.mask_mode, w.window)
    return run


def _other():
    w = wl.random_workload(90, [100, 37], [150, 37], 4, 2, 128, "bf16",
                           wl.MASK_CAUSAL_BOTTOM_RIGHT, name="disturb")
    return w, to_device(w)


@pytest.mark.parametrize("kind", ["ragged_prefill", "splitk_decode"])
def test_forward_graph_replay(kind):
    """Forward of a ragged GQA pack (cost-sorted prefill: the order kernel writes the
    workspace, then the prefill reads it) or of a decode pack (split-K kernel and combine,
    partials in the workspace), captured once and replayed on new Q, K and V."""
    import torch
    import exact_attention_tiled_amd as eat
    if kind == "ragged_prefill":
        w = wl.random_workload(91, [300, 1, 129, 64, 0, 200], [300, 5, 129, 64, 7, 250], 8, 2,
                               128, "bf16", wl.MASK_CAUSAL_BOTTOM_RIGHT, name="graph-ragged")
        path = eat.ATTN_PATH_PREFILL
    else:
        w = wl.random_workload(92, [1, 4, 16, 3], [3000, 129, 1000, 2], 8, 2, 128, "bf16",
                               wl.MASK_CAUSAL_BOTTOM_RIGHT, name="graph-decode")
        path = eat.ATTN_PATH_SPLITK
    print(f"graph forward {kind}", flush=True)
    t = to_device(w)
    args = (w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window)
    plan = eat.attn_describe_plan(t["q"], t["k"], t["cu_q"], *args[:2], w.mask_mode, w.window,
                                  path=path)
    assert ("path=splitk" in plan) == (kind == "splitk_decode"), plan
    need = eat.attn_fwd_workspace_size(t["q"], t["k"], t["cu_q"], *args[:2], w.mask_mode,
                                       w.window, path=path)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty((w.hq, w.total_q), dtype=torch.float32, device="cuda")

    def call(o=None, l=None, wsp=None):
        return eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args, path=path,
                            out=o, lse=l, workspace=wsp)
    call(out, lse, ws)  # first call on the device outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse, ws)
    _replay_and_check(g, [t["q"], t["k"], t["v"]], [out, lse], lambda: call(),
                      lambda i: _fresh_like(t, (93, int(kind == "splitk_decode"), i),
                                            ["q", "k", "v"]),
                      _disturb(_other()))


def test_backward_graph_replay():
    """Backward (the dQ kernel forming D and the base-2 LSE, then dK/dV) on ragged edge
    lengths with GQA 4:2, captured once and replayed on a new loss gradient."""
    import torch
    import exact_attention_tiled_amd as eat
    w = wl.random_workload(94, [0, 1, 63, 65, 128, 200], [5, 129, 64, 63, 300, 129], 4, 2,
                           128, "bf16", wl.MASK_CAUSAL_TOP_LEFT, with_dout=True,
                           name="graph-bwd")
    print("graph backward", flush=True)
    t = to_device(w)
    args = (w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window)
    out, lse = eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args)
    need = eat.attn_bwd_workspace_size(t["q"], t["k"], t["cu_q"], *args[:2], w.mask_mode,
                                       w.window)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(t[n]) for n in ("q", "k", "v"))

    def call(a=None, b=None, c=None, wsp=None):
        return eat.attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], t["cu_q"], t["cu_k"],
                            *args, dq=a, dk=b, dv=c, workspace=wsp)
    call(dq, dk, dv, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(dq, dk, dv, ws)
    _replay_and_check(g, [t["dout"]], [dq, dk, dv], lambda: call(),
                      lambda i: _fresh_like(t, (95, i), ["dout"]), _disturb(_other()))


def test_dropout_pair_graph_replay():
    """Dropout forward writing the output residual and the backward reading it (p = 0.2),
    captured together in one graph and replayed on new Q, K, V and loss gradient."""
    import torch
    import exact_attention_tiled_amd as eat
    w = wl.random_workload(96, [200, 64, 7], [300, 64, 70], 4, 2, 128, "bf16",
                           wl.MASK_CAUSAL_BOTTOM_RIGHT, with_dout=True, name="graph-drop")
    print("graph dropout pair", flush=True)
    t = to_device(w)
    args = (t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
            w.window, 0.2, 1234)
    fneed = eat.attn_fwd_dropout_workspace_size(t["q"], t["k"], t["cu_q"], w.max_seqlen_q,
                                                w.max_seqlen_k, w.mask_mode, w.window)
    bneed = eat.attn_bwd_workspace_size(t["q"], t["k"], t["cu_q"], w.max_seqlen_q,
                                        w.max_seqlen_k, w.mask_mode, w.window)
    fws = torch.empty(max(fneed, 1), dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(bneed, 1), dtype=torch.uint8, device="cuda")
    out, res = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    lse = torch.empty((w.hq, w.total_q), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(t[n]) for n in ("q", "k", "v"))

    def call(bufs=None):
        if bufs is None:
            r = torch.empty_like(t["q"])
            o, l = eat.attn_fwd_dropout(t["q"], t["k"], t["v"], *args, out_residual=r)
            return (o, l, r) + tuple(eat.attn_bwd_dropout(t["q"], t["k"], t["v"], o, l,
                                                          t["dout"], *args, out_residual=r))
        eat.attn_fwd_dropout(t["q"], t["k"], t["v"], *args, out=out, lse=lse, workspace=fws,
                             out_residual=res)
        eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out, lse, t["dout"], *args, dq=dq, dk=dk,
                             dv=dv, workspace=bws, out_residual=res)
    call(True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(True)
    _replay_and_check(g, [t["q"], t["k"], t["v"], t["dout"]], [out, lse, res, dq, dk, dv],
                      lambda: call(), lambda i: _fresh_like(t, (97, i), ["q", "k", "v", "dout"]),
                      _disturb(_other()))


def test_no_workspace_forward_graph_replay():
    """attn_fwd_no_workspace (the library's fixed device scratch instead of a workspace) on a
    ragged pack, captured and replayed: the entry point for callers that cannot allocate."""
    import torch
    import exact_attention_tiled_amd as eat
    w = wl.random_workload(98, [300, 1, 129, 0, 77], [300, 5, 129, 7, 500], 8, 2, 128, "bf16",
                           wl.MASK_CAUSAL_BOTTOM_RIGHT, name="graph-noalloc")
    print("graph no-workspace forward", flush=True)
    t = to_device(w)
    args = (w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window)
    out = torch.empty_like(t["q"])
    lse = torch.empty((w.hq, w.total_q), dtype=torch.float32, device="cuda")

    def call(o, l):
        eat.attn_fwd_no_workspace(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], *args, out=o,
                                  lse=l)

    def eager():
        o, l = torch.empty_like(out), torch.empty_like(lse)
        call(o, l)
        return o, l
    call(out, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    _replay_and_check(g, [t["q"], t["k"], t["v"]], [out, lse], eager,
                      lambda i: _fresh_like(t, (99, i), ["q", "k", "v"]), _disturb(_other()))

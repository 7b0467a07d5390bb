"""Race exposure: the parity subset on the build that poisons every LDS buffer before each
refill (lib/libattn_poison.so, compiled with ATTN_DEBUG_POISON_LDS).

A missing barrier often still gives the right answer, because the stale or early data it
exposes is plausible ("Efficient Attention: Formal Correctness", introduction). In the
poisoned build every thread writes a finite sentinel (about 3e4) into exactly the LDS bytes
it is about to refill, so a read that is not ordered after the refill by a barrier sees the
sentinel every time. The poisoned build must give bitwise the same outputs as the release
build, and match the oracle, on ragged forward, split-K decode, backward and dropout cases.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import (BF16_TOL, DROPOUT_GRAD_TOL, LSE_TOL, assert_close, to_device, to_np,
                      tol_for)

pytestmark = pytest.mark.gpu

EDGE_Q = [0, 1, 63, 64, 65, 127, 128, 129, 200, 7]
EDGE_K = [5, 129, 128, 64, 63, 1, 300, 129, 0, 70]


@pytest.fixture(scope="module")
def poison_lib():
    import torch
    import exact_attention_tiled_amd as eat
    from exact_attention_tiled_amd import build as eat_build
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    eat.load()
    if not os.path.exists(eat_build.POISON_LIB_PATH):
        pytest.fail(f"{eat_build.POISON_LIB_PATH} missing: build it with __graft_entry__.build()")
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    with eat.use_library(eat_build.POISON_LIB_PATH):
        plan = eat.attn_describe_plan(q, q, cu, 4, 4, 1)
    assert plan.endswith("lds=poisoned"), plan
    assert "poisoned" not in eat.attn_describe_plan(q, q, cu, 4, 4, 1)
    return eat_build.POISON_LIB_PATH


def _bitwise(a, b):
    import torch
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.contiguous().view(view), b.contiguous().view(view))


def _both(poison_lib, fn):
    """fn() on the release build, then on the poisoned build; the two result tuples."""
    import torch
    import exact_attention_tiled_amd as eat
    rel = fn()
    torch.cuda.synchronize()
    with eat.use_library(poison_lib):
        poi = fn()
        torch.cuda.synchronize()
    return rel, poi


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (2, 97)])
def test_prefill_race_exposure(poison_lib, dtype, d, mode, window):
    import exact_attention_tiled_amd as eat
    w = wl.random_workload((51, d, mode), EDGE_Q, EDGE_K, 4, 2, d, dtype, mode, window,
                           name="poison-fwd", v_offsets=True)
    print(f"poisoned prefill {dtype} d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    (o1, l1), (o2, l2) = _both(poison_lib, lambda: eat.attn_fwd(
        t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale,
        w.mask_mode, w.window, path=eat.ATTN_PATH_PREFILL))
    assert _bitwise(o1, o2) and _bitwise(l1, l2)
    ro, rl = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window)
    assert_close(to_np(o2), ro, *tol_for(w), "poisoned O")
    assert_close(to_np(l2), rl, LSE_TOL, 0.0, "poisoned LSE")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nq,group,splits", [(1, 4, 0), (16, 4, 3), (64, 1, 2)])
def test_splitk_race_exposure(poison_lib, dtype, nq, group, splits):
    import exact_attention_tiled_amd as eat
    d = 128 if dtype == "bf16" else 64
    w = wl.random_workload((52, nq, group), [nq, nq, 0, nq], [2000, 700, 50, 1], 2 * group, 2,
                           d, dtype, wl.MASK_CAUSAL_BOTTOM_RIGHT, name="poison-splitk",
                           v_offsets=True)
    print(f"poisoned split-K {dtype} nq={nq} group={group} splits={splits}", flush=True)
    t = to_device(w)
    (o1, l1), (o2, l2) = _both(poison_lib, lambda: eat.attn_fwd(
        t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale,
        w.mask_mode, w.window, path=eat.ATTN_PATH_SPLITK, num_splits=splits))
    assert _bitwise(o1, o2) and _bitwise(l1, l2)
    ro, rl = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window)
    assert_close(to_np(o2), ro, *tol_for(w), "poisoned split-K O")
    assert_close(to_np(l2), rl, LSE_TOL, 0.0, "poisoned split-K LSE")


# Backward workloads whose gradient bounds are derived on the CPU by the rounding model
# (tests/test_tolerance_derivation.py): the seed-21 edges stay inside the standard bound,
# the seed-42 dropout edges need DROPOUT_GRAD_TOL. The last flag runs the forward that also
# writes the output residual (its second PV contraction) and the backward that forms D from
# it, with dropout or (p = 0) without.
BWD_CASES = [(64, 1, 0, 0.0, False), (128, 2, 0, 0.0, False), (128, 0, 0, 0.0, False),
             (64, 1, 70, 0.0, False), (64, 1, 0, 0.2, False), (128, 2, 0, 0.2, False),
             (128, 1, 70, 0.2, False), (64, 1, 0, 0.2, True), (128, 0, 0, 0.2, True),
             (64, 2, 33, 0.0, True), (128, 1, 0, 0.0, True)]


@pytest.mark.parametrize("d,mode,window,dropout_p,residual", BWD_CASES)
def test_backward_race_exposure(poison_lib, d, mode, window, dropout_p, residual):
    import exact_attention_tiled_amd as eat
    if dropout_p == 0.0:
        w = wl.random_workload((21, d, mode), EDGE_Q, EDGE_K, 4, 2, d, "bf16", mode, window,
                               with_dout=True, name="bwd-edge")
    else:
        edge = [0, 1, 63, 64, 65, 127, 128, 129]
        w = wl.random_workload((42, d, mode), edge + [5, 200], edge[::-1] + [300, 3], 4, 2, d,
                               "bf16", mode, window, with_dout=True, name="drop-bwd")
    print(f"poisoned backward d={d} mode={mode} window={window} p={dropout_p} "
          f"residual={residual}", flush=True)
    t = to_device(w)
    args = (t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
            w.scale, w.mask_mode, w.window)

    def run():
        if dropout_p == 0.0 and not residual:
            out, lse = eat.attn_fwd(*args)
            g = eat.attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], *args[3:])
        else:
            import torch
            res = torch.empty_like(t["q"]) if residual else None
            out, lse = eat.attn_fwd_dropout(*args, dropout_p, 99, out_residual=res)
            g = eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out, lse, t["dout"], *args[3:],
                                     dropout_p, 99, out_residual=res)
            if residual:
                return (out, lse) + tuple(g) + (res,)
        return (out, lse) + tuple(g)

    rel, poi = _both(poison_lib, run)
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV", "residual"), rel, poi):
        assert _bitwise(a, b), f"poisoned {name} differs from the release build"
    kw = {} if dropout_p == 0.0 else {"dropout_p": dropout_p, "seed": 99}
    ref = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                               w.window, **kw)
    tol = BF16_TOL if dropout_p == 0.0 else DROPOUT_GRAD_TOL
    for name, g, r in zip(("dQ", "dK", "dV"), poi[2:], ref):
        assert_close(to_np(g), r, *tol, f"poisoned {name}")

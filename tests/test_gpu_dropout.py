"""GPU parity of attention dropout: the kernels' realisation bit-exactly against the oracle's,
and forward / backward against the fp64 oracle replaying the same realisation."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import (BF16_TOL, DROPOUT_GRAD_TOL, LSE_TOL, assert_close, to_device, to_np,
                      tol_for)
from rounding_model import required_atol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import exact_attention_tiled_amd as eat
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    eat.load()


def fwd_drop(w, t, p, seed, res=None):
    import exact_attention_tiled_amd as eat
    return eat.attn_fwd_dropout(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                                w.max_seqlen_k, w.scale, w.mask_mode, w.window, p, seed,
                                out_residual=res)


def bwd_drop(w, t, out, lse, p, seed, res=None):
    import exact_attention_tiled_amd as eat
    return eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out, lse, t["dout"], t["cu_q"],
                                t["cu_k"], w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
                                w.window, p, seed, out_residual=res)


def residual_buffer(t):
    """Output-residual buffer of the bf16 dropout forward (None: no residual)."""
    import torch
    return torch.full_like(t["q"], float("nan"))


@pytest.mark.parametrize("seed,p,seq,head,q0,nq,k0,nk", [
    (0, 0.1, 0, 0, 0, 64, 0, 64),
    (0x0123456789ABCDEF, 0.5, 3, 7, 5, 37, 2, 91),
    (2**64 - 1, 0.9, 16383, 31, 131000, 40, 130950, 120),
    (42, 1.0 / 256, 1, 2, 1, 3, 1, 3),
    (42, 255.0 / 256, 1, 2, 0, 16, 0, 16),
    (7, 0.2, 2, 5, 32, 96, 64, 160),          # several 32-aligned blocks in each direction
    (99, 0.2, 9, 3, 8160, 64, 256, 64),        # deep in a long sequence, aligned
    (2**40 + 3, 0.5, 1, 0, 4064, 65, 33, 127),  # ragged tails on both sides
])
def test_dropout_probe_bit_exact(seed, p, seq, head, q0, nq, k0, nk):
    """The kernels' keep flags, computed in both lane layouts the kernels use (rows of the
    forward and dQ; columns of dK/dV), equal the oracle's element for element (integer work)."""
    import exact_attention_tiled_amd as eat
    print(f"dropout probe seed={seed} p={p} seq={seq} head={head} q0={q0} k0={k0}", flush=True)
    got = eat.attn_dropout_probe(seq, head, q0, nq, k0, nk, p, seed).cpu().numpy()
    ref = oracle.dropout_keep(seed, seq, head, np.arange(q0, q0 + nq)[:, None],
                              np.arange(k0, k0 + nk)[None, :], oracle.dropout_threshold(p))
    assert not np.any(got & ~np.uint8(3)), "bits 2-7 must be zero"
    assert np.array_equal((got & 1).astype(bool), ref), "row form (forward, dQ)"
    assert np.array_equal((got >> 1 & 1).astype(bool), ref), "column form (dK, dV)"


EDGE = [0, 1, 63, 64, 65, 127, 128, 129]

# The backward's contractions take Z = P * keep / (1 - p) (dV) and dS (dK, dQ) as bf16
# operands. On the edge workloads below - one sequence sums about 400 rounded weights near
# 0.4 into every dV entry of its 3 keys - those roundings alone move some gradients beyond
# 2e-2 + 2e-2 |ref|. The edge backward is held to DROPOUT_GRAD_TOL (gpu_util), the bound the
# CPU rounding model derives for exactly these workloads (test_tolerance_derivation.py);
# outputs, LSE, the realisation, the canary workload and the full-size gradients keep the
# standard bounds.



@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (2, 70)])
def test_dropout_forward_edges(dtype, d, mode, window):
    """Ragged lengths around the tile edges, GQA 4:2: O against the oracle with the same
    realisation, LSE against the undropped oracle LSE."""
    lq = EDGE + [5, 200]
    lk = EDGE[::-1] + [300, 3]
    w = wl.random_workload((41, d, mode), lq, lk, 4, 2, d, dtype, mode, window, name="drop-edge",
                           v_offsets=True)
    print(f"dropout fwd dtype={dtype} d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    for p, seed in ((0.1, 7), (0.5, 2**40 + 3)):
        out, lse = fwd_drop(w, t, p, seed)
        ro, rl = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                                  dropout_p=p, seed=seed)
        assert_close(to_np(out), ro, *tol_for(w), f"dropout O p={p}")
        assert_close(to_np(lse), rl, LSE_TOL, 0.0, f"dropout LSE p={p}")


@pytest.mark.parametrize("residual", [False, True], ids=["exact_d_pass", "residual"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (1, 70)])
def test_dropout_backward_edges(d, mode, window, residual):
    """dQ, dK, dV (GQA group sums) against the oracle replaying the forward's realisation,
    with D from the backward's own pass or from the forward's output plus its residual."""
    lq = EDGE + [5, 200]
    lk = EDGE[::-1] + [300, 3]
    # N(0,1) values: the backward forms D = rowsum(dO * O) from the stored bf16 output, so
    # the forward tests' large per-sequence value offsets would put its rounding (spacing
    # 0.5 near |O| = 90) far above the gradient tolerance.
    w = wl.random_workload((42, d, mode), lq, lk, 4, 2, d, "bf16", mode, window,
                           with_dout=True, name="drop-bwd")
    print(f"dropout bwd d={d} mode={mode} window={window} residual={residual}", flush=True)
    t = to_device(w)
    p, seed = 0.2, 99
    res = residual_buffer(t) if residual else None
    out, lse = fwd_drop(w, t, p, seed, res)
    got = bwd_drop(w, t, out, lse, p, seed, res)
    ref = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                               w.window, dropout_p=p, seed=seed)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        worst = assert_close(to_np(g), r, *DROPOUT_GRAD_TOL, f"dropout {name}")
        print(f"dropout {name}: max |err| {worst:.4f}, required atol at rtol 2e-2 "
              f"{required_atol(to_np(g), r):.4f} (bound {DROPOUT_GRAD_TOL[0]})", flush=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,window", [(1, 0), (2, 0), (0, 0), (2, 70)])
def test_dropout_output_residual(d, mode, window):
    """The forward's output residual: out + residual is the unrounded output (within 1e-4 +
    1e-4 |ref| of the oracle, against 2e-2 for out alone), the residual is at most half a
    bf16 spacing of out (out is the nearest bf16 to out + residual, up to a tie made by the
    residual's own rounding), and rows with no allowed key have +0.0 in both."""
    import torch
    lq = EDGE + [5, 200]
    lk = EDGE[::-1] + [300, 3]
    w = wl.random_workload((41, d, mode), lq, lk, 4, 2, d, "bf16", mode, window,
                           name="drop-edge", v_offsets=True)
    print(f"dropout residual d={d} mode={mode} window={window}", flush=True)
    t = to_device(w)
    res = residual_buffer(t)
    out, lse = fwd_drop(w, t, 0.1, 7, res)
    ro, _ = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                             dropout_p=0.1, seed=7)
    o, r = to_np(out), to_np(res)
    assert np.all(np.isfinite(r))
    assert_close(o, ro, *BF16_TOL, "dropout O (rounded)")
    assert_close(o.astype(np.float64) + r, ro, 1e-4, 1e-4, "dropout O + residual")
    # spacing above |out|: the next bf16 magnitude minus |out| (the spacing below is never
    # larger, so |residual| <= half of it on both sides)
    mag = out.view(torch.int16) & 0x7FFF
    up = (mag + 1).view(torch.bfloat16).float() - mag.view(torch.bfloat16).float()
    assert torch.all(res.float().abs() <= 0.5 * up)
    empty = ~oracle.explicit_mask(w.cu_q, w.cu_k, w.mask_mode, w.window).any(axis=1)
    if empty.any():
        rows = torch.from_numpy(np.nonzero(empty)[0]).cuda()
        assert torch.all(out[rows].view(torch.int16) == 0)
        assert torch.all(res[rows].view(torch.int16) == 0)


def test_dropout_replays_across_packings():
    """A sequence's dropout output and gradients are bitwise the same when the other
    sequences of the pack change length (its storage offsets move; its index, heads and
    positions do not)."""
    a = wl.random_workload(43, [300, 0, 257, 5], [310, 3, 257, 9], 4, 2, 128, "bf16",
                           wl.MASK_CAUSAL_TOP_LEFT, with_dout=True, name="pack-a")
    b = wl.random_workload(44, [17, 129, 257, 64], [1, 200, 257, 64], 4, 2, 128, "bf16",
                           wl.MASK_CAUSAL_TOP_LEFT, with_dout=True, name="pack-b")
    qa, ka, qb, kb = int(a.cu_q[2]), int(a.cu_k[2]), int(b.cu_q[2]), int(b.cu_k[2])
    for name in ("q", "dout"):
        getattr(b, name)[qb:qb + 257] = getattr(a, name)[qa:qa + 257]
    for name in ("k", "v"):
        getattr(b, name)[kb:kb + 257] = getattr(a, name)[ka:ka + 257]
    res = []
    for w in (a, b):
        t = to_device(w)
        out, lse = fwd_drop(w, t, 0.3, 1234)
        res.append((to_np(out), to_np(lse)) + tuple(to_np(x) for x in bwd_drop(w, t, out, lse,
                                                                                0.3, 1234)))
    (oa, la, dqa, dka, dva), (ob, lb, dqb, dkb, dvb) = res
    assert np.array_equal(oa[qa:qa + 257], ob[qb:qb + 257])
    assert np.array_equal(la[:, qa:qa + 257], lb[:, qb:qb + 257])
    assert np.array_equal(dqa[qa:qa + 257], dqb[qb:qb + 257])
    assert np.array_equal(dka[ka:ka + 257], dkb[kb:kb + 257])
    assert np.array_equal(dva[ka:ka + 257], dvb[kb:kb + 257])


def test_dropout_zero_probability_is_attn_fwd():
    """p = 0 is the deterministic operator: attn_fwd_dropout then runs attn_fwd's kernels."""
    import exact_attention_tiled_amd as eat
    w = wl.random_workload(45, [200, 77], [200, 90], 4, 2, 128, "bf16",
                           wl.MASK_CAUSAL_BOTTOM_RIGHT, name="p0")
    t = to_device(w)
    out, lse = fwd_drop(w, t, 0.0, 5)
    out2, lse2 = eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                              w.max_seqlen_k, w.scale, w.mask_mode, w.window,
                              path=eat.ATTN_PATH_PREFILL)
    assert np.array_equal(to_np(out), to_np(out2)) and np.array_equal(to_np(lse), to_np(lse2))


@pytest.mark.parametrize("residual", [False, True], ids=["exact_d_pass", "residual"])
def test_dropout_train_full_size(residual):
    """The training workload (B=2, Hq=32, Hkv=8, N=8192, d=128, top-left) with p = 0.1:
    full GPU forward + backward (D from the backward's own pass, or from the forward's
    output residual as the bench runs it); the oracle replays the realisation on one
    (sequence, K/V head group): O and LSE of its 4 query heads, dQ, dK, dV of the group."""
    w = wl.train_bf16()
    t = to_device(w)
    p, seed = 0.1, 2026
    print(f"dropout train full size residual={residual}", flush=True)
    res = residual_buffer(t) if residual else None
    out, lse = fwd_drop(w, t, p, seed, res)
    dq, dk, dv = bwd_drop(w, t, out, lse, p, seed, res)
    del res
    o, l, gq, gk, gv = (to_np(x) for x in (out, lse, dq, dk, dv))
    for x in (o, l, gq, gk, gv):
        assert np.all(np.isfinite(x))
    s, g = 0, 5
    heads = list(range(4 * g, 4 * g + 4))
    ro, rl = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                              seqs=[s], heads=heads, dropout_p=p, seed=seed)
    rq, rk, rv = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale,
                                      w.mask_mode, w.window, seqs=[s], kv_heads=[g],
                                      dropout_p=p, seed=seed)
    rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
    assert_close(o[rows][:, heads], ro[rows][:, heads], *BF16_TOL, "dropout train O")
    assert_close(l[heads][:, rows], rl[heads][:, rows], LSE_TOL, 0.0, "dropout train LSE")
    assert_close(gq[rows][:, heads], rq[rows][:, heads], *BF16_TOL, "dropout train dQ")
    assert_close(gk[rows][:, g], rk[rows][:, g], *BF16_TOL, "dropout train dK")
    assert_close(gv[rows][:, g], rv[rows][:, g], *BF16_TOL, "dropout train dV")


@pytest.mark.parametrize("residual", [False, True], ids=["exact_d_pass", "residual"])
def test_dropout_canaries_no_out_of_bounds_writes(residual):
    """The dropout forward and backward write only inside their outputs: O, LSE, the output
    residual, dQ, dK, dV land inside larger buffers whose slack holds sentinels, and every
    sentinel survives. Keys no query can see get exactly zero dK/dV, whatever the
    realisation."""
    import torch
    import exact_attention_tiled_amd as eat
    lq, lk = [40, 3, 90], [10, 200, 90]
    w = wl.random_workload(46, lq, lk, 4, 1, 64, "bf16", wl.MASK_CAUSAL_BOTTOM_RIGHT, 16,
                           with_dout=True, name="drop-canary")
    t = to_device(w)
    pad, sentinel = 4096, -12345.0

    def padded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * pad,), sentinel, dtype=dtype, device="cuda")
        return buf, buf[pad:pad + n].view(shape)

    bo, out = padded(t["q"].shape, t["q"].dtype)
    bl, lse = padded((w.hq, w.total_q), torch.float32)
    br, res = padded(t["q"].shape, t["q"].dtype) if residual else (None, None)
    eat.attn_fwd_dropout(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                         w.max_seqlen_k, w.scale, w.mask_mode, w.window, 0.25, 777, out=out,
                         lse=lse, out_residual=res)
    bq, dq = padded(t["q"].shape, t["q"].dtype)
    bk, dk = padded(t["k"].shape, t["k"].dtype)
    bv, dv = padded(t["v"].shape, t["v"].dtype)
    eat.attn_bwd_dropout(t["q"], t["k"], t["v"], out, lse, t["dout"], t["cu_q"], t["cu_k"],
                         w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode, w.window, 0.25,
                         777, dq=dq, dk=dk, dv=dv, out_residual=res)
    torch.cuda.synchronize()
    for buf in (bo, bl, bq, bk, bv) + ((br,) if residual else ()):
        assert torch.all(buf[:pad] == sentinel) and torch.all(buf[-pad:] == sentinel)
    m = oracle.explicit_mask(w.cu_q, w.cu_k, w.mask_mode, w.window)
    unseen = torch.from_numpy(np.nonzero(~m.any(axis=0))[0]).cuda()
    assert len(unseen) > 50
    assert torch.all(dk[unseen].float() == 0) and torch.all(dv[unseen].float() == 0)
    ro, rl = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                              dropout_p=0.25, seed=777)
    assert_close(to_np(out), ro, *BF16_TOL, "dropout canary O")
    assert_close(to_np(lse), rl, LSE_TOL, 0.0, "dropout canary LSE")
    ref = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                               w.window, dropout_p=0.25, seed=777)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(to_np(g), r, *BF16_TOL, f"dropout canary {name}")

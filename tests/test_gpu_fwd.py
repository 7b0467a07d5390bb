"""GPU forward parity against the fp64 oracle (both forward paths), bit-exact mask checks."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import (BF16_TOL, F32_TOL, LSE_TOL, assert_close, check_fwd, run_fwd, to_device,
                      to_np)

pytestmark = pytest.mark.gpu

PREFILL, SPLITK = 1, 2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import exact_attention_tiled_amd as eat
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    eat.load()


def _oracle(w, seqs=None, heads=None):
    return oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window,
                            seqs=seqs, heads=heads)


# ----------------------------------------------------------------------------------------
# mask unit: bit-exact against the explicit mask from sequence ids and positions
# ----------------------------------------------------------------------------------------

MASK_PACKS = [
    ([63, 64, 65], [63, 64, 65]),
    ([127, 128, 129, 1, 0, 5], [127, 128, 129, 1, 3, 0]),
    ([40, 300], [200, 100]),
    ([257], [1]),
    ([1, 2, 3], [300, 64, 129]),
]


PROBE_UNITS = {0: "prefill_bf16", 1: "prefill_generic", 3: "bwd_dk_dv", 4: "bwd_dq",
               5: "bwd_dk_dv_f32", 6: "bwd_dq_f32"}


@pytest.mark.parametrize("unit", sorted(PROBE_UNITS), ids=lambda u: PROBE_UNITS[u])
@pytest.mark.parametrize("pack", range(len(MASK_PACKS)))
@pytest.mark.parametrize("mode,window", [(0, 0), (1, 0), (2, 0), (1, 1), (1, 64), (2, 7), (2, 130)])
def test_mask_probe_bit_exact(pack, mode, window, unit):
    """Each kernel unit's own mask decisions (stage range, block classes, per-lane tests)
    against the explicit mask from sequence ids and positions, bit for bit ("Causal Mask
    and Ragged Sequence Layouts", sections 1-4; section 6 for the backward units)."""
    import torch
    import exact_attention_tiled_amd as eat
    lq, lk = MASK_PACKS[pack]
    cu_q, cu_k = wl.cu_from_lengths(lq), wl.cu_from_lengths(lk)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    print(f"mask probe unit={PROBE_UNITS[unit]} pack={pack} mode={mode} window={window}", flush=True)
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    if unit == eat.ATTN_PROBE_PREFILL:
        bits = eat.attn_mask_probe(cq, ck, tq, tk, mode, window, 0, tq, 0, tk)
    else:
        bits = eat.attn_mask_probe_ex(cq, ck, tq, tk, max(lq), max(lk), 1, 1, mode, window, unit,
                                      0, tq, 0, tk)
    got = bits.cpu().numpy().astype(bool)
    want = oracle.explicit_mask(cu_q, cu_k, mode, window)
    assert np.array_equal(got, want), np.argwhere(got != want)[:10].tolist()


# Decode-shaped packs for the split-K unit: query lengths, key lengths, Hq, Hkv (G * max
# query length <= 64 rows per K/V head, one or two 32-row blocks).
SPLITK_PACKS = [
    ([1, 4, 16, 0, 3], [300, 129, 1000, 5, 2], 8, 2),
    ([64, 1, 7], [32, 300, 7], 2, 2),
    ([16, 16], [4096, 3000], 8, 2),
    ([5, 9], [700, 9], 6, 1),
]


@pytest.mark.parametrize("pack", range(len(SPLITK_PACKS)))
@pytest.mark.parametrize("mode,window", [(2, 0), (1, 0), (0, 0), (2, 300), (2, 7)])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_mask_probe_splitk_bit_exact(pack, mode, window, splits):
    """The split-K decode's decisions (chunk ranges, the chunk clip, block classes of the
    row blocks, per-lane tests) for every query head of the group against the explicit
    mask, for the automatic and forced split counts."""
    import torch
    import exact_attention_tiled_amd as eat
    lq, lk, hq, hkv = SPLITK_PACKS[pack]
    cu_q, cu_k = wl.cu_from_lengths(lq), wl.cu_from_lengths(lk)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    want = oracle.explicit_mask(cu_q, cu_k, mode, window)
    print(f"split-K mask probe pack={pack} mode={mode} window={window} splits={splits}", flush=True)
    for h in range(hq // hkv):
        bits = eat.attn_mask_probe_ex(cq, ck, tq, tk, max(lq), max(lk), hq, hkv, mode, window,
                                      eat.ATTN_PROBE_SPLITK, 0, tq, 0, tk, head=h,
                                      num_splits=splits)
        got = bits.cpu().numpy().astype(bool)
        assert np.array_equal(got, want), (h, np.argwhere(got != want)[:10].tolist())


# ----------------------------------------------------------------------------------------
# tiny fp32 workload (B=2, H=2, N=128, d=64), bottom-right and no mask
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [wl.MASK_CAUSAL_BOTTOM_RIGHT, wl.MASK_NONE])
@pytest.mark.parametrize("path", [0, PREFILL])
def test_tiny_f32(mode, path):
    w = wl.tiny_f32(mode)
    print(f"tiny_f32 mode={mode} path={path}", flush=True)
    ref_o, ref_l = _oracle(w)
    out, lse = run_fwd(w, path=path)
    check_fwd(w, out, lse, ref_o, ref_l, f"tiny f32 mode {mode} path {path}")


# ----------------------------------------------------------------------------------------
# ragged edge lengths around tile boundaries, both dtypes, all alignments, GQA, both paths
# ----------------------------------------------------------------------------------------

EDGE = [0, 1, 63, 64, 65, 127, 128, 129]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,window", [(0, 0), (1, 0), (2, 0), (1, 50), (2, 97)])
def test_edge_lengths_prefill(dtype, d, mode, window):
    lq = EDGE + [5, 200]
    lk = EDGE[::-1] + [300, 3]
    w = wl.random_workload((11, d, mode), lq, lk, 4, 2, d, dtype, mode, window, name="edge",
                           v_offsets=True)
    print(f"edge prefill dtype={dtype} d={d} mode={mode} window={window}", flush=True)
    ref_o, ref_l = _oracle(w)
    out, lse = run_fwd(w, path=PREFILL)
    check_fwd(w, out, lse, ref_o, ref_l, "edge prefill")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,window", [(2, 0), (1, 0), (0, 0), (2, 300)])
@pytest.mark.parametrize("nq,group", [(1, 4), (3, 8), (16, 4), (64, 1)])
def test_splitk_decode_shapes(dtype, mode, window, nq, group):
    lk = [1, 129, 700, 2048, 0, 333]
    lq = [min(nq, x) if mode == 1 else nq for x in lk]
    d = 128 if dtype == "bf16" else 64   # fp32 split-K stages of head_dim 128 exceed LDS
    w = wl.random_workload((12, nq, mode), lq, lk, 2 * group, 2, d, dtype, mode, window,
                           name="decode-small", v_offsets=True)
    print(f"splitk dtype={dtype} mode={mode} window={window} nq={nq} group={group}", flush=True)
    ref_o, ref_l = _oracle(w)
    for splits in (0, 1, 3):
        out, lse = run_fwd(w, path=SPLITK, num_splits=splits)
        check_fwd(w, out, lse, ref_o, ref_l, f"splitk splits={splits}")
    out, lse = run_fwd(w, path=PREFILL)
    check_fwd(w, out, lse, ref_o, ref_l, "same shapes via prefill")


# ----------------------------------------------------------------------------------------
# equal-length batches: the prefill enumerates tiles largest-first across (sequence, head)
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("lq,lk,mode,window", [
    (300, 450, 2, 0), (300, 450, 1, 0), (450, 300, 2, 0), (450, 300, 1, 0), (257, 257, 0, 0),
    (384, 384, 1, 100), (200, 600, 2, 129), (1, 1, 1, 0)])
@pytest.mark.parametrize("hq,hkv", [(6, 2), (8, 8), (12, 3)])
@pytest.mark.parametrize("d", [64, 128])
def test_equal_length_batches(lq, lk, mode, window, hq, hkv, d):
    """Every sequence of the pack has the same lengths (ragged tails inside the last tile),
    head counts that are and are not multiples of 8; against the oracle, and bitwise equal
    to the same sequences preceded by a one-token sequence (which forces the cost-sorted order)."""
    import exact_attention_tiled_amd as eat
    import torch
    nseq = 3
    w = wl.random_workload((14, lq, lk, mode, hq), [lq] * nseq, [lk] * nseq, hq, hkv, d,
                           "bf16", mode, window, name="equal", v_offsets=True)
    print(f"equal-length lq={lq} lk={lk} mode={mode} window={window} hq={hq} hkv={hkv} d={d}",
          flush=True)
    t = to_device(w)
    plan = eat.attn_describe_plan(t["q"], t["k"], t["cu_q"], w.max_seqlen_q, w.max_seqlen_k,
                                  w.mask_mode, w.window)
    assert "order=largest_first" in plan, plan
    out, lse = run_fwd(w, t, path=PREFILL)
    check_fwd(w, out, lse, *_oracle(w), "equal-length")
    if lq == 1 and lk == 1:
        return  # a one-token prefix would keep the batch equal-length
    # The same pack after a one-token sequence: not equal-length, so the slot order runs.
    q1 = torch.cat([t["q"][:1], t["q"]])
    k1 = torch.cat([t["k"][:1], t["k"]])
    v1 = torch.cat([t["v"][:1], t["v"]])
    cu_q1 = torch.cat([t["cu_q"][:1], t["cu_q"] + 1])
    cu_k1 = torch.cat([t["cu_k"][:1], t["cu_k"] + 1])
    plan1 = eat.attn_describe_plan(q1, k1, cu_q1, w.max_seqlen_q, w.max_seqlen_k, w.mask_mode,
                                   w.window)
    assert "order=cost_sorted" in plan1, plan1
    out1, lse1 = eat.attn_fwd(q1, k1, v1, cu_q1, cu_k1, w.max_seqlen_q, w.max_seqlen_k, w.scale,
                              w.mask_mode, w.window, path=PREFILL)
    torch.cuda.synchronize()
    assert torch.equal(out1[1:].view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse1[:, 1:], lse)


# ----------------------------------------------------------------------------------------
# bit-exact behaviour: empty rows, masked K/V perturbation, packing, determinism
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("path", [PREFILL, SPLITK])
def test_empty_rows_are_exact_zero(path):
    """Nq = 64 > Nk = 32 under bottom-right alignment: the first 32 rows of every sequence
    are empty -> O = +0.0 (all bits zero) and LSE = -inf exactly."""
    if path == PREFILL:
        w = wl.decode(64, nk=32)            # the full Nq = 64 > Nk = 32 edge workload
        n_empty = 32
    else:                                   # split-K holds at most 64 rows per K/V head
        w = wl.random_workload(16, [16] * 5, [8, 8, 1, 16, 9], 8, 2, 128, "bf16",
                               wl.MASK_CAUSAL_BOTTOM_RIGHT, name="empty-rows-splitk")
        n_empty = None
    print(f"empty rows path={path}", flush=True)
    out, lse = run_fwd(w, path=path)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    for s in range(w.num_seqs):
        lq, lk = int(w.cu_q[s + 1] - w.cu_q[s]), int(w.cu_k[s + 1] - w.cu_k[s])
        ne = n_empty if n_empty is not None else max(0, lq - lk)
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s]) + ne)
        assert np.all(o[rows].view(np.uint32) == 0), "empty rows must be +0.0"
        assert np.all(l[:, rows] == -np.inf)
        assert np.all(np.isfinite(l[:, int(w.cu_q[s]) + ne:int(w.cu_q[s + 1])]))
    ref_o, ref_l = _oracle(w)
    check_fwd(w, out, lse, ref_o, ref_l, "edge decode")


@pytest.mark.parametrize("path", [PREFILL, SPLITK])
def test_masked_kv_changes_nothing(path):
    """Overwriting K/V entries no query may see (other sequences' neighbours, future keys,
    keys beyond the window) with large finite values leaves every output bit unchanged."""
    import torch
    lq, lk = [100, 1, 50, 7], [130, 200, 50, 1500]
    w = wl.random_workload(13, lq, lk, 4, 2, 128, "bf16", wl.MASK_CAUSAL_BOTTOM_RIGHT, 64,
                           name="perturb")
    t = to_device(w)
    if path == SPLITK:
        w = wl.random_workload(13, [3, 1, 2, 7], lk, 4, 2, 128, "bf16",
                               wl.MASK_CAUSAL_BOTTOM_RIGHT, 64, name="perturb")
        t = to_device(w)
    out1, lse1 = run_fwd(w, t, path=path)
    m = oracle.explicit_mask(w.cu_q, w.cu_k, w.mask_mode, w.window)
    unseen = ~m.any(axis=0)
    assert unseen.sum() > 100
    k2, v2 = t["k"].clone(), t["v"].clone()
    idx = torch.from_numpy(np.nonzero(unseen)[0]).cuda()
    k2[idx] = 1.0e4
    v2[idx] = -3.0e4
    t2 = dict(t, k=k2, v=v2)
    out2, lse2 = run_fwd(w, t2, path=path)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))


def test_packing_order_is_bitwise_neutral():
    """Each sequence's forward result is bitwise independent of where it sits in the pack
    (tiles start at each sequence's first token)."""
    import torch
    lens = [70, 129, 5, 300]
    w = wl.random_workload(14, lens, lens, 4, 4, 128, "bf16", wl.MASK_CAUSAL_TOP_LEFT,
                           name="pack")
    out, lse = run_fwd(w, path=PREFILL)
    perm = [2, 0, 3, 1]
    cu = w.cu_q
    q = np.concatenate([w.q[cu[s]:cu[s + 1]] for s in perm])
    k = np.concatenate([w.k[cu[s]:cu[s + 1]] for s in perm])
    v = np.concatenate([w.v[cu[s]:cu[s + 1]] for s in perm])
    lp = [lens[s] for s in perm]
    w2 = wl.Workload("pack2", "bf16", q, k, v, wl.cu_from_lengths(lp), wl.cu_from_lengths(lp),
                     w.scale, w.mask_mode)
    out2, lse2 = run_fwd(w2, path=PREFILL)
    cu2 = w2.cu_q
    for j, s in enumerate(perm):
        a = out[cu[s]:cu[s + 1]].view(torch.int16)
        b = out2[cu2[j]:cu2[j + 1]].view(torch.int16)
        assert torch.equal(a, b), f"sequence {s}"
        assert torch.equal(lse[:, cu[s]:cu[s + 1]].contiguous().view(torch.int32),
                           lse2[:, cu2[j]:cu2[j + 1]].contiguous().view(torch.int32))


def test_forward_is_deterministic():
    import torch
    w = wl.dense_bf16(batch=2, seqlen=1024, heads=4)
    t = to_device(w)
    a = run_fwd(w, t)
    b = run_fwd(w, t)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_unusual_scales(scale):
    w = wl.random_workload(15, [7, 20], [90, 150], 2, 1, 64, "f32", wl.MASK_CAUSAL_BOTTOM_RIGHT,
                           name="scale", scale=scale)
    ref_o, ref_l = _oracle(w)
    for path in (PREFILL, SPLITK):
        out, lse = run_fwd(w, path=path)
        check_fwd(w, out, lse, ref_o, ref_l, f"scale {scale} path {path}")


@pytest.mark.parametrize("scale", [50.0, 1e-3, -2.0])
def test_extreme_scales_splitk_bf16(scale):
    """The bf16 split-K decode forward at extreme scales (GQA 4:2, 1 to 16 queries over 2 to
    3000 keys, bottom-right): scale 50 gives logit gaps of hundreds, so a chunk's running
    offset moves at almost every 128-key stage and the log-sum-exp merge of the chunks
    combines partials whose maxima differ by hundreds; 1e-3 gives nearly uniform weights.
    Automatic and 3 splits, against the oracle at the standard bounds."""
    w = wl.random_workload((67, int(abs(scale) * 1000)), [1, 4, 16, 3], [3000, 129, 1000, 2],
                           8, 2, 128, "bf16", wl.MASK_CAUSAL_BOTTOM_RIGHT, name="scale-splitk",
                           scale=scale)
    with np.errstate(over="ignore"):
        ref_o, ref_l = _oracle(w)
    for splits in (0, 3):
        out, lse = run_fwd(w, path=SPLITK, num_splits=splits)
        check_fwd(w, out, lse, ref_o, ref_l, f"split-K scale {scale} splits {splits}")


# ----------------------------------------------------------------------------------------
# the named workloads at full size (oracle on sampled sequences / heads)
# ----------------------------------------------------------------------------------------

def test_dense_bf16_full_size():
    """B=4, H=16, N=2048, d=128, causal top-left: O and LSE of every (sequence, head) slice
    against the oracle (slices evaluated in parallel CPU workers)."""
    import oracle_pool as op
    w = wl.dense_bf16()
    out, lse = run_fwd(w)
    o, l = to_np(out), to_np(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    tasks = [(op.fwd_slice, (s, list(range(h0, h0 + 4)))) for s in range(4) for h0 in range(0, 16, 4)]
    print(f"dense full size: {len(tasks)} oracle tasks", flush=True)
    for (_, (s, heads)), (ro, rl) in zip(tasks, op.run("dense_bf16", {}, tasks)):
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        assert_close(o[rows][:, heads], ro, *BF16_TOL, f"dense O s{s} h{heads}")
        assert_close(l[heads][:, rows], rl, LSE_TOL, 0.0, f"dense LSE s{s} h{heads}")


def test_ragged_gqa_full_size():
    """16384 packed tokens, ragged lengths incl. 63/64/65/127/128/129, Hq=32, Hkv=8, V offset
    per sequence: every sequence on one query head of each of the 8 GQA groups, and all 32
    heads of the three longest sequences, against the oracle ("Causal Mask and Ragged
    Sequence Layouts", fifth section: packed against per-sequence with distinct value
    ranges)."""
    import oracle_pool as op
    w = wl.ragged_gqa()
    out, lse = run_fwd(w)
    o, l = to_np(out), to_np(lse)
    assert np.all(np.isfinite(o))
    lens = np.diff(w.cu_q)
    longest = [int(x) for x in np.argsort(lens)[-3:]]
    tasks = []
    for s in range(w.num_seqs):
        if s in longest:
            tasks += [(op.fwd_slice, (s, list(range(h0, h0 + 8)))) for h0 in range(0, 32, 8)]
        else:
            tasks.append((op.fwd_slice, (s, [4 * g + g % 4 for g in range(8)])))
    print(f"ragged full size: {w.num_seqs} sequences, {len(tasks)} oracle tasks", flush=True)
    for (_, (s, heads)), (ro, rl) in zip(tasks, op.run("ragged_gqa", {}, tasks)):
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        assert_close(o[rows][:, heads], ro, *BF16_TOL, f"ragged O s{s} h{heads}")
        assert_close(l[heads][:, rows], rl, LSE_TOL, 0.0, f"ragged LSE s{s} h{heads}")


@pytest.mark.parametrize("nq", [1, 4, 16])
def test_decode_full_size(nq):
    """B=16, Hq=32, Hkv=8, d=128, Nk=32768, bottom-right: every sequence, each on one K/V
    head group (all of the group's query heads), against the oracle; the auto plan must
    pick the split-K path."""
    import exact_attention_tiled_amd as eat
    import oracle_pool as op
    w = wl.decode(nq)
    t = to_device(w)
    plan = eat.attn_describe_plan(t["q"], t["k"], t["cu_q"], w.max_seqlen_q, w.max_seqlen_k,
                                  w.mask_mode)
    assert plan.startswith("path=splitk"), plan
    out, lse = run_fwd(w, t)
    o, l = to_np(out), to_np(lse)
    del t
    tasks = [(op.fwd_slice, (s, list(range(4 * (s % 8), 4 * (s % 8) + 4)))) for s in range(16)]
    # two workers: each regenerates the 2 GiB cache, and the slices themselves are small
    for (_, (s, heads)), (ro, rl) in zip(tasks, op.run("decode", {"nq": nq}, tasks, procs=2)):
        rows = slice(int(w.cu_q[s]), int(w.cu_q[s + 1]))
        assert_close(o[rows][:, heads], ro, *BF16_TOL, f"decode O s{s} h{heads}")
        assert_close(l[heads][:, rows], rl, LSE_TOL, 0.0, f"decode LSE s{s} h{heads}")
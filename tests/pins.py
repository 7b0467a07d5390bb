"""Checks that pin an attention implementation to facts fixed by the pages and by mathematics.

Each check takes the implementation under test as a function
    fwd(q, k, v, cu_q, cu_k, scale, mode, window) -> (O [Tq,Hq,d], LSE [Hq,Tq])
or  bwd(q, k, v, dout, cu_q, cu_k, scale, mode, window) -> (dQ, dK, dV)
working in float64, and raises AssertionError when the fact does not hold. The same checks
run against the fp64 oracle (where every one must pass) and against deliberately broken
variants of a tiled model (where each mutant must fail at least one), so a plausible
mistake in the oracle would be caught by them.

The expected values here never come from the function under test: they are closed forms,
hand-written fixtures under tests/golden/, invariants relating two calls, finite
differences, or torch's CPU float64 scaled_dot_product_attention.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

NONE, TL, BR = 0, 1, 2


# ----------------------------------------------------------------------------------------
# fixtures
# ----------------------------------------------------------------------------------------

def load_golden_masks():
    cases = []
    cur = None
    with open(os.path.join(GOLDEN, "masks.txt")) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case "):
                cur = {"name": line.split()[1], "rows": []}
            elif line.startswith("cu_q "):
                cur["cu_q"] = [int(x) for x in line.split()[1:]]
            elif line.startswith("cu_k "):
                cur["cu_k"] = [int(x) for x in line.split()[1:]]
            elif line.startswith("mode "):
                cur["mode"] = int(line.split()[1])
            elif line.startswith("window "):
                cur["window"] = int(line.split()[1])
            elif line == "end":
                cur["mask"] = np.array([[c == "1" for c in r] for r in cur["rows"]], dtype=bool)
                if cur["mask"].size == 0:
                    cur["mask"] = np.zeros((cur["cu_q"][-1], cur["cu_k"][-1]), dtype=bool)
                cases.append(cur)
                cur = None
            else:
                cur["rows"].append(line)
    return cases


def load_two_tile_recurrence():
    rows = []
    with open(os.path.join(GOLDEN, "two_tile_recurrence.txt")) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            v1, v2, ok, no_l, no_acc = line.split()
            rows.append({"v": (int(v1), int(v2)), "correct": Fraction(ok),
                         "no_l_rescale": Fraction(no_l), "no_acc_rescale": Fraction(no_acc)})
    return rows


def cu_of(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


def allowed_interval(pos_q, len_q, len_k, mode, window):
    """Closed-form allowed key-position interval [lo, hi] (empty when lo > hi).

    Written as an interval, not as the oracle's pairwise predicate: NONE keeps every key;
    top-left ends at the query position; bottom-right ends at pos_q + Nk - Nq; a window of
    width W starts W - 1 positions before the end.
    """
    if mode == NONE:
        return 0, len_k - 1
    end = pos_q if mode == TL else pos_q + len_k - len_q
    hi = min(end, len_k - 1)
    lo = 0 if window <= 0 else max(0, end - window + 1)
    return lo, hi


def row_count_closed_form(pos_q, len_q, len_k, mode, window):
    lo, hi = allowed_interval(pos_q, len_q, len_k, mode, window)
    return max(0, hi - lo + 1)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    bad = ~(diff <= tol * (1.0 + np.abs(b)))
    assert not bad.any(), f"{what}: max diff {np.nanmax(diff)} at {np.argwhere(bad)[:5].tolist()}"


# ----------------------------------------------------------------------------------------
# forward checks
# ----------------------------------------------------------------------------------------

def check_golden_masks(fwd):
    """Uniform logits (q = 0) give the average of the allowed values, ln(count) as LSE, and
    zero output / -inf LSE for empty rows, on every hand-written mask fixture.
    ("Attention Algorithm Error and Complexity Tests", first section: uniform logits test
    the allowed-key average; "Causal Mask and Ragged Sequence Layouts", fourth section.)"""
    rng = np.random.default_rng(100)
    for case in load_golden_masks():
        cu_q, cu_k = np.array(case["cu_q"]), np.array(case["cu_k"])
        tq, tk = int(cu_q[-1]), int(cu_k[-1])
        hq, hkv, d = 2, 1, 3
        q = np.zeros((tq, hq, d))
        k = _rand(rng, tk, hkv, d)
        v = _rand(rng, tk, hkv, d) + 5.0 * np.arange(tk)[:, None, None]
        o, lse = fwd(q, k, v, cu_q, cu_k, 0.5, case["mode"], case["window"])
        m = case["mask"]
        for t in range(tq):
            n = int(m[t].sum())
            for h in range(hq):
                if n == 0:
                    assert np.all(o[t, h] == 0.0), (case["name"], t, h, o[t, h])
                    assert lse[h, t] == -np.inf, (case["name"], t, h, lse[h, t])
                else:
                    want = v[m[t], 0, :].mean(axis=0)
                    _close(o[t, h], want, 1e-12, f"{case['name']} O row {t}")
                    _close(lse[h, t], math.log(n), 1e-12, f"{case['name']} LSE row {t}")


def check_uniform_brute_force(fwd, seed=101, trials=60):
    """Uniform logits over random packs of short sequences (lengths 0..5, all modes, several
    windows): output is the allowed-key average with the allowed set from the closed-form
    interval; LSE = ln(count)."""
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        nseq = int(rng.integers(1, 4))
        lq = [int(x) for x in rng.integers(0, 6, nseq)]
        lk = [int(x) for x in rng.integers(0, 6, nseq)]
        mode = int(rng.integers(0, 3))
        window = 0 if mode == NONE else int(rng.choice([0, 1, 2, 3, 7]))
        cu_q, cu_k = cu_of(lq), cu_of(lk)
        tq, tk = int(cu_q[-1]), int(cu_k[-1])
        q = np.zeros((tq, 2, 2))
        v = _rand(rng, tk, 1, 2) + 7.0 * np.arange(tk)[:, None, None]
        k = _rand(rng, tk, 1, 2)
        o, lse = fwd(q, k, v, cu_q, cu_k, 0.3, mode, window)
        for s in range(nseq):
            for i in range(lq[s]):
                t = int(cu_q[s]) + i
                lo, hi = allowed_interval(i, lq[s], lk[s], mode, window)
                n = max(0, hi - lo + 1)
                if n == 0:
                    assert np.all(o[t] == 0.0) and np.all(lse[:, t] == -np.inf), (trial, s, i)
                else:
                    keys = int(cu_k[s]) + np.arange(lo, hi + 1)
                    for h in range(2):
                        _close(o[t, h], v[keys, 0].mean(axis=0), 1e-12, f"trial {trial} O")
                        _close(lse[h, t], math.log(n), 1e-12, f"trial {trial} LSE")


def check_dominant_score(fwd):
    """A single dominant score: logits are exactly {a*scale at key j*, 0 elsewhere}, so
    O = (e^x v_j* + sum of the other v) / (e^x + n - 1) with x = a*scale. x = 1024 overflows
    an unnormalised exponential and must still give v_j* ("Attention Algorithm Error and
    Complexity Tests", first section: a single dominant score tests stable normalisation)."""
    rng = np.random.default_rng(102)
    n, d = 6, 4
    for x, jstar in ((32.0, 2), (1024.0, 4), (-3.0, 0)):
        scale = 0.25
        a = x / scale
        q = np.zeros((1, 1, d)); q[0, 0, 0] = a
        k = np.zeros((n, 1, d)); k[:, 0, 1:] = _rand(rng, n, d - 1); k[jstar, 0, :] = 0.0
        k[jstar, 0, 0] = 1.0
        v = _rand(rng, n, 1, d)
        o, lse = fwd(q, k, v, np.array([0, 1]), np.array([0, n]), scale, NONE, 0)
        others = [j for j in range(n) if j != jstar]
        if x > 700:   # e^x overflows float64: take the limit exactly
            want = v[jstar, 0]
            want_lse = x + math.log1p((n - 1) * math.exp(-x))
        else:
            w = math.exp(x)
            want = (w * v[jstar, 0] + v[others, 0].sum(axis=0)) / (w + n - 1)
            want_lse = math.log(w + n - 1)
        _close(o[0, 0], want, 1e-12, f"dominant x={x}")
        _close(lse[0, 0], want_lse, 1e-12, f"dominant lse x={x}")


def check_masked_dominant_score(fwd):
    """A dominant score on a *disallowed* key (a future key, a key of another packed sequence,
    a key beyond the window) must not enter the maximum or the denominator: the allowed
    logits are all 0, so O is exactly the mean of the allowed values, even when the masked
    logit is 1024 ("Attention Algorithm Error and Complexity Tests", first section;
    "Causal Mask and Ragged Sequence Layouts", second section)."""
    rng = np.random.default_rng(103)
    d, scale = 4, 0.5
    big = 1024.0 / scale
    # one query row at position 2 of a 4-token sequence (TL), window 2; a second sequence
    # follows in the pack.
    cu_q, cu_k = np.array([0, 4, 6]), np.array([0, 4, 6])
    q = np.zeros((6, 1, d)); q[2, 0, 0] = big
    k = np.zeros((6, 1, d)); k[:, 0, 1:] = _rand(rng, 6, d - 1)
    v = _rand(rng, 6, 1, d)
    for masked_key in (3, 4, 0):      # future key, other sequence, beyond the window
        kk = k.copy(); kk[masked_key, 0, 0] = 1.0
        o, lse = fwd(q, kk, v, cu_q, cu_k, scale, TL, 2)
        want = v[[1, 2], 0].mean(axis=0)
        _close(o[2, 0], want, 1e-12, f"masked dominant key {masked_key}")
        _close(lse[0, 2], math.log(2.0), 1e-12, f"masked dominant lse key {masked_key}")


def _random_pack(rng, lq, lk, hq, hkv, d, voff=True):
    cu_q, cu_k = cu_of(lq), cu_of(lk)
    q = _rand(rng, int(cu_q[-1]), hq, d)
    k = _rand(rng, int(cu_k[-1]), hkv, d)
    v = _rand(rng, int(cu_k[-1]), hkv, d)
    if voff:
        for s in range(len(lk)):
            v[cu_k[s]:cu_k[s + 1]] = v[cu_k[s]:cu_k[s + 1]] * (s + 1) + 10 * s
    return q, k, v, cu_q, cu_k


def check_shift_invariance(fwd):
    """Adding w to every key of one (sequence, K/V head) adds the constant scale*q_t.w to all
    logits of each row using that head: O is unchanged and LSE moves by that constant
    ("Attention Algorithm Error and Complexity Tests", third section)."""
    rng = np.random.default_rng(104)
    lq, lk = [5, 3, 4], [5, 6, 2]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 4, 2, 3)
    scale = 0.7
    for mode, window in ((TL, 0), (BR, 0), (BR, 2), (NONE, 0)):
        o, lse = fwd(q, k, v, cu_q, cu_k, scale, mode, window)
        w = _rand(rng, 3)
        s, g = 1, 1
        k2 = k.copy(); k2[cu_k[s]:cu_k[s + 1], g, :] += w
        o2, lse2 = fwd(q, k2, v, cu_q, cu_k, scale, mode, window)
        _close(o2, o, 1e-12, "shift O")
        lse_want = lse.copy()
        for h in (2, 3):   # query heads of K/V head 1
            for t in range(cu_q[s], cu_q[s + 1]):
                if np.isfinite(lse[h, t]):
                    lse_want[h, t] += scale * float(q[t, h] @ w)
        _close(lse2, lse_want, 1e-12, "shift LSE")


def check_key_permutation(fwd):
    """Without a causal relation, permuting the keys and values of a sequence together leaves
    every output unchanged ("Attention Algorithm Error and Complexity Tests", third
    section)."""
    rng = np.random.default_rng(105)
    lq, lk = [4, 3], [6, 5]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 2, 2, 3)
    o, lse = fwd(q, k, v, cu_q, cu_k, 0.6, NONE, 0)
    perm = np.arange(k.shape[0])
    perm[cu_k[1]:cu_k[2]] = cu_k[1] + rng.permutation(lk[1])
    perm[cu_k[0]:cu_k[1]] = rng.permutation(lk[0])
    o2, lse2 = fwd(q, k[perm], v[perm], cu_q, cu_k, 0.6, NONE, 0)
    _close(o2, o, 1e-12, "perm O")
    _close(lse2, lse, 1e-12, "perm LSE")


def check_gqa_matches_repeat(fwd):
    """Shared-KV heads equal an MHA run on explicitly repeated K/V with the consecutive
    grouping h -> h // (Hq/Hkv) ("Attention Algorithm Error and Complexity Tests", third
    section)."""
    rng = np.random.default_rng(106)
    lq, lk = [4, 6], [7, 3]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 6, 2, 3)
    for mode, window in ((BR, 0), (TL, 2), (NONE, 0)):
        o, lse = fwd(q, k, v, cu_q, cu_k, 0.4, mode, window)
        o2, lse2 = fwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), cu_q, cu_k,
                       0.4, mode, window)
        _close(o, o2, 1e-12, "gqa O")
        _close(lse, lse2, 1e-12, "gqa LSE")


def check_packing_matches_separate(fwd):
    """A packed call reproduces one call per sequence (each with its own one-sequence
    cumulative array), so no global offset can act as a position ("Causal Mask and Ragged
    Sequence Layouts", first and second sections)."""
    rng = np.random.default_rng(107)
    lq, lk = [3, 5, 1, 4], [6, 5, 0, 2]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 2, 1, 3)
    for mode, window in ((TL, 0), (BR, 0), (BR, 3), (NONE, 0)):
        o, lse = fwd(q, k, v, cu_q, cu_k, 0.5, mode, window)
        for s in range(len(lq)):
            qa, qb, ka, kb = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
            os_, ls_ = fwd(q[qa:qb], k[ka:kb], v[ka:kb], np.array([0, qb - qa]),
                           np.array([0, kb - ka]), 0.5, mode, window)
            _close(o[qa:qb], os_, 1e-12, f"pack O seq {s}")
            _close(lse[:, qa:qb], ls_, 1e-12, f"pack LSE seq {s}")


def torch_sdpa_reference(q, k, v, cu_q, cu_k, scale, mode, window):
    """torch CPU float64 scaled_dot_product_attention per sequence with an explicit boolean
    mask built from positions (interval form) and K/V repeated to all query heads. torch's
    own is_causal flag is never used: it is top-left only ("Causal Mask and Ragged Sequence
    Layouts", fourth section)."""
    import torch
    tq, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    o = np.zeros((tq, hq, v.shape[2]))
    lse = np.full((hq, tq), -np.inf)
    for s in range(len(cu_q) - 1):
        qa, qb, ka, kb = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        lqs, lks = qb - qa, kb - ka
        if lqs == 0:
            continue
        m = np.zeros((lqs, lks), dtype=bool)
        for i in range(lqs):
            lo, hi = allowed_interval(i, lqs, lks, mode, window)
            if hi >= lo:
                m[i, lo:hi + 1] = True
        if lks == 0:
            continue
        tq_ = torch.from_numpy(q[qa:qb]).permute(1, 0, 2)[None]
        tk_ = torch.from_numpy(np.repeat(k[ka:kb], grp, axis=1)).permute(1, 0, 2)[None]
        tv_ = torch.from_numpy(np.repeat(v[ka:kb], grp, axis=1)).permute(1, 0, 2)[None]
        out = torch.nn.functional.scaled_dot_product_attention(
            tq_, tk_, tv_, attn_mask=torch.from_numpy(m), scale=scale)
        o[qa:qb] = out[0].permute(1, 0, 2).numpy()
        logits = torch.einsum("hqd,hkd->hqk", tq_[0], tk_[0]) * scale
        logits = logits.masked_fill(~torch.from_numpy(m), float("-inf"))
        lse[:, qa:qb] = torch.logsumexp(logits, dim=-1).numpy()
    return o, lse


def check_torch_sdpa(fwd):
    """Agreement with torch's CPU float64 SDPA (a separate implementation of the same
    operator) on random packs in every mode, with GQA."""
    rng = np.random.default_rng(108)
    for lq, lk in (([5, 3, 7], [5, 6, 4]), ([1, 4], [9, 2]), ([6], [6])):
        q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 4, 2, 5)
        for mode, window in ((NONE, 0), (TL, 0), (BR, 0), (TL, 3), (BR, 2)):
            o, lse = fwd(q, k, v, cu_q, cu_k, 0.45, mode, window)
            o2, lse2 = torch_sdpa_reference(q, k, v, cu_q, cu_k, 0.45, mode, window)
            _close(o, o2, 1e-10, f"torch O mode {mode} w {window}")
            _close(lse, lse2, 1e-10, f"torch LSE mode {mode} w {window}")


FWD_CHECKS = [check_golden_masks, check_uniform_brute_force, check_dominant_score,
              check_masked_dominant_score, check_shift_invariance, check_key_permutation,
              check_gqa_matches_repeat, check_packing_matches_separate, check_torch_sdpa]


# ----------------------------------------------------------------------------------------
# backward checks
# ----------------------------------------------------------------------------------------

def check_finite_differences(fwd, bwd):
    """Central differences of L = sum(R * O) on tiny smooth cases against the analytic
    gradients, for every input scalar. Masks depend only on indices, so no step crosses a
    mask change ("Attention Algorithm Error and Complexity Tests", fourth section)."""
    rng = np.random.default_rng(109)
    lq, lk = [3, 4, 2], [5, 4, 0]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 4, 2, 3, voff=False)
    r = _rand(rng, *q.shape)
    h = 1e-6
    for mode, window in ((TL, 0), (BR, 0), (BR, 2), (NONE, 0)):
        dq, dk, dv = bwd(q, k, v, r, cu_q, cu_k, 0.8, mode, window)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args = {"q": q, "k": k, "v": v}
                args[name] = xp
                lp = float((fwd(args["q"], args["k"], args["v"], cu_q, cu_k, 0.8, mode,
                                window)[0] * r).sum())
                args[name] = xm
                lm = float((fwd(args["q"], args["k"], args["v"], cu_q, cu_k, 0.8, mode,
                                window)[0] * r).sum())
                fd[idx] = (lp - lm) / (2 * h)
            err = np.abs(fd - g)
            assert np.all(err <= 1e-7 * (1 + np.abs(g))), \
                f"FD d{name} mode {mode} w {window}: max err {err.max()}"


def check_gqa_bwd_sums(bwd):
    """GQA gradients equal the MHA gradients on repeated K/V with dK, dV summed over each
    group ("Attention Algorithm Error and Complexity Tests", third section)."""
    rng = np.random.default_rng(110)
    lq, lk = [4, 5], [6, 3]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 6, 2, 3)
    do = _rand(rng, *q.shape)
    for mode, window in ((BR, 0), (TL, 2), (NONE, 0)):
        dq, dk, dv = bwd(q, k, v, do, cu_q, cu_k, 0.3, mode, window)
        dq2, dk2, dv2 = bwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), do,
                            cu_q, cu_k, 0.3, mode, window)
        _close(dq, dq2, 1e-12, "gqa dQ")
        _close(dk, dk2.reshape(dk.shape[0], 2, 3, -1).sum(axis=2), 1e-12, "gqa dK")
        _close(dv, dv2.reshape(dv.shape[0], 2, 3, -1).sum(axis=2), 1e-12, "gqa dV")


def check_shift_bwd(bwd):
    """Under the key shift of the forward check, dQ, dK and dV are unchanged: every row of
    dS sums to zero, so the shift adds nothing to dQ."""
    rng = np.random.default_rng(111)
    lq, lk = [5, 3], [5, 6]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 2, 1, 3)
    do = _rand(rng, *q.shape)
    for mode, window in ((TL, 0), (BR, 3)):
        g1 = bwd(q, k, v, do, cu_q, cu_k, 0.5, mode, window)
        k2 = k.copy(); k2[cu_k[1]:cu_k[2], 0, :] += _rand(rng, 3)
        g2 = bwd(q, k2, v, do, cu_q, cu_k, 0.5, mode, window)
        for a, b, nm in zip(g1, g2, ("dQ", "dK", "dV")):
            _close(b, a, 1e-11, f"shift {nm}")


def check_torch_autograd(bwd):
    """Agreement with torch autograd through CPU float64 SDPA on repeated K/V (gradients of
    repeated heads summed back), every mode, with empty rows present."""
    import torch
    rng = np.random.default_rng(112)
    lq, lk = [5, 4, 3], [3, 6, 4]
    q, k, v, cu_q, cu_k = _random_pack(rng, lq, lk, 4, 2, 3)
    do = _rand(rng, *q.shape)
    for mode, window in ((BR, 0), (TL, 0), (NONE, 0), (BR, 2)):
        dq, dk, dv = bwd(q, k, v, do, cu_q, cu_k, 0.55, mode, window)
        tq_ = torch.tensor(q, requires_grad=True)
        tk_ = torch.tensor(k, requires_grad=True)
        tv_ = torch.tensor(v, requires_grad=True)
        outs = []
        for s in range(len(lq)):
            qa, qb, ka, kb = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
            m = np.zeros((qb - qa, kb - ka), dtype=bool)
            for i in range(qb - qa):
                lo, hi = allowed_interval(i, qb - qa, kb - ka, mode, window)
                if hi >= lo:
                    m[i, lo:hi + 1] = True
            qq = tq_[qa:qb].permute(1, 0, 2)[None]
            kk = tk_[ka:kb].repeat_interleave(2, dim=1).permute(1, 0, 2)[None]
            vv = tv_[ka:kb].repeat_interleave(2, dim=1).permute(1, 0, 2)[None]
            out = torch.nn.functional.scaled_dot_product_attention(
                qq, kk, vv, attn_mask=torch.from_numpy(m), scale=0.55)
            outs.append(out[0].permute(1, 0, 2))
        loss = (torch.cat(outs) * torch.from_numpy(do)).sum()
        loss.backward()
        _close(dq, tq_.grad.numpy(), 1e-10, f"autograd dQ mode {mode}")
        _close(dk, tk_.grad.numpy(), 1e-10, f"autograd dK mode {mode}")
        _close(dv, tv_.grad.numpy(), 1e-10, f"autograd dV mode {mode}")


BWD_CHECKS = [check_gqa_bwd_sums, check_shift_bwd, check_torch_autograd]

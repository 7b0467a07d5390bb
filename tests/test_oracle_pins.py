"""Pins of the fp64 oracle against facts the pages and mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import pins
from workloads import round_to_bf16


def ofwd(q, k, v, cu_q, cu_k, scale, mode, window):
    return oracle.attention(q, k, v, cu_q, cu_k, scale, mode, window)


def obwd(q, k, v, do, cu_q, cu_k, scale, mode, window):
    return oracle.attention_bwd(q, k, v, do, cu_q, cu_k, scale, mode, window)


def ofwd_explicit(q, k, v, cu_q, cu_k, scale, mode, window):
    return oracle.attention_explicit(q, k, v, oracle.explicit_mask(cu_q, cu_k, mode, window),
                                     scale)


def obwd_explicit(q, k, v, do, cu_q, cu_k, scale, mode, window):
    """The explicit-mask backward over the whole pack (one [Tq, Tk] mask for every head),
    fed the mask that sequence ids and positions give."""
    return oracle.attention_explicit_bwd(q, k, v, do,
                                         oracle.explicit_mask(cu_q, cu_k, mode, window), scale)


@pytest.mark.parametrize("check", pins.FWD_CHECKS, ids=lambda f: f.__name__)
def test_oracle_forward_pins(check):
    check(ofwd)


@pytest.mark.parametrize("check", pins.BWD_CHECKS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("bwd", [obwd, obwd_explicit], ids=["per_sequence", "explicit_mask"])
def test_oracle_backward_pins(check, bwd):
    check(bwd)


@pytest.mark.parametrize("fwd,bwd", [(ofwd, obwd), (ofwd_explicit, obwd_explicit)],
                         ids=["per_sequence", "explicit_mask"])
def test_oracle_finite_differences(fwd, bwd):
    pins.check_finite_differences(fwd, bwd)


def test_explicit_mask_matches_golden():
    for case in pins.load_golden_masks():
        m = oracle.explicit_mask(case["cu_q"], case["cu_k"], case["mode"], case["window"])
        assert m.shape == case["mask"].shape, case["name"]
        assert np.array_equal(m, case["mask"]), case["name"]


def test_mask_row_counts_brute_force():
    """Exhaustive over 1-3 sequences with lengths 0..5, every mode and several windows:
    oracle mask row counts equal the closed forms, and no pair crosses sequences."""
    for nseq in (1, 2, 3):
        rng = np.random.default_rng(nseq)
        combos = [(a, b) for a in range(6) for b in range(6)]
        for trial in range(40 if nseq > 1 else 36):
            if nseq == 1:
                lq, lk = [combos[trial][0]], [combos[trial][1]]
            else:
                lq = [int(x) for x in rng.integers(0, 6, nseq)]
                lk = [int(x) for x in rng.integers(0, 6, nseq)]
            cu_q, cu_k = pins.cu_of(lq), pins.cu_of(lk)
            for mode in (0, 1, 2):
                for window in ((0,) if mode == 0 else (0, 1, 2, 3, 7)):
                    m = oracle.explicit_mask(cu_q, cu_k, mode, window)
                    for s in range(nseq):
                        for i in range(lq[s]):
                            t = cu_q[s] + i
                            want = pins.row_count_closed_form(i, lq[s], lk[s], mode, window)
                            assert m[t].sum() == want, (lq, lk, mode, window, s, i)
                            outside = np.ones(m.shape[1], bool)
                            outside[cu_k[s]:cu_k[s + 1]] = False
                            assert not m[t, outside].any()


def test_packing_matches_per_sequence_oracle():
    """The packed evaluation (global sequence ids) equals the purely local per-sequence one."""
    rng = np.random.default_rng(7)
    lq, lk = [5, 0, 9, 3], [4, 2, 9, 7]
    q, k, v, cu_q, cu_k = pins._random_pack(rng, lq, lk, 4, 2, 3)
    for mode, window in ((1, 0), (2, 0), (2, 4), (0, 0)):
        a = oracle.attention(q, k, v, cu_q, cu_k, 0.3, mode, window)
        b = oracle.attention_per_sequence(q, k, v, cu_q, cu_k, 0.3, mode, window)
        pins._close(a[0], b[0], 1e-13, "O")
        pins._close(a[1], b[1], 1e-13, "LSE")


def test_padded_layout_matches_packed():
    """A padded [B, Lmax] layout whose mask combines token validity with the causal relation
    gives the packed results on valid tokens ("Causal Mask and Ragged Sequence Layouts",
    second section: padding is an exclusion rule)."""
    rng = np.random.default_rng(8)
    lens = [5, 2, 7]
    lmax = max(lens)
    q, k, v, cu_q, cu_k = pins._random_pack(rng, lens, lens, 2, 1, 4)
    o_pack, lse_pack = oracle.attention(q, k, v, cu_q, cu_k, 0.5, 1, 0)
    for b, L in enumerate(lens):
        # padded sequence: valid tokens then garbage padding
        qp = rng.standard_normal((lmax, 2, 4)) * 100
        kp = rng.standard_normal((lmax, 1, 4)) * 100
        vp = rng.standard_normal((lmax, 1, 4)) * 100
        qp[:L], kp[:L], vp[:L] = q[cu_q[b]:cu_q[b + 1]], k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]]
        valid = np.arange(lmax) < L
        causal = np.arange(lmax)[None, :] <= np.arange(lmax)[:, None]
        mask = causal & valid[None, :] & valid[:, None]
        o, lse = oracle.attention_explicit(qp, kp, vp, mask, 0.5)
        pins._close(o[:L], o_pack[cu_q[b]:cu_q[b + 1]], 1e-13, "padded O")
        pins._close(lse[:, :L], lse_pack[:, cu_q[b]:cu_q[b + 1]], 1e-13, "padded LSE")


def test_causal_permutation_with_explicit_mask():
    """With a causal relation, permuting keys/values is only an invariance when the mask
    columns are permuted too ("Attention Algorithm Error and Complexity Tests", third
    section: causal relations must be transformed consistently)."""
    rng = np.random.default_rng(9)
    q, k, v, cu_q, cu_k = pins._random_pack(rng, [6], [8], 2, 2, 3)
    m = oracle.explicit_mask(cu_q, cu_k, 2, 0)
    o, lse = oracle.attention_explicit(q, k, v, m, 0.7)
    perm = rng.permutation(8)
    o2, lse2 = oracle.attention_explicit(q, k[perm], v[perm], m[:, perm], 0.7)
    pins._close(o2, o, 1e-13, "O")
    pins._close(lse2, lse, 1e-13, "LSE")
    o3, _ = oracle.attention_explicit(q, k[perm], v[perm], m, 0.7)
    assert np.abs(o3 - o).max() > 1e-3   # permuting without the mask changes the operator


def test_causal_permutation_backward_with_explicit_mask():
    """The same consistent permutation of keys, values and mask columns leaves dQ unchanged
    and permutes dK and dV the same way (the backward rebuilds the permuted mask: "Causal
    Mask and Ragged Sequence Layouts", sixth section)."""
    rng = np.random.default_rng(19)
    q, k, v, cu_q, cu_k = pins._random_pack(rng, [6], [8], 4, 2, 3)
    do = rng.standard_normal(q.shape)
    for mode, window in ((2, 0), (1, 3)):
        m = oracle.explicit_mask(cu_q, cu_k, mode, window)
        dq, dk, dv = oracle.attention_explicit_bwd(q, k, v, do, m, 0.7)
        perm = rng.permutation(8)
        dq2, dk2, dv2 = oracle.attention_explicit_bwd(q, k[perm], v[perm], do, m[:, perm], 0.7)
        pins._close(dq2, dq, 1e-13, "permuted dQ")
        pins._close(dk2, dk[perm], 1e-13, "permuted dK")
        pins._close(dv2, dv[perm], 1e-13, "permuted dV")
        dq3, _, _ = oracle.attention_explicit_bwd(q, k[perm], v[perm], do, m, 0.7)
        assert np.abs(dq3 - dq).max() > 1e-3   # without the mask columns it is another operator


def test_split_key_ranges_combine_to_full():
    """Attention over disjoint key ranges, combined by log-sum-exp, equals the unsplit result,
    including chunks that are wholly masked and rows that are empty (Nq > Nk)."""
    rng = np.random.default_rng(10)
    for lq, lk, mode, window in (([4, 4], [13, 13], 2, 0), ([6, 6], [3, 3], 2, 0),
                                 ([3, 5], [11, 9], 1, 4), ([2, 2], [10, 10], 0, 0)):
        q, k, v, cu_q, cu_k = pins._random_pack(rng, lq, lk, 4, 2, 3)
        full = oracle.attention(q, k, v, cu_q, cu_k, 0.6, mode, window)
        bounds = [0, 2, 5, 9, 100]
        parts = [oracle.attention_key_range(q, k, v, cu_q, cu_k, 0.6, mode, window, a, b)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        comb = oracle.lse_combine(parts)
        pins._close(comb[0], full[0], 1e-12, "split O")
        pins._close(comb[1], full[1], 1e-12, "split LSE")


def test_lse_units_natural_log_of_scaled_logits():
    """LSE is ln(sum exp(scale * q.k)) over allowed keys, checked on a two-key row."""
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[2.0, 0.0]], [[0.0, 1.0]]])
    v = np.zeros((2, 1, 2))
    _, lse = oracle.attention(q, k, v, [0, 1], [0, 2], 0.5, 0, 0)
    assert abs(lse[0, 0] - math.log(math.e + 1.0)) < 1e-15


def test_empty_batch_and_zero_lengths():
    q = np.zeros((0, 2, 4)); k = np.zeros((0, 1, 4)); v = np.zeros((0, 1, 4))
    o, lse = oracle.attention(q, k, v, [0], [0], 0.5, 1, 0)
    assert o.shape == (0, 2, 4) and lse.shape == (2, 0)
    dq, dk, dv = oracle.attention_bwd(q, k, v, q, [0], [0], 0.5, 1, 0)
    assert dq.shape == q.shape and dk.shape == k.shape


def test_restricted_evaluation_matches_full():
    """Evaluating a subset of sequences / heads gives the same numbers as the full call."""
    rng = np.random.default_rng(11)
    q, k, v, cu_q, cu_k = pins._random_pack(rng, [4, 6, 3], [5, 6, 3], 4, 2, 3)
    do = rng.standard_normal(q.shape)
    o, lse = oracle.attention(q, k, v, cu_q, cu_k, 0.5, 2, 0)
    o2, lse2 = oracle.attention(q, k, v, cu_q, cu_k, 0.5, 2, 0, seqs=[1], heads=[3])
    sl = slice(cu_q[1], cu_q[2])
    assert np.array_equal(o2[sl, 3], o[sl, 3]) and np.array_equal(lse2[3, sl], lse[3, sl])
    g = oracle.attention_bwd(q, k, v, do, cu_q, cu_k, 0.5, 2, 0)
    g2 = oracle.attention_bwd(q, k, v, do, cu_q, cu_k, 0.5, 2, 0, seqs=[1], kv_heads=[1])
    assert np.allclose(g2[0][sl, 2:4], g[0][sl, 2:4], rtol=0, atol=1e-14)
    ks = slice(cu_k[1], cu_k[2])
    assert np.allclose(g2[1][ks, 1], g[1][ks, 1], rtol=0, atol=1e-14)
    assert np.allclose(g2[2][ks, 1], g[2][ks, 1], rtol=0, atol=1e-14)


def test_bf16_rounding_matches_torch():
    """The input generator's round-to-nearest-even bf16 cast equals torch's."""
    import torch
    x = np.random.default_rng(12).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # ties
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)

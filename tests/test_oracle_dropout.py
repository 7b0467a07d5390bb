"""Pins of the oracle's dropout against what the generator's publication, the pages and the
mathematics fix (CPU only).

Dropout is validated separately from the deterministic operator ("Attention Algorithm
Error and Complexity Tests" page, first section), its realisation must replay in the
backward and across layouts by logical index ("Causal Mask and Ragged Sequence Layouts"
page, sixth section), and finite differences use the same realisation (same page as the
first, fourth section).
"""
import os

import numpy as np
import pytest

import oracle
import pins
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            rows.append([int(x, 16) for x in line])
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for r in rows:
        got = oracle.philox4x32_10(r[0], r[1], r[2], r[3], r[4], r[5])
        assert [int(x) for x in got] == r[6:], [hex(int(x)) for x in got]


def test_keep_flags_brute_force():
    """The vectorised keep flags equal one scalar generator call per element (Python ints,
    no numpy), including patches cut by non-multiple-of-4 ranges."""
    seed, seq, head, thr = 0x0123456789ABCDEF, 3, 5, 77
    pq = np.arange(5, 19)
    pk = np.arange(2, 23)
    got = oracle.dropout_keep(seed, seq, head, pq[:, None], pk[None, :], thr)

    def philox(c, k):
        c = list(c)
        k = list(k)
        for r in range(10):
            if r:
                k = [(k[0] + 0x9E3779B9) % 2**32, (k[1] + 0xBB67AE85) % 2**32]
            a, b = 0xD2511F53 * c[0], 0xCD9E8D57 * c[2]
            c = [(b >> 32) ^ c[1] ^ k[0], b % 2**32, (a >> 32) ^ c[3] ^ k[1], a % 2**32]
        return c

    for i, q in enumerate(pq):
        for j, kk in enumerate(pk):
            w = philox([int(q) // 4, int(kk) // 4, head, seq], [seed % 2**32, seed >> 32])
            byte = (w[int(q) % 4] >> (8 * (int(kk) % 4))) & 0xFF
            assert bool(got[i, j]) == (byte >= thr), (q, kk)


def test_threshold_rounding():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.1) == 26          # 25.6 -> 26
    assert oracle.dropout_threshold(0.5) == 128
    assert oracle.dropout_threshold(1.0 / 512) == 1     # 0.5 rounds up
    assert oracle.dropout_threshold(255.0 / 256) == 255
    with pytest.raises(ValueError):
        oracle.dropout_threshold(1.0)
    with pytest.raises(ValueError):
        oracle.dropout_threshold(-0.01)


@pytest.mark.parametrize("thr", [26, 128, 200])
def test_keep_rate_and_byte_lanes(thr):
    """Over 512 x 512 positions the dropped fraction is t/256 within 6 binomial standard
    deviations, for every (word, byte) lane of the patch separately: a wrong byte or word
    selection (e.g. one byte reused for a whole patch) shifts or correlates these rates."""
    pq = np.arange(512)[:, None]
    pk = np.arange(512)[None, :]
    keep = oracle.dropout_keep(987654321, 1, 2, pq, pk, thr)
    pdrop = thr / 256.0
    for wq in range(4):
        for bk in range(4):
            sub = ~keep[wq::4, bk::4]
            n = sub.size
            assert abs(sub.mean() - pdrop) <= 6 * np.sqrt(pdrop * (1 - pdrop) / n), (wq, bk)
    # neighbouring elements of one patch are independent draws: P(both dropped) = p^2
    both = (~keep[:, 0::4] & ~keep[:, 1::4]).mean()
    n = keep[:, 0::4].size
    assert abs(both - pdrop**2) <= 6 * np.sqrt(pdrop**2 * (1 - pdrop**2) / n)


def test_keys_select_distinct_streams():
    """Seed, sequence, head and positions each change the realisation."""
    pq = np.arange(64)[:, None]
    pk = np.arange(64)[None, :]
    base = oracle.dropout_keep(11, 0, 0, pq, pk, 128)
    for kw in ({"seed": 12}, {"seq": 1}, {"head": 1}):
        args = {"seed": 11, "seq": 0, "head": 0}
        args.update(kw)
        other = oracle.dropout_keep(args["seed"], args["seq"], args["head"], pq, pk, 128)
        assert 0.35 < (other != base).mean() < 0.65, kw
    shifted = oracle.dropout_keep(11, 0, 0, pq + 4, pk, 128)
    assert 0.35 < (shifted != base).mean() < 0.65


def _pack(seed):
    w = wl.random_workload(seed, [7, 0, 13, 5], [9, 3, 13, 2], 4, 2, 8, "f32",
                           wl.MASK_CAUSAL_BOTTOM_RIGHT, with_dout=True, name="dropout-pin")
    return w


def test_zero_probability_is_the_plain_operator():
    w = _pack(120)
    o, l = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    od, ld = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                              dropout_p=0.0, seed=99)
    assert np.array_equal(o, od) and np.array_equal(l, ld)
    g = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    gd = oracle.attention_bwd(w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                              dropout_p=0.0, seed=99)
    for a, b in zip(g, gd):
        assert np.array_equal(a, b)


def test_explicit_realisation():
    """Dropout output equals (P * keep / (1 - p)) V built by hand from the plain
    operator's probabilities (recovered as the output of one-hot values) and the keep
    flags; the LSE is unchanged."""
    w = _pack(121)
    p_drop = 0.3
    thr = oracle.dropout_threshold(p_drop)
    od, ld = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                              dropout_p=p_drop, seed=5)
    _, l = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    assert np.array_equal(l, ld)
    sq, pq, _ = oracle.token_metadata(w.cu_q)
    sk, pk, _ = oracle.token_metadata(w.cu_k)
    tk = w.k.shape[0]
    eye = np.eye(tk)[:, None, :].repeat(w.k.shape[1], axis=1)      # V = one-hot per key
    probs, _ = oracle.attention(w.q, w.k, eye, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    for h in range(w.q.shape[1]):
        keep = np.zeros((w.q.shape[0], tk), dtype=bool)
        for s in range(len(w.cu_q) - 1):
            qa, qb, ka, kb = w.cu_q[s], w.cu_q[s + 1], w.cu_k[s], w.cu_k[s + 1]
            keep[qa:qb, ka:kb] = oracle.dropout_keep(5, s, h, pq[qa:qb, None], pk[None, ka:kb],
                                                     thr)
        z = probs[:, h, :] * keep * (256.0 / (256.0 - thr))
        ref = z @ np.asarray(w.v, np.float64)[:, h // 2, :]
        assert np.allclose(od[:, h, :], ref, rtol=1e-12, atol=1e-12)


def test_unbiased_over_seeds():
    """Inverted dropout is unbiased: the mean output over 400 seeds approaches the plain
    output within 6 standard errors of the per-seed samples."""
    w = _pack(122)
    o, _ = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    samples = np.stack([oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode,
                                         dropout_p=0.25, seed=s)[0] for s in range(400)])
    mean = samples.mean(axis=0)
    se = samples.std(axis=0, ddof=1) / np.sqrt(len(samples))
    assert np.all(np.abs(mean - o) <= 6 * se + 1e-12)


def test_storage_offsets_do_not_enter():
    """Sequence 2's dropout output and gradients do not change when the other sequences'
    lengths change (its storage offset moves; its index, positions and head stay)."""
    a = wl.random_workload(123, [7, 0, 13, 5], [9, 3, 13, 2], 4, 2, 8, "f32",
                           wl.MASK_CAUSAL_TOP_LEFT, with_dout=True, name="layout-a")
    lq, lk = [20, 6, 13, 1], [11, 9, 13, 8]
    b = wl.random_workload(124, lq, lk, 4, 2, 8, "f32", wl.MASK_CAUSAL_TOP_LEFT,
                           with_dout=True, name="layout-b")
    qa, qb, ka, kb = a.cu_q[2], a.cu_q[3], a.cu_k[2], a.cu_k[3]
    qa2, ka2 = b.cu_q[2], b.cu_k[2]
    for name in ("q", "dout"):
        getattr(b, name)[qa2:qa2 + 13] = getattr(a, name)[qa:qb]
    for name in ("k", "v"):
        getattr(b, name)[ka2:ka2 + 13] = getattr(a, name)[ka:kb]
    kw = dict(dropout_p=0.4, seed=77)
    oa, _ = oracle.attention(a.q, a.k, a.v, a.cu_q, a.cu_k, a.scale, a.mask_mode, **kw)
    ob, _ = oracle.attention(b.q, b.k, b.v, b.cu_q, b.cu_k, b.scale, b.mask_mode, **kw)
    assert np.array_equal(oa[qa:qb], ob[qa2:qa2 + 13])
    ga = oracle.attention_bwd(a.q, a.k, a.v, a.dout, a.cu_q, a.cu_k, a.scale, a.mask_mode, **kw)
    gb = oracle.attention_bwd(b.q, b.k, b.v, b.dout, b.cu_q, b.cu_k, b.scale, b.mask_mode, **kw)
    assert np.array_equal(ga[0][qa:qb], gb[0][qa2:qa2 + 13])
    assert np.array_equal(ga[1][ka:kb], gb[1][ka2:ka2 + 13])


def test_dropout_finite_differences():
    """Central differences of sum(R * O) with a fixed realisation against the backward."""
    kw = dict(dropout_p=0.3, seed=2024)
    pins.check_finite_differences(
        lambda *a: oracle.attention(*a, **kw),
        lambda *a: oracle.attention_bwd(*a, **kw))


def test_backward_from_a_given_output():
    """``out=``: D is formed from the given output. With the oracle's own output the
    gradients are unchanged; shifting one stored element O[t, h, m] by c shifts dQ[t, h] by
    -scale c dO[t, h, m] sum_u P[t, u] k_u (the attention output with V = K), the keys' dK
    summed over the sequence by -scale c dO[t, h, m] q[t, h] (the weights sum to 1), and
    leaves dV unchanged (D does not enter it)."""
    w = wl.random_workload(125, [6, 9], [7, 9], 4, 2, 8, "f32", wl.MASK_CAUSAL_BOTTOM_RIGHT,
                           with_dout=True, name="given-out")
    args = (w.q, w.k, w.v, w.dout, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    o, _ = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    base = oracle.attention_bwd(*args)
    same = oracle.attention_bwd(*args, out=o)
    for a, b in zip(base, same):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
    t, h, m, c = 8, 3, 5, 0.37        # token 8 is position 2 of sequence 1; K/V head 1
    o2 = o.copy()
    o2[t, h, m] += c
    dq2, dk2, dv2 = oracle.attention_bwd(*args, out=o2)
    g = h // 2
    coef = -w.scale * c * float(np.asarray(w.dout, np.float64)[t, h, m])
    ok_, _ = oracle.attention(w.q, w.k, w.k, w.cu_q, w.cu_k, w.scale, w.mask_mode)
    assert np.allclose(dq2[t, h] - base[0][t, h], coef * ok_[t, h], rtol=1e-10, atol=1e-12)
    others = np.ones(len(dq2), dtype=bool)
    others[t] = False
    assert np.allclose(dq2[others], base[0][others], rtol=0, atol=1e-14)
    ka, kb = int(w.cu_k[1]), int(w.cu_k[2])
    assert np.allclose((dk2 - base[1])[ka:kb, g].sum(axis=0),
                       coef * np.asarray(w.q, np.float64)[t, h], rtol=1e-10, atol=1e-12)
    assert np.array_equal(dv2, base[2])

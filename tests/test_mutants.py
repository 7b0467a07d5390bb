"""The pins catch every modelled tiling mistake, and the unmutated tiled recurrence satisfies
the online-softmax invariant and matches the oracle (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import sympy

import oracle
import pins
from tiled_model import BWD_MUTANTS, FWD_MUTANTS, TiledModel, two_tile_value


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_clean_model_passes_all_pins():
    m = TiledModel(bm=2, bn=3)
    for check in pins.FWD_CHECKS:
        check(m.fwd_fn())
    for check in pins.BWD_CHECKS:
        check(m.bwd_fn())
    pins.check_finite_differences(m.fwd_fn(), m.bwd_fn())


def test_clean_model_matches_oracle_and_invariant():
    """After every tile the running denominator equals the recomputed denominator at the
    current max ("Efficient Attention: Formal Correctness", "The FlashAttention Proof")."""
    rng = np.random.default_rng(5)
    q, k, v, cu_q, cu_k = pins._random_pack(rng, [7, 4, 9], [5, 8, 9], 4, 2, 3)
    do = rng.standard_normal(q.shape)
    for mode, window in ((1, 0), (2, 0), (2, 3), (0, 0)):
        log = []
        m = TiledModel(bm=3, bn=2, invariant_log=log)
        o, lse = m.forward(q, k, v, cu_q, cu_k, 0.9, mode, window)
        ro, rl = oracle.attention(q, k, v, cu_q, cu_k, 0.9, mode, window)
        pins._close(o, ro, 1e-12, "model O")
        pins._close(lse, rl, 1e-12, "model LSE")
        assert log and max(log) < 1e-13
        g = m.backward(q, k, v, do, cu_q, cu_k, 0.9, mode, window)
        rg = oracle.attention_bwd(q, k, v, do, cu_q, cu_k, 0.9, mode, window)
        for a, b in zip(g, rg):
            pins._close(a, b, 1e-11, "model grads")


@pytest.mark.parametrize("mutant", FWD_MUTANTS)
def test_forward_mutant_is_caught(mutant):
    fwd = TiledModel(bm=2, bn=3, mutants=[mutant]).fwd_fn()
    caught = [c.__name__ for c in pins.FWD_CHECKS if _fails(lambda c=c: c(fwd))]
    assert caught, f"no pin catches {mutant}"


@pytest.mark.parametrize("mutant", BWD_MUTANTS)
def test_backward_mutant_is_caught(mutant):
    m = TiledModel(bm=2, bn=3, mutants=[mutant])
    clean = TiledModel(bm=2, bn=3)
    caught = [c.__name__ for c in pins.BWD_CHECKS if _fails(lambda c=c: c(m.bwd_fn()))]
    if _fails(lambda: pins.check_finite_differences(clean.fwd_fn(), m.bwd_fn())):
        caught.append("finite_differences")
    assert caught, f"no pin catches {mutant}"


def test_two_tile_fixture_values():
    for row in pins.load_two_tile_recurrence():
        assert abs(two_tile_value(row["v"]) - float(row["correct"])) < 1e-12
        assert abs(two_tile_value(row["v"], ["no_l_rescale"]) - float(row["no_l_rescale"])) < 1e-12
        assert abs(two_tile_value(row["v"], ["no_acc_rescale"]) - float(row["no_acc_rescale"])) < 1e-12


def test_two_tile_fixture_exact_in_sympy():
    """The fixture's rationals follow exactly from exp(ln 3) = 3 in exact arithmetic."""
    s1, s2 = sympy.Integer(0), sympy.log(3)
    for row in pins.load_two_tile_recurrence():
        v1, v2 = (sympy.Integer(x) for x in row["v"])
        m1 = s1
        l1, acc1 = sympy.exp(s1 - m1), sympy.exp(s1 - m1) * v1
        m2 = sympy.Max(m1, s2)
        alpha = sympy.exp(m1 - m2)
        p2 = sympy.exp(s2 - m2)
        correct = sympy.nsimplify((alpha * acc1 + p2 * v2) / (alpha * l1 + p2))
        no_l = sympy.nsimplify((alpha * acc1 + p2 * v2) / (l1 + p2))
        no_acc = sympy.nsimplify((acc1 + p2 * v2) / (alpha * l1 + p2))
        assert Fraction(str(correct)) == row["correct"]
        assert Fraction(str(no_l)) == row["no_l_rescale"]
        assert Fraction(str(no_acc)) == row["no_acc_rescale"]


def test_recurrence_invariant_symbolic():
    """For three tiles of one key with symbolic logits and every order of their maxima, the
    running denominator equals sum exp(s_i - m) at the current max and the final output equals
    the recomputed softmax average, exactly."""
    a, b, c = sympy.symbols("a b c", real=True)
    v = sympy.symbols("v0:3", real=True)
    logits = [a, b, c]
    import itertools
    for order in itertools.permutations(range(3)):
        # impose an ordering of the logits: logits[order[0]] < logits[order[1]] < ...
        subs_rank = {logits[order[i]]: i for i in range(3)}
        m, l, acc = None, 0, 0
        for j, sj in enumerate(logits):
            if m is None:
                m_new = sj
            else:
                m_new = m if subs_rank[m] > subs_rank[sj] else sj
            alpha = sympy.exp(m - m_new) if m is not None else 0
            p = sympy.exp(sj - m_new)
            l = alpha * l + p
            acc = alpha * acc + p * v[j]
            m = m_new
            want_l = sum(sympy.exp(logits[i] - m) for i in range(j + 1))
            assert sympy.simplify(sympy.expand(l - want_l)) == 0
        full = sum(sympy.exp(x) * vv for x, vv in zip(logits, v)) / sum(sympy.exp(x) for x in logits)
        assert sympy.simplify(acc / l - full) == 0

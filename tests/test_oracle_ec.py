"""Pins for the Expert Choice oracle (``oracle.expert_choice``, ``oracle.moe_forward_ec``).

The capacity-factor section of the routing-principles page
("MoE混合专家模型路由机制原理与稀疏激活实现", "Expert Choice路由策略与容量因子调优")
fixes what is pinned here: experts choose tokens, each expert takes a fixed
number of them (capacity = tokens / E * factor), and tokens nobody takes
keep only the residual. Each check reaches the expected value by another
route: brute force over token subsets, a library softmax, the token-choice
oracle at k = E, closed forms, and a hand-worked example in exact arithmetic.
A second group plants plausible mistakes in copies of the selection and
shows that a pin catches each.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

from oracle import oracle as orc


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _layer(rng, T, d, h, E):
    x = _f32(rng.standard_normal((T, d)))
    wg = _f32(rng.standard_normal((E, d)) / math.sqrt(d))
    w1 = _f32(rng.standard_normal((E, h, d)) / math.sqrt(d))
    b1 = _f32(rng.standard_normal((E, h)) * 0.1)
    w2 = _f32(rng.standard_normal((E, d, h)) / math.sqrt(h))
    b2 = _f32(rng.standard_normal((E, d)) * 0.1)
    return x, wg, w1, b1, w2, b2


# ---------------------------------------------------------------- checks ----
# Each takes a selection function with the signature of oracle.expert_choice,
# so the same checks run against the oracle and against planted mistakes.

def check_brute_force(select):
    """For tiny T, each expert's set is the C-subset with the largest score sum
    (unique for distinct scores), found by enumerating every subset."""
    rng = np.random.default_rng(11)
    for T, E, C in [(6, 3, 2), (7, 2, 3), (5, 4, 1)]:
        score = softmax(rng.standard_normal((T, E)), axis=1)
        offsets, st, dest, gate = select(score, C)
        for e in range(E):
            best = max(itertools.combinations(range(T), C), key=lambda s: sum(score[list(s), e]))
            assert sorted(st[offsets[e]:offsets[e + 1]].tolist()) == sorted(best)


def check_ties_lowest_index(select):
    """One expert: every probability is exactly 1, so the tie rule alone decides."""
    score = softmax(np.zeros((9, 1)), axis=1)
    offsets, st, dest, gate = select(score, 4)
    assert st.tolist() == [0, 1, 2, 3]
    # equal scores inside one expert among other distinct ones
    score = np.array([[0.3, 0.7], [0.5, 0.5], [0.3, 0.7], [0.9, 0.1]])
    offsets, st, dest, gate = select(score, 2)
    assert st[0:2].tolist() == [1, 3]      # 0.9, 0.5
    assert st[2:4].tolist() == [0, 2]      # 0.7, 0.7 (beats 0.5)
    offsets, st, dest, gate = select(score, 3)
    assert st[0:3].tolist() == [0, 1, 3]   # 0.9, 0.5, then 0.3 of token 0 before token 2


def check_hand_example(select):
    """Worked by hand: logits (0,0), (ln 3, 0), (0, ln 3) give probabilities
    (1/2, 1/2), (3/4, 1/4), (1/4, 3/4) exactly."""
    score = np.array([[float(Fraction(1, 2)), float(Fraction(1, 2))],
                      [float(Fraction(3, 4)), float(Fraction(1, 4))],
                      [float(Fraction(1, 4)), float(Fraction(3, 4))]])
    offsets, st, dest, gate = select(score, 1)
    assert offsets.tolist() == [0, 1, 2] and st.tolist() == [1, 2]
    assert dest.tolist() == [[-1, -1], [0, -1], [-1, 1]]
    assert gate.tolist() == [[0, 0], [0.75, 0], [0, 0.75]]
    offsets, st, dest, gate = select(score, 2)
    assert st.tolist() == [0, 1, 0, 2]
    assert dest.tolist() == [[0, 2], [1, -1], [-1, 3]]
    assert gate.tolist() == [[0.5, 0.5], [0.75, 0], [0, 0.75]]


def check_balance_and_bijection(select):
    """Every expert takes exactly min(C, T) tokens; dest_row maps the chosen
    pairs one to one onto [0, E*min(C,T)) and agrees with sorted_token."""
    rng = np.random.default_rng(5)
    T, E = 40, 6
    score = softmax(rng.standard_normal((T, E)) * 2, axis=1)
    for C in (0, 1, 7, 40, 55):
        offsets, st, dest, gate = select(score, C)
        Cc = min(C, T)
        assert offsets.tolist() == [e * Cc for e in range(E + 1)]
        rows = dest[dest >= 0]
        assert sorted(rows.tolist()) == list(range(E * Cc))
        for t, e in zip(*np.nonzero(dest >= 0)):
            assert st[dest[t, e]] == t and offsets[e] <= dest[t, e] < offsets[e + 1]
            assert gate[t, e] == score[t, e]
        assert np.all(gate[dest < 0] == 0)
        for e in range(E):
            seg = st[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(seg) > 0)  # ascending token order


CHECKS = [check_brute_force, check_ties_lowest_index, check_hand_example,
          check_balance_and_bijection]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_selection(check):
    check(orc.expert_choice)


def check_scores(scores):
    """Against scipy's softmax over each token's experts, and rows summing to 1."""
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((50, 9)) * 3
    p = scores(lg)
    np.testing.assert_allclose(p, softmax(lg, axis=1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)


def test_scores_are_the_softmax_of_each_token():
    check_scores(orc.ec_scores)


@pytest.mark.parametrize("mutant", [lambda lg: softmax(lg, axis=0),         # over tokens
                                    lambda lg: np.exp(lg) / np.exp(lg).sum()])  # over all
def test_a_wrong_softmax_axis_fails_the_score_pin(mutant):
    with pytest.raises(AssertionError):
        check_scores(mutant)


def test_full_capacity_is_the_soft_mixture_of_token_choice_with_k_equal_E():
    """C = T: every expert takes every token, so the layer equals the
    token-choice oracle with k = E and no renormalisation: sum_e p_e E_e(x)."""
    rng = np.random.default_rng(3)
    T, d, h, E = 12, 16, 24, 4
    x, wg, w1, b1, w2, b2 = _layer(rng, T, d, h, E)
    ec = orc.moe_forward_ec(x, wg, w1, b1, w2, b2, C=T, residual=True)
    tc = orc.moe_forward(x, wg, w1, b1, w2, b2, k=E, renorm=False, residual=True)
    np.testing.assert_allclose(ec["out"], tc["out"], rtol=1e-12, atol=1e-12)


def test_zero_capacity_passes_the_residual_exactly():
    rng = np.random.default_rng(4)
    x, wg, w1, b1, w2, b2 = _layer(rng, 10, 8, 8, 3)
    res = orc.moe_forward_ec(x, wg, w1, b1, w2, b2, C=0, residual=True)
    assert np.array_equal(res["out"], x.astype(np.float64))
    res = orc.moe_forward_ec(x, wg, w1, b1, w2, b2, C=0, residual=False)
    assert not np.any(res["out"])


def test_output_is_the_gated_sum_over_choosing_experts():
    """Against a direct float64 numpy evaluation of y = x + sum_{e chooses t} p[t,e] E_e(x_t)."""
    rng = np.random.default_rng(6)
    T, d, h, E, C = 30, 16, 32, 5, 7
    x, wg, w1, b1, w2, b2 = _layer(rng, T, d, h, E)
    res = orc.moe_forward_ec(x, wg, w1, b1, w2, b2, C=C, residual=True)
    X = x.astype(np.float64)
    p = softmax(X @ wg.astype(np.float64).T, axis=1)
    want = X.copy()
    for e in range(E):
        top = sorted(range(T), key=lambda t: (-p[t, e], t))[:C]
        for t in top:
            z = w1[e].astype(np.float64) @ X[t] + b1[e]
            a = z / (1 + np.exp(-z))
            want[t] += p[t, e] * (w2[e].astype(np.float64) @ a + b2[e])
    np.testing.assert_allclose(res["out"], want, rtol=1e-11, atol=1e-11)


def test_token_sample_matches_full_evaluation():
    rng = np.random.default_rng(8)
    x, wg, w1, b1, w2, b2 = _layer(rng, 25, 8, 16, 4)
    full = orc.moe_forward_ec(x, wg, w1, b1, w2, b2, C=6, residual=True)
    toks = np.array([1, 4, 9, 20, 24], np.int32)
    part = orc.moe_forward_ec(x, wg, w1, b1, w2, b2, C=6, residual=True, tokens=toks)
    np.testing.assert_array_equal(part["out"], full["out"][toks])


# ------------------------------------------------------- planted mistakes ----

def _mutant(kind):
    def select(score, C):
        score = np.asarray(score, dtype=np.float64)
        T, E = score.shape
        Cc = max(0, min(int(C), T))
        offsets = np.arange(E + 1, dtype=np.int32) * Cc
        st = np.full(E * Cc, -1, np.int32)
        dest = np.full((T, E), -1, np.int32)
        gate = np.zeros((T, E))
        t_idx = np.arange(T)
        for e in range(E):
            key = score[:, e]
            if kind == "ascending":
                order = np.lexsort((t_idx, key))
            elif kind == "ties_high_index":
                order = np.lexsort((-t_idx, -key))
            else:
                order = np.lexsort((t_idx, -key))
            chosen = order[:max(Cc - 1, 0)] if kind == "one_short" else order[:Cc]
            if kind != "unsorted_rows":
                chosen = np.sort(chosen)
            st[e * Cc:e * Cc + chosen.size] = chosen
            dest[chosen, e] = e * Cc + np.arange(chosen.size)
            gate[chosen, e] = score[chosen, e] if kind != "renormalised" else \
                score[chosen, e] / score[chosen, e].sum()
        return offsets, st, dest, gate
    return select


@pytest.mark.parametrize("kind", ["ascending", "ties_high_index", "one_short",
                                  "unsorted_rows", "renormalised"])
def test_each_planted_mistake_fails_a_pin(kind):
    select = _mutant(kind)
    failed = []
    for check in CHECKS:
        try:
            check(select)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin catches the {kind} mistake"

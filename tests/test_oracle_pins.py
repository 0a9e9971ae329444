"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Nothing here re-types the oracle's formulas. Each test uses an independent
route to the same number: a closed form, an invariant, a special case that
reduces to a library routine (numpy / scipy), a hand-worked example in exact
rational arithmetic, or brute force on tiny inputs written from the gate
equation of the routing-principles page ("MoE混合专家模型路由机制原理与稀疏激活实现",
section "MoE混合专家模型架构与门控路由原理": G(x) = softmax(TopK(x.W_g)) with
the non-selected logits set to -inf, and y = sum_i G(x)_i E_i(x)).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _rand_layer(rng, T, d, h, E, scale_b=0.1):
    x = _f32(rng.standard_normal((T, d)))
    wg = _f32(rng.standard_normal((E, d)) / math.sqrt(d))
    w1 = _f32(rng.standard_normal((E, h, d)) / math.sqrt(d))
    b1 = _f32(rng.standard_normal((E, h)) * scale_b)
    w2 = _f32(rng.standard_normal((E, d, h)) / math.sqrt(h))
    b2 = _f32(rng.standard_normal((E, d)) * scale_b)
    return x, wg, w1, b1, w2, b2


def _np_expert(x, w1, b1, w2, b2):
    """Library route: numpy float64 matmuls and scipy's logistic function."""
    z = x.astype(np.float64) @ w1.astype(np.float64).T + b1.astype(np.float64)
    a = z * expit(z)
    return a @ w2.astype(np.float64).T + b2.astype(np.float64)


# ---------------------------------------------------------------- SiLU ----

def test_silu_identities():
    z = np.linspace(-30, 30, 2001)
    s = orc.silu(z)
    sn = orc.silu(-z)
    # SiLU(z) - SiLU(-z) = z  (z*sig(z) - (-z)*sig(-z) = z*(sig(z)+sig(-z)) = z)
    np.testing.assert_allclose(s - sn, z, rtol=0, atol=1e-12)
    assert orc.silu(np.zeros(1))[0] == 0.0
    # library routine: z * expit(z)
    np.testing.assert_allclose(s, z * expit(z), rtol=1e-14, atol=1e-300)


# ------------------------------------------------------ hand-worked case ----

def test_hand_worked_router_and_dispatch():
    """E=3, k=2, four tokens with logits chosen so that softmax is rational.

    token 0: [0, ln2, ln3]     -> p = [1/6, 2/6, 3/6], top-2 = (2, 1)
    token 1: [ln3, ln3, 0]     -> p = [3/7, 3/7, 1/7], tie: (0, 1)
    token 2: [0, 0, 0]         -> p = [1/3]*3,         tie: (0, 1)
    token 3: [-0.0, +0.0, ln(1/2)] -> p = [2/5, 2/5, 1/5]; +0 == -0 so (0, 1)
    """
    lg = np.array([[0.0, math.log(2), math.log(3)],
                   [math.log(3), math.log(3), 0.0],
                   [0.0, 0.0, 0.0],
                   [-0.0, 0.0, math.log(0.5)]])
    F = Fraction
    probs = [[F(1, 6), F(2, 6), F(3, 6)], [F(3, 7), F(3, 7), F(1, 7)],
             [F(1, 3)] * 3, [F(2, 5), F(2, 5), F(1, 5)]]
    sel = [[2, 1], [0, 1], [0, 1], [0, 1]]
    idx, gate, ps, p = orc.route(lg, 2, renorm=True, want_probs=True)
    assert idx.tolist() == sel
    for t in range(4):
        tot = sum(probs[t][e] for e in sel[t])
        for j, e in enumerate(sel[t]):
            assert gate[t, j] == pytest.approx(float(probs[t][e] / tot), abs=1e-15)
            assert p[t, e] == pytest.approx(float(probs[t][e]), abs=1e-15)
    for e in range(3):
        assert ps[e] == pytest.approx(float(sum(probs[t][e] for t in range(4))), abs=1e-14)
    _, gate0, _ = orc.route(lg, 2, renorm=False)
    for t in range(4):
        for j, e in enumerate(sel[t]):
            assert gate0[t, j] == pytest.approx(float(probs[t][e]), abs=1e-15)

    # flat order of assignments: e2 e1 | e0 e1 | e0 e1 | e0 e1
    counts, offsets, dest, st = orc.permute(idx, 3, capacity=-1)
    assert counts.tolist() == [3, 4, 1]
    assert offsets.tolist() == [0, 3, 7, 8]
    assert dest.tolist() == [7, 3, 0, 4, 1, 5, 2, 6]
    assert st.tolist() == [1, 2, 3, 0, 1, 2, 3, 0]
    # capacity 2: e0 keeps tokens 1,2; e1 keeps 0,1; e2 keeps 0
    counts, offsets, dest, st = orc.permute(idx, 3, capacity=2)
    assert counts.tolist() == [3, 4, 1]
    assert offsets.tolist() == [0, 2, 4, 5]
    assert dest.tolist() == [4, 2, 0, 3, 1, -1, -1, -1]
    assert st.tolist() == [1, 2, 0, 1, 0]

    f, P, loss = orc.aux(ps, counts, 4)
    fs = [sum(probs[t][e] for t in range(4)) / 4 for e in range(3)]
    Ps = [F(3, 4), F(4, 4), F(1, 4)]
    assert loss == pytest.approx(float(3 * sum(a * b for a, b in zip(fs, Ps))), abs=1e-14)
    assert P.tolist() == [float(v) for v in Ps]


def test_bf16_widening_exact():
    """bf16 bit patterns widen exactly: 0x3F80=1, 0xC000=-2, 0x3F81=1+2^-7, 0x0001=2^-133."""
    x = np.array([[0x3F80, 0xC000, 0x3F81, 0x0001]], np.uint16)
    wg = np.array([[0x3F80, 0, 0, 0], [0, 0x3F80, 0, 0], [0, 0, 0x3F80, 0],
                   [0, 0, 0, 0x3F80]], np.uint16)
    lg = orc.logits(x, wg)
    assert lg[0].tolist() == [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133]


def test_logits_router_bias_and_library_matmul():
    rng = np.random.default_rng(1)
    x = _f32(rng.standard_normal((37, 19)))
    wg = _f32(rng.standard_normal((5, 19)))
    gb = _f32(rng.standard_normal(5))
    ref = x.astype(np.float64) @ wg.astype(np.float64).T + gb.astype(np.float64)
    np.testing.assert_allclose(orc.logits(x, wg, gb), ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------- golden: printed shapes ----

def test_golden_router_output_shapes():
    g = json.load(open(os.path.join(GOLDEN, "sparse_inference_router_shapes.json")))
    B, S, D = g["x_shape"]
    rng = np.random.default_rng(2)
    x = _f32(rng.standard_normal((B * S, D)))
    wg = _f32(rng.standard_normal((g["num_experts"], g["dim"])) / math.sqrt(D))
    idx, gate, _ = orc.route(orc.logits(x, wg), g["k"], renorm=True)
    assert list(gate.reshape(B, S, -1).shape) == g["weights_shape"]
    assert list(idx.reshape(B, S, -1).shape) == g["indices_shape"]
    assert idx.min() >= 0 and idx.max() < g["num_experts"]


# ------------------------------------------------------ router forms ----

@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (64, 2), (256, 8), (5, 5)])
def test_router_three_forms_agree(E, k):
    """softmax->topk->renormalise == softmax(TopK-masked logits) == softmax(top-k logits)."""
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.standard_normal((500, E)) * 2.0
    idx, gate, ps, probs = orc.route(lg, k, renorm=True, want_probs=True)
    # masked form (gate equation): non-selected logits -> -inf, softmax over E
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert np.array_equal(order, idx)
    masked = np.full_like(lg, -np.inf)
    np.put_along_axis(masked, order, np.take_along_axis(lg, order, 1), 1)
    G = softmax(masked, axis=1)
    np.testing.assert_allclose(np.take_along_axis(G, order, 1), gate, rtol=1e-13, atol=1e-15)
    assert np.all(G[masked == -np.inf] == 0)
    # top-k on logits, then softmax over the k logits
    gk = softmax(np.take_along_axis(lg, order, 1), axis=1)
    np.testing.assert_allclose(gk, gate, rtol=1e-13, atol=1e-15)
    # renormalised gates sum to one
    np.testing.assert_allclose(gate.sum(1), 1.0, rtol=0, atol=1e-12)
    # non-renormalised gates are the full-softmax probabilities
    _, g0, _ = orc.route(lg, k, renorm=False)
    P = softmax(lg, axis=1)
    np.testing.assert_allclose(g0, np.take_along_axis(P, order, 1), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(probs, P, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(ps, P.sum(0), rtol=1e-12)


def test_top1_renorm_gate_is_one():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((300, 16))
    _, gate, _ = orc.route(lg, 1, renorm=True)
    assert np.all(gate == 1.0)


# ------------------------------------------------------ permutation ----

@pytest.mark.parametrize("cap", [-1, 0, 1, 7, 40, 10**6])
def test_permute_invariants(cap):
    rng = np.random.default_rng(11 + max(cap, 0) % 97)
    T, k, E = 301, 3, 12
    # skewed routing so some experts overflow small capacities
    w = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    idx = np.stack([rng.choice(E, size=k, replace=False, p=w / w.sum()) for _ in range(T)]).astype(np.int32)
    counts, offsets, dest, st = orc.permute(idx, E, cap)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    kept = np.diff(offsets)
    assert offsets[0] == 0 and np.all(kept >= 0)
    if cap >= 0:
        assert np.all(kept <= cap)
        assert np.array_equal(kept, np.minimum(counts, cap))
    else:
        assert np.array_equal(kept, counts)
    R = offsets[E]
    drops = int((dest < 0).sum())
    assert R == T * k - drops
    valid = dest >= 0
    # bijection from kept assignments onto [0, R)
    assert np.array_equal(np.sort(dest[valid]), np.arange(R))
    # each row knows its token and lies in its expert's segment
    f = np.nonzero(valid)[0]
    assert np.array_equal(st[dest[f]], f // k)
    e = flat[f]
    assert np.all((dest[f] >= offsets[e]) & (dest[f] < offsets[e + 1]))
    # stable: within an expert, rows follow ascending flat index, and the kept
    # ones are exactly the first kept[e] of that expert's assignments
    for ee in range(E):
        fe = np.nonzero(flat == ee)[0]
        de = dest[fe]
        assert np.array_equal(de[: kept[ee]], offsets[ee] + np.arange(kept[ee]))
        assert np.all(de[kept[ee]:] == -1)
    if cap >= T * k:
        assert drops == 0


# ------------------------------------------------------------- aux ----

def test_aux_closed_forms():
    T, E, k = 64, 8, 2
    # uniform probabilities (all logits equal): f = 1/E, so loss = sum P = k
    lg = np.zeros((T, E))
    idx, _, ps = orc.route(lg, k, renorm=True)
    counts, *_ = orc.permute(idx, E, -1)
    f, P, loss = orc.aux(ps, counts, T)
    assert np.allclose(f, 1.0 / E, atol=1e-15) and loss == pytest.approx(k, abs=1e-12)
    # uniform counts (each expert gets T*k/E), arbitrary probs: loss = k
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((T, E))
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], np.int32)
    _, _, ps = orc.route(lg, k, renorm=True)
    counts, *_ = orc.permute(idx, E, -1)
    assert np.all(counts == T * k // E)
    _, _, loss = orc.aux(ps, counts, T)
    assert loss == pytest.approx(k, abs=1e-12)
    # full collapse onto expert 0 with top-1: f_0 = 1, P_0 = 1 -> loss = E
    lg = np.zeros((T, E))
    lg[:, 0] = 1000.0
    idx, _, ps = orc.route(lg, 1, renorm=False)
    counts, *_ = orc.permute(idx, E, -1)
    _, _, loss = orc.aux(ps, counts, T)
    assert loss == float(E)


# ---------------------------------------------------- whole-layer pins ----

def test_zero_gate_ties_and_drop_set():
    """W_g = 0: every logit ties, so S_t = (0..k-1); with a cap the drops are tokens >= cap."""
    rng = np.random.default_rng(5)
    T, d, h, E, k, cap = 40, 6, 10, 6, 3, 17
    x, wg, w1, b1, w2, b2 = _rand_layer(rng, T, d, h, E)
    wg[:] = 0.0
    for renorm in (True, False):
        r = orc.moe_forward(x, wg, w1, b1, w2, b2, k, renorm, capacity=cap)
        assert np.all(r["idx"] == np.arange(k))
        assert np.allclose(r["gate"], 1.0 / k if renorm else 1.0 / E, atol=1e-15)
        assert r["counts"].tolist() == [T] * k + [0] * (E - k)
        dest = r["dest_row"].reshape(T, k)
        assert np.all((dest >= 0) == (np.arange(T)[:, None] < cap))


def test_capacity_zero_gives_residual():
    rng = np.random.default_rng(6)
    x, wg, w1, b1, w2, b2 = _rand_layer(rng, 30, 8, 12, 4)
    r = orc.moe_forward(x, wg, w1, b1, w2, b2, 2, True, capacity=0, residual=True)
    assert r["offsets"][-1] == 0
    assert np.array_equal(r["out"], x.astype(np.float64))
    r = orc.moe_forward(x, wg, w1, b1, w2, b2, 2, True, capacity=0, residual=False)
    assert np.all(r["out"] == 0.0)


def test_k_equals_E_identical_experts_is_dense_ffn():
    rng = np.random.default_rng(7)
    T, d, h, E = 50, 16, 24, 4
    x, wg, w1, b1, w2, b2 = _rand_layer(rng, T, d, h, E)
    w1[:] = w1[0]
    b1[:] = b1[0]
    w2[:] = w2[0]
    b2[:] = b2[0]
    r = orc.moe_forward(x, wg, w1, b1, w2, b2, E, True)
    dense = _np_expert(x, w1[0], b1[0], w2[0], b2[0])
    np.testing.assert_allclose(r["out"], dense, rtol=1e-12, atol=1e-12)


def test_k_equals_E_distinct_experts_is_soft_mixture():
    rng = np.random.default_rng(8)
    T, d, h, E = 50, 16, 24, 5
    x, wg, w1, b1, w2, b2 = _rand_layer(rng, T, d, h, E)
    r = orc.moe_forward(x, wg, w1, b1, w2, b2, E, True)
    p = softmax(x.astype(np.float64) @ wg.astype(np.float64).T, axis=1)
    mix = sum(p[:, e:e + 1] * _np_expert(x, w1[e], b1[e], w2[e], b2[e]) for e in range(E))
    np.testing.assert_allclose(r["out"], mix, rtol=1e-11, atol=1e-12)


def test_single_expert_is_dense_ffn():
    rng = np.random.default_rng(9)
    x, wg, w1, b1, w2, b2 = _rand_layer(rng, 20, 8, 16, 1)
    for renorm in (True, False):
        r = orc.moe_forward(x, wg, w1, b1, w2, b2, 1, renorm)
        assert np.all(r["gate"] == 1.0)
        np.testing.assert_allclose(r["out"], _np_expert(x, w1[0], b1[0], w2[0], b2[0]),
                                   rtol=1e-12, atol=1e-12)


def _brute_layer(x, wg, gb, w1, b1, w2, b2, k, renorm, cap, residual):
    """Per-token direct evaluation in pure Python from the gate equation.

    Logits by explicit sums; TopK keeps the k largest (lower index first on
    ties) and sets the rest to -inf, then softmax (renorm) -- or the gate is the
    full-softmax probability of the selected expert (renorm off). Capacity is
    first-come in token order, then slot order. No permutation is built.
    """
    T, d = x.shape
    E, h = w1.shape[0], w1.shape[1]
    used = [0] * E
    out = np.zeros((T, d))
    for t in range(T):
        xt = [float(v) for v in x[t]]
        lg = [sum(xt[i] * float(wg[e, i]) for i in range(d)) + (float(gb[e]) if gb is not None else 0.0)
              for e in range(E)]
        S = sorted(range(E), key=lambda e: (-lg[e], e))[:k]
        if renorm:
            masked = [lg[e] if e in S else -math.inf for e in range(E)]
            m = max(masked)
            ex = [math.exp(v - m) if v != -math.inf else 0.0 for v in masked]
        else:
            m = max(lg)
            ex = [math.exp(v - m) for v in lg]
        G = [v / sum(ex) for v in ex]
        acc = list(xt) if residual else [0.0] * d
        for e in S:
            if cap >= 0 and used[e] >= cap:
                continue
            used[e] += 1
            a = []
            for n in range(h):
                z = sum(float(w1[e, n, i]) * xt[i] for i in range(d)) + float(b1[e, n])
                a.append(z / (1.0 + math.exp(-z)))
            for mm in range(d):
                ye = sum(float(w2[e, mm, n]) * a[n] for n in range(h)) + float(b2[e, mm])
                acc[mm] += G[e] * ye
        out[t] = acc
    return out


@pytest.mark.parametrize("T,E,k,renorm,cap,residual", [
    (6, 4, 1, True, -1, False), (6, 4, 2, True, -1, False), (5, 4, 3, True, -1, True),
    (6, 4, 4, True, -1, False), (6, 3, 1, False, 2, True), (6, 4, 2, True, 1, True),
    (4, 2, 2, False, -1, False), (6, 4, 2, True, 0, True)])
def test_brute_force_tiny(T, E, k, renorm, cap, residual):
    rng = np.random.default_rng(T * 1000 + E * 100 + k * 10 + cap + 3)
    d, h = 5, 7
    x, wg, w1, b1, w2, b2 = _rand_layer(rng, T, d, h, E)
    gb = _f32(rng.standard_normal(E) * 0.5)
    r = orc.moe_forward(x, wg, w1, b1, w2, b2, k, renorm, capacity=cap, gate_bias=gb,
                        residual=residual)
    ref = _brute_layer(x, wg, gb, w1, b1, w2, b2, k, renorm, cap, residual)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-13)


def test_tiny_config_against_library_pipeline():
    """The fp32 tiny workload end to end against numpy/scipy float64 library routines."""
    import moe_inputs as mi
    cfg = mi.CONFIGS["tiny_fp32"]
    inp = mi.make_inputs(cfg, "cpu")
    a = {k_: mi.to_host_array(v) for k_, v in inp.items()}
    r = orc.moe_forward(a["x"], a["w_gate"], a["w1"], a["b1"], a["w2"], a["b2"], cfg.k, cfg.renorm)
    x = a["x"].astype(np.float64)
    lg = x @ a["w_gate"].astype(np.float64).T
    np.testing.assert_allclose(r["logits"], lg, rtol=1e-12, atol=1e-12)
    order = np.argsort(-lg, axis=1, kind="stable")[:, :cfg.k]
    assert np.array_equal(order, r["idx"])
    p = softmax(lg, axis=1)
    g = np.take_along_axis(p, order, 1)
    g = g / g.sum(1, keepdims=True)
    out = np.zeros_like(x)
    for e in range(cfg.E):
        y = _np_expert(a["x"], a["w1"][e], a["b1"][e], a["w2"][e], a["b2"][e])
        for j in range(cfg.k):
            m = order[:, j] == e
            out[m] += g[m, j:j + 1] * y[m]
    np.testing.assert_allclose(r["out"], out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["f"], p.mean(0), rtol=1e-12)
    assert r["loss"] == pytest.approx(cfg.E * float((p.mean(0) * np.bincount(order.ravel(), minlength=cfg.E) / cfg.T).sum()), rel=1e-12)


def test_token_subset_matches_full_and_per_expert_fetch():
    rng = np.random.default_rng(10)
    x, wg, w1, b1, w2, b2 = _rand_layer(rng, 64, 12, 20, 6)
    full = orc.moe_forward(x, wg, w1, b1, w2, b2, 2, True, capacity=20, residual=True)
    toks = np.array([0, 5, 17, 63, 40], np.int32)
    sub = orc.moe_forward(x, wg, w1, b1, w2, b2, 2, True, capacity=20, residual=True,
                          tokens=toks, expert_weights=lambda e: (w1[e], b1[e], w2[e], b2[e]))
    assert np.array_equal(sub["out"], full["out"][toks])
    assert np.array_equal(sub["dest_row"], full["dest_row"])

"""Pins for the error yardsticks the GPU tolerances are built on.

Two oracle outputs are not gradients but scales:
  - the per-element magnitude M that ``moe_backward(..., want_scale=True)``
    returns beside every gradient (the backward evaluated on absolute
    values, with the extra terms for a rounded pre-activation),
  - the same for ``moe_backward_ec`` (Expert Choice layers).
A GPU test passes when its error stays under tol * RMS + c * M, so an
inflated M would widen the bound without any test noticing. The checks
below rebuild every element of every scale from its definition with plain
Python loops, token by token and slot by slot (the oracle works expert by
expert with matrix products), and require agreement to rtol 1e-12.

The definitions, per kept (token t, slot j) with expert e and gate g,
z = W1[e] x[t] + b1[e], y = W2[e] SiLU(z) + b2[e], |dy[n]| = |g| |dout[t][n]|:
  M_dW2[e][n][c] += |dy[n]| (|SiLU(z[c])| + |SiLU'(z[c]) z[c]| / 4)
  M_db2[e][n]    += |dy[n]|
  M_dz[c]         = (sum_n |dy[n]| |W2[e][n][c]|) (|SiLU'(z[c])| + |z[c]| / 8)
  M_dW1[e][c][i] += M_dz[c] |x[t][i]|,   M_db1[e][c] += M_dz[c]
  M_dx[t][i]     += sum_c M_dz[c] |W1[e][c][i]|
  M_dgate[t][j]   = sum_n |dout[t][n]| |y[n]|
then per token the router: renormalised gates M_dl[S_j] += |g_j| (M_dgate_j +
sum_i |g_i| M_dgate_i); full-softmax gates and the aux term M_dl[e] = p[e]
(m[e] + sum_e' p[e'] m[e']) with m the gate magnitudes summed per expert, or
|daux| E counts[e] / T^2; finally M_dx += |dout| (residual) + sum_e M_dl |W_g|,
M_dW_g[e][i] = sum_t M_dl[t][e] |x[t][i]|, M_db_g[e] = sum_t M_dl[t][e].

MOE_ORACLE_BWD may name a copy of the backward oracle module to test in its
place (the mutation tests plant mistakes in such copies).
"""
import importlib.util
import math
import os

import numpy as np
import pytest


def _module(env, default):
    path = os.environ.get(env)
    if not path:
        return default
    spec = importlib.util.spec_from_file_location(f"oracle_under_test_{env}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


from oracle import backward as _bwd  # noqa: E402
from oracle import oracle as _orc  # noqa: E402

bwd = _module("MOE_ORACLE_BWD", _bwd)
orc = _orc


def _layer(seed, T, d, h, E, gate_bias):
    rng = np.random.default_rng(seed)
    p = dict(
        x=np.float32(rng.standard_normal((T, d))),
        w_gate=np.float32(rng.standard_normal((E, d)) * 1.5 / math.sqrt(d)),
        w1=np.float32(rng.standard_normal((E, h, d)) / math.sqrt(d)),
        b1=np.float32(rng.standard_normal((E, h)) * 0.3),
        w2=np.float32(rng.standard_normal((E, d, h)) / math.sqrt(h)),
        b2=np.float32(rng.standard_normal((E, d)) * 0.3),
        gate_bias=np.float32(rng.standard_normal(E) * 0.5) if gate_bias else None,
    )
    dout = rng.standard_normal((T, d))
    return p, dout


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _silu(z):
    return z * _sig(z)


def _dsilu(z):
    s = _sig(z)
    return s * (1.0 + z * (1.0 - s))


def _expert_terms(X, W1, B1, W2, B2, dO, t, e, g, M, Mdx):
    """Add the magnitudes of one kept (token t, expert e, gate g) pair into M
    and Mdx, element by element; returns (M_dgate of the pair, y)."""
    h, d = len(W1[e]), len(X[t])
    z = [sum(W1[e][c][i] * X[t][i] for i in range(d)) + (B1[e][c] if B1 is not None else 0.0)
         for c in range(h)]
    y = [sum(W2[e][n][c] * _silu(z[c]) for c in range(h)) + (B2[e][n] if B2 is not None else 0.0)
         for n in range(d)]
    ady = [abs(g) * abs(dO[t][n]) for n in range(d)]
    for n in range(d):
        for c in range(h):
            M["dw2"][e][n][c] += ady[n] * (abs(_silu(z[c])) + abs(_dsilu(z[c]) * z[c]) / 4.0)
        if M["db2"] is not None:
            M["db2"][e][n] += ady[n]
    for c in range(h):
        mdz = sum(ady[n] * abs(W2[e][n][c]) for n in range(d)) * (abs(_dsilu(z[c])) + abs(z[c]) / 8.0)
        for i in range(d):
            M["dw1"][e][c][i] += mdz * abs(X[t][i])
            Mdx[t][i] += mdz * abs(W1[e][c][i])
        if M["db1"] is not None:
            M["db1"][e][c] += mdz
    mdg = sum(abs(dO[t][n]) * abs(y[n]) for n in range(d))
    return mdg, y


def _empty(E, d, h, has_b1, has_b2):
    z3 = lambda a, b, c: [[[0.0] * c for _ in range(b)] for _ in range(a)]  # noqa: E731
    z2 = lambda a, b: [[0.0] * b for _ in range(a)]  # noqa: E731
    return dict(dw1=z3(E, h, d), dw2=z3(E, d, h), db1=z2(E, h) if has_b1 else None,
                db2=z2(E, d) if has_b2 else None)


def _router_tail(X, Wg, dO, Mdl, residual, has_gate_bias, M, Mdx):
    T, d, E = len(X), len(X[0]), len(Wg)
    for t in range(T):
        for i in range(d):
            Mdx[t][i] += (abs(dO[t][i]) if residual else 0.0) + \
                sum(Mdl[t][e] * abs(Wg[e][i]) for e in range(E))
    M["dx"] = Mdx
    M["dlogits"] = Mdl
    M["dw_gate"] = [[sum(Mdl[t][e] * abs(X[t][i]) for t in range(T)) for i in range(d)]
                    for e in range(E)]
    M["dgate_bias"] = [sum(Mdl[t][e] for t in range(T)) for e in range(E)] if has_gate_bias else None


def brute_scales(p, dout, k, renorm, capacity, daux, residual):
    """Every magnitude of moe_backward, element by element (see the module docstring)."""
    lg = orc.logits(p["x"], p["w_gate"], p["gate_bias"])
    idx, gate, _ = orc.route(lg, k, renorm)
    counts, offsets, dest, _ = orc.permute(idx, p["w_gate"].shape[0], capacity)
    X, Wg = bwd.widen(p["x"]).tolist(), bwd.widen(p["w_gate"]).tolist()
    W1, W2 = bwd.widen(p["w1"]).tolist(), bwd.widen(p["w2"]).tolist()
    B1, B2 = bwd.widen(p["b1"]).tolist(), bwd.widen(p["b2"]).tolist()
    dO = np.asarray(dout, np.float64).tolist()
    T, d, E, h = len(X), len(X[0]), len(Wg), len(W1[0])
    M = _empty(E, d, h, True, True)
    Mdx = [[0.0] * d for _ in range(T)]
    Mdg = [[0.0] * k for _ in range(T)]
    Mdl = [[0.0] * E for _ in range(T)]
    for t in range(T):
        for j in range(k):
            if dest[t * k + j] < 0:
                continue
            Mdg[t][j], _ = _expert_terms(X, W1, B1, W2, B2, dO, t, int(idx[t, j]), gate[t, j], M, Mdx)
        z = [math.exp(v - max(lg[t])) for v in lg[t]]
        prob = [v / sum(z) for v in z]
        if renorm:
            inner = sum(abs(gate[t, i]) * Mdg[t][i] for i in range(k))
            for j in range(k):
                Mdl[t][int(idx[t, j])] += abs(gate[t, j]) * (Mdg[t][j] + inner)
        else:
            m = [0.0] * E
            for j in range(k):
                m[int(idx[t, j])] += Mdg[t][j]
            pm = sum(prob[e] * m[e] for e in range(E))
            for e in range(E):
                Mdl[t][e] += prob[e] * (m[e] + pm)
        if daux:
            dpa = [abs(daux) * E * counts[e] / (float(T) * T) for e in range(E)]
            pd = sum(prob[e] * dpa[e] for e in range(E))
            for e in range(E):
                Mdl[t][e] += prob[e] * (dpa[e] + pd)
    M["dgate"] = Mdg
    _router_tail(X, Wg, dO, Mdl, residual, p["gate_bias"] is not None, M, Mdx)
    return M


def brute_scales_ec(p, dout, C, residual):
    """Every magnitude of moe_backward_ec, element by element: each chosen
    (token, expert) pair with its probability as the gate, then the
    full-softmax backward of the gate magnitudes."""
    lg = orc.logits(p["x"], p["w_gate"], p["gate_bias"])
    prob = orc.ec_scores(lg)
    offsets, st, _, _ = orc.expert_choice(prob, C)
    X, Wg = bwd.widen(p["x"]).tolist(), bwd.widen(p["w_gate"]).tolist()
    W1, W2 = bwd.widen(p["w1"]).tolist(), bwd.widen(p["w2"]).tolist()
    B1, B2 = bwd.widen(p["b1"]).tolist(), bwd.widen(p["b2"]).tolist()
    dO = np.asarray(dout, np.float64).tolist()
    T, d, E, h = len(X), len(X[0]), len(Wg), len(W1[0])
    M = _empty(E, d, h, True, True)
    Mdx = [[0.0] * d for _ in range(T)]
    Mdg = [[0.0] * E for _ in range(T)]
    for e in range(E):
        for t in st[offsets[e]:offsets[e + 1]].tolist():
            Mdg[t][e], _ = _expert_terms(X, W1, B1, W2, B2, dO, t, e, prob[t, e], M, Mdx)
    Mdl = [[0.0] * E for _ in range(T)]
    for t in range(T):
        pm = sum(prob[t, e] * Mdg[t][e] for e in range(E))
        for e in range(E):
            Mdl[t][e] = prob[t, e] * (Mdg[t][e] + pm)
    M["dgate"] = Mdg
    _router_tail(X, Wg, dO, Mdl, residual, p["gate_bias"] is not None, M, Mdx)
    return M


def _compare(M, got, names):
    for n in names:
        want = M[n]
        if want is None:
            assert got[n] is None, n
            continue
        np.testing.assert_allclose(got[n], np.array(want), rtol=1e-12, atol=1e-300, err_msg=n)


NAMES = ("dx", "dw_gate", "dgate_bias", "dw1", "db1", "dw2", "db2", "dgate", "dlogits")

# name: (seed, T, d, h, E, k, renorm, capacity, daux, residual, gate_bias)
TC_CASES = {
    "top2_renorm_aux": (31, 7, 4, 5, 4, 2, True, -1, 0.3, False, False),
    "top2_renorm_drops": (32, 8, 3, 4, 3, 2, True, 3, 0.0, True, True),
    "top1_prob_gate_drops_aux": (33, 9, 4, 3, 3, 1, False, 2, 0.7, True, True),
    "top2_prob_gate": (34, 6, 3, 5, 4, 2, False, -1, -0.4, False, True),
}


@pytest.mark.parametrize("name", sorted(TC_CASES))
def test_token_choice_scales_are_their_definition(name):
    seed, T, d, h, E, k, renorm, cap, daux, res, gb = TC_CASES[name]
    p, dout = _layer(seed, T, d, h, E, gb)
    r = bwd.moe_backward(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], k, renorm, cap,
                         dout, daux, gate_bias=p["gate_bias"], residual=res, want_scale=True)
    if cap >= 0:
        assert (r["dest_row"] < 0).any(), "case must drop some assignments"
    _compare(brute_scales(p, dout, k, renorm, cap, daux, res), r["scale"], NAMES)


@pytest.mark.parametrize("C,res,gb", [(2, False, False), (4, True, True), (9, True, False)])
def test_expert_choice_scales_are_their_definition(C, res, gb):
    p, dout = _layer(40 + C, 9, 3, 4, 3, gb)
    r = bwd.moe_backward_ec(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], C, dout,
                            gate_bias=p["gate_bias"], residual=res, want_scale=True)
    _compare(brute_scales_ec(p, dout, C, res), r["scale"], NAMES)

"""Pins for the backward oracle: gradients checked by routes that do not use its formulas.

- Central finite differences of L = <dout, out> + daux * aux_loss through the
  forward oracle (the C library), for every input element of tiny layers
  that cover renormalised top-2, top-1 with capacity drops, a router bias,
  the residual path and k = E. Inputs sit on a 2^-10 grid so that x +- 2^-10
  is exact in float32, and each case asserts that no perturbation changes
  the routing (the gradient is that of the fixed-routing branch).
- torch.autograd in float64 through the forward written a second time with
  torch ops (masked-logit softmax for the gates, as in the gate equation).
- Closed forms and invariants: each row of dlogits sums to 0; the
  aux-only gradient at uniform router probabilities; k = E with identical
  experts, where the layer is a dense FFN whatever the gates are, so the
  gate path gives the router no gradient and the summed expert gradients
  equal the dense ones.

MOE_ORACLE_BWD may name a copy of the backward module to test in its
place (the mutation tests plant mistakes in such copies).
"""
import importlib.util
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc


def _bwd_module():
    path = os.environ.get("MOE_ORACLE_BWD")
    if not path:
        from oracle import backward
        return backward
    spec = importlib.util.spec_from_file_location("oracle.backward_under_test", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


bwd = _bwd_module()

H = 2.0 ** -10  # finite-difference step; inputs are multiples of it


def _grid(a):
    return np.ascontiguousarray(np.round(np.asarray(a) / H) * H, dtype=np.float32)


def _layer(seed, T, d, h, E, gate_bias=False):
    rng = np.random.default_rng(seed)
    p = dict(
        x=_grid(rng.standard_normal((T, d))),
        w_gate=_grid(rng.standard_normal((E, d)) * 1.5 / math.sqrt(d)),
        w1=_grid(rng.standard_normal((E, h, d)) / math.sqrt(d)),
        b1=_grid(rng.standard_normal((E, h)) * 0.3),
        w2=_grid(rng.standard_normal((E, d, h)) / math.sqrt(h)),
        b2=_grid(rng.standard_normal((E, d)) * 0.3),
    )
    if gate_bias:
        p["gate_bias"] = _grid(rng.standard_normal(E) * 0.5)
    dout = rng.standard_normal((T, d))
    return p, dout


def _forward(p, k, renorm, capacity, residual):
    return orc.moe_forward(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], k, renorm,
                           capacity, gate_bias=p.get("gate_bias"), residual=residual)


def _loss(p, dout, daux, k, renorm, capacity, residual):
    r = _forward(p, k, renorm, capacity, residual)
    return float((dout * r["out"]).sum() + daux * r["loss"]), r


def _backward(p, dout, daux, k, renorm, capacity, residual):
    return bwd.moe_backward(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], k, renorm,
                            capacity, dout, daux, gate_bias=p.get("gate_bias"), residual=residual)


GRAD_OF = dict(x="dx", w_gate="dw_gate", gate_bias="dgate_bias", w1="dw1", b1="db1", w2="dw2",
               b2="db2")

# name: (seed, T, d, h, E, k, renorm, capacity, residual, gate_bias, daux)
FD_CASES = {
    "top2_renorm": (11, 7, 6, 5, 4, 2, True, -1, False, False, 0.3),
    "top1_capacity_bias_residual": (12, 9, 5, 6, 3, 1, False, 2, True, True, 0.7),
    "top2_renorm_capacity": (13, 8, 5, 4, 3, 2, True, 3, False, False, 0.5),
    "top2_no_renorm_residual": (14, 6, 4, 5, 4, 2, False, -1, True, True, 0.0),
    "k_equals_E": (15, 5, 4, 6, 3, 3, True, -1, True, False, 1.1),
}


@pytest.mark.parametrize("name", sorted(FD_CASES))
def test_finite_differences(name):
    seed, T, d, h, E, k, renorm, cap, res, gb, daux = FD_CASES[name]
    p, dout = _layer(seed, T, d, h, E, gb)
    L0, r0 = _loss(p, dout, daux, k, renorm, cap, res)
    if cap >= 0:
        assert (r0["dest_row"] < 0).any(), "case must drop some assignments"
    g = _backward(p, dout, daux, k, renorm, cap, res)
    for pname, gname in GRAD_OF.items():
        if pname not in p:
            assert g[gname] is None
            continue
        a = p[pname]
        num = np.zeros(a.shape, np.float64)
        for i in np.ndindex(a.shape):
            keep = a[i]
            a[i] = keep + H
            Lp, rp = _loss(p, dout, daux, k, renorm, cap, res)
            a[i] = keep - H
            Lm, rm = _loss(p, dout, daux, k, renorm, cap, res)
            a[i] = keep
            for rr in (rp, rm):
                assert np.array_equal(rr["idx"], r0["idx"]), f"{pname}{i} changes the routing"
                assert np.array_equal(rr["dest_row"], r0["dest_row"])
            num[i] = (Lp - Lm) / (2 * H)
        ana = g[gname]
        scale = max(1.0, float(np.abs(ana).max()))
        err = float(np.abs(num - ana).max())
        assert err <= 2e-5 * scale, f"{name} {gname}: max |fd - oracle| = {err} (scale {scale})"


# --------------------------------------------------------------- autograd --

def _torch_forward(p, dout, daux, k, renorm, capacity, residual, idx, dest):
    """The layer in torch float64 ops with the routing held fixed."""
    t = {n: torch.tensor(bwd.widen(v), dtype=torch.float64, requires_grad=True)
         for n, v in p.items()}
    X, Wg = t["x"], t["w_gate"]
    T, d = X.shape
    E = Wg.shape[0]
    lg = X @ Wg.T + (t["gate_bias"] if "gate_bias" in t else 0.0)
    prob = torch.softmax(lg, dim=1)
    sel = torch.tensor(idx, dtype=torch.long)
    if renorm:
        masked = torch.full_like(lg, -torch.inf).scatter(1, sel, lg.gather(1, sel))
        gates = torch.softmax(masked, dim=1).gather(1, sel)
    else:
        gates = prob.gather(1, sel)
    out = X.clone() if residual else torch.zeros_like(X)
    dest = dest.reshape(T, k)
    for tt in range(T):
        for j in range(k):
            if dest[tt, j] < 0:
                continue
            e = int(idx[tt, j])
            z = t["w1"][e] @ X[tt] + t["b1"][e]
            y = t["w2"][e] @ torch.nn.functional.silu(z) + t["b2"][e]
            out = out.index_add(0, torch.tensor([tt]), (gates[tt, j] * y)[None])
    counts = torch.tensor(np.bincount(idx.ravel(), minlength=E), dtype=torch.float64)
    aux = E * ((prob.sum(0) / T) * (counts / T)).sum()
    L = (torch.tensor(dout) * out).sum() + daux * aux
    L.backward()
    return {GRAD_OF[n]: v.grad.numpy() for n, v in t.items()}


@pytest.mark.parametrize("renorm,cap,res,gb,k", [(True, -1, False, False, 2),
                                                  (False, 5, True, True, 1),
                                                  (True, 9, True, True, 3)])
def test_matches_autograd(renorm, cap, res, gb, k):
    p, dout = _layer(21 + k, 40, 16, 24, 6, gb)
    g = _backward(p, dout, 0.4, k, renorm, cap, res)
    ref = _torch_forward(p, dout, 0.4, k, renorm, cap, res, g["idx"], g["dest_row"])
    for name, v in ref.items():
        scale = max(1e-30, float(np.abs(v).max()))
        err = float(np.abs(g[name] - v).max())
        assert err <= 1e-11 * scale, f"{name}: {err} vs scale {scale}"


# ------------------------------------------------ closed forms, invariants --

def test_logit_gradient_rows_sum_to_zero():
    p, dout = _layer(31, 50, 12, 10, 8, True)
    for renorm, k in ((True, 2), (False, 1), (False, 3)):
        g = _backward(p, dout, 0.9, k, renorm, 20, True)
        np.testing.assert_allclose(g["dlogits"].sum(axis=1), 0.0, atol=1e-13)
        np.testing.assert_allclose(g["dgate_bias"].sum(), 0.0, atol=1e-12)


def test_aux_gradient_at_uniform_probabilities():
    """W_g = 0 and no bias: p = 1/E, ties route every token to experts 0..k-1,
    and dl[t,e] = daux * (counts_e - k T / E) / T^2 (the gate path is
    switched off with dout = 0)."""
    T, d, h, E, k, daux = 24, 8, 6, 5, 2, 1.7
    p, _ = _layer(41, T, d, h, E)
    p["w_gate"][:] = 0
    g = _backward(p, np.zeros((T, d)), daux, k, True, -1, False)
    counts = np.array([T] * k + [0] * (E - k), np.float64)
    want = np.broadcast_to(daux * (counts - k * T / E) / T ** 2, (T, E))
    np.testing.assert_allclose(g["dlogits"], want, rtol=0, atol=1e-15)
    np.testing.assert_allclose(g["dw1"], 0.0, atol=0)
    np.testing.assert_allclose(g["dx"], g["dlogits"] @ np.zeros((E, d)), atol=0)


def test_identical_experts_make_a_dense_ffn():
    """k = E, renormalised: sum_j g_j = 1, so with one FFN in every slot the
    layer is that FFN; the gates get equal gradients, the router none, and
    the expert gradients summed over experts are the dense FFN's gradients
    (written here with torch autograd on the dense FFN)."""
    T, d, h, E = 16, 8, 12, 4
    p, dout = _layer(51, T, d, h, E)
    for n in ("w1", "b1", "w2", "b2"):
        p[n][:] = p[n][0]
    g = _backward(p, dout, 0.0, E, True, -1, False)
    np.testing.assert_allclose(g["dlogits"], 0.0, atol=1e-12)
    X = torch.tensor(bwd.widen(p["x"]), requires_grad=True)
    W1 = torch.tensor(bwd.widen(p["w1"][0]), requires_grad=True)
    b1 = torch.tensor(bwd.widen(p["b1"][0]), requires_grad=True)
    W2 = torch.tensor(bwd.widen(p["w2"][0]), requires_grad=True)
    b2 = torch.tensor(bwd.widen(p["b2"][0]), requires_grad=True)
    y = torch.nn.functional.silu(X @ W1.T + b1) @ W2.T + b2
    (torch.tensor(dout) * y).sum().backward()
    for mine, ref in ((g["dw1"].sum(0), W1.grad), (g["db1"].sum(0), b1.grad),
                      (g["dw2"].sum(0), W2.grad), (g["db2"].sum(0), b2.grad), (g["dx"], X.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_dropped_assignments_get_no_expert_gradient():
    """Capacity 0 drops everything: the experts see no rows, the gates get
    no gradient, only the aux loss and the residual reach the inputs."""
    p, dout = _layer(61, 10, 6, 5, 3)
    g = _backward(p, dout, 0.5, 1, False, 0, True)
    assert np.all(g["dw1"] == 0) and np.all(g["db2"] == 0) and np.all(g["dgate"] == 0)
    want = bwd.widen(dout) + g["dlogits"] @ bwd.widen(p["w_gate"])
    np.testing.assert_allclose(g["dx"], want, rtol=1e-14, atol=1e-14)


def test_error_scales_bound_the_gradients():
    """The magnitudes returned with want_scale are sums of absolute values
    of the terms of each element, so they bound the gradient itself."""
    p, dout = _layer(71, 40, 12, 10, 6, True)
    for renorm, k, cap in ((True, 2, -1), (False, 1, 8), (True, 3, 15)):
        g = _backward(p, dout, 0.3, k, renorm, cap, True)
        g2 = bwd.moe_backward(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], k, renorm,
                              cap, dout, 0.0, gate_bias=p["gate_bias"], residual=True,
                              want_scale=True)
        for name, M in g2["scale"].items():
            ref = g2[name]
            assert M.shape == ref.shape, name
            assert np.all(M >= np.abs(ref) * (1 - 1e-12) - 1e-15), name
        # daux only moves dlogits and what follows from it
        np.testing.assert_allclose(g2["dw1"], g["dw1"], rtol=0, atol=0)


def test_sampled_backward_matches_the_whole_one():
    """moe_backward_sampled picks the same numbers out of the same chain as
    moe_backward, for tokens, dW1 rows, dW2 columns and db2 of several
    experts, in both gate modes, with drops and the aux term."""
    for renorm, k, cap, res in ((True, 2, 9, False), (False, 1, 6, True)):
        p, dout = _layer(81 + k, 30, 8, 12, 5, not renorm)
        lg = orc.logits(p["x"], p["w_gate"], p.get("gate_bias"))
        full = bwd.moe_backward(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], k,
                                renorm, cap, dout, 0.7, gate_bias=p.get("gate_bias"), residual=res,
                                lg=lg, want_scale=True)
        fetch = lambda e: (p["w1"][e], p["b1"][e], p["w2"][e], p["b2"][e])  # noqa: E731
        toks = [0, 3, 17, 29]
        rows = [(0, 1), (2, 11), (4, 0)]
        cols = [(1, 5), (3, 0)]
        sm = bwd.moe_backward_sampled(p["x"], p["w_gate"], fetch, k, renorm, cap, dout, 0.7, lg,
                                      gate_bias=p.get("gate_bias"), residual=res, tokens=toks,
                                      w1_rows=rows, w2_cols=cols, b2_experts=[0, 4])
        sc = full["scale"]
        for name in ("dx", "dgate", "dlogits"):
            v, m = sm[name]
            np.testing.assert_allclose(v, full[name][toks], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(m, sc[name][toks], rtol=1e-12, atol=1e-13)
        for (e, n) in rows:
            np.testing.assert_allclose(sm["dw1"][(e, n)][0], full["dw1"][e][n], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sm["dw1"][(e, n)][1], sc["dw1"][e][n], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sm["db1"][(e, n)][0], full["db1"][e][n], rtol=1e-12, atol=1e-13)
        for (e, n) in cols:
            np.testing.assert_allclose(sm["dw2"][(e, n)][0], full["dw2"][e][:, n], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sm["dw2"][(e, n)][1], sc["dw2"][e][:, n], rtol=1e-12, atol=1e-13)
        for e in (0, 4):
            np.testing.assert_allclose(sm["db2"][e][0], full["db2"][e], rtol=1e-12, atol=1e-13)


def test_router_backward_over_every_token_matches_the_whole_one():
    """router_backward_all, which takes each expert's outputs from the forward
    oracle's expert_rows, gives moe_backward's dgate, dlogits, dW_g and db_g
    and their magnitudes, in both gate modes, with drops, a router bias and
    the aux term."""
    for renorm, k, cap, gb, daux in ((True, 2, 9, False, 0.7), (False, 1, 6, True, 0.7),
                                     (True, 3, -1, True, 0.0), (False, 2, 0, False, 0.3)):
        p, dout = _layer(95 + k, 30, 8, 12, 5, gb)
        lg = orc.logits(p["x"], p["w_gate"], p.get("gate_bias"))
        full = bwd.moe_backward(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], k,
                                renorm, cap, dout, daux, gate_bias=p.get("gate_bias"), lg=lg,
                                want_scale=True)
        fetch = lambda e: (p["w1"][e], p["b1"][e], p["w2"][e], p["b2"][e])  # noqa: E731
        rb = bwd.router_backward_all(p["x"], p["w_gate"], fetch, k, renorm, cap, dout, daux, lg,
                                     gate_bias=p.get("gate_bias"))
        sc = full["scale"]
        names = ("dgate", "dlogits", "dw_gate") + (("dgate_bias",) if gb else ())
        for name in names:
            v, m = rb[name]
            np.testing.assert_allclose(v, full[name], rtol=1e-10, atol=1e-12, err_msg=name)
            np.testing.assert_allclose(m, sc[name], rtol=1e-10, atol=1e-12, err_msg=name)
        if not gb:
            assert rb["dgate_bias"] is None
        if cap == 0:
            assert not np.any(rb["dgate"][0])


# ------------------------------------------------------------ Expert Choice --

def _ec_loss(p, dout, C, res):
    r = orc.moe_forward_ec(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], C,
                           gate_bias=p.get("gate_bias"), residual=res)
    return float((dout * r["out"]).sum()), r


@pytest.mark.parametrize("C,res,gb", [(3, False, False), (5, True, True), (9, True, False)])
def test_expert_choice_finite_differences(C, res, gb):
    """Central differences of <dout, out> through the Expert Choice forward
    oracle, every input element of a tiny layer (selection unchanged by
    every perturbation)."""
    p, dout = _layer(91 + C, 9, 5, 6, 3, gb)
    L0, r0 = _ec_loss(p, dout, C, res)
    g = bwd.moe_backward_ec(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], C, dout,
                            gate_bias=p.get("gate_bias"), residual=res)
    for pname, gname in GRAD_OF.items():
        if pname not in p:
            assert g[gname] is None
            continue
        a = p[pname]
        num = np.zeros(a.shape)
        for i in np.ndindex(a.shape):
            keep = a[i]
            a[i] = keep + H
            Lp, rp = _ec_loss(p, dout, C, res)
            a[i] = keep - H
            Lm, rm = _ec_loss(p, dout, C, res)
            a[i] = keep
            for rr in (rp, rm):
                assert np.array_equal(rr["dest_row"], r0["dest_row"]), f"{pname}{i} changes the selection"
            num[i] = (Lp - Lm) / (2 * H)
        scale = max(1.0, float(np.abs(g[gname]).max()))
        err = float(np.abs(num - g[gname]).max())
        assert err <= 2e-5 * scale, f"C={C} {gname}: max |fd - oracle| = {err}"


def test_expert_choice_backward_invariants():
    """Rows of dlogits sum to 0; C = T (every expert takes every token) is
    the token-choice layer at k = E without renormalisation, so the two
    backward oracles agree there; magnitudes bound the gradients."""
    p, dout = _layer(97, 12, 6, 8, 4, True)
    g = bwd.moe_backward_ec(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], 4, dout,
                            gate_bias=p["gate_bias"], residual=True, want_scale=True)
    np.testing.assert_allclose(g["dlogits"].sum(axis=1), 0.0, atol=1e-13)
    for name, M in g["scale"].items():
        assert np.all(M >= np.abs(g[name]) * (1 - 1e-12) - 1e-15), name
    ec = bwd.moe_backward_ec(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], 12, dout,
                             gate_bias=p["gate_bias"], residual=True)
    tc = bwd.moe_backward(p["x"], p["w_gate"], p["w1"], p["b1"], p["w2"], p["b2"], 4, False, -1,
                          dout, 0.0, gate_bias=p["gate_bias"], residual=True)
    for name in ("dx", "dw_gate", "dgate_bias", "dw1", "db1", "dw2", "db2", "dlogits"):
        np.testing.assert_allclose(ec[name], tc[name], rtol=1e-11, atol=1e-12)

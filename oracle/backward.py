"""CPU oracle for the backward pass of one MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. It shares nothing with the GPU library.

What it computes: the gradients of the scalar

    L = sum_t <dout[t], out[t]> + daux * aux_loss

with respect to every input of the layer (x, W_g, b_g, W1, b1, W2, b2), where
out and aux_loss are the forward of ``oracle.moe_forward``: the gate equation
G(x) = softmax(TopK(x . W_g)) and output sum_i G_i E_i(x) of the routing page
"MoE混合专家模型路由机制原理与稀疏激活实现" (section "MoE混合专家模型架构与门控路由原理"),
its Expert w2(silu(w1 x + b1)) + b2 and load_balancing_loss E * sum f * P
(section "Top-K门控路由的PyTorch实现"), and its capacity rule (section
"Expert Choice路由策略与容量因子调优"). The aux loss exists to be trained
against (same section; the router of "MoE模型稀疏推理原理与生产落地实战",
section 2.3, is trained jointly with the experts and keeps its two largest
logits before the softmax so that gradients reach them).

Readings (where the pages say nothing about gradients):
  - the top-k selection, the expert counts and the capacity drop are
    piecewise constant in the inputs: no gradient flows through them, only
    through the gate values, the expert FFNs and the probabilities of the
    aux loss;
  - a dropped (token, slot) contributes nothing to out, so its gate gets no
    gradient; with renormalised gates the kept gates still depend on the
    dropped slot's logit through the renormalisation;
  - aux_loss = E * sum_e (prob_sum_e / T) * (counts_e / T): the gradient
    reaches the probabilities, d aux / d p[t,e] = E * counts_e / T^2.

The chain rule is written out step by step, in reverse order of the forward,
in double precision from the exact input values; a library matmul does each
contraction. Every function below names the forward step it differentiates.
"""
from __future__ import annotations

import numpy as np

from . import oracle as fwd


def widen(a) -> np.ndarray:
    """float32 -> float64, bf16 bit patterns (uint16) -> float64, both exact."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (np.ascontiguousarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """SiLU(z) = z / (1 + e^-z) (the Expert's activation)."""
    return z * sigmoid(z)


def silu_grad(z):
    """d/dz [z s(z)] = s(z) + z s(z) (1 - s(z)), s the logistic function."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def softmax(lg):
    """p[t,e] = exp(l - max) / sum_e exp(l - max): the router's softmax over all experts."""
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def softmax_grad(p, dp):
    """Backward of a row softmax: dl = p * (dp - sum_e p dp)."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def gate_grad(lg, idx, gate, dgate, renorm: bool):
    """Backward of the gates to the logits.

    renorm: g_j = exp(l_{S_j}) / sum_{i in S} exp(l_{S_i}), the softmax over
    the k selected logits (the masked-softmax form of the gate equation):
    dl[S_j] = g_j (dg_j - sum_i g_i dg_i), zero for unselected experts.
    Otherwise g_j = p[t, S_j] (the full softmax): the gate gradients land on
    p and go through the softmax backward.
    """
    T, E = lg.shape
    k = idx.shape[1]
    dl = np.zeros((T, E), np.float64)
    rows = np.repeat(np.arange(T), k)
    if renorm:
        inner = (gate * dgate).sum(axis=1, keepdims=True)
        np.add.at(dl, (rows, idx.ravel()), (gate * (dgate - inner)).ravel())
        return dl
    dp = np.zeros((T, E), np.float64)
    np.add.at(dp, (rows, idx.ravel()), dgate.ravel())
    return softmax_grad(softmax(lg), dp)


def aux_grad(lg, counts, daux: float):
    """Backward of aux = E * sum_e (sum_t p[t,e] / T) (counts_e / T) to the logits."""
    T, E = lg.shape
    dp = np.broadcast_to(daux * E * counts.astype(np.float64) / (float(T) * T), (T, E))
    return softmax_grad(softmax(lg), dp)


def expert_backward(xe, w1e, b1e, w2e, b2e, dy):
    """Backward of y = W2 SiLU(W1 x + b1) + b2 over the rows of one expert.

    xe [n, d] (the expert's input rows), dy [n, d]. Returns (y, dx, dW1, db1,
    dW2, db2) with y the forward output of the rows (the gate's gradient needs
    it).
    """
    z = xe @ w1e.T + (0.0 if b1e is None else b1e)
    a = silu(z)
    y = a @ w2e.T + (0.0 if b2e is None else b2e)
    dw2 = dy.T @ a
    db2 = dy.sum(axis=0)
    da = dy @ w2e
    dz = da * silu_grad(z)
    dw1 = dz.T @ xe
    db1 = dz.sum(axis=0)
    dx = dz @ w1e
    return y, dx, dw1, db1, dw2, db2


def moe_backward(x, w_gate, w1, b1, w2, b2, k: int, renorm: bool, capacity: int, dout,
                 daux: float = 0.0, gate_bias=None, residual: bool = False, lg=None,
                 want_scale: bool = False):
    """Gradients of L = <dout, out> + daux * aux_loss for the whole layer.

    ``lg``: logits to route from (same-logits mode, e.g. the GPU's fp32
    logits); computed in double when None. Routing, counts and the
    permutation come from the forward oracle. Returns a dict with dx,
    dw_gate, dgate_bias (None without a router bias), dw1, db1, dw2, db2 and
    the intermediates dlogits [T,E], dgate [T,k], y_rows [R,d] (the forward
    output of each kept row, in permuted order).

    ``want_scale``: also return ``scale``, a dict with the same keys holding
    for every element the sum of the absolute values of the products it is
    made of, carried through the chain (see ``_scales``): the yardstick of a
    rounding-error bound, not a gradient.
    """
    X = widen(x)
    Wg = widen(w_gate)
    W1, W2 = widen(w1), widen(w2)
    B1, B2 = widen(b1), widen(b2)
    dO = widen(dout)
    T, d = X.shape
    E, h = W1.shape[0], W1.shape[1]
    if lg is None:
        lg = fwd.logits(x, w_gate, gate_bias)
    lg = np.asarray(lg, dtype=np.float64)
    idx, gate, _ = fwd.route(lg, k, renorm)
    counts, offsets, dest, st = fwd.permute(idx, E, capacity)
    R = int(offsets[E])
    slot_of_row = np.empty(R, np.int64)  # flat slot t*k + j of each kept row
    kept = np.nonzero(dest >= 0)[0]
    slot_of_row[dest[kept]] = kept

    dx = dO.copy() if residual else np.zeros((T, d), np.float64)
    dw1 = np.zeros((E, h, d), np.float64)
    dw2 = np.zeros((E, d, h), np.float64)
    db1 = np.zeros((E, h), np.float64)
    db2 = np.zeros((E, d), np.float64)
    dgate = np.zeros(T * k, np.float64)
    y_rows = np.zeros((R, d), np.float64)
    gflat = gate.ravel()
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        tok = st[r0:r1]
        slots = slot_of_row[r0:r1]
        # combine: out[t] += g[t,j] y[row]  ->  dy[row] = g dout[t]
        dy = gflat[slots][:, None] * dO[tok]
        y, dxe, dw1[e], db1[e], dw2[e], db2[e] = expert_backward(
            X[tok], W1[e], None if B1 is None else B1[e], W2[e], None if B2 is None else B2[e], dy)
        # ... and dg[t,j] = <dout[t], y[row]>
        dgate[slots] = (dO[tok] * y).sum(axis=1)
        y_rows[r0:r1] = y
        # the expert's input rows are gathered from x: scatter-add back
        np.add.at(dx, tok, dxe)
    dgate = dgate.reshape(T, k)
    dl = gate_grad(lg, idx, gate, dgate, renorm)
    if daux:
        dl = dl + aux_grad(lg, counts, daux)
    # logits = x W_g^T + b_g
    dw_gate = dl.T @ X
    dgate_bias = None if gate_bias is None else dl.sum(axis=0)
    dx += dl @ Wg
    res = dict(dx=dx, dw_gate=dw_gate, dgate_bias=dgate_bias, dw1=dw1, db1=db1, dw2=dw2,
               db2=db2, dlogits=dl, dgate=dgate, y_rows=y_rows, idx=idx, gate=gate,
               counts=counts, offsets=offsets, dest_row=dest, sorted_token=st, logits=lg)
    if want_scale:
        res["scale"] = _scales(X, Wg, W1, B1, W2, dO, lg, idx, gate, dest, st, offsets,
                               slot_of_row, y_rows, renorm, residual, gate_bias is not None,
                               B2 is not None, counts, daux)
    return res


def _scales(X, Wg, W1, B1, W2, dO, lg, idx, gate, dest, st, offsets, slot_of_row, y_rows,
            renorm, residual, has_gate_bias, has_b2, counts, daux):
    """Per-element magnitude M of every gradient: the backward run again on
    absolute values, so that |result| <= M (triangle inequality) and each
    rounded operand or product that feeds an element contributes at most
    its own relative error times M. Where z, the pre-activation, is itself
    a rounded value, the magnitudes also carry the change of the function
    of z under a relative change u of z: SiLU moves by at most
    |SiLU'(z) z| u, counted as |SiLU(z)| + |SiLU'(z) z| / 4, and SiLU'
    by at most |z| u / 2 (|SiLU''| <= 1/2), counted as |SiLU'(z)| + |z| / 8
    (so that four relative errors u of the magnitude cover the roundings
    of z, of the operands and of the result)."""
    T, d = X.shape
    E, h = W1.shape[0], W1.shape[1]
    k = idx.shape[1]
    aX, aO = np.abs(X), np.abs(dO)
    m_dx = aO.copy() if residual else np.zeros((T, d))
    m = {n: np.zeros(s) for n, s in (("dw1", (E, h, d)), ("dw2", (E, d, h)), ("db1", (E, h)),
                                     ("db2", (E, d)))}
    m_dg = np.zeros(T * k)
    gflat = gate.ravel()
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        tok = st[r0:r1]
        slots = slot_of_row[r0:r1]
        z = X[tok] @ W1[e].T + (0.0 if B1 is None else B1[e])
        ady = np.abs(gflat[slots])[:, None] * aO[tok]
        m["dw2"][e] = ady.T @ (np.abs(silu(z)) + np.abs(silu_grad(z) * z) / 4.0)
        m["db2"][e] = ady.sum(axis=0)
        adz = (ady @ np.abs(W2[e])) * (np.abs(silu_grad(z)) + np.abs(z) / 8.0)
        m["dw1"][e] = adz.T @ aX[tok]
        m["db1"][e] = adz.sum(axis=0)
        np.add.at(m_dx, tok, adz @ np.abs(W1[e]))
        m_dg[slots] = (aO[tok] * np.abs(y_rows[r0:r1])).sum(axis=1)
    m_dg = m_dg.reshape(T, k)
    m_dl = _router_scales(lg, idx, gate, m_dg, renorm, counts, daux)
    m_dx += m_dl @ np.abs(Wg)
    m.update(dx=m_dx, dw_gate=m_dl.T @ aX, dgate_bias=m_dl.sum(axis=0) if has_gate_bias else None,
             dgate=m_dg, dlogits=m_dl)
    if not has_b2:
        m["db2"] = None
    if B1 is None:
        m["db1"] = None
    return m


def _router_scales(lg, idx, gate, m_dg, renorm, counts, daux):
    """Magnitude of dlogits [T, E] from the magnitude m_dg [T, k] of the
    gate gradients: the gate and aux-loss backward of ``gate_grad`` and
    ``aux_grad`` run on absolute values (the centring term added, not
    subtracted)."""
    T, E = lg.shape
    k = idx.shape[1]
    ag = np.abs(gate)
    rows = np.repeat(np.arange(T), k)
    m_dl = np.zeros((T, E))
    if renorm:
        inner = (ag * m_dg).sum(axis=1, keepdims=True)
        np.add.at(m_dl, (rows, idx.ravel()), (ag * (m_dg + inner)).ravel())
    else:
        p = softmax(lg)
        mdp = np.zeros((T, E))
        np.add.at(mdp, (rows, idx.ravel()), m_dg.ravel())
        m_dl = p * (mdp + (p * mdp).sum(axis=1, keepdims=True))
    if daux:
        p = softmax(lg)
        dpa = np.broadcast_to(abs(daux) * E * counts.astype(np.float64) / (float(T) * T), (T, E))
        m_dl = m_dl + p * (dpa + (p * dpa).sum(axis=1, keepdims=True))
    return m_dl


def router_backward_all(x, w_gate, fetch, k: int, renorm: bool, capacity: int, dout,
                        daux: float, lg, gate_bias=None):
    """The router's gradients over every token, for layers too large for
    ``moe_backward``: dgate [T, k], dlogits [T, E], dW_g [E, d] and db_g [E]
    (None without a router bias), each a (value, magnitude) pair with the
    magnitude as in ``_scales``.

    The gate gradient of a kept slot (t, j) is <dout[t], y>, y the forward
    output of token t in its j-th expert; y comes from the forward oracle's
    ``expert_rows``, one expert at a time over all of its rows (fetch(e) ->
    (w1e, b1e, w2e, b2e) gives the expert's weights). The rest is
    ``gate_grad`` and ``aux_grad`` on all T rows, then logits = x W_g^T + b_g
    backwards.
    """
    X = widen(x)
    dO = widen(dout)
    T = X.shape[0]
    E = np.asarray(w_gate).shape[0]
    lg = np.asarray(lg, dtype=np.float64)
    idx, gate, _ = fwd.route(lg, k, renorm)
    counts, offsets, dest, st = fwd.permute(idx, E, capacity)
    R = int(offsets[E])
    slot_of_row = np.empty(R, np.int64)
    kept = np.nonzero(dest >= 0)[0]
    slot_of_row[dest[kept]] = kept
    dgate = np.zeros(T * k)
    m_dg = np.zeros(T * k)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        tok = st[r0:r1]
        y = fwd.expert_rows(x, tok, *fetch(e))
        dgate[slot_of_row[r0:r1]] = (dO[tok] * y).sum(axis=1)
        m_dg[slot_of_row[r0:r1]] = (np.abs(dO[tok]) * np.abs(y)).sum(axis=1)
    dgate, m_dg = dgate.reshape(T, k), m_dg.reshape(T, k)
    dl = gate_grad(lg, idx, gate, dgate, renorm)
    if daux:
        dl = dl + aux_grad(lg, counts, daux)
    m_dl = _router_scales(lg, idx, gate, m_dg, renorm, counts, daux)
    return dict(dgate=(dgate, m_dg), dlogits=(dl, m_dl), dw_gate=(dl.T @ X, m_dl.T @ np.abs(X)),
                dgate_bias=None if gate_bias is None else (dl.sum(axis=0), m_dl.sum(axis=0)),
                counts=counts, offsets=offsets, idx=idx)


def moe_backward_sampled(x, w_gate, fetch, k: int, renorm: bool, capacity: int, dout, daux: float,
                         lg, gate_bias=None, residual: bool = False, tokens=(), w1_rows=(),
                         w2_cols=(), b2_experts=()):
    """Selected elements of the same gradients, each computed on its own, for
    layers too large for ``moe_backward``.

    fetch(e) -> (w1e, b1e, w2e, b2e) gives one expert's weights. Returns a
    dict of (value, magnitude) pairs, the magnitude as in ``_scales``:
      "dx":      [len(tokens), d] rows of dx, with "dgate" [n, k] and
                 "dlogits" [n, E] of the same tokens;
      "dw1":     {(e, n): row n of dW1[e] ([d])},  "db1": {(e, n): db1[e][n]};
      "dw2":     {(e, n): column n of dW2[e] ([d])};
      "db2":     {e: db2[e] ([d])}.
    Every value follows the expert's rows r (token t_r, slot j_r, gate g_r):
    dy_r = g_r dout[t_r], z_r = W1[e] x[t_r] + b1[e], dZ_r = (dy_r W2[e]) *
    SiLU'(z_r).
    """
    X = widen(x)
    Wg = widen(w_gate)
    dO = widen(dout)
    T, d = X.shape
    E = Wg.shape[0]
    lg = np.asarray(lg, dtype=np.float64)
    idx, gate, _ = fwd.route(lg, k, renorm)
    counts, offsets, dest, st = fwd.permute(idx, E, capacity)
    R = int(offsets[E])
    slot_of_row = np.empty(R, np.int64)
    kept = np.nonzero(dest >= 0)[0]
    slot_of_row[dest[kept]] = kept
    gflat = gate.ravel()
    cache = {}

    def weights(e):
        if e not in cache:
            cache[e] = tuple(widen(a) for a in fetch(e))
        return cache[e]

    def rows_of(e):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        tok = st[r0:r1]
        return tok, gflat[slot_of_row[r0:r1]]

    out = {}
    tokens = np.asarray(tokens, np.int64)
    p = softmax(lg[tokens]) if tokens.size else np.zeros((0, E))
    dxs, mdxs, dgs, mdgs, dls, mdls = [], [], [], [], [], []
    for i, t in enumerate(tokens):
        dx = dO[t].copy() if residual else np.zeros(d)
        mdx = np.abs(dO[t]) if residual else np.zeros(d)
        dg = np.zeros(k)
        mdg = np.zeros(k)
        for j in range(k):
            r = dest[t * k + j]
            if r < 0:
                continue
            w1e, b1e, w2e, b2e = weights(int(idx[t, j]))
            z = w1e @ X[t] + (0.0 if b1e is None else b1e)
            y = w2e @ silu(z) + (0.0 if b2e is None else b2e)
            dg[j] = dO[t] @ y
            mdg[j] = np.abs(dO[t]) @ np.abs(y)
            dy = gflat[t * k + j] * dO[t]
            dz = (dy @ w2e) * silu_grad(z)
            dx += dz @ w1e
            mdz = (np.abs(dy) @ np.abs(w2e)) * (np.abs(silu_grad(z)) + np.abs(z) / 8.0)
            mdx += mdz @ np.abs(w1e)
        # the router row of this token: gates, then the aux term
        ag = np.abs(gate[t])
        dl = np.zeros(E)
        mdl = np.zeros(E)
        if renorm:
            inner = gate[t] @ dg
            np.add.at(dl, idx[t], gate[t] * (dg - inner))
            np.add.at(mdl, idx[t], ag * (mdg + ag @ mdg))
        else:
            dp = np.zeros(E)
            mdp = np.zeros(E)
            np.add.at(dp, idx[t], dg)
            np.add.at(mdp, idx[t], mdg)
            dl += p[i] * (dp - p[i] @ dp)
            mdl += p[i] * (mdp + p[i] @ mdp)
        if daux:
            dpa = daux * E * counts.astype(np.float64) / (float(T) * T)
            dl += p[i] * (dpa - p[i] @ dpa)
            mdl += p[i] * (np.abs(dpa) + p[i] @ np.abs(dpa))
        dx += dl @ Wg
        mdx += mdl @ np.abs(Wg)
        dxs.append(dx)
        mdxs.append(mdx)
        dgs.append(dg)
        mdgs.append(mdg)
        dls.append(dl)
        mdls.append(mdl)
    out["dx"] = (np.array(dxs).reshape(-1, d), np.array(mdxs).reshape(-1, d))
    out["dgate"] = (np.array(dgs).reshape(-1, k), np.array(mdgs).reshape(-1, k))
    out["dlogits"] = (np.array(dls).reshape(-1, E), np.array(mdls).reshape(-1, E))

    out["dw1"], out["db1"], out["dw2"], out["db2"] = {}, {}, {}, {}
    for e, n in w1_rows:
        w1e, b1e, w2e, _ = weights(e)
        tok, g = rows_of(e)
        xe = X[tok]
        dy = g[:, None] * dO[tok]
        z = xe @ w1e[n] + (0.0 if b1e is None else b1e[n])
        dzn = (dy @ w2e[:, n]) * silu_grad(z)
        mdzn = (np.abs(dy) @ np.abs(w2e[:, n])) * (np.abs(silu_grad(z)) + np.abs(z) / 8.0)
        out["dw1"][(e, n)] = (dzn @ xe, mdzn @ np.abs(xe))
        out["db1"][(e, n)] = (dzn.sum(), mdzn.sum())
    for e, n in w2_cols:
        w1e, b1e, _, _ = weights(e)
        tok, g = rows_of(e)
        dy = g[:, None] * dO[tok]
        z = X[tok] @ w1e[n] + (0.0 if b1e is None else b1e[n])
        hn = silu(z)
        mhn = np.abs(hn) + np.abs(silu_grad(z) * z) / 4.0
        out["dw2"][(e, n)] = (hn @ dy, mhn @ np.abs(dy))
    for e in b2_experts:
        tok, g = rows_of(e)
        dy = g[:, None] * dO[tok]
        out["db2"][e] = (dy.sum(axis=0), np.abs(dy).sum(axis=0))
    out.update(offsets=offsets, counts=counts, idx=idx)
    return out


def moe_backward_ec(x, w_gate, w1, b1, w2, b2, C: int, dout, gate_bias=None,
                    residual: bool = False, lg=None, score=None, want_scale: bool = False):
    """Gradients of L = <dout, out> for an Expert Choice layer (``oracle.moe_forward_ec``).

    The selection (each expert's C tokens) is piecewise constant; the gate of
    a chosen pair (t, e) is p[t,e], the softmax over experts of token t's
    logits, so the gate gradients land on p and go through the softmax
    backward. ``lg`` / ``score``: as in ``moe_forward_ec`` (the selection is
    made on ``score``, the gradient flows through the softmax of ``lg``).
    Returns the keys of ``moe_backward`` (dgate is [T, E], 0 where not
    chosen).
    """
    X = widen(x)
    Wg = widen(w_gate)
    W1, W2 = widen(w1), widen(w2)
    B1, B2 = widen(b1), widen(b2)
    dO = widen(dout)
    T, d = X.shape
    E, h = W1.shape[0], W1.shape[1]
    if lg is None:
        lg = fwd.logits(x, w_gate, gate_bias)
    lg = np.asarray(lg, dtype=np.float64)
    p = softmax(lg)
    sel = p if score is None else np.asarray(score, dtype=np.float64)
    offsets, st, dest, gate = fwd.expert_choice(sel, C)
    gate = np.where(dest >= 0, p, 0.0)  # the gate is the probability itself
    dx = dO.copy() if residual else np.zeros((T, d))
    dw1 = np.zeros((E, h, d))
    dw2 = np.zeros((E, d, h))
    db1 = np.zeros((E, h))
    db2 = np.zeros((E, d))
    dgate = np.zeros((T, E))
    mag = dict(dx=np.abs(dO) if residual else np.zeros((T, d)), dw1=np.zeros((E, h, d)),
               dw2=np.zeros((E, d, h)), db1=np.zeros((E, h)), db2=np.zeros((E, d)),
               dgate=np.zeros((T, E)))
    for e in range(E):
        tok = st[offsets[e]:offsets[e + 1]]
        if tok.size == 0:
            continue
        dy = gate[tok, e][:, None] * dO[tok]
        y, dxe, dw1[e], db1[e], dw2[e], db2[e] = expert_backward(
            X[tok], W1[e], None if B1 is None else B1[e], W2[e], None if B2 is None else B2[e], dy)
        dgate[tok, e] = (dO[tok] * y).sum(axis=1)
        np.add.at(dx, tok, dxe)
        if want_scale:
            z = X[tok] @ W1[e].T + (0.0 if B1 is None else B1[e])
            ady = np.abs(dy)
            mag["dw2"][e] = ady.T @ (np.abs(silu(z)) + np.abs(silu_grad(z) * z) / 4.0)
            mag["db2"][e] = ady.sum(axis=0)
            adz = (ady @ np.abs(W2[e])) * (np.abs(silu_grad(z)) + np.abs(z) / 8.0)
            mag["dw1"][e] = adz.T @ np.abs(X[tok])
            mag["db1"][e] = adz.sum(axis=0)
            np.add.at(mag["dx"], tok, adz @ np.abs(W1[e]))
            mag["dgate"][tok, e] = (np.abs(dO[tok]) * np.abs(y)).sum(axis=1)
    dl = softmax_grad(p, dgate)
    dw_gate = dl.T @ X
    dgate_bias = None if gate_bias is None else dl.sum(axis=0)
    dx += dl @ Wg
    res = dict(dx=dx, dw_gate=dw_gate, dgate_bias=dgate_bias, dw1=dw1, db1=db1, dw2=dw2,
               db2=db2, dlogits=dl, dgate=dgate, offsets=offsets, sorted_token=st, dest_row=dest,
               gate=gate, logits=lg)
    if want_scale:
        mdl = p * (mag["dgate"] + (p * mag["dgate"]).sum(axis=1, keepdims=True))
        mag["dx"] += mdl @ np.abs(Wg)
        mag.update(dlogits=mdl, dw_gate=mdl.T @ np.abs(X),
                   dgate_bias=None if gate_bias is None else mdl.sum(axis=0))
        if B1 is None:
            mag["db1"] = None
        if B2 is None:
            mag["db2"] = None
        res["scale"] = mag
    return res

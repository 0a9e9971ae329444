"""CPU oracle for one MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. It drives ``libmoe_oracle.so`` (plain C, double
accumulation, built from ``moe_oracle.c`` in this folder by ``build.py``) and
shares nothing with the GPU library: no kernels, headers, helpers or
constants.

Sources: the routing-principles page "MoE混合专家模型路由机制原理与稀疏激活实现"
(yunthe.com) -- the gate equation G(x)=softmax(TopK(x.W_g)), the output
y=sum_i G_i E_i(x), the TopKRouter / Expert / MoELayer / load_balancing_loss
code section, and the capacity-factor section -- plus the router bias of
section 5.2 of "MoE 架构完整指南" (walkerchi.com). The readings taken where the
pages are silent are listed in the header of ``moe_oracle.c``.

Arrays: floating inputs are numpy ``float32`` arrays, or ``uint16`` arrays
holding bf16 bit patterns (which the C code widens exactly). Every floating
result is ``float64``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB lets the mutation tests load a deliberately broken build
LIB_PATH = os.environ.get("MOE_ORACLE_LIB", os.path.join(_HERE, "libmoe_oracle.so"))

F32, BF16 = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"oracle library not built: {LIB_PATH} (run oracle/build.py)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.orc_silu.argtypes = [P, I, P]
        lib.orc_logits.argtypes = [P, I, I, I, P, I, P, I, P]
        lib.orc_route.argtypes = [P, I, I, I, I, P, P, P, P]
        lib.orc_permute.argtypes = [P, I, I, I, I, P, P, P, P]
        lib.orc_expert_rows.argtypes = [P, I, I, I, P, I, P, P, P, P, I, P]
        lib.orc_combine.argtypes = [P, P, P, I, I, I, P, P, I, P]
        lib.orc_aux.argtypes = [P, P, I, I, P, P, P]
        for f in ("orc_silu", "orc_logits", "orc_route", "orc_permute",
                  "orc_expert_rows", "orc_combine", "orc_aux"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def silu(z: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float64).ravel()
    out = np.empty_like(z)
    _load().orc_silu(_p(z), z.size, _p(out))
    return out


def logits(x, w_gate, gate_bias=None) -> np.ndarray:
    """l[t,e] = sum_i x[t,i] W_g[e,i] (+ b_g[e]); x [T,d], W_g [E,d]."""
    x, w_gate = _c(x), _c(w_gate)
    gb = None if gate_bias is None else np.ascontiguousarray(gate_bias, dtype=np.float32)
    T, d = x.shape
    E = w_gate.shape[0]
    assert w_gate.shape[1] == d
    out = np.empty((T, E), np.float64)
    _load().orc_logits(_p(x), _dt(x), T, d, _p(w_gate), _dt(w_gate), _p(gb), E, _p(out))
    return out


def route(lg, k: int, renorm: bool, want_probs: bool = False):
    """Top-k selection, softmax gates and per-expert probability sums.

    Returns (idx [T,k] int32, gate [T,k] f64, prob_sum [E] f64[, probs [T,E]]).
    ``lg`` may be float32 (GPU logits, widened exactly) or float64.
    """
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float64)
    ps = np.empty(E, np.float64)
    probs = np.empty((T, E), np.float64) if want_probs else None
    _load().orc_route(_p(lg), T, E, k, int(bool(renorm)), _p(idx), _p(gate), _p(ps), _p(probs))
    return (idx, gate, ps, probs) if want_probs else (idx, gate, ps)


def permute(idx, E: int, capacity: int):
    """Counting sort by expert with capacity (capacity < 0: unlimited).

    Returns (counts [E], offsets [E+1], dest_row [T*k], sorted_token [R]).
    """
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    dest = np.empty(T * k, np.int32)
    st = np.full(T * k, -1, np.int32)
    _load().orc_permute(_p(idx), T, k, E, int(capacity), _p(counts), _p(offsets), _p(dest), _p(st))
    return counts, offsets, dest, st[: offsets[E]].copy()


def expert_rows(x, tok, w1e, b1e, w2e, b2e) -> np.ndarray:
    """y[r] = W2 SiLU(W1 x[tok_r] + b1) + b2 for one expert; returns [n, d] f64."""
    x = _c(x)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    w1e, w2e, b1e, b2e = _c(w1e), _c(w2e), _c(b1e), _c(b2e)
    d = x.shape[1]
    h = w1e.shape[0]
    assert w1e.shape == (h, d) and w2e.shape == (d, h)
    wdt = _dt(w1e)
    for a in (w2e, b1e, b2e):
        if a is not None and _dt(a) != wdt:
            raise TypeError("expert tensors must share one dtype")
    y = np.empty((tok.size, d), np.float64)
    _load().orc_expert_rows(_p(x), _dt(x), d, h, _p(tok), tok.size, _p(w1e), _p(b1e),
                            _p(w2e), _p(b2e), wdt, _p(y))
    return y


def combine(y_slots, dest, gate, tok, residual=None) -> np.ndarray:
    """out[i] = residual[tok_i] + sum_{j kept} gate[i,j] y_slots[i,j] (j ascending)."""
    y_slots = np.ascontiguousarray(y_slots, dtype=np.float64)
    ntok, k, d = y_slots.shape
    dest = np.ascontiguousarray(dest, dtype=np.int32).reshape(ntok, k)
    gate = np.ascontiguousarray(gate, dtype=np.float64).reshape(ntok, k)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    residual = _c(residual)
    out = np.empty((ntok, d), np.float64)
    _load().orc_combine(_p(y_slots), _p(dest), _p(gate), ntok, k, d, _p(tok), _p(residual),
                        _dt(residual) if residual is not None else 0, _p(out))
    return out


def aux(prob_sum, counts, T: int):
    """Returns (f [E], P [E], loss) with loss = E * sum f*P."""
    prob_sum = np.ascontiguousarray(prob_sum, dtype=np.float64)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    E = prob_sum.size
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    loss = np.empty(1, np.float64)
    _load().orc_aux(_p(prob_sum), _p(counts), T, E, _p(f), _p(P), _p(loss))
    return f, P, float(loss[0])


def moe_forward(x, w_gate, w1, b1, w2, b2, k: int, renorm: bool, capacity: int = -1,
                gate_bias=None, residual: bool = False, lg=None, tokens=None,
                expert_weights=None):
    """Whole layer: route -> permute -> experts (expert-major) -> combine -> aux.

    ``lg``: logits to route from (same-logits mode); computed in double when None.
    ``tokens``: evaluate the expert FFN and combine for these tokens only
    (routing, permutation and aux always cover all T tokens).
    ``expert_weights``: optional callable e -> (w1e, b1e, w2e, b2e) used instead
    of slicing w1/b1/w2/b2 (lets a caller fetch one expert at a time).
    Returns a dict with every intermediate.
    """
    T, d = x.shape
    E = w_gate.shape[0]
    if lg is None:
        lg = logits(x, w_gate, gate_bias)
    idx, gate, prob_sum = route(lg, k, renorm)
    counts, offsets, dest, sorted_token = permute(idx, E, capacity)
    f, P, loss = aux(prob_sum, counts, T)
    tokens = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    ntok = tokens.size
    dest_s = dest.reshape(T, k)[tokens]
    y_slots = np.zeros((ntok, k, d), np.float64)
    # expert-major: each expert's weights are visited once for all its rows
    for e in range(E):
        sel_i, sel_j = np.nonzero((idx[tokens] == e) & (dest_s >= 0))
        if sel_i.size == 0:
            continue
        if expert_weights is not None:
            w1e, b1e, w2e, b2e = expert_weights(e)
        else:
            w1e, w2e = w1[e], w2[e]
            b1e = None if b1 is None else b1[e]
            b2e = None if b2 is None else b2[e]
        y = expert_rows(x, tokens[sel_i], w1e, b1e, w2e, b2e)
        y_slots[sel_i, sel_j] = y
    out = combine(y_slots, dest_s, gate[tokens], tokens, x if residual else None)
    return dict(logits=lg, idx=idx, gate=gate, prob_sum=prob_sum, counts=counts,
                offsets=offsets, dest_row=dest, sorted_token=sorted_token, f=f, P=P,
                loss=loss, out=out, tokens=tokens)


# ------------------------------------------------------- Expert Choice ----
# The capacity-factor section of the routing-principles page
# ("Expert Choice路由策略与容量因子调优") reverses the direction of selection:
# each expert takes a fixed number of tokens, capacity = tokens / E * factor,
# and tokens no expert takes pass through the residual. Readings taken where
# the page is silent: an expert ranks tokens by the router probability
# p[t,e] = softmax over experts of token t's logits (the gate equation's
# softmax without the top-k mask); ties go to the lower token index; the
# gate of a chosen (token, expert) pair is p[t,e] itself; a token's output
# sums its experts' contributions in ascending expert order.

def ec_scores(lg) -> np.ndarray:
    """p[t,e] = exp(l[t,e] - max_e l[t,:]) / sum_e exp(l[t,e] - max_e l[t,:]), in double."""
    lg = np.asarray(lg, dtype=np.float64)
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def expert_choice(score, C: int):
    """Each expert takes the min(C, T) tokens of highest score[t, e] (ties: lower t).

    Returns (offsets [E+1], sorted_token [E*Cc] with each expert's tokens in
    ascending order, dest_row [T, E] = row of (t, e) or -1, gate [T, E] =
    score of a chosen pair or 0), Cc = min(C, T).
    """
    score = np.asarray(score)
    T, E = score.shape
    Cc = max(0, min(int(C), T))
    offsets = np.arange(E + 1, dtype=np.int32) * Cc
    sorted_token = np.empty(E * Cc, np.int32)
    dest = np.full((T, E), -1, np.int32)
    gate = np.zeros((T, E), np.float64)
    t_idx = np.arange(T)
    for e in range(E):
        # primary key: score descending; secondary: token index ascending
        order = np.lexsort((t_idx, -score[:, e].astype(np.float64)))
        chosen = np.sort(order[:Cc])
        sorted_token[e * Cc:(e + 1) * Cc] = chosen
        dest[chosen, e] = e * Cc + np.arange(Cc)
        gate[chosen, e] = score[chosen, e]
    return offsets, sorted_token, dest, gate


def moe_forward_ec(x, w_gate, w1, b1, w2, b2, C: int, gate_bias=None, residual: bool = False,
                   lg=None, score=None, tokens=None, expert_weights=None):
    """Whole Expert Choice layer: logits -> scores -> per-expert selection ->
    experts (expert-major) -> combine.

    ``lg``: logits (same-logits mode); computed in double when None.
    ``score``: selection scores and gates to use verbatim (same-score mode);
    the double-precision softmax of ``lg`` when None.
    ``tokens``: evaluate the expert FFN and combine for these tokens only.
    ``expert_weights``: optional callable e -> (w1e, b1e, w2e, b2e).
    """
    T, d = x.shape
    E = w_gate.shape[0]
    if lg is None:
        lg = logits(x, w_gate, gate_bias)
    p = ec_scores(lg)
    sel = p if score is None else np.asarray(score, dtype=np.float64)
    offsets, sorted_token, dest, gate = expert_choice(sel, C)
    tokens = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    pos = np.full(T, -1, np.int64)
    pos[tokens] = np.arange(tokens.size)
    if residual:
        xr = x.astype(np.float64) if x.dtype == np.float32 else _bf16_to_f64(x)
        out = xr[tokens].copy()
    else:
        out = np.zeros((tokens.size, d), np.float64)
    for e in range(E):  # ascending expert order for every token
        rows = sorted_token[offsets[e]:offsets[e + 1]]
        mine = rows[pos[rows] >= 0]
        if mine.size == 0:
            continue
        if expert_weights is not None:
            w1e, b1e, w2e, b2e = expert_weights(e)
        else:
            w1e, w2e = w1[e], w2[e]
            b1e = None if b1 is None else b1[e]
            b2e = None if b2 is None else b2[e]
        y = expert_rows(x, mine, w1e, b1e, w2e, b2e)
        out[pos[mine]] += gate[mine, e][:, None] * y
    return dict(logits=lg, p=p, score=sel, offsets=offsets, sorted_token=sorted_token,
                dest_row=dest, gate=gate, out=out, tokens=tokens)


def _bf16_to_f64(a) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to double."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

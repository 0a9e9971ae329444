"""GPU parity of the layer backward at the full workload sizes, on sampled outputs.

The training step runs as the benchmark runs it (forward keeping Z and H,
then the five backward calls, aux-loss weight 0.01). The oracle computes
selected outputs one by one (oracle.backward.moe_backward_sampled) from the
GPU's fp32 logits: whole rows of dx, dgate and dlogits for sampled tokens,
rows of dW1, columns of dW2 and db1 / db2 entries of sampled experts
(always including the expert with the most rows). Each is held to the
element-wise bar of the reduced-size tests, |err| <= 2e-2 RMS + 2^-6 M with
RMS over the sampled reference values of that tensor. The router's
gradients are checked over every token: the oracle's router_backward_all
gives dgate and dlogits of all T tokens (each expert's outputs over all of
its rows), and from them dW_g and db_g, held to the same bar with RMS over
the whole tensor.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from _parity import sample_tokens
from oracle import backward as bwd
from top_routing_expert_topk_amd import moe_layer_backward, moe_layer_forward

pytestmark = pytest.mark.gpu

DAUX = 0.01
TOL, C = 2e-2, 2.0 ** -6


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(label, got, want, mag, rms):
    err = np.abs(got - want)
    bound = TOL * rms + C * mag
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    assert worst <= 1.0, f"{label}: worst err/bound {worst} (max err {err.max()}, RMS {rms})"
    return worst


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_prefill", "switch_top1_cap", "deepseek_v3"])
def test_full_size_backward_samples(name):
    cfg = mi.CONFIGS[name]
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    print(f"[bwd-full] {name}: T={T} d={d} h={h} E={E} k={k}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    dout = mi.make_dout(cfg, "cuda")
    fwd = moe_layer_forward(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                            inp["w2"], inp["b2"], k, cfg.renorm, cfg.capacity, cfg.residual,
                            out_dtype=cfg.torch_dtype, train=True)
    g = moe_layer_backward(fwd, inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                           inp["w2"], inp["b2"], dout, cfg.renorm, cfg.residual, DAUX)
    torch.cuda.synchronize()
    counts = np.diff(fwd.offsets.cpu().numpy())
    rng = np.random.default_rng(cfg.cfg_id + 100)
    nonempty = np.nonzero(counts > 0)[0]
    experts = sorted({int(np.argmax(counts))} | set(rng.choice(nonempty, 2, replace=False).tolist()))
    rows = [(e, int(n)) for e in experts for n in rng.choice(h, 2, replace=False)]
    cols = [(e, int(n)) for e in experts for n in rng.choice(h, 2, replace=False)]
    toks = sample_tokens(T, 6, seed=cfg.cfg_id)

    def fetch(e):
        return tuple(None if inp[n] is None else mi.to_host_array(inp[n][e])
                     for n in ("w1", "b1", "w2", "b2"))
    ref = bwd.moe_backward_sampled(
        mi.to_host_array(inp["x"]), mi.to_host_array(inp["w_gate"]), fetch, k, cfg.renorm,
        cfg.capacity, mi.to_host_array(dout), DAUX, fwd.logits.cpu().numpy(),
        gate_bias=None if inp["gate_bias"] is None else inp["gate_bias"].cpu().numpy(),
        residual=cfg.residual, tokens=toks, w1_rows=rows, w2_cols=cols, b2_experts=experts)
    worst = {}
    for n, got in (("dx", _np(g.dx)[toks]), ("dgate", _np(g.dgate)[toks]),
                   ("dlogits", _np(g.dlogits)[toks])):
        want, mag = ref[n]
        worst[n] = _check(f"{name} {n}", got, want, mag, float(np.sqrt(np.mean(want ** 2))))
    for n, table, pick in (("dw1", ref["dw1"], lambda e, j: _np(g.dw1[e, j])),
                           ("dw2", ref["dw2"], lambda e, j: _np(g.dw2[e, :, j]))):
        rms = float(np.sqrt(np.mean(np.concatenate([v[0] for v in table.values()]) ** 2)))
        worst[n] = max(_check(f"{name} {n}{key}", pick(*key), v, m, rms)
                       for key, (v, m) in table.items())
    if g.db1 is not None:
        vals = np.array([v for v, _ in ref["db1"].values()])
        rms = float(np.sqrt(np.mean(vals ** 2)))
        worst["db1"] = max(_check(f"{name} db1{key}", float(g.db1[key].float()), v, m, rms)
                           for key, (v, m) in ref["db1"].items())
        rms = float(np.sqrt(np.mean(np.concatenate([v for v, _ in ref["db2"].values()]) ** 2)))
        worst["db2"] = max(_check(f"{name} db2[{e}]", _np(g.db2[e]), v, m, rms)
                           for e, (v, m) in ref["db2"].items())
    # the router's gradients over every token
    rb = bwd.router_backward_all(
        mi.to_host_array(inp["x"]), mi.to_host_array(inp["w_gate"]), fetch, k, cfg.renorm,
        cfg.capacity, mi.to_host_array(dout), DAUX, fwd.logits.cpu().numpy(),
        gate_bias=None if inp["gate_bias"] is None else inp["gate_bias"].cpu().numpy())
    for n, got in (("dgate", _np(g.dgate)), ("dlogits", _np(g.dlogits)),
                   ("dw_gate", _np(g.dw_gate)),
                   ("dgate_bias", None if g.dgate_bias is None else _np(g.dgate_bias))):
        if got is None:
            assert rb[n] is None
            continue
        want, mag = rb[n]
        worst[n + "_all"] = _check(f"{name} {n} (every token)", got, want, mag,
                                   float(np.sqrt(np.mean(want ** 2))))
    print(f"[bwd-full] {name}: experts {experts} rows {counts[experts].tolist()} worst "
          + ", ".join(f"{n}={w:.2f}" for n, w in worst.items()), flush=True)

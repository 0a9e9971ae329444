"""Helpers for the GPU parity tests: run the HIP path, then check it against the oracle.

Routing is compared in same-logits mode: the oracle routes from the fp32
logits the GPU produced, so top-k indices, counts, offsets, dest_row,
sorted_token and the drop set must be bit-exact. End to end, the oracle's
double-precision logits must pick the same experts on every token whose
k-th / (k+1)-th logit gap exceeds 1e-3. Outputs are compared element by
element on the checked tokens: max |err| <= 1e-5 * RMS (fp32 layers) or
2e-2 * RMS (bf16 layers), RMS taken over the oracle outputs of the checked
tokens; out is fp32 (the product contract for bf16 layers too). A second
run of the same layer that stores out in bf16 must hold exactly the first
run's fp32 out rounded to nearest even; its error against the oracle is
reported next to the floor any bf16 storage has (the oracle's output rounded
once), which at 10^7 - 10^8 elements reaches most of the 2e-2 * RMS bar by
itself. Gates: 1e-6 (fp32) / 1e-5 (bf16) absolute. Aux: f and loss within
1e-5 relative, P exact.
"""
import numpy as np
import torch

import moe_inputs as mi
from oracle import oracle as orc
from top_routing_expert_topk_amd import moe_layer_forward

TOL = {"f32": dict(out=1e-5, gate=1e-6, logit=1e-5),
       "bf16": dict(out=2e-2, gate=1e-5, logit=1e-4)}
GAP = 1e-3


def run_gpu(cfg, inp, bufs=None, want_logits=True, out_dtype=torch.float32):
    b = moe_layer_forward(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                          inp["w2"], inp["b2"], cfg.k, cfg.renorm, cfg.capacity, cfg.residual,
                          want_logits=want_logits, bufs=bufs, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return b


def _np(t):
    return t.detach().cpu().numpy()


def _out64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def sample_tokens(T, n, seed=0, must=()):
    if n is None or n >= T:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=n, replace=False).tolist()) | {0, T - 1} | set(must)
    return np.array(sorted(pick), dtype=np.int32)


def expert_fetcher(inp):
    def fetch(e):
        return tuple(None if inp[n] is None else mi.to_host_array(inp[n][e])
                     for n in ("w1", "b1", "w2", "b2"))
    return fetch


def check_layer(cfg, inp, b, tokens=None, e2e_tokens=None, label="", b_bf16=None):
    """Every comparison of one layer run; returns a dict of the measured errors.

    ``b_bf16``: optional second run of the same layer with a bf16 ``out``;
    its routing must equal the first run's and its out be the first run's
    fp32 out rounded to bf16."""
    tol = TOL[cfg.dtype]
    T, E, k = cfg.T, cfg.E, cfg.k
    lg = _np(b.logits)
    gi, gg = _np(b.topk_idx), _np(b.topk_gate).astype(np.float64)
    # -- routing from the same fp32 logits: bit-exact selection
    o_idx, o_gate, o_ps = orc.route(lg, k, cfg.renorm)
    assert np.array_equal(gi, o_idx), f"{label}: top-k indices differ on the same logits"
    gate_err = float(np.abs(gg - o_gate).max()) if T else 0.0
    assert gate_err <= tol["gate"], f"{label}: gate err {gate_err}"
    # -- permutation: bit-exact
    counts, offsets, dest, st = orc.permute(o_idx, E, cfg.capacity)
    assert np.array_equal(_np(b.counts), counts), f"{label}: counts"
    assert np.array_equal(_np(b.offsets), offsets), f"{label}: offsets"
    assert np.array_equal(_np(b.dest_row), dest), f"{label}: dest_row / drop set"
    R = int(offsets[-1])
    assert np.array_equal(_np(b.sorted_token)[:R], st), f"{label}: sorted_token"
    # -- aux statistics
    f, P, loss = orc.aux(o_ps, counts, T)
    gf, gP, gl = _np(b.f).astype(np.float64), _np(b.P).astype(np.float64), float(_np(b.loss)[0])
    f_err = float(np.max(np.abs(gf - f) / np.maximum(np.abs(f), 1e-30)))
    assert np.allclose(gf, f, rtol=1e-5, atol=1e-7), f"{label}: f rel err {f_err}"
    assert np.array_equal(gP, (counts / np.float64(T)).astype(np.float32).astype(np.float64)), \
        f"{label}: P"
    assert abs(gl - loss) <= 1e-5 * abs(loss) + 1e-7, f"{label}: loss {gl} vs {loss}"
    x_h = mi.to_host_array(inp["x"])
    wg_h = mi.to_host_array(inp["w_gate"])
    gb_h = None if inp["gate_bias"] is None else _np(inp["gate_bias"])
    # -- end to end: double logits choose the same experts where the gap is clear
    e2e = sample_tokens(T, None) if e2e_tokens is None else e2e_tokens
    lg_o = orc.logits(x_h[e2e], wg_h, gb_h)
    logit_err = float(np.abs(lg[e2e] - lg_o).max()) if e2e.size else 0.0
    assert logit_err <= tol["logit"] * max(1.0, float(np.abs(lg_o).max(initial=0.0))), \
        f"{label}: logit err {logit_err}"
    srt = np.sort(lg_o, axis=1)[:, ::-1]
    gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(e2e.size, np.inf)
    clear = gap > GAP
    e_idx, _, _ = orc.route(lg_o, k, cfg.renorm)
    # the contract is which experts are selected: the order inside the top-k
    # may flip between fp32 and double logits (same-logits mode above checks
    # the order bit for bit)
    assert np.array_equal(np.sort(gi[e2e][clear], axis=1), np.sort(e_idx[clear], axis=1)), \
        f"{label}: end-to-end selection"
    # -- outputs on the checked tokens
    toks = sample_tokens(T, None) if tokens is None else tokens
    res = orc.moe_forward(x_h, wg_h, None, None, None, None, k, cfg.renorm, cfg.capacity,
                          gate_bias=gb_h, residual=cfg.residual, lg=lg, tokens=toks,
                          expert_weights=expert_fetcher(inp))
    ref = res["out"]
    got = _out64(b.out)[toks]
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    out_err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert out_err <= tol["out"] * rms, f"{label}: out max err {out_err} vs {tol['out']}*RMS {rms}"
    r = dict(gate_err=gate_err, f_err=f_err, logit_err=logit_err, out_err=out_err, rms=rms,
             out_rel=out_err / rms if rms else 0.0, rows=R, drops=int((dest < 0).sum()),
             unclear=int((~clear).sum()), checked_tokens=int(toks.size))
    if b_bf16 is not None:
        # bf16 storage of out: the same fp32 sums, rounded to nearest even
        assert b_bf16.out.dtype == torch.bfloat16
        assert np.array_equal(_np(b_bf16.topk_idx), gi), f"{label}: bf16-output run routed apart"
        assert torch.equal(b_bf16.out, b.out.to(torch.bfloat16)), \
            f"{label}: bf16 out is not the fp32 out rounded"
        # reported, not asserted: against the plain bar, and the floor that
        # any bf16 storage of out has (the oracle's output rounded once)
        got16 = _out64(b_bf16.out)[toks]
        exact16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        if rms:
            r["bf16_out_rel"] = float(np.abs(got16 - ref).max()) / rms
            r["bf16_rounding_floor_rel"] = float(np.abs(exact16 - ref).max()) / rms
    return r


def decode_expert_outputs(y, d):
    """The block fixed point of a bf16 layer's y_perm (uint8 [rows][row
    bytes]): returns (values [rows][d] float64, mantissas int16 [rows][d],
    exponents int [rows][d/8]), value = mantissa * 2^(exponent - 14)."""
    a = y.detach().cpu().numpy()
    mant = np.ascontiguousarray(a[:, :2 * d]).view("<i2")
    ex = a[:, 2 * d:2 * d + d // 8].view(np.int8).astype(np.int64)
    vals = mant.astype(np.float64) * np.exp2(np.repeat(ex, 8, axis=1) - 14)
    return vals, mant, ex

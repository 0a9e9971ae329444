"""GPU parity of Expert Choice routing: the HIP path through the C-ABI against the oracle.

Selection is compared in same-score mode: the oracle selects from the fp32
scores the GPU produced (the decision is taken in the kernel's precision),
so offsets, sorted_token, dest_row and gates must be bit-exact. The GPU's
scores must match the oracle's double softmax of the same logits within
1e-6, and the oracle's double scores must choose the same tokens for every
expert whose C-th / (C+1)-th score gap exceeds 1e-6. Outputs are compared
element by element on every token: max |err| <= 1e-5 * RMS (fp32 layers) or
2e-2 * RMS (bf16 layers), the bar of the token-choice layers (the expert
outputs reach the combine in fp32; H is the only rounded intermediate).
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from _parity import TOL, expert_fetcher, sample_tokens
from oracle import oracle as orc
from top_routing_expert_topk_amd import moe_layer_forward_ec

pytestmark = pytest.mark.gpu

EC = mi.CONFIGS["switch_expert_choice"]
SCORE_TOL = 1e-6


def _np(t):
    return t.detach().cpu().numpy()


def run_ec(cfg, inp, C=None):
    b = moe_layer_forward_ec(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                             inp["w2"], inp["b2"], cfg.capacity if C is None else C,
                             residual=cfg.residual)
    torch.cuda.synchronize()
    return b


def check_ec(cfg, inp, b, C, tokens=None, label=""):
    tol = TOL[cfg.dtype]
    T, E = cfg.T, cfg.E
    Cc = max(0, min(C, T))
    lg = _np(b.logits)
    sc = _np(b.scores).T  # [T][E]
    # scores against the double softmax of the same fp32 logits
    p = orc.ec_scores(lg)
    score_err = float(np.abs(sc - p).max()) if T else 0.0
    assert score_err <= SCORE_TOL, f"{label}: score err {score_err}"
    # selection from the same fp32 scores: bit-exact
    offsets, st, dest, gate = orc.expert_choice(sc, C)
    assert np.array_equal(_np(b.offsets), offsets), f"{label}: offsets"
    assert np.array_equal(_np(b.sorted_token)[:E * Cc], st), f"{label}: sorted_token"
    assert np.array_equal(_np(b.dest_row), dest), f"{label}: dest_row"
    assert np.array_equal(_np(b.gate).astype(np.float64), gate), f"{label}: gates"
    # the double scores choose the same tokens wherever the cut is clear
    unclear = 0
    if 0 < Cc < T:
        _, st64, _, _ = orc.expert_choice(p, C)
        srt = np.sort(p, axis=0)[::-1]
        gap = srt[Cc - 1] - srt[Cc]
        for e in range(E):
            if gap[e] > SCORE_TOL:
                assert np.array_equal(st64[e * Cc:(e + 1) * Cc], st[e * Cc:(e + 1) * Cc]), \
                    f"{label}: expert {e} selection from double scores"
            else:
                unclear += 1
    # outputs on the checked tokens
    x_h = mi.to_host_array(inp["x"])
    wg_h = mi.to_host_array(inp["w_gate"])
    gb_h = None if inp["gate_bias"] is None else _np(inp["gate_bias"])
    toks = sample_tokens(T, None) if tokens is None else tokens
    res = orc.moe_forward_ec(x_h, wg_h, None, None, None, None, C, gate_bias=gb_h,
                             residual=cfg.residual, lg=lg, score=sc, tokens=toks,
                             expert_weights=expert_fetcher(inp))
    ref = res["out"]
    got = b.out.detach().float().cpu().numpy().astype(np.float64)[toks]
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(got - ref)
    out_err = float(err.max()) if ref.size else 0.0
    assert out_err <= tol["out"] * rms, f"{label}: out err {out_err} vs {tol['out']}*RMS {rms}"
    return dict(score_err=score_err, out_err=out_err, rms=rms, unclear=unclear,
                rows=E * Cc, uncovered=int(((dest >= 0).sum(axis=1) == 0).sum()),
                bar_ratio=out_err / (tol["out"] * rms) if rms else 0.0)


def _run(cfg, C=None, nsample=None, mutate=None, label=None):
    C = cfg.capacity if C is None else C
    print(f"[ec] {label or cfg.name}: T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} C={C} "
          f"{cfg.dtype}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    if mutate:
        mutate(inp)
    b = run_ec(cfg, inp, C)
    r = check_ec(cfg, inp, b, C, sample_tokens(cfg.T, nsample, seed=cfg.cfg_id),
                 label or cfg.name)
    print(f"[ec] {label or cfg.name}: {r}", flush=True)
    return inp, b, r


@pytest.mark.timeout(600)
def test_full_switch_shaped_workload():
    """Switch-shaped layer with the Zipf-skewed router, every token: every
    expert takes exactly 80 tokens although token choice would drop ~60% of
    assignments."""
    _, b, r = _run(EC)
    assert r["rows"] == EC.E * EC.capacity


SMALL = {
    "ec_switch_small": EC.with_(name="ec_switch_small", T=1000, d=256, h=512, E=16, capacity=79),
    "ec_fp32": EC.with_(name="ec_fp32", T=77, d=96, h=200, E=5, capacity=20, dtype="f32",
                        zipf_gate_bias=False),
    "ec_e100": EC.with_(name="ec_e100", T=700, d=256, h=256, E=100, capacity=9,
                        zipf_gate_bias=False),
    "ec_e512": EC.with_(name="ec_e512", T=600, d=256, h=128, E=512, capacity=3,
                        zipf_gate_bias=False, residual=False),
    "ec_few_tokens": EC.with_(name="ec_few_tokens", T=7, d=256, h=256, E=8, capacity=3),
    "ec_ring_tiles": EC.with_(name="ec_ring_tiles", T=2048, d=512, h=512, E=8, capacity=400,
                              zipf_gate_bias=False),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_reduced_shape_every_element(name):
    _run(SMALL[name])


def test_zero_capacity_passes_the_residual_exactly():
    cfg = SMALL["ec_switch_small"]
    inp, b, r = _run(cfg, C=0, label="ec_c0")
    assert torch.equal(b.out, inp["x"].float())


@pytest.mark.parametrize("extra", [0, 5])
def test_capacity_at_least_T_takes_every_token(extra):
    cfg = SMALL["ec_switch_small"].with_(T=200, E=6)
    inp, b, r = _run(cfg, C=cfg.T + extra, label=f"ec_all_{extra}")
    assert r["rows"] == cfg.E * cfg.T
    assert bool((b.dest_row >= 0).all())


def test_equal_scores_take_the_lowest_tokens():
    cfg = SMALL["ec_switch_small"].with_(T=300, E=8, zipf_gate_bias=False)

    def zero_router(inp):
        inp["w_gate"].zero_()
    inp, b, r = _run(cfg, C=37, mutate=zero_router, label="ec_ties")
    st = _np(b.sorted_token)[:8 * 37].reshape(8, 37)
    assert np.array_equal(st, np.tile(np.arange(37, dtype=np.int32), (8, 1)))


def test_determinism_bitwise():
    cfg = SMALL["ec_switch_small"]
    inp = mi.make_inputs(cfg, "cuda")
    b1 = run_ec(cfg, inp)
    o1 = b1.out.clone()
    b2 = run_ec(cfg, inp)
    assert torch.equal(o1, b2.out)

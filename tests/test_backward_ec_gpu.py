"""GPU parity of the Expert Choice layer backward against the backward oracle.

The forward keeps Z and H (train=True); the oracle selects from the GPU's
fp32 scores (the selection is taken in the kernel's precision, as in the
forward parity tests) and differentiates through the softmax of the GPU's
logits. Every element of every gradient and of dgate / dlogits is held to
the bar of the token-choice backward tests: |err| <= tol RMS(ref) + c M,
tol 2e-2 / 1e-5 and c 2^-6 / 2^-16 for bf16 / fp32 layers, M the oracle's
magnitude of the element.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import backward as bwd
from top_routing_expert_topk_amd import moe_layer_backward_ec, moe_layer_forward_ec

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 2.0 ** -16), "bf16": (2e-2, 2.0 ** -6)}
EC = mi.CONFIGS["switch_expert_choice"]
CASES = {
    "ec_switch_small": (EC.with_(name="ec_switch_small", T=1000, d=256, h=512, E=16), 79),
    "ec_e100": (EC.with_(name="ec_e100", T=700, d=256, h=256, E=100, zipf_gate_bias=False), 9),
    "ec_few_tokens": (EC.with_(name="ec_few_tokens", T=7, d=256, h=256, E=8), 3),
    "ec_every_token": (EC.with_(name="ec_every_token", T=200, d=256, h=256, E=6,
                                zipf_gate_bias=False), 205),
    "ec_fp32": (EC.with_(name="ec_fp32", T=77, d=96, h=200, E=5, dtype="f32",
                         zipf_gate_bias=False, residual=False), 20),
    # every expert takes every token: 24 kept slots per token, more than the
    # gather lists per token in LDS, and three passes of eight in the combine
    "ec_many_slots": (EC.with_(name="ec_many_slots", T=40, d=256, h=256, E=24,
                               zipf_gate_bias=False), 40),
    # the Switch-shaped workload as benched (T=8192, d=768, h=3072, E=128, C=80)
    "ec_switch_full": (EC, EC.capacity),
}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_expert_choice_backward_every_element(name):
    cfg, C = CASES[name]
    print(f"[bwd-ec] {name}: T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} C={C} {cfg.dtype}",
          flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    dout = mi.make_dout(cfg, "cuda")
    fwd = moe_layer_forward_ec(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                               inp["w2"], inp["b2"], C, residual=cfg.residual,
                               out_dtype=cfg.torch_dtype, train=True)
    g = moe_layer_backward_ec(fwd, inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"],
                              inp["b1"], inp["w2"], inp["b2"], dout, residual=cfg.residual)
    torch.cuda.synchronize()
    h = {n: mi.to_host_array(v) for n, v in inp.items() if v is not None}
    ref = bwd.moe_backward_ec(h["x"], h["w_gate"], h["w1"], h.get("b1"), h["w2"], h.get("b2"), C,
                              mi.to_host_array(dout), gate_bias=h.get("gate_bias"),
                              residual=cfg.residual, lg=fwd.logits.cpu().numpy(),
                              score=fwd.scores.cpu().numpy().T, want_scale=True)
    assert np.array_equal(fwd.dest_row.cpu().numpy(), ref["dest_row"]), "selection"
    tol, c = TOL[cfg.dtype]
    worst = {}
    for n in ("dx", "dw_gate", "dgate_bias", "dw1", "db1", "dw2", "db2", "dgate", "dlogits"):
        want = ref[n]
        got = getattr(g, n)
        if want is None:
            assert got is None, n
            continue
        got = _np(got).reshape(want.shape)
        rms = float(np.sqrt(np.mean(want ** 2)))
        bound = tol * rms + c * ref["scale"][n]
        ratio = float((np.abs(got - want) / np.maximum(bound, 1e-300)).max())
        worst[n] = ratio
        assert ratio <= 1.0, f"{name} {n}: error {ratio:.2f} of its bound (RMS {rms})"
    print(f"[bwd-ec] {name}: " + ", ".join(f"{n}={w:.2f}" for n, w in worst.items()), flush=True)

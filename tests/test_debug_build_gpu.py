"""The debug build (libmoe_debug.so, MOE_HOST_BOUNDS_CHECK) on the GPU.

It runs whole layers (token choice with capacity drops, Expert Choice, and
a training step) with the host-side permutation checks in front of every
launch that indexes with offsets, sorted_token or dest_row, and matches the
oracle as the release build does. Given a corrupted permutation it refuses
the call with status 1 before launching anything. Each corrupted array is
built so that even an unchecked launch would stay inside its allocations:
the out-of-range token and row indices point into spare rows allocated past
the end of x and y_perm, and the bad offsets only move expert 0's first
row.
"""
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
from _parity import check_layer, run_gpu
from top_routing_expert_topk_amd import layer as moe_layer
from top_routing_expert_topk_amd import native as N

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(N.LIB_PATH), "libmoe_debug.so")
CFG = mi.CONFIGS


@pytest.fixture
def debug_lib():
    old = N.use_library(DEBUG_LIB)
    try:
        assert N.debug_checks(), "libmoe_debug.so was not built with MOE_HOST_BOUNDS_CHECK"
        yield
    finally:
        N.use_library(old)


@pytest.mark.parametrize("cfg", [
    CFG["switch_top1_cap"].with_(name="dbg_switch", T=1000, d=256, h=512, E=16, capacity=79),
    CFG["deepseek_v3"].with_(name="dbg_deepseek", T=513, d=384, h=256, E=64),
    CFG["decode"].with_(name="dbg_decode", T=7, d=576, h=768, E=16),
], ids=lambda c: c.name)
def test_debug_build_runs_layers_to_the_oracle(debug_lib, cfg):
    print(f"[debug] {cfg.name}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    b = run_gpu(cfg, inp)
    check_layer(cfg, inp, b, label=cfg.name)


def test_debug_build_runs_expert_choice_and_a_training_step(debug_lib):
    cfg = CFG["switch_expert_choice"].with_(T=600, d=256, h=256, E=32, capacity=20)
    inp = mi.make_inputs(cfg, "cuda")
    b = moe_layer.moe_layer_forward_ec(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"],
                                       inp["b1"], inp["w2"], inp["b2"], cfg.capacity,
                                       residual=cfg.residual)
    torch.cuda.synchronize()
    assert torch.isfinite(b.out).all()
    cfg = CFG["mixtral_prefill"].with_(T=300, d=256, h=512)
    inp = mi.make_inputs(cfg, "cuda")
    fwd = moe_layer.moe_layer_forward(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"],
                                      inp["b1"], inp["w2"], inp["b2"], cfg.k, cfg.renorm,
                                      cfg.capacity, cfg.residual, train=True)
    g = moe_layer.moe_layer_backward(fwd, inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"],
                                     inp["b1"], inp["w2"], inp["b2"], mi.make_dout(cfg, "cuda"),
                                     cfg.renorm, cfg.residual, 0.01)
    torch.cuda.synchronize()
    assert torch.isfinite(g.dx.float()).all() and torch.isfinite(g.dw_gate).all()


def test_debug_build_refuses_corrupted_permutations(debug_lib):
    cfg = CFG["mixtral_prefill"].with_(T=256, d=256, h=512, E=8, k=2)
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    inp = mi.make_inputs(cfg, "cuda")
    spare = 8
    xs = torch.zeros((T + spare, d), dtype=torch.bfloat16, device="cuda")
    xs[:T] = inp["x"]
    x = xs[:T]
    b = run_gpu(cfg, dict(inp, x=x))
    R = int(b.offsets[-1])
    ys = N.expert_output_buffer(torch.bfloat16, T * k + spare, d, "cuda")
    y = ys[:T * k]

    def ffn(offsets, sorted_token):
        N.moe_grouped_ffn(x, T, d, h, E, k, offsets, sorted_token, inp["w1"], inp["b1"],
                          inp["w2"], inp["b2"], y, b.ws_ffn)

    def combine(dest):
        N.moe_combine(y, x.dtype, dest, b.topk_gate, T, k, d, None, b.out)

    ffn(b.offsets, b.sorted_token)  # the layer's own arrays pass
    combine(b.dest_row)
    torch.cuda.synchronize()
    st = b.sorted_token.clone()
    st[R // 2] = T + spare // 2  # a token past x (inside the spare rows)
    with pytest.raises(N.MoEError) as err:
        ffn(b.offsets, st)
    assert err.value.status == N.MOE_ERR_INVALID
    off = b.offsets.clone()
    off[0] = 1  # offsets not starting at row 0 (an unchecked launch would skip row 0)
    with pytest.raises(N.MoEError) as err:
        ffn(off, b.sorted_token)
    assert err.value.status == N.MOE_ERR_INVALID
    dest = b.dest_row.clone()
    dest[5] = T * k + spare // 2  # a row past y_perm (inside its spare rows)
    with pytest.raises(N.MoEError) as err:
        combine(dest)
    assert err.value.status == N.MOE_ERR_INVALID
    torch.cuda.synchronize()
    # the library still runs the real layer afterwards
    b2 = run_gpu(cfg, inp)
    check_layer(cfg, inp, b2, label="after_refusals")
    assert np.isfinite(b2.out.cpu().numpy()).all()

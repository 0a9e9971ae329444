"""GPU: the layer over host-resident experts streamed into an LRU of device slots.

Each step reads the routing's counts back, copies the missing experts from
pinned host memory into the least recently used slots on a copy stream while
the resident experts run, then runs the loaded ones. The output must equal
the all-resident layer bit for bit (same kernels, same arithmetic) on every
step of a sequence that hits, misses and evicts, and match the oracle.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from _parity import check_layer
from top_routing_expert_topk_amd import ExpertCache, moe_layer_forward, moe_layer_forward_cached

pytestmark = pytest.mark.gpu

DEC = mi.CONFIGS["decode"]


def _x(cfg, seed):
    g = torch.Generator(device="cuda").manual_seed(1000 + seed)
    return torch.randn((cfg.T, cfg.d), generator=g, device="cuda").to(cfg.torch_dtype)


@pytest.mark.parametrize("T,E,k,S", [(32, 64, 2, 56), (8, 16, 2, 14), (5, 8, 1, 8)])
def test_cached_layer_equals_the_resident_layer_step_by_step(T, E, k, S):
    cfg = DEC.with_(name="cache", T=T, d=512, h=256, E=E, k=k)
    print(f"[cache] T={T} E={E} k={k} S={S}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    cache = ExpertCache(inp["w1"], inp["b1"], inp["w2"], inp["b2"], S, "cuda")
    loads = []
    for step in range(6):
        x = _x(cfg, step % 4)  # repeats: later steps hit what earlier ones loaded
        ref = moe_layer_forward(x, inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                                inp["w2"], inp["b2"], k, cfg.renorm, cfg.capacity, cfg.residual)
        got = moe_layer_forward_cached(x, inp["w_gate"], inp["gate_bias"], cache, k, cfg.renorm,
                                       cfg.capacity, cfg.residual)
        torch.cuda.synchronize()
        loads.append(cache.loaded)
        assert torch.equal(got.topk_idx, ref.topk_idx)
        assert torch.equal(got.out, ref.out), f"step {step}"
        assert torch.equal(got.loss, ref.loss)
    print(f"[cache] experts loaded per step: {loads}", flush=True)
    assert loads[0] > 0


def test_cached_layer_matches_the_oracle():
    cfg = DEC.with_(name="cache_oracle", T=16, d=512, h=256, E=32, k=2)
    inp = mi.make_inputs(cfg, "cuda")
    cache = ExpertCache(inp["w1"], inp["b1"], inp["w2"], inp["b2"], 20, "cuda")
    b = moe_layer_forward_cached(inp["x"], inp["w_gate"], inp["gate_bias"], cache, cfg.k,
                                 cfg.renorm, cfg.capacity, cfg.residual, want_logits=True)
    torch.cuda.synchronize()
    r = check_layer(cfg, inp, b, label="cache_oracle")
    print(f"[cache] oracle: {r}", flush=True)


def test_a_second_identical_step_loads_nothing():
    cfg = DEC.with_(name="cache_hits", T=32, d=512, h=256, E=64, k=2)
    inp = mi.make_inputs(cfg, "cuda")
    cache = ExpertCache(inp["w1"], inp["b1"], inp["w2"], inp["b2"], 64, "cuda")
    moe_layer_forward_cached(inp["x"], inp["w_gate"], inp["gate_bias"], cache, 2)
    first = cache.loaded
    moe_layer_forward_cached(inp["x"], inp["w_gate"], inp["gate_bias"], cache, 2)
    torch.cuda.synchronize()
    assert first > 0 and cache.loaded == 0

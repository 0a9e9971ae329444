"""The layer forward captured in a HIP graph and replayed.

The five calls launch kernels only (no allocation, memset or host read), so
one step can be captured on a stream and replayed. Each replay must give the
eager step's outputs bit for bit. Between replays the test poisons every
output with eager fill kernels, synchronises, and also runs the eager step on
the same buffers, so a replay that reused stale memory or skipped a kernel
would show. Shapes cover the 256-row ring GEMM (whole and split tiles, and
taller last tiles), the persistent 128-row GEMM with capacity drops and a
residual, the decode weight-streaming kernel and an fp32 layer.
"""
import pytest
import torch

import moe_inputs as mi
import top_routing_expert_topk_amd as moe

pytestmark = pytest.mark.gpu

CFG = mi.CONFIGS
CASES = {
    "ring_full_tail": CFG["mixtral_prefill"].with_(name="ring_full_tail", T=4096, d=512, h=2048),
    "ring_taller": CFG["deepseek_v3"].with_(name="ring_taller", T=1100, d=512, h=256, E=32),
    "pring_capacity": CFG["switch_top1_cap"].with_(name="pring_capacity", T=6000, d=512,
                                                    h=1536, E=64),
    "decode": CFG["decode"].with_(name="decode_graph", T=7, d=576, h=768, E=16),
    "fp32": CFG["tiny_fp32"].with_(name="fp32_graph", T=77, d=96, h=200, E=5),
}
REPLAYS = 3


def _outputs(b):
    return {"out": b.out, "topk_idx": b.topk_idx, "topk_gate": b.topk_gate,
            "prob_sum": b.prob_sum, "counts": b.counts, "offsets": b.offsets,
            "dest_row": b.dest_row, "sorted_token": b.sorted_token, "y_perm": b.y_perm,
            "f": b.f, "P": b.P, "loss": b.loss}


def _poison(ts):
    for t in ts.values():
        if t.is_floating_point():
            t.fill_(float("nan"))
        elif t.dtype == torch.uint8:
            t.fill_(0xAB)
        else:
            t.fill_(-7)


def _snapshot(ts, R):
    snap = {}
    for name, t in ts.items():
        v = t[:R] if name in ("sorted_token", "y_perm") else t
        snap[name] = v.clone()
    return snap


def _equal(a, b):
    if a.is_floating_point():
        return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)
    return torch.equal(a, b)


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replay_equals_eager(name):
    cfg = CASES[name]
    print(f"[graph] {name}: T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} k={cfg.k} {cfg.dtype}",
          flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    s = torch.cuda.Stream()  # default priority
    b = moe.MoEBuffers(cfg.T, cfg.d, cfg.h, cfg.E, cfg.k, cfg.torch_dtype, torch.device("cuda"))

    def step():
        moe.moe_layer_forward(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                              inp["w2"], inp["b2"], cfg.k, cfg.renorm, cfg.capacity,
                              cfg.residual, bufs=b, stream=s)

    outs = _outputs(b)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        _poison(outs)
        step()
    torch.cuda.synchronize()
    R = int(b.offsets[-1])
    ref = _snapshot(outs, R)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        with torch.cuda.stream(s):
            _poison(outs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(outs, R)
        for key in ref:
            assert _equal(got[key], ref[key]), f"{name}: replay {rep} differs in {key}"
        # the program's own eager work between replays
        with torch.cuda.stream(s):
            step()
        torch.cuda.synchronize()
        for key, v in _snapshot(outs, R).items():
            assert _equal(v, ref[key]), f"{name}: eager step after replay {rep} differs in {key}"
    print(f"[graph] {name}: {REPLAYS} replays equal the eager step (R={R})", flush=True)

"""The layer forward captured in a HIP graph and replayed.

The five calls launch kernels only (no allocation, memset or host read), so
one step can be captured on a stream and replayed. Each replay must give the
eager step's outputs bit for bit. Between replays the test poisons every
output with eager fill kernels, synchronises, and also runs the eager step on
the same buffers, so a replay that reused stale memory or skipped a kernel
would show. The same holds for a training step (the forward keeping Z and
H, then the five backward calls). Shapes cover the 256-row ring GEMM (whole and split tiles, and
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
    # bit patterns, so that NaN poison left behind would not compare equal
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
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


# ------------------------------------------------------- training step ----
TRAIN_CASES = {
    "ring_taller": CASES["ring_taller"],
    "switch_small": CFG["switch_top1_cap"].with_(name="switch_train_graph", T=1024, d=256,
                                                  h=512, E=16, capacity=80),
    "fp32": CASES["fp32"],
}


@pytest.mark.parametrize("name", sorted(TRAIN_CASES))
def test_training_step_graph_replay_equals_eager(name):
    """Forward keeping Z and H, then the five backward calls, captured once:
    every replay gives the eager step's gradients bit for bit."""
    cfg = TRAIN_CASES[name]
    print(f"[graph-train] {name}: T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} k={cfg.k} "
          f"{cfg.dtype}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    dout = mi.make_dout(cfg, "cuda")
    dev = torch.device("cuda")
    s = torch.cuda.Stream()  # default priority
    fwd = moe.MoEBuffers(cfg.T, cfg.d, cfg.h, cfg.E, cfg.k, cfg.torch_dtype, dev,
                         cfg.torch_dtype, train=True)
    grads = moe.MoEGrads(cfg.T, cfg.d, cfg.h, cfg.E, cfg.k, cfg.torch_dtype, dev,
                         inp["b1"] is not None, inp["b2"] is not None,
                         inp["gate_bias"] is not None)
    args = (inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"], inp["w2"],
            inp["b2"])

    def step():
        moe.moe_layer_forward(*args, cfg.k, cfg.renorm, cfg.capacity, cfg.residual, bufs=fwd,
                              stream=s, train=True)
        moe.moe_layer_backward(fwd, *args, dout, cfg.renorm, cfg.residual, 0.01, grads=grads,
                               stream=s)

    outs = {n: v for n, v in dict(dx=grads.dx, dw_gate=grads.dw_gate,
                                  dgate_bias=grads.dgate_bias, dw1=grads.dw1, db1=grads.db1,
                                  dw2=grads.dw2, db2=grads.db2, dgate=grads.dgate,
                                  dlogits=grads.dlogits, out=fwd.out, loss=fwd.loss).items()
            if v is not None}
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        _poison(outs)
        step()
    torch.cuda.synchronize()
    ref = {n: v.clone() for n, v in outs.items()}
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
        for key, v in outs.items():
            assert _equal(v, ref[key]), f"{name}: replay {rep} differs in {key}"
        with torch.cuda.stream(s):
            step()
        torch.cuda.synchronize()
        for key, v in outs.items():
            assert _equal(v, ref[key]), f"{name}: eager step after replay {rep} differs in {key}"
    print(f"[graph-train] {name}: {REPLAYS} replays equal the eager step", flush=True)


# ------------------------------------------------------- Expert Choice ----
EC_CASES = {
    "ec_switch_small": CFG["switch_expert_choice"].with_(name="ec_graph", T=1000, d=256, h=512,
                                                         E=16, capacity=70),
}


@pytest.mark.parametrize("name", sorted(EC_CASES))
def test_expert_choice_graph_replay_equals_eager(name):
    """The Expert Choice forward (router logits, selection per expert, grouped
    FFN, combine) captured once: every replay equals the eager step."""
    cfg = EC_CASES[name]
    print(f"[graph-ec] {name}: T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} C={cfg.capacity}",
          flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    s = torch.cuda.Stream()  # default priority
    b = moe.ECBuffers(cfg.T, cfg.d, cfg.h, cfg.E, cfg.capacity, cfg.torch_dtype,
                      torch.device("cuda"))

    def step():
        moe.moe_layer_forward_ec(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"],
                                 inp["b1"], inp["w2"], inp["b2"], cfg.capacity, cfg.residual,
                                 bufs=b, stream=s)

    outs = {"out": b.out, "logits": b.logits, "scores": b.scores, "offsets": b.offsets,
            "sorted_token": b.sorted_token, "dest_row": b.dest_row, "gate": b.gate,
            "y_perm": b.y_perm}
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
        for key, v in _snapshot(outs, R).items():
            assert _equal(v, ref[key]), f"{name}: replay {rep} differs in {key}"
        with torch.cuda.stream(s):
            step()
        torch.cuda.synchronize()
        for key, v in _snapshot(outs, R).items():
            assert _equal(v, ref[key]), f"{name}: eager step after replay {rep} differs in {key}"
    print(f"[graph-ec] {name}: {REPLAYS} replays equal the eager step (R={R})", flush=True)

"""GPU parity of the layer backward: the HIP path through the C-ABI against the backward oracle.

The forward runs first (want_logits) and the oracle differentiates the layer
routed from the same fp32 logits, so selection, counts and drops are those
of the GPU run (checked bit-exact by the forward tests). Every element of
every gradient tensor, and of the intermediates dgate and dlogits, is
compared with the oracle's float64 value:

    |err_i| <= tol * RMS(ref) + c * M_i

tol is the forward's bar (1e-5 fp32, 2e-2 bf16), RMS over the whole tensor.
M_i is the oracle's magnitude of element i (the sum of the absolute values
of the products it is made of, carried through the chain). bf16 layers
round dY, Z, SiLU(Z), dZ (twice), dX_perm and every gradient to bf16 (2^-9
relative each); a chain of up to eight such roundings bounds the error by
2^-6 M_i, so c = 2^-6. fp32 layers: c = 2^-16 covers fp32 accumulation in
any order over up to 256 terms (256 * 2^-24). With one or two rows per
expert the rounding of a single product is the whole error, which is why an
RMS-only bar cannot hold there (a 1-row weight gradient carries 2-3 relative
roundings of 2^-9 on an element several times the tensor's RMS).
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import backward as bwd
from top_routing_expert_topk_amd import moe_layer_backward, moe_layer_forward

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 2.0 ** -16), "bf16": (2e-2, 2.0 ** -6)}
DAUX = 0.5

BASE = mi.CONFIGS["mixtral_prefill"]
SW = mi.CONFIGS["switch_top1_cap"]
CASES = {
    # about 128 rows per expert: short tiles in every GEMM
    "mix_small": BASE.with_(name="mix_small", T=512, d=256, h=512),
    # about 768 rows per expert: whole tiles, split tail tiles, ragged ends
    "mix_rows": BASE.with_(name="mix_rows", T=1536, d=256, h=768, E=4),
    # top-1 without renormalisation, capacity drops, router bias, residual
    "switch_small": SW.with_(name="switch_small", T=1024, d=256, h=512, E=16, capacity=80),
    # top-8 of 32
    "deepseek_small": mi.CONFIGS["deepseek_v3"].with_(name="deepseek_small", T=256, d=512, h=256,
                                                      E=32),
    # 32 experts of about 275 rows: an expert's last row block is one taller
    # tile of up to 288 rows, in the forward and in the Z recompute; few
    # tiles, so they are split along K
    "taller_tiles": mi.CONFIGS["deepseek_v3"].with_(name="taller_tiles", T=1100, d=512, h=256,
                                                    E=32),
    # the same with top-2 of 32 at d = 256, h = 768 (~281 rows per expert)
    "taller_top2": BASE.with_(name="taller_top2", T=4500, d=256, h=768, E=32),
    # top-16 of 40 (the router's largest k): as many kept slots per token as
    # the gather lists in LDS, two of the combine's passes of eight, and 40
    # experts ending in a partial 16-expert MFMA step of the router products
    "many_slots": mi.CONFIGS["deepseek_v3"].with_(name="many_slots", T=96, d=256, h=256, E=40,
                                                  k=16),
    # most experts receive no row: their weight gradients must be zero
    "sparse_experts": BASE.with_(name="sparse_experts", T=24, d=256, h=256, E=64),
    # every assignment dropped: only the residual and the aux loss remain
    "capacity_zero": SW.with_(name="capacity_zero", T=300, d=256, h=256, E=8, capacity=0),
    "tiny_fp32": mi.CONFIGS["tiny_fp32"],
    # widths that are not multiples of anything, fp32
    "f32_ragged": mi.CONFIGS["tiny_fp32"].with_(name="f32_ragged", T=77, d=96, h=200, E=5,
                                                capacity=25, residual=True),
}


def _np(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def run_backward(cfg, daux=DAUX, train=True):
    """train: the forward keeps Z and H for the backward; otherwise the
    backward recomputes Z."""
    inp = mi.make_inputs(cfg, "cuda")
    dout = mi.make_dout(cfg, "cuda")
    fwd = moe_layer_forward(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                            inp["w2"], inp["b2"], cfg.k, cfg.renorm, cfg.capacity, cfg.residual,
                            want_logits=True, out_dtype=cfg.torch_dtype, train=train)
    g = moe_layer_backward(fwd, inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                           inp["w2"], inp["b2"], dout, cfg.renorm, cfg.residual, daux)
    torch.cuda.synchronize()
    return inp, dout, fwd, g


def oracle_backward(cfg, inp, dout, fwd, daux=DAUX):
    h = {n: mi.to_host_array(v) for n, v in inp.items() if v is not None}
    return bwd.moe_backward(h["x"], h["w_gate"], h["w1"], h.get("b1"), h["w2"], h.get("b2"),
                            cfg.k, cfg.renorm, cfg.capacity, mi.to_host_array(dout), daux,
                            gate_bias=h.get("gate_bias"), residual=cfg.residual,
                            lg=fwd.logits.cpu().numpy(), want_scale=True)


def compare(cfg, g, ref, label):
    tol, c = TOL[cfg.dtype]
    errs = {}
    pairs = dict(dx=g.dx, dw_gate=g.dw_gate, dgate_bias=g.dgate_bias, dw1=g.dw1, db1=g.db1,
                 dw2=g.dw2, db2=g.db2, dgate=g.dgate, dlogits=g.dlogits)
    for name, got in pairs.items():
        want = ref[name]
        if want is None:
            assert got is None, name
            continue
        got = _np(got).reshape(want.shape)
        if not want.size:
            continue
        rms = float(np.sqrt(np.mean(want ** 2)))
        err = np.abs(got - want)
        bound = tol * rms + c * ref["scale"][name]
        worst = float((err / np.maximum(bound, 1e-300)).max())
        errs[name] = (float(err.max()), rms, worst)
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        assert worst <= 1.0, (f"{label} {name}: err {err[i]} at {i} exceeds its bound {bound[i]} "
                              f"(RMS {rms}, ref {want[i]}, got {got[i]})")
    return errs


@pytest.mark.parametrize("name", list(CASES))
def test_backward_every_element(name):
    cfg = CASES[name]
    print(f"[bwd] {name}: T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} k={cfg.k} cap={cfg.capacity} "
          f"{cfg.dtype}", flush=True)
    inp, dout, fwd, g = run_backward(cfg)
    ref = oracle_backward(cfg, inp, dout, fwd)
    errs = compare(cfg, g, ref, name)
    print(f"[bwd] {name}: " + ", ".join(f"{k}={e / r if r else 0:.2e}/{w:.2f}"
                                        for k, (e, r, w) in errs.items()), flush=True)
    # experts without rows have exactly zero weight gradients
    empty = np.nonzero(np.diff(ref["offsets"]) == 0)[0]
    for e in empty:
        assert not bool(g.dw1[e].any()) and not bool(g.dw2[e].any()), f"expert {e}"


def test_backward_is_deterministic():
    cfg = CASES["mix_rows"]
    _, _, _, g1 = run_backward(cfg)
    keep = {n: getattr(g1, n).clone() for n in ("dx", "dw1", "dw2", "db1", "db2", "dw_gate")}
    _, _, _, g2 = run_backward(cfg)
    for n, v in keep.items():
        assert torch.equal(v, getattr(g2, n)), n


@pytest.mark.parametrize("name", ["mix_rows", "taller_tiles", "switch_small", "tiny_fp32",
                                  "sparse_experts"])
def test_kept_and_recomputed_preactivations_agree(name):
    """With the forward's Z the backward skips recomputing it. Z is the same
    bf16(acc + b1) either way, so everything that follows from dZ is
    identical; dW2 reads H, which the forward rounds from the unrounded z,
    so it only agrees within the bar (fp32 layers: identical)."""
    cfg = CASES[name]
    inp, dout, fwd, g_keep = run_backward(cfg, train=True)
    _, _, _, g_re = run_backward(cfg, train=False)
    for n in ("dx", "dw1", "db1", "db2", "dgate", "dlogits", "dw_gate"):
        assert torch.equal(getattr(g_keep, n), getattr(g_re, n)), n
    if cfg.dtype == "f32":
        assert torch.equal(g_keep.dw2, g_re.dw2)
    ref = oracle_backward(cfg, inp, dout, fwd)
    compare(cfg, g_re, ref, name + " recomputed")


TRAIN_PATHS = {
    "ring": CASES["mix_rows"],                        # 768 rows per expert
    "taller": CASES["taller_tiles"],                  # taller last tiles
    "persistent": CASES["switch_small"],              # about 64 rows per expert
    "streaming": CASES["sparse_experts"],             # 48 rows over 64 experts
    "tiles128": BASE.with_(name="tiles128", T=300, d=384, h=640),
    "tiles64": BASE.with_(name="tiles64", T=200, d=192, h=320),
    "fp32": CASES["f32_ragged"],
}


@pytest.mark.parametrize("path", list(TRAIN_PATHS))
def test_training_forward_keeps_z_and_h(path):
    """moe_grouped_ffn_train on every FFN path: y_perm equals
    moe_grouped_ffn's bit for bit; z_perm is W1 x + b1 rounded once to the
    layer dtype (|err| <= 2^-8 |z| + 1.1 d 2^-24 M, M = sum |x w1| + |b1|:
    one rounding plus fp32 accumulation over d terms in any order); h_perm is
    SiLU of the unrounded z (|SiLU'| <= 1.1). fp32 layers: 2^-16 |z| instead
    of 2^-8 |z|."""
    import moe_inputs as mi2
    from top_routing_expert_topk_amd import native as N
    cfg = TRAIN_PATHS[path]
    inp = mi2.make_inputs(cfg, "cuda")
    b = moe_layer_forward(inp["x"], inp["w_gate"], inp["gate_bias"], inp["w1"], inp["b1"],
                          inp["w2"], inp["b2"], cfg.k, cfg.renorm, cfg.capacity, cfg.residual,
                          train=True)
    y_train = b.y_perm.clone()
    N.moe_grouped_ffn(inp["x"], cfg.T, cfg.d, cfg.h, cfg.E, cfg.k, b.offsets, b.sorted_token,
                      inp["w1"], inp["b1"], inp["w2"], inp["b2"], b.y_perm, b.ws_ffn)
    torch.cuda.synchronize()
    R = int(b.offsets[-1])
    assert torch.equal(y_train[:R], b.y_perm[:R])
    X = bwd.widen(mi2.to_host_array(inp["x"]))
    W1 = bwd.widen(mi2.to_host_array(inp["w1"]))
    B1 = bwd.widen(mi2.to_host_array(inp["b1"]))
    off = b.offsets.cpu().numpy()
    st = b.sorted_token.cpu().numpy()
    z_gpu = _np(b.z_perm[:R])
    h_gpu = _np(b.h_perm[:R])
    c = 2.0 ** -16 if cfg.dtype == "f32" else 2.0 ** -8
    for e in range(cfg.E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        xe = X[st[r0:r1]]
        z = xe @ W1[e].T + B1[e]
        M = np.abs(xe) @ np.abs(W1[e]).T + np.abs(B1[e])
        hz = bwd.silu(z)
        acc = 1.1 * cfg.d * 2.0 ** -24 * M  # fp32 accumulation over d terms, through SiLU'
        assert np.all(np.abs(z_gpu[r0:r1] - z) <= c * np.abs(z) + acc), f"z, expert {e}"
        assert np.all(np.abs(h_gpu[r0:r1] - hz) <= c * np.abs(hz) + acc), f"h, expert {e}"


EDGE = {
    "one_token": BASE.with_(name="one_token", T=1, d=256, h=256),
    "one_expert": BASE.with_(name="one_expert", T=64, d=256, h=256, E=1, k=1),
    "k_equals_E": BASE.with_(name="k_equals_E", T=64, d=256, h=512, E=4, k=4),
    "top3_of_5_no_renorm": BASE.with_(name="top3_of_5_no_renorm", T=80, d=256, h=256, E=5, k=3,
                                      renorm=False, residual=True),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_backward_edge_cases(name):
    cfg = EDGE[name]
    inp, dout, fwd, g = run_backward(cfg)
    ref = oracle_backward(cfg, inp, dout, fwd)
    compare(cfg, g, ref, name)


def test_backward_of_an_empty_batch():
    """T = 0: the backward calls accept the empty batch, every weight and
    bias gradient comes out zero (the calls still write them), and so does
    the router's."""
    from top_routing_expert_topk_amd import MoEGrads
    from top_routing_expert_topk_amd import native as N
    E, k, d, h = 8, 2, 256, 256
    cfg = BASE.with_(name="empty", T=4, d=d, h=h, E=E)
    inp = mi.make_inputs(cfg, "cuda")
    x = inp["x"][:0]
    g = MoEGrads(0, d, h, E, k, torch.bfloat16, torch.device("cuda"), True, True, True)
    for n in ("dw1", "dw2", "db1", "db2", "dw_gate", "dgate_bias"):
        getattr(g, n).fill_(7)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    none_i = torch.empty(0, dtype=torch.int32, device="cuda")
    none_f = torch.empty((0, k), dtype=torch.float32, device="cuda")
    N.moe_combine_backward(g.dy_perm, none_i, none_f, 0, k, d, x, g.dy_perm, g.dgate)
    N.moe_router_backward(g.dlogits, none_i, none_f, g.dgate, offsets[:E], 0, E, k, True, 0.5,
                          g.dlogits)
    N.moe_grouped_ffn_backward(x, 0, d, h, E, k, offsets, none_i, inp["w1"], inp["b1"], inp["w2"],
                               g.dy_perm, None, None, g.dx_perm, g.dw1, g.db1, g.dw2, g.db2,
                               g.ws_ffn)
    N.moe_gather_backward(g.dx_perm, none_i, 0, k, d, None, g.dlogits, inp["w_gate"], E, g.dx)
    N.moe_router_weight_backward(x, 0, d, E, g.dlogits, g.dw_gate, g.dgate_bias, g.ws_router)
    torch.cuda.synchronize()
    for n in ("dw1", "dw2", "db1", "db2", "dw_gate", "dgate_bias"):
        assert not bool(getattr(g, n).any()), n

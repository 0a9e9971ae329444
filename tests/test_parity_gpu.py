"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Full-size workloads are checked on every routing / permutation / aux output
and on every token's output (out in fp32; a bf16 out must be the fp32 out
rounded); reduced shapes that still span several tiles and a ragged tail are
checked on every output element; the edge cases cover ties, capacity 0, k = E, E = 1, a single hot expert, the
largest E and k, T = 0, missing biases and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from _parity import check_layer, run_gpu, sample_tokens

pytestmark = pytest.mark.gpu

CFG = mi.CONFIGS


def _run_and_check(cfg, nsample=None, e2e=None, mutate=None, label=None, bf16_out=False):
    print(f"[parity] {label or cfg.name}: T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} k={cfg.k} "
          f"cap={cfg.capacity} {cfg.dtype}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    if mutate:
        mutate(inp)
    b = run_gpu(cfg, inp)
    b16 = run_gpu(cfg, inp, out_dtype=torch.bfloat16) if bf16_out else None
    toks = sample_tokens(cfg.T, nsample, seed=cfg.cfg_id)
    e2e_t = sample_tokens(cfg.T, e2e, seed=cfg.cfg_id + 100)
    r = check_layer(cfg, inp, b, tokens=toks, e2e_tokens=e2e_t, label=label or cfg.name,
                    b_bf16=b16)
    print(f"[parity] {label or cfg.name}: {r}", flush=True)
    return inp, b, r


# ------------------------------------------------------- full workloads ----
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_fp32", "mixtral_prefill", "switch_top1_cap", "decode",
                                  "deepseek_v3"])
def test_full_workload(name):
    """Every token of the full layer, logits chosen end to end included; the
    bf16 layers run a second time with out stored in bf16, which must be the
    fp32 out rounded (its distance to the oracle is reported). The oracle visits each expert once for all its rows
    (about a minute for the 8192 x 8 DeepSeek-shaped layer on 16 threads)."""
    cfg = CFG[name]
    _run_and_check(cfg, bf16_out=cfg.dtype == "bf16")


# ------------------------------------------- reduced shapes, every element ----
SMALL = {
    "mixtral_small": CFG["mixtral_prefill"].with_(name="mixtral_small", T=300, d=512, h=1024),
    "switch_small": CFG["switch_top1_cap"].with_(name="switch_small", T=1000, d=256, h=512, E=16,
                                                  capacity=79),
    "decode_small": CFG["decode"].with_(name="decode_small", T=7, d=576, h=768, E=16),
    "deepseek_small": CFG["deepseek_v3"].with_(name="deepseek_small", T=513, d=384, h=256, E=64),
    "bn64_small": CFG["mixtral_prefill"].with_(name="bn64_small", T=129, d=448, h=320, E=6, k=3),
    "fp32_ragged": CFG["tiny_fp32"].with_(name="fp32_ragged", T=77, d=96, h=200, E=5, k=2),
    "renorm_off_k2": CFG["mixtral_prefill"].with_(name="renorm_off_k2", T=200, d=256, h=384,
                                                   renorm=False),
    "no_bias": CFG["deepseek_v3"].with_(name="no_bias", T=100, d=256, h=128, E=32, k=4,
                                        expert_bias=False),
    # 256 x 256 tiles: every tile is a tail tile split along K
    "big_tail_only": CFG["mixtral_prefill"].with_(name="big_tail_only", T=1024, d=512, h=1024,
                                                   E=4),
    # 256 x 256 tiles: whole rounds of tiles plus a split tail
    "big_full_tail": CFG["mixtral_prefill"].with_(name="big_full_tail", T=4096, d=512, h=2048),
    # the same without expert biases (the whole tiles' epilogue stages zeros)
    "big_full_tail_no_bias": CFG["mixtral_prefill"].with_(name="big_full_tail_no_bias", T=4096,
                                                           d=512, h=2048, expert_bias=False),
    # 256 x 256 tiles over experts of ~256 rows: many last row blocks hold a
    # few rows, whose idle waves and activation DMAs are skipped
    "big_ragged": CFG["deepseek_v3"].with_(name="big_ragged", T=2048, d=512, h=512, E=64),
    # 32 experts of ~275 rows: an expert's last row block runs as one taller
    # tile of up to 288 rows; few tiles, so the taller tiles are split along K
    "big_taller_split": CFG["deepseek_v3"].with_(name="big_taller_split", T=1100, d=512,
                                                  h=256, E=32),
    # taller last tiles at other widths and expert counts: 48 experts of ~267
    # rows (d = 768, h = 512), and top-2 of 32 with ~281 rows per expert
    "big_taller_e48": CFG["deepseek_v3"].with_(name="big_taller_e48", T=1600, d=768, h=512,
                                                E=48),
    "big_taller_top2": CFG["mixtral_prefill"].with_(name="big_taller_top2", T=4500, d=256,
                                                     h=768, E=32),
    # experts of ~150 rows: persistent 256 x 128 tiles, two row blocks per expert
    "mid_rows_multi": CFG["mixtral_prefill"].with_(name="mid_rows_multi", T=600, d=512, h=1536),
    # 64 experts under a capacity of 80 rows: persistent 256 x 128 tiles, a
    # split tail, capacity drops
    "mid_rows_capacity": CFG["switch_top1_cap"].with_(name="mid_rows_capacity", T=6000, d=512,
                                                       h=1536, E=64),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_reduced_shape_every_element(name):
    _run_and_check(SMALL[name])


def test_taller_tiles_are_planned():
    """The big_taller_split shape does reach the taller-tile path: the first
    product's work list (FFN workspace from byte 256, 32-byte entries e, row0,
    rows, n0, kbeg, kend, unit, ms) holds tiles of 257..288 rows, among them
    K ranges of split tiles, and covers every permuted row of every expert
    exactly once per output panel."""
    cfg = SMALL["big_taller_split"]
    inp = mi.make_inputs(cfg, "cuda")
    b = run_gpu(cfg, inp)
    R, E = int(b.offsets[-1]), cfg.E
    nt = cfg.h // 256
    n_ent = -(-((-(-R // 256) + min(R, E)) * nt + 256) // 8) * 8  # entries of the list
    ent = b.ws_ffn[256:256 + 32 * n_ent].view(torch.int32).reshape(-1, 8).cpu().numpy()
    ent = ent[ent[:, 0] >= 0]
    assert ent[:, 2].max() > 256 and ent[:, 2].max() <= 288
    assert ((ent[:, 2] > 256) & (ent[:, 6] >= 0)).any()
    off = b.offsets.cpu().numpy()
    whole = ent[(ent[:, 6] < 0) | (ent[:, 4] == 0)]  # one entry per tile
    for e in range(E):
        for n0 in range(0, cfg.h, 256):
            t = whole[(whole[:, 0] == e) & (whole[:, 3] == n0)]
            if off[e + 1] == off[e]:
                assert len(t) == 0
                continue
            covered = np.sort(np.concatenate([np.arange(r0, r0 + n) for r0, n in t[:, 1:3]]))
            assert np.array_equal(covered, np.arange(off[e], off[e + 1])), (e, n0)


@pytest.mark.parametrize("name", ["big_full_tail", "big_taller_split", "mid_rows_capacity",
                                  "bn64_small", "decode_small"])
def test_expert_outputs_are_block_fixed_point(name):
    """y_perm of a bf16 layer on the 256 x 256 ring (whole and split tiles),
    taller tiles, the persistent ring, 64-wide tiles and the streaming path:
    every block of 8 features of a written row is normalised (its largest
    mantissa in [2^14, 2^15), or all zero with exponent -127), and the decoded
    rows match the oracle's expert outputs (each expert over its rows, double
    precision) within 2e-2 of their RMS, as the layer outputs do."""
    from _parity import decode_expert_outputs, expert_fetcher
    from oracle import oracle as orc
    cfg = SMALL[name]
    inp = mi.make_inputs(cfg, "cuda")
    b = run_gpu(cfg, inp)
    d = cfg.d
    assert b.y_perm.dtype == torch.uint8
    assert b.y_perm.shape[1] == 2 * d + (-(-(d // 8) // 16)) * 16
    off = b.offsets.cpu().numpy()
    R = int(off[-1])
    vals, mant, ex = decode_expert_outputs(b.y_perm[:R], d)
    top = np.abs(mant.astype(np.int64)).reshape(R, d // 8, 8).max(axis=2)
    zero = ex == -127
    assert np.all(top[zero] == 0)
    assert np.all((top[~zero] >= 1 << 14) & (top[~zero] <= 32767))
    st = b.sorted_token.cpu().numpy()
    fetch = expert_fetcher(inp)
    x_h = mi.to_host_array(inp["x"])
    ref = np.zeros((R, d))
    for e in range(cfg.E):
        if off[e + 1] > off[e]:
            ref[off[e]:off[e + 1]] = orc.expert_rows(x_h, st[off[e]:off[e + 1]], *fetch(e))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.abs(vals - ref).max())
    print(f"[yq] {name}: rows {R} max err {err:.3g} = {err / rms:.4f} RMS", flush=True)
    assert err <= 2e-2 * rms


# ------------------------------------------------------------ edge cases ----
def test_single_token():
    _run_and_check(CFG["mixtral_prefill"].with_(T=1, d=256, h=512), label="single_token")


def test_zero_gate_ties_and_drop_set():
    cfg = CFG["switch_top1_cap"].with_(T=500, d=256, h=256, E=8, k=3, renorm=True, capacity=37,
                                       zipf_gate_bias=False)

    def zero(inp):
        inp["w_gate"].zero_()
    _, b, _ = _run_and_check(cfg, mutate=zero, label="zero_gate")
    idx = b.topk_idx.cpu().numpy()
    assert np.all(idx == np.arange(cfg.k))
    dest = b.dest_row.cpu().numpy().reshape(cfg.T, cfg.k)
    assert np.array_equal(dest >= 0, np.broadcast_to(np.arange(cfg.T)[:, None] < 37, dest.shape))


def test_capacity_zero_passes_residual_exactly():
    cfg = CFG["switch_top1_cap"].with_(T=300, d=256, h=256, E=8, capacity=0)
    inp, b, _ = _run_and_check(cfg, label="capacity_zero")
    assert int(b.offsets[-1]) == 0
    assert torch.equal(b.out, inp["x"].float())


def test_k_equals_E():
    _run_and_check(CFG["mixtral_prefill"].with_(T=100, d=256, h=256, E=4, k=4), label="k_eq_E")


def test_single_expert():
    _run_and_check(CFG["mixtral_prefill"].with_(T=100, d=128, h=256, E=1, k=1), label="E1")


@pytest.mark.parametrize("T,E", [(40, 64), (700, 8)])
def test_one_hot_expert(T, E):
    """A huge router bias sends every token to expert 3 (decode path: rows > 4 per pass;
    GEMM path: many tiles of one expert)."""
    cfg = CFG["decode"].with_(T=T, d=512, h=512, E=E, zipf_gate_bias=False)

    def bias(inp):
        gb = torch.zeros(E, device="cuda")
        gb[3] = 100.0
        inp["gate_bias"] = gb
    _, b, _ = _run_and_check(cfg, mutate=bias, label=f"hot_expert_T{T}_E{E}")
    assert int(b.counts[3]) == T


def test_largest_E_and_k():
    _run_and_check(CFG["deepseek_v3"].with_(T=300, d=256, h=128, E=512, k=16), label="E512_k16")


def test_determinism_bitwise():
    cfg = SMALL["deepseek_small"]
    inp = mi.make_inputs(cfg, "cuda")
    a = run_gpu(cfg, inp)
    snap = {n: getattr(a, n).clone() for n in ("out", "topk_gate", "prob_sum", "loss", "y_perm")}
    b = run_gpu(cfg, inp)
    for n, v in snap.items():
        assert torch.equal(v, getattr(b, n)), n


def test_empty_batch():
    from top_routing_expert_topk_amd import native as N
    E, k, d, h = 8, 2, 128, 256
    x = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    wg = torch.randn(E, d, device="cuda").to(torch.bfloat16)
    idx = torch.empty((0, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((0, k), dtype=torch.float32, device="cuda")
    ps = torch.full((E,), 7.0, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    N.moe_router_topk(x, wg, None, E, k, True, None, idx, gate, ps, ws)
    counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    N.moe_permute(idx, 0, k, E, -1, counts, offsets, idx.view(-1), idx.view(-1), None)
    torch.cuda.synchronize()
    assert torch.all(ps == 0) and torch.all(counts == 0) and torch.all(offsets == 0)


@pytest.mark.parametrize("name", ["mixtral_small", "switch_small", "deepseek_small",
                                  "bn64_small", "big_ragged", "mid_rows_capacity"])
def test_bf16_output_is_the_rounded_fp32_output(name):
    """out stored as bf16 on reduced shapes: every element is the fp32-output
    run's value rounded to nearest even (the fp32 run meets the bar)."""
    _run_and_check(SMALL[name], label=f"{name}_bf16_out", bf16_out=True)


@pytest.mark.parametrize("E,k", [(8, 2), (100, 3), (130, 1), (200, 4), (300, 2), (400, 6),
                                 (450, 2), (512, 8)])
def test_router_expert_counts(E, k):
    """Every expert-tile shape of the bf16 router (E padded to 64, 128, ..., 512)."""
    cfg = CFG["deepseek_v3"].with_(T=300, d=320, h=64, E=E, k=k)
    _run_and_check(cfg, label=f"router_E{E}_k{k}")


@pytest.mark.parametrize("T,E,k,d,bias", [(4100, 256, 8, 448, False), (2048, 512, 16, 256, True),
                                          (4096, 256, 1, 320, True), (8192, 256, 8, 7168, False)])
def test_router_at_scale(T, E, k, d, bias):
    """The bf16 router at thousands of tokens and 256 or 512 experts: a ragged
    last token tile, the largest k, a router bias, and the DeepSeek-shaped
    width. Logits, every token's selection (same logits: bit-exact; end to
    end: where the gap is clear), gates, the permutation and the aux
    statistics against the oracle; the FFN outputs of these shapes are not
    what is tested here."""
    cfg = CFG["deepseek_v3"].with_(name=f"router_T{T}_E{E}", T=T, d=d, h=256, E=E, k=k,
                                   zipf_gate_bias=bias)
    print(f"[parity] {cfg.name}: T={T} d={d} E={E} k={k} bias={bias}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    b = run_gpu(cfg, inp)
    r = check_layer(cfg, inp, b, tokens=np.zeros(0, np.int32),
                    e2e_tokens=sample_tokens(T, 2048, seed=7))
    print(f"[parity] {cfg.name}: {r}", flush=True)


@pytest.mark.parametrize("dtype,T,d,E,k,bias", [("bf16", 1000, 96, 100, 5, True),
                                                ("bf16", 777, 320, 130, 2, False),
                                                ("f32", 333, 72, 7, 3, True)])
def test_router_alone_and_logits_only(dtype, T, d, E, k, bias):
    """moe_router_topk on its own: a width that is not a multiple of 64 (the
    16x16x32 logits kernel), one that is, and fp32 with E % 4 != 0. The
    selection is bit-exact with the oracle's on the same logits and the
    logits match the oracle's double ones; a call with no top-k, gate or
    probability outputs writes the same logits bit for bit."""
    from oracle import oracle as orc
    from top_routing_expert_topk_amd import native as N
    cfg = CFG["deepseek_v3"].with_(name="router_alone", T=T, d=d, h=64, E=E, k=k, dtype=dtype,
                                   zipf_gate_bias=bias)
    print(f"[parity] router alone: {dtype} T={T} d={d} E={E} k={k} bias={bias}", flush=True)
    inp = mi.make_inputs(cfg, "cuda")
    x, wg, gb = inp["x"], inp["w_gate"], inp["gate_bias"]
    ws = torch.empty(N.moe_workspace_size(N.MOE_OP_ROUTER, T, d, 0, E, k), dtype=torch.uint8,
                     device="cuda")
    lg = torch.empty((T, E), device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), device="cuda")
    ps = torch.empty((E,), device="cuda")
    N.moe_router_topk(x, wg, gb, E, k, True, lg, idx, gate, ps, ws)
    lg2 = torch.full((T, E), float("nan"), device="cuda")
    N.moe_router_topk(x, wg, gb, E, k, True, lg2, None, None, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(lg, lg2), "logits-only call"
    lg_h = lg.cpu().numpy()
    o_idx, o_gate, o_ps = orc.route(lg_h, k, True)
    assert np.array_equal(idx.cpu().numpy(), o_idx), "top-k indices on the same logits"
    assert np.abs(gate.cpu().numpy() - o_gate).max() <= 1e-5
    assert np.allclose(ps.cpu().numpy(), o_ps, rtol=1e-5, atol=1e-6)
    lg_o = orc.logits(mi.to_host_array(x), mi.to_host_array(wg), None if gb is None else gb.cpu().numpy())
    tol = 1e-4 if dtype == "bf16" else 1e-5
    assert np.abs(lg_h - lg_o).max() <= tol * max(1.0, float(np.abs(lg_o).max()))

"""Benchmark: one MoE layer forward on one MI355X, routed tokens per second.

A step is one pass of the whole layer over one batch of synthetic, seeded
inputs already resident in HBM: router -> permute -> grouped FFN -> combine
-> aux loss, five library calls enqueued on one stream. W untimed warm-up
steps, then K timed steps bracketed by device synchronisation. Per-call
durations come from HIP events recorded on the same stream around every
call of every timed step.

The default workload is the DeepSeek-V3-shaped routed-expert layer (T=8192,
d=7168, expert hidden 2048, 256 experts, top-8, bf16): the largest of the
workloads that fits one GPU. Prints one JSON line, with the dominant call
(the grouped FFN) against both rooflines (dense bf16 MFMA at the published
2.5 PFLOP/s and at 2.3 PFLOP/s, HBM at 8 TB/s), the binding one named in
"bound", and the shader clock sampled during the timed steps.

--backward times a training step instead: the forward (keeping the logits,
pre-activations and hidden rows) followed by the backward calls (combine, router, grouped FFN, gather,
router weights) on a seeded upstream gradient, and reports the backward's
grouped FFN against the MFMA roofline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_BF16_ALT_TFLOPS = 2300.0  # the dense bf16 figure the workload statement quotes
METRIC = "routed tokens/sec per MoE layer fwd (bf16, 1 GPU) + % of MFMA/HBM roofline"
ROOT = os.path.dirname(os.path.abspath(__file__))
CALLS = ("router", "permute", "ffn", "combine", "aux")
EC_CALLS = ("router", "choice", "ffn", "combine")  # Expert Choice layer
BWD_CALLS = ("combine_bwd", "router_bwd", "ffn_bwd", "gather_bwd", "router_weight_bwd")
TRAIN_METRIC = "routed tokens/sec per MoE layer fwd+bwd (bf16, 1 GPU) + % of MFMA roofline"
# tokens whose expert FFN the CPU baseline evaluates (routing always covers all T)
CPU_SAMPLE = {"tiny_fp32": 256, "mixtral_prefill": 2048, "switch_top1_cap": 8192, "decode": 32,
              "deepseek_v3": 2048, "switch_expert_choice": 2048, "decode_offload": 32}
# tokens of the sub-batch the backward CPU baseline differentiates
BWD_CPU_SAMPLE = {"tiny_fp32": 256, "mixtral_prefill": 1024, "switch_top1_cap": 2048,
                  "deepseek_v3": 64, "switch_expert_choice": 2048}
PCIE_GBS = 64.0             # PCIe 5.0 x16, one direction
OFFLOAD_BATCHES = 16        # distinct token batches the offload workload cycles through


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first: on a fresh process the first heavy calls run up to 30%% slower and settle after about ten")
    ap.add_argument("--config", default="deepseek_v3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 3 s run after the timed steps that reads the shader clock "
                         "(for counter runs, where every dispatch is serialised)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (a 'graph' "
                         "object beside the eager line's figures)")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (a training step) instead of the forward")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="JSON with HBM bytes per dominant-call launch from rocprofv3 counters")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES bytes (counter calibration)")
    ap.add_argument("--summarize-counters", default="", metavar="DIR",
                    help="only turn the rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR (subfolders "
                         "pmc_FETCH_SIZE, pmc_WRITE_SIZE, pmc_copy_FETCH_SIZE, pmc_copy_WRITE_SIZE) "
                         "into the --traffic record of --config, scaled by the copy calibration "
                         "(--copy-calibration BYTES gives its size)")
    return ap.parse_args()


def ffn_source_hash() -> str:
    """Hash of the grouped-FFN kernel sources; counter data for another source is stale."""
    import hashlib
    h = hashlib.sha256()
    for f in ("ffn.hip", "ring_gemm.h", "tile_map.h", "moe_internal.h"):
        h.update(open(os.path.join(ROOT, "top_routing_expert_topk_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(path, workload):
    """HBM bytes per moe_grouped_ffn call, if measured for this kernel source, else None."""
    if not path or not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if not rec or rec.get("ffn_source") != ffn_source_hash():
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


# kernels of one moe_grouped_ffn call, by name prefix
FFN_KERNELS = ("big_plan", "gemm_bf16_ring", "gemm_bf16_pring", "big_tail_reduce", "gemm_bf16<",
               "build_tile_map", "decode_bf16", "gemm_f32")


def _counter_means(folder, counter):
    """Mean value of `counter` per dispatch, per kernel name, from the rocprofv3
    counter-collection CSV files under folder."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            name = row["Kernel_Name"]
            for pre in ("void ", "moe::(anonymous namespace)::", "moe::"):
                name = name.replace(pre, "")
            vals.setdefault(name.split("(")[0], []).append(float(row["Counter_Value"]))
    return {k: float(np.mean(v)) for k, v in vals.items()}


def summarize_counters(folder, workload, copy_bytes, out_path):
    """Writes the traffic record of one workload: the FFN call's HBM-side
    bytes per call (FETCH_SIZE + WRITE_SIZE, KiB per dispatch, summed over
    the call's kernels), each counter divided by what it reads for a plain
    device copy of copy_bytes bytes (FETCH_SIZE reads about half the bytes
    a copy reads, WRITE_SIZE all it writes)."""
    factor = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cal = _counter_means(os.path.join(folder, f"pmc_copy_{c}"), c)
        copy_kib = max(cal.values())  # the copy kernel dominates its run
        factor[c] = copy_kib * 1024.0 / copy_bytes
    per_kernel, tot = {}, {"FETCH_SIZE": 0.0, "WRITE_SIZE": 0.0}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        for name, kib in _counter_means(os.path.join(folder, f"pmc_{c}"), c).items():
            b = kib * 1024.0 / factor[c]
            per_kernel.setdefault(name, {})["fetch_bytes" if c == "FETCH_SIZE" else "write_bytes"] = b
            if name.startswith(FFN_KERNELS):
                tot[c] += b
    rec = json.load(open(out_path)) if os.path.exists(out_path) else {}
    rec[workload] = {"ffn_source": ffn_source_hash(), "fetch_bytes": tot["FETCH_SIZE"],
                     "write_bytes": tot["WRITE_SIZE"], "fetch_factor": factor["FETCH_SIZE"],
                     "write_factor": factor["WRITE_SIZE"], "per_kernel": per_kernel}
    json.dump(rec, open(out_path, "w"), indent=1)
    print(json.dumps({"workload": workload, **{k: v for k, v in rec[workload].items()
                                                if k != "per_kernel"}}), flush=True)


def copy_calibration(nbytes, steps):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "steps": steps}), flush=True)


class ClockSampler:
    """Samples amdsmi's GPU metrics table in a background thread: the current
    shader clock of every XCD (current_gfxclks). The firmware refreshes that
    table about once a second, so a sample only describes the load if the
    table was refreshed while the load ran; see clock_window."""

    def __init__(self, period_s=0.02):
        import threading
        self.period, self.samples, self.err = period_s, [], None
        self._stop = threading.Event()
        self._th = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            try:
                h = amdsmi.amdsmi_get_processor_handles()[0]
                while not self._stop.is_set():
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    xcd = [float(v) for v in (m.get("current_gfxclks") or [])
                           if isinstance(v, (int, float)) and 0 < v < 65535]
                    if xcd:
                        self.samples.append((time.perf_counter(), m.get("system_clock_counter"),
                                             float(np.mean(xcd)), min(xcd), max(xcd)))
                    self._stop.wait(self.period)
            finally:
                amdsmi.amdsmi_shut_down()
        except Exception as exc:  # no amdsmi or no permission: report none
            self.err = repr(exc)[:200]

    def __enter__(self):
        self._th.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        self._th.join(timeout=5)

    def summary(self, t_load):
        """Table refreshes first seen at least 0.25 s after the load began."""
        seen, upd = set(), []
        for t, cnt, mean, lo, hi in self.samples:
            if cnt in seen:
                continue
            seen.add(cnt)
            if t >= t_load + 0.25:
                upd.append((mean, lo, hi))
        if not upd:
            return {"mhz": None, "note": self.err or "no table refresh during the load"}
        v = np.array(upd)
        return {"mhz": float(np.median(v[:, 0])), "mean_mhz": float(v[:, 0].mean()),
                "min_xcd_mhz": float(v[:, 1].min()), "max_xcd_mhz": float(v[:, 2].max()),
                "refreshes": int(len(upd)),
                "source": "amdsmi gpu_metrics current_gfxclks (mean of the 8 XCDs, table "
                          "refreshed ~1/s) while the same step runs for 3 s after the timed "
                          "steps; median over the refreshes"}


CLOCK_SECONDS = 3.0


def clock_window(step, seconds=None):
    """Runs step() back to back for `seconds` (untimed, after the timed
    region) and returns the shader clock the metrics table reported meanwhile."""
    import torch
    seconds = CLOCK_SECONDS if seconds is None else seconds
    if seconds <= 0:
        return {"mhz": None, "note": "not measured (--no-clock)"}
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            step()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    return clk.summary(t0)


def graph_replay(step, stream, steps, warmup, T):
    """The same step captured once in a HIP graph on `stream` and replayed:
    `steps` timed replays after `warmup` untimed ones, HIP events on the
    stream around the whole timed region."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "replays": steps,
            "note": "the step's calls captured once in a HIP graph and replayed"}


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(cfg, inp, sample_n):
    """The oracle timed on this host: routing/permute/aux on all T tokens, expert FFN +
    combine on a seeded token sample; the rate is extrapolated to the full batch."""
    import moe_inputs as mi
    from oracle import oracle as orc
    x = mi.to_host_array(inp["x"])
    wg = mi.to_host_array(inp["w_gate"])
    gb = None if inp["gate_bias"] is None else inp["gate_bias"].cpu().numpy()
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(cfg.T, size=min(sample_n, cfg.T), replace=False)).astype(np.int32)
    host_w = {}

    def fetch(e):  # host copies are made before the clock starts
        return host_w[e]
    # which experts the sample needs: route once untimed to know what to copy to the host
    lg_all = orc.logits(x, wg, gb)
    if cfg.routing == "expert_choice":
        _, _, dest, _ = orc.expert_choice(orc.ec_scores(lg_all), cfg.capacity)
        need = set(np.nonzero((dest[toks] >= 0).any(axis=0))[0].tolist())
    else:
        lg0 = orc.logits(x[toks], wg, gb)
        need = set(orc.route(lg0, cfg.k, cfg.renorm)[0].ravel().tolist())
        need |= set(orc.route(lg_all, cfg.k, cfg.renorm)[0][toks].ravel().tolist())
    for e in sorted(need):
        host_w[e] = tuple(None if inp[n] is None else mi.to_host_array(inp[n][e])
                          for n in ("w1", "b1", "w2", "b2"))
    if cfg.routing == "expert_choice":
        return _cpu_baseline_ec(cfg, inp, x, wg, gb, toks, host_w, fetch)
    t0 = time.perf_counter()
    lg = orc.logits(x, wg, gb)
    t1 = time.perf_counter()
    idx, gate, ps = orc.route(lg, cfg.k, cfg.renorm)
    counts, offsets, dest, st = orc.permute(idx, cfg.E, cfg.capacity)
    orc.aux(ps, counts, cfg.T)
    t2 = time.perf_counter()
    # moe_forward re-runs route/permute/aux on all tokens, then FFN + combine on the sample
    orc.moe_forward(x, wg, None, None, None, None, cfg.k, cfg.renorm, cfg.capacity, gate_bias=gb,
                    residual=cfg.residual, lg=lg, tokens=toks, expert_weights=fetch)
    t3 = time.perf_counter()
    t_route = (t1 - t0) + (t2 - t1)
    t_ffn = max((t3 - t2) - (t2 - t1), 1e-9)
    full = t_route + t_ffn * cfg.T / toks.size
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": cfg.T / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"routing, permute and aux on all {cfg.T} tokens ({t_route:.2f} s); expert "
                       f"FFN + combine on {toks.size} seeded tokens ({t_ffn:.2f} s), extrapolated "
                       f"to {cfg.T}; double precision, {threads} threads on {cpu_model()}"),
            "extrapolated": toks.size < cfg.T, "seconds": t3 - t0}


def _cpu_baseline_ec(cfg, inp, x, wg, gb, toks, host_w, fetch):
    """Expert Choice layer on the oracle: logits, scores and every expert's
    selection on all T tokens; expert FFN + combine on the token sample."""
    from oracle import oracle as orc
    t0 = time.perf_counter()
    lg = orc.logits(x, wg, gb)
    ta = time.perf_counter()
    orc.expert_choice(orc.ec_scores(lg), cfg.capacity)
    t1 = time.perf_counter()
    orc.moe_forward_ec(x, wg, None, None, None, None, cfg.capacity, gate_bias=gb,
                       residual=cfg.residual, lg=lg, tokens=toks, expert_weights=fetch)
    t2 = time.perf_counter()
    t_route = t1 - t0
    t_ffn = max((t2 - t1) - (t1 - ta), 1e-9)  # moe_forward_ec redoes scores and selection
    full = t_route + t_ffn * cfg.T / toks.size
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": cfg.T / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"logits, scores and Expert Choice selection on all {cfg.T} tokens "
                       f"({t_route:.2f} s); expert FFN + combine on {toks.size} seeded tokens "
                       f"({t_ffn:.2f} s), extrapolated to {cfg.T}; double precision, {threads} "
                       f"threads on {cpu_model()}"),
            "extrapolated": toks.size < cfg.T, "seconds": t2 - t0}


def bench_offload(args, cfg, inp, dev):
    """Layer over host-resident experts: each step routes a new batch (cycling
    through OFFLOAD_BATCHES seeded batches resident in HBM), reads the counts
    back, copies the missing experts from pinned host memory into the LRU
    slots while the resident ones run, then runs the loaded ones."""
    import torch
    import top_routing_expert_topk_amd as moe
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    gen = torch.Generator(device=dev)
    xs = []
    for i in range(OFFLOAD_BATCHES):
        gen.manual_seed(int(np.random.SeedSequence([20261203, cfg.cfg_id, 99, i]).generate_state(1)[0]))
        xs.append(torch.randn((T, d), generator=gen, device=dev).to(cfg.torch_dtype))
    cache = moe.ExpertCache(inp["w1"], inp["b1"], inp["w2"], inp["b2"], cfg.offload_slots, dev)
    del inp["w1"], inp["w2"]  # the experts now live in host memory and device slots only
    torch.cuda.empty_cache()
    bufs = moe.MoEBuffers(T, d, h, E, k, cfg.torch_dtype, dev)
    stream = torch.cuda.Stream(dev)  # default priority
    expert_bytes = sum(t[0].numel() * t.element_size() for t in cache.host if t is not None)

    def step(i):
        moe.moe_layer_forward_cached(xs[i % OFFLOAD_BATCHES], inp["w_gate"], inp["gate_bias"],
                                     cache, k, cfg.renorm, cfg.capacity, cfg.residual,
                                     bufs=bufs, stream=stream)
        return cache.loaded

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    loads, touched = [], []
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.warmup, args.warmup + args.steps):
        loads.append(step(i))
        touched.append(int((bufs.counts.cpu() > 0).sum()))
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ctr = iter(range(args.warmup + args.steps, 1 << 30))
    sclk = clock_window(lambda: step(next(ctr)))
    ms_step = e0.elapsed_time(e1) / args.steps
    loaded = float(np.mean(loads))
    pcie_bytes = loaded * expert_bytes
    out = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "d": d, "h": h, "E": E, "k": k,
                   "renorm": bool(cfg.renorm), "capacity": cfg.capacity,
                   "residual": bool(cfg.residual), "routing": cfg.routing,
                   "offload_slots": cfg.offload_slots, "parallelism": "single GPU"},
        "offload": {"experts_loaded_per_step": loaded,
                    "experts_touched_per_step": float(np.mean(touched)),
                    "hit_rate": 1.0 - float(np.sum(loads)) / max(1, int(np.sum(touched))),
                    "expert_bytes": expert_bytes, "pcie_bytes_per_step": pcie_bytes,
                    "pcie_GBps_over_step": pcie_bytes / (ms_step * 1e-3) / 1e9,
                    "pcie_peak_GBps": PCIE_GBS},
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "device": torch.cuda.get_device_name(dev),
        "sclk": sclk,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_backward(cfg, inp, dout, sample_n):
    """The backward oracle timed on this host over the first sample_n tokens
    (routing, every expert's forward and backward products and the router
    gradients of that sub-batch), extrapolated to T tokens."""
    import moe_inputs as mi
    from oracle import backward as bwd
    n = min(sample_n, cfg.T)
    h = {k: mi.to_host_array(v) for k, v in inp.items() if v is not None}
    x = h["x"][:n]
    g = mi.to_host_array(dout)[:n]
    t0 = time.perf_counter()
    if cfg.routing == "expert_choice":
        # the sub-batch keeps the ratio of capacity to tokens
        c = max(1, round(cfg.capacity * n / cfg.T))
        bwd.moe_backward_ec(x, h["w_gate"], h["w1"], h.get("b1"), h["w2"], h.get("b2"), c, g,
                            gate_bias=h.get("gate_bias"), residual=cfg.residual)
    else:
        bwd.moe_backward(x, h["w_gate"], h["w1"], h.get("b1"), h["w2"], h.get("b2"), cfg.k,
                         cfg.renorm, cfg.capacity, g, 0.01, gate_bias=h.get("gate_bias"),
                         residual=cfg.residual)
    t = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"forward products and full backward of the layer over the first {n} of "
                       f"{cfg.T} tokens ({t:.2f} s; weight gradients over those tokens' rows), "
                       f"rate per token; double precision numpy, {threads} threads on "
                       f"{cpu_model()}"),
            "extrapolated": n < cfg.T, "seconds": t}


def bench_backward(args, cfg, inp, dev):
    """Training step: forward with the logits kept, then the five backward
    calls on a seeded upstream gradient (aux-loss weight 0.01)."""
    import torch
    import moe_inputs as mi
    import top_routing_expert_topk_amd as moe
    from top_routing_expert_topk_amd import native as N
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    ec = cfg.routing == "expert_choice"
    daux = 0.0 if ec else 0.01
    dout = mi.make_dout(cfg, dev)
    if ec:
        bufs = moe.ECBuffers(T, d, h, E, cfg.capacity, cfg.torch_dtype, dev, cfg.torch_dtype,
                             train=True)
        k = bufs.k_ffn  # FFN rows per token; the combine and router run with E slots
    else:
        bufs = moe.MoEBuffers(T, d, h, E, k, cfg.torch_dtype, dev, cfg.torch_dtype, train=True)
    grads = moe.MoEGrads(T, d, h, E, k, cfg.torch_dtype, dev, inp["b1"] is not None,
                         inp["b2"] is not None, inp["gate_bias"] is not None,
                         slots=E if ec else 0)
    slots = E if ec else k
    stream = torch.cuda.Stream(dev)  # default priority
    x, wg, gb = inp["x"], inp["w_gate"], inp["gate_bias"]
    w1, b1, w2, b2 = inp["w1"], inp["b1"], inp["w2"], inp["b2"]

    def step(ev=None):
        b, g = bufs, grads
        if ev is not None:
            ev[0].record(stream)
        if ec:
            moe.moe_layer_forward_ec(x, wg, gb, w1, b1, w2, b2, cfg.capacity, cfg.residual,
                                     bufs=b, stream=stream, train=True)
        else:
            moe.moe_layer_forward(x, wg, gb, w1, b1, w2, b2, k, cfg.renorm, cfg.capacity,
                                  cfg.residual, bufs=b, stream=stream, train=True)
        if ev is not None:
            ev[1].record(stream)
        gate = b.gate if ec else b.topk_gate
        N.moe_combine_backward(b.y_perm, b.dest_row, gate, T, slots, d, dout, g.dy_perm, g.dgate,
                               stream)
        if ev is not None:
            ev[2].record(stream)
        N.moe_router_backward(b.logits, None if ec else b.topk_idx, gate, g.dgate,
                              None if ec else b.counts, T, E, slots, False if ec else cfg.renorm,
                              daux, g.dlogits, stream)
        if ev is not None:
            ev[3].record(stream)
        N.moe_grouped_ffn_backward(x, T, d, h, E, k, b.offsets, b.sorted_token, w1, b1, w2,
                                   g.dy_perm, b.z_perm, b.h_perm, g.dx_perm, g.dw1, g.db1, g.dw2,
                                   g.db2, g.ws_ffn, stream)
        if ev is not None:
            ev[4].record(stream)
        N.moe_gather_backward(g.dx_perm, b.dest_row, T, slots, d,
                              dout if cfg.residual else None, g.dlogits, wg, E, g.dx, stream)
        if ev is not None:
            ev[5].record(stream)
        N.moe_router_weight_backward(x, T, d, E, g.dlogits, g.dw_gate, g.dgate_bias,
                                     g.ws_router, stream)
        if ev is not None:
            ev[6].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    calls = ("forward",) + BWD_CALLS
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = clock_window(step)
    graph = graph_replay(step, stream, args.steps, args.warmup, T) if args.graph else None
    ms = {c: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in events]))
          for j, c in enumerate(calls)}
    ms_step = events[0][0].elapsed_time(events[-1][len(calls)]) / args.steps
    R = int(bufs.offsets[-1])
    counts = np.diff(bufs.offsets.cpu().numpy())
    touched = int((counts > 0).sum())
    # algorithmic work of the backward FFN: dH, dX, dW1, dW2 (2 R d h each);
    # its unavoidable HBM bytes: the touched experts' W1 and W2 read for the
    # data gradients, and every expert's dW1, dW2, db1, db2 written
    ebytes = 2 if cfg.dtype == "bf16" else 4
    flop = 8.0 * R * d * h
    wbytes = (touched * 2 * d * h + E * (2 * d * h + d + h)) * ebytes
    t_bwd = ms["ffn_bwd"] * 1e-3
    if cfg.dtype != "bf16":
        roof = {"bound": "alu", "achieved": flop / t_bwd / 1e12, "peak": PEAK_F32_TFLOPS,
                "unit": "TFLOP/s"}
    elif flop / max(wbytes, 1) > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": flop / t_bwd / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": wbytes / t_bwd / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = ("moe_grouped_ffn_backward (dZ and dX_perm on the MFMA ring GEMM, dW1 and dW2 "
                      "on the weight-gradient GEMM, gathered input rows, bias sums)")
    roof["per_launch"] = {"flop": flop, "weight_bytes": wbytes, "rows": R,
                          "touched_experts": touched}
    out = {
        "metric": TRAIN_METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name + "_train", "T": T, "d": d, "h": h, "E": E, "k": k,
                   "renorm": bool(cfg.renorm), "capacity": cfg.capacity,
                   "residual": bool(cfg.residual), "routing": cfg.routing, "daux": daux,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "ms_per_call": ms,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "device": torch.cuda.get_device_name(dev),
        "sclk": sclk,
    }
    if graph is not None:
        out["graph"] = graph
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(cfg, inp, dout, BWD_CPU_SAMPLE.get(cfg.name, 64))
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer forward runs on a single MI355X "
              "(no expert or data parallelism across GPUs); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.config, args.copy_calibration or (1 << 30),
                           args.traffic)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    global CLOCK_SECONDS
    if args.no_clock:
        CLOCK_SECONDS = 0.0
    import torch
    import moe_inputs as mi
    import top_routing_expert_topk_amd as moe
    from top_routing_expert_topk_amd import native as N

    cfg = mi.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = mi.make_inputs(cfg, dev)
    torch.cuda.synchronize()
    if cfg.offload_slots > 0:
        return bench_offload(args, cfg, inp, dev)
    if args.backward:
        return bench_backward(args, cfg, inp, dev)
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    ec = cfg.routing == "expert_choice"
    calls = EC_CALLS if ec else CALLS
    if ec:
        bufs = moe.ECBuffers(T, d, h, E, cfg.capacity, cfg.torch_dtype, dev)
    else:
        bufs = moe.MoEBuffers(T, d, h, E, k, cfg.torch_dtype, dev)
    stream = torch.cuda.Stream(dev)  # default priority
    x = inp["x"]
    resid = x if cfg.residual else None

    def step_ec(ev=None):
        b = bufs
        if ev is not None:
            ev[0].record(stream)
        N.moe_router_topk(x, inp["w_gate"], inp["gate_bias"], E, 1, True, b.logits, None, None,
                          None, b.ws_router, stream)
        if ev is not None:
            ev[1].record(stream)
        N.moe_expert_choice(b.logits, T, E, cfg.capacity, b.scores, b.offsets, b.sorted_token,
                            b.dest_row, b.gate, stream)
        if ev is not None:
            ev[2].record(stream)
        N.moe_grouped_ffn(x, T, d, h, E, b.k_ffn, b.offsets, b.sorted_token, inp["w1"],
                          inp["b1"], inp["w2"], inp["b2"], b.y_perm, b.ws_ffn, stream)
        if ev is not None:
            ev[3].record(stream)
        N.moe_combine(b.y_perm, x.dtype, b.dest_row, b.gate, T, E, d, resid, b.out, stream)
        if ev is not None:
            ev[4].record(stream)

    def step(ev=None):
        if ec:
            return step_ec(ev)
        b = bufs
        if ev is not None:
            ev[0].record(stream)
        N.moe_router_topk(x, inp["w_gate"], inp["gate_bias"], E, k, cfg.renorm, None, b.topk_idx,
                          b.topk_gate, b.prob_sum, b.ws_router, stream)
        if ev is not None:
            ev[1].record(stream)
        N.moe_permute(b.topk_idx, T, k, E, cfg.capacity, b.counts, b.offsets, b.dest_row,
                      b.sorted_token, b.ws_permute, stream)
        if ev is not None:
            ev[2].record(stream)
        N.moe_grouped_ffn(x, T, d, h, E, k, b.offsets, b.sorted_token, inp["w1"], inp["b1"],
                          inp["w2"], inp["b2"], b.y_perm, b.ws_ffn, stream)
        if ev is not None:
            ev[3].record(stream)
        N.moe_combine(b.y_perm, x.dtype, b.dest_row, b.topk_gate, T, k, d, resid, b.out, stream)
        if ev is not None:
            ev[4].record(stream)
        N.moe_aux_loss(b.prob_sum, b.counts, T, E, b.f, b.P, b.loss, stream)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = clock_window(step)
    graph = graph_replay(step, stream, args.steps, args.warmup, T) if args.graph else None
    nc = len(calls)
    per_call = {c: [] for c in calls}
    for ev in events:
        for j, c in enumerate(calls):
            per_call[c].append(ev[j].elapsed_time(ev[j + 1]))
    ms = {c: float(np.mean(v)) for c, v in per_call.items()}
    # whole timed region (gaps between steps included) over K steps
    ms_step = events[0][0].elapsed_time(events[-1][nc]) / args.steps

    R = int(bufs.offsets[-1])
    if ec:
        touched = E if R > 0 else 0
    else:
        counts = bufs.counts.cpu().numpy()
        touched = int((np.minimum(counts, cfg.capacity if cfg.capacity >= 0 else counts) > 0).sum())
    ebytes = 2 if cfg.dtype == "bf16" else 4
    ffn_flop = 4.0 * R * d * h
    expert_bytes = touched * (2 * d * h + d + h) * ebytes
    t_ffn = ms["ffn"] * 1e-3
    mfma_bound = cfg.dtype == "bf16" and ffn_flop / max(expert_bytes, 1) > \
        PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(args.traffic, cfg.name)
    if cfg.dtype != "bf16":
        roof = {"bound": "alu", "achieved": ffn_flop / t_ffn / 1e12, "peak": PEAK_F32_TFLOPS,
                "unit": "TFLOP/s"}
    elif mfma_bound:
        roof = {"bound": "mfma", "achieved": ffn_flop / t_ffn / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": expert_bytes / t_ffn / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    if cfg.dtype == "bf16":
        # both rooflines of the call: time at 100% of each peak, and the
        # fraction reached of each (the binding one is the longer time)
        tflops = ffn_flop / t_ffn / 1e12
        roof["both"] = {
            "mfma_ms_at_peak": ffn_flop / (PEAK_BF16_TFLOPS * 1e12) * 1e3,
            "hbm_ms_at_peak": expert_bytes / (PEAK_HBM_GBS * 1e9) * 1e3,
            "mfma_frac": tflops / PEAK_BF16_TFLOPS,
            "mfma_frac_at_2300": tflops / PEAK_BF16_ALT_TFLOPS,
            "hbm_frac": expert_bytes / t_ffn / 1e9 / PEAK_HBM_GBS,
            "ffn_ms": ms["ffn"],
        }
    roof["kernel"] = "moe_grouped_ffn (expert GEMM1+SiLU and GEMM2, both grouped MFMA launches)"
    roof["per_launch"] = {"flop": ffn_flop, "expert_weight_bytes": expert_bytes, "rows": R,
                          "touched_experts": touched}

    out = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "d": d, "h": h, "E": E, "k": k,
                   "renorm": bool(cfg.renorm), "capacity": cfg.capacity,
                   "residual": bool(cfg.residual), "routing": cfg.routing,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kept_rows_per_s": R / (ms_step * 1e-3),
        "ms_per_call": ms,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "device": torch.cuda.get_device_name(dev),
        "sclk": sclk,
    }
    if graph is not None:
        out["graph"] = graph
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, CPU_SAMPLE.get(cfg.name, 64))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

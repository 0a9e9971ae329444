"""Seeded synthetic inputs for one MoE layer forward.

This module is shared by the tests, the benchmark and the smoke check. It
holds the workload shapes and draws the random tensors; it computes nothing
of the layer itself (no routing, no expert arithmetic).

Distributions follow the workloads on the pages: x ~ N(0, 1); router and
expert weights ~ N(0, 1/d_in); expert biases ~ N(0, 0.01) read as a variance
(std 0.1). The Switch-style workload adds a router bias that follows a Zipf
law over expert rank so that hot experts overflow their capacity.

Every tensor is drawn with ``torch.randn`` from a ``torch.Generator`` on the
target device, seeded per (workload, tensor, expert). Values are therefore
fixed per device type (the CPU and GPU generators differ), and the expert
weights can be drawn one expert at a time. bf16 tensors are drawn in fp32
and rounded to nearest-even by ``Tensor.to``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BASE_SEED = 20261203

TENSOR_IDS = {"x": 0, "w_gate": 1, "w1": 2, "b1": 3, "w2": 4, "b2": 5, "dout": 6}


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    T: int
    d: int
    h: int
    E: int
    k: int
    renorm: bool = True
    capacity: int = -1          # < 0: unlimited
    dtype: str = "bf16"         # "bf16" or "f32"
    residual: bool = False      # combine adds x (dropped tokens pass through)
    zipf_gate_bias: bool = False
    expert_bias: bool = True
    routing: str = "topk"       # "topk" (tokens choose k experts) or "expert_choice"
    offload_slots: int = 0      # > 0: experts live in host memory, this many device slots

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # tiny fp32 layer: parity in fp32, launch-latency bound
    "tiny_fp32": MoEConfig("tiny_fp32", 0, T=256, d=128, h=256, E=8, k=2, dtype="f32"),
    # Mixtral-8x7B-shaped prefill: d=4096, expert hidden 14336, 8 experts, top-2
    "mixtral_prefill": MoEConfig("mixtral_prefill", 1, T=4096, d=4096, h=14336, E=8, k=2),
    # Switch-style top-1, capacity factor 1.25: ceil(8192 / 128 * 1.25) = 80 slots per
    # expert, and a Zipf router bias so that hot experts overflow
    "switch_top1_cap": MoEConfig("switch_top1_cap", 2, T=8192, d=768, h=3072, E=128, k=1,
                                 renorm=False, capacity=80,
                                 residual=True, zipf_gate_bias=True),
    # decode: 32 tokens over 64 experts, weight streaming dominates
    "decode": MoEConfig("decode", 3, T=32, d=4096, h=4096, E=64, k=2),
    # DeepSeek-V3-shaped routed experts: 256 experts, top-8, d=7168, hidden 2048
    "deepseek_v3": MoEConfig("deepseek_v3", 4, T=8192, d=7168, h=2048, E=256, k=8),
    # decode with the experts in pinned host memory and 56 of 64 in device
    # slots (LRU); each step routes a new batch of 32 tokens
    "decode_offload": MoEConfig("decode_offload", 3, T=32, d=4096, h=4096, E=64, k=2,
                                offload_slots=56),
    # Expert Choice on the Switch-shaped layer (same inputs, same Zipf-skewed
    # router): each of the 128 experts takes its 80 highest-probability tokens
    "switch_expert_choice": MoEConfig("switch_expert_choice", 2, T=8192, d=768, h=3072, E=128,
                                      k=1, renorm=False, capacity=80, residual=True,
                                      zipf_gate_bias=True, routing="expert_choice"),
}

CONFIG_ORDER = ["tiny_fp32", "mixtral_prefill", "switch_top1_cap", "decode", "deepseek_v3"]


def _seed(cfg_id: int, tensor: str, expert: int = 0) -> int:
    st = np.random.SeedSequence([BASE_SEED, cfg_id, TENSOR_IDS[tensor], expert]).generate_state(2)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def _randn(shape, std, cfg_id, tensor, expert, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg_id, tensor, expert))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def zipf_gate_bias(E: int, s: float = 1.1, scale: float = 0.5) -> torch.Tensor:
    """b_e = scale * ln(w_{e+1}),  w_r = r^-s / sum_{r'<=E} r'^-s  (expert e has rank e+1)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    w = r ** (-s)
    w /= w.sum()
    return torch.from_numpy((scale * np.log(w)).astype(np.float32))


def expert_tensors(cfg: MoEConfig, e: int, device="cpu"):
    """(w1 [h,d], b1 [h], w2 [d,h], b2 [d]) of expert e, drawn independently."""
    dt = cfg.torch_dtype
    w1 = _randn((cfg.h, cfg.d), 1.0 / math.sqrt(cfg.d), cfg.cfg_id, "w1", e, device, dt)
    w2 = _randn((cfg.d, cfg.h), 1.0 / math.sqrt(cfg.h), cfg.cfg_id, "w2", e, device, dt)
    if cfg.expert_bias:
        b1 = _randn((cfg.h,), 0.1, cfg.cfg_id, "b1", e, device, dt)
        b2 = _randn((cfg.d,), 0.1, cfg.cfg_id, "b2", e, device, dt)
    else:
        b1 = b2 = None
    return w1, b1, w2, b2


def make_inputs(cfg: MoEConfig, device="cpu") -> dict:
    """All layer inputs as torch tensors on ``device``.

    Keys: x [T,d], w_gate [E,d], gate_bias [E] fp32 or None, w1 [E,h,d],
    b1 [E,h] or None, w2 [E,d,h], b2 [E,d] or None.
    """
    dt = cfg.torch_dtype
    x = _randn((cfg.T, cfg.d), 1.0, cfg.cfg_id, "x", 0, device, dt)
    wg = _randn((cfg.E, cfg.d), 1.0 / math.sqrt(cfg.d), cfg.cfg_id, "w_gate", 0, device, dt)
    gb = zipf_gate_bias(cfg.E).to(device) if cfg.zipf_gate_bias else None
    w1 = torch.empty((cfg.E, cfg.h, cfg.d), dtype=dt, device=device)
    w2 = torch.empty((cfg.E, cfg.d, cfg.h), dtype=dt, device=device)
    b1 = torch.empty((cfg.E, cfg.h), dtype=dt, device=device) if cfg.expert_bias else None
    b2 = torch.empty((cfg.E, cfg.d), dtype=dt, device=device) if cfg.expert_bias else None
    for e in range(cfg.E):
        a, b, c, dd = expert_tensors(cfg, e, device)
        w1[e].copy_(a)
        w2[e].copy_(c)
        if cfg.expert_bias:
            b1[e].copy_(b)
            b2[e].copy_(dd)
    return dict(x=x, w_gate=wg, gate_bias=gb, w1=w1, b1=b1, w2=w2, b2=b2)


def make_dout(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """Upstream gradient of the layer output for the backward pass: [T, d] ~ N(0, 1)."""
    return _randn((cfg.T, cfg.d), 1.0, cfg.cfg_id, "dout", 0, device, cfg.torch_dtype)


def to_host_array(t):
    """torch tensor -> numpy for the oracle: fp32 stays fp32, bf16 -> uint16 bit patterns."""
    if t is None:
        return None
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")

"""One MoE layer forward through the libmoe calls.

Allocation (torch device tensors for outputs and workspaces) and call order
only; the arithmetic runs in libmoe.so. Token choice (top-k):
  moe_router_topk -> moe_permute -> moe_grouped_ffn -> moe_combine -> moe_aux_loss
Expert Choice (each expert takes C tokens):
  moe_router_topk (logits) -> moe_expert_choice -> moe_grouped_ffn -> moe_combine
all enqueued on one stream, with no device-to-host read in between.
"""
from __future__ import annotations

import dataclasses

import torch

from . import native as N


@dataclasses.dataclass
class MoEBuffers:
    """Every output and workspace of one layer forward at fixed sizes."""
    T: int
    d: int
    h: int
    E: int
    k: int
    dtype: torch.dtype
    device: torch.device
    out_dtype: torch.dtype = torch.float32  # combine output; fp32 keeps the sum unrounded

    def __post_init__(self):
        T, d, h, E, k = self.T, self.d, self.h, self.E, self.k
        dev = self.device
        f32, i32 = torch.float32, torch.int32
        self.logits = torch.empty((T, E), dtype=f32, device=dev)
        self.topk_idx = torch.empty((T, k), dtype=i32, device=dev)
        self.topk_gate = torch.empty((T, k), dtype=f32, device=dev)
        self.prob_sum = torch.empty((E,), dtype=f32, device=dev)
        self.counts = torch.empty((E,), dtype=i32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=i32, device=dev)
        self.dest_row = torch.empty((T * k,), dtype=i32, device=dev)
        self.sorted_token = torch.empty((T * k,), dtype=i32, device=dev)
        self.y_perm = torch.empty((T * k, d), dtype=self.dtype, device=dev)
        self.out = torch.empty((T, d), dtype=self.out_dtype, device=dev)
        self.f = torch.empty((E,), dtype=f32, device=dev)
        self.P = torch.empty((E,), dtype=f32, device=dev)
        self.loss = torch.empty((1,), dtype=f32, device=dev)

        def ws(op):
            n = N.moe_workspace_size(op, T, d, h, E, k)
            return torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)

        self.ws_router = ws(N.MOE_OP_ROUTER)
        self.ws_permute = ws(N.MOE_OP_PERMUTE)
        self.ws_ffn = ws(N.MOE_OP_FFN)


def moe_layer_forward(x, w_gate, gate_bias, w1, b1, w2, b2, k, renorm=True, capacity=-1,
                      residual=False, want_logits=False, bufs: MoEBuffers | None = None,
                      stream=None, out_dtype=torch.float32) -> MoEBuffers:
    """Enqueue the whole layer; returns the buffers (outputs valid once the stream runs)."""
    T, d = x.shape
    E = w_gate.shape[0]
    h = w1.shape[1]
    if bufs is None:
        bufs = MoEBuffers(T, d, h, E, k, x.dtype, x.device, out_dtype)
    b = bufs
    N.moe_router_topk(x, w_gate, gate_bias, E, k, renorm, b.logits if want_logits else None,
                      b.topk_idx, b.topk_gate, b.prob_sum, b.ws_router, stream)
    N.moe_permute(b.topk_idx, T, k, E, capacity, b.counts, b.offsets, b.dest_row,
                  b.sorted_token, b.ws_permute, stream)
    N.moe_grouped_ffn(x, T, d, h, E, k, b.offsets, b.sorted_token, w1, b1, w2, b2, b.y_perm,
                      b.ws_ffn, stream)
    N.moe_combine(b.y_perm, b.dest_row, b.topk_gate, T, k, d, x if residual else None, b.out,
                  stream)
    N.moe_aux_loss(b.prob_sum, b.counts, T, E, b.f, b.P, b.loss, stream)
    return b


def ec_ffn_k(T: int, E: int, C: int) -> int:
    """Rows per token the FFN is sized for when each of E experts takes min(C, T) tokens."""
    if T == 0:
        return 1
    return max(1, -(-E * min(C, T) // T))


@dataclasses.dataclass
class ECBuffers:
    """Every output and workspace of one Expert Choice layer forward."""
    T: int
    d: int
    h: int
    E: int
    C: int
    dtype: torch.dtype
    device: torch.device
    out_dtype: torch.dtype = torch.float32

    def __post_init__(self):
        T, d, h, E = self.T, self.d, self.h, self.E
        dev = self.device
        f32, i32 = torch.float32, torch.int32
        self.Cc = max(0, min(self.C, T))
        self.k_ffn = ec_ffn_k(T, E, self.C)
        self.logits = torch.empty((T, E), dtype=f32, device=dev)
        self.topk_idx = torch.empty((T, 1), dtype=i32, device=dev)
        self.topk_gate = torch.empty((T, 1), dtype=f32, device=dev)
        self.scores = torch.empty((E, T), dtype=f32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=i32, device=dev)
        self.sorted_token = torch.empty((max(E * self.Cc, 1),), dtype=i32, device=dev)
        self.dest_row = torch.empty((T, E), dtype=i32, device=dev)
        self.gate = torch.empty((T, E), dtype=f32, device=dev)
        self.y_perm = torch.empty((T * self.k_ffn, d), dtype=self.dtype, device=dev)
        self.out = torch.empty((T, d), dtype=self.out_dtype, device=dev)

        def ws(op, k):
            n = N.moe_workspace_size(op, T, d, h, E, k)
            return torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)

        self.ws_router = ws(N.MOE_OP_ROUTER, 1)
        self.ws_ffn = ws(N.MOE_OP_FFN, self.k_ffn)


def moe_layer_forward_ec(x, w_gate, gate_bias, w1, b1, w2, b2, C, residual=False,
                         bufs: ECBuffers | None = None, stream=None,
                         out_dtype=torch.float32) -> ECBuffers:
    """Enqueue an Expert Choice layer; returns the buffers."""
    T, d = x.shape
    E = w_gate.shape[0]
    h = w1.shape[1]
    if bufs is None:
        bufs = ECBuffers(T, d, h, E, C, x.dtype, x.device, out_dtype)
    b = bufs
    N.moe_router_topk(x, w_gate, gate_bias, E, 1, True, b.logits, b.topk_idx, b.topk_gate, None,
                      b.ws_router, stream)
    N.moe_expert_choice(b.logits, T, E, C, b.scores, b.offsets, b.sorted_token, b.dest_row,
                        b.gate, stream)
    N.moe_grouped_ffn(x, T, d, h, E, b.k_ffn, b.offsets, b.sorted_token, w1, b1, w2, b2,
                      b.y_perm, b.ws_ffn, stream)
    N.moe_combine(b.y_perm, b.dest_row, b.gate, T, E, d, x if residual else None, b.out, stream)
    return b

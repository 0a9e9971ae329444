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
    train: bool = False  # keep the pre-activations and hidden rows for the backward

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
        self.y_perm = N.expert_output_buffer(self.dtype, T * k, d, dev)
        self.out = torch.empty((T, d), dtype=self.out_dtype, device=dev)
        self.f = torch.empty((E,), dtype=f32, device=dev)
        self.P = torch.empty((E,), dtype=f32, device=dev)
        self.loss = torch.empty((1,), dtype=f32, device=dev)
        self.z_perm = self.h_perm = None
        if self.train:
            self.z_perm = torch.empty((T * k, self.h), dtype=self.dtype, device=dev)
            self.h_perm = torch.empty((T * k, self.h), dtype=self.dtype, device=dev)

        def ws(op):
            n = N.moe_workspace_size(op, T, d, h, E, k)
            return torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)

        self.ws_router = ws(N.MOE_OP_ROUTER)
        self.ws_permute = ws(N.MOE_OP_PERMUTE)
        self.ws_ffn = ws(N.MOE_OP_FFN)


def moe_layer_forward(x, w_gate, gate_bias, w1, b1, w2, b2, k, renorm=True, capacity=-1,
                      residual=False, want_logits=False, bufs: MoEBuffers | None = None,
                      stream=None, out_dtype=torch.float32, train=False) -> MoEBuffers:
    """Enqueue the whole layer; returns the buffers (outputs valid once the stream runs).
    train: keep the logits, pre-activations and hidden rows for moe_layer_backward."""
    T, d = x.shape
    E = w_gate.shape[0]
    h = w1.shape[1]
    if bufs is None:
        bufs = MoEBuffers(T, d, h, E, k, x.dtype, x.device, out_dtype, train)
    want_logits = want_logits or train
    b = bufs
    N.moe_router_topk(x, w_gate, gate_bias, E, k, renorm, b.logits if want_logits else None,
                      b.topk_idx, b.topk_gate, b.prob_sum, b.ws_router, stream)
    N.moe_permute(b.topk_idx, T, k, E, capacity, b.counts, b.offsets, b.dest_row,
                  b.sorted_token, b.ws_permute, stream)
    if b.train:
        N.moe_grouped_ffn_train(x, T, d, h, E, k, b.offsets, b.sorted_token, w1, b1, w2, b2,
                                b.y_perm, b.z_perm, b.h_perm, b.ws_ffn, stream)
    else:
        N.moe_grouped_ffn(x, T, d, h, E, k, b.offsets, b.sorted_token, w1, b1, w2, b2, b.y_perm,
                          b.ws_ffn, stream)
    N.moe_combine(b.y_perm, x.dtype, b.dest_row, b.topk_gate, T, k, d, x if residual else None,
                  b.out, stream)
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
    train: bool = False  # keep the pre-activations and hidden rows for the backward

    def __post_init__(self):
        T, d, h, E = self.T, self.d, self.h, self.E
        dev = self.device
        f32, i32 = torch.float32, torch.int32
        self.Cc = max(0, min(self.C, T))
        self.k_ffn = ec_ffn_k(T, E, self.C)
        self.logits = torch.empty((T, E), dtype=f32, device=dev)
        self.scores = torch.empty((E, T), dtype=f32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=i32, device=dev)
        self.sorted_token = torch.empty((max(E * self.Cc, 1),), dtype=i32, device=dev)
        self.dest_row = torch.empty((T, E), dtype=i32, device=dev)
        self.gate = torch.empty((T, E), dtype=f32, device=dev)
        self.y_perm = N.expert_output_buffer(self.dtype, T * self.k_ffn, d, dev)
        self.out = torch.empty((T, d), dtype=self.out_dtype, device=dev)
        self.z_perm = self.h_perm = None
        if self.train:
            self.z_perm = torch.empty((T * self.k_ffn, h), dtype=self.dtype, device=dev)
            self.h_perm = torch.empty((T * self.k_ffn, h), dtype=self.dtype, device=dev)

        def ws(op, k):
            n = N.moe_workspace_size(op, T, d, h, E, k)
            return torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)

        self.ws_router = ws(N.MOE_OP_ROUTER, 1)
        self.ws_ffn = ws(N.MOE_OP_FFN, self.k_ffn)


def moe_layer_forward_ec(x, w_gate, gate_bias, w1, b1, w2, b2, C, residual=False,
                         bufs: ECBuffers | None = None, stream=None,
                         out_dtype=torch.float32, train=False) -> ECBuffers:
    """Enqueue an Expert Choice layer; returns the buffers (train: keep Z and
    H for moe_layer_backward_ec)."""
    T, d = x.shape
    E = w_gate.shape[0]
    h = w1.shape[1]
    if bufs is None:
        bufs = ECBuffers(T, d, h, E, C, x.dtype, x.device, out_dtype, train)
    b = bufs
    N.moe_router_topk(x, w_gate, gate_bias, E, 1, True, b.logits, None, None, None,
                      b.ws_router, stream)
    N.moe_expert_choice(b.logits, T, E, C, b.scores, b.offsets, b.sorted_token, b.dest_row,
                        b.gate, stream)
    if b.train:
        N.moe_grouped_ffn_train(x, T, d, h, E, b.k_ffn, b.offsets, b.sorted_token, w1, b1, w2,
                                b2, b.y_perm, b.z_perm, b.h_perm, b.ws_ffn, stream)
    else:
        N.moe_grouped_ffn(x, T, d, h, E, b.k_ffn, b.offsets, b.sorted_token, w1, b1, w2, b2,
                          b.y_perm, b.ws_ffn, stream)
    N.moe_combine(b.y_perm, x.dtype, b.dest_row, b.gate, T, E, d, x if residual else None, b.out,
                  stream)
    return b


class ExpertCache:
    """Experts held in pinned host memory, S of them in device slots (LRU).

    Allocation and bookkeeping only: the slot policy and the copies run in
    libmoe (moe_cache_step), the FFN over the slots in moe_grouped_ffn_cached.
    """

    def __init__(self, w1, b1, w2, b2, S: int, device):
        import numpy as np
        self.E, self.h, self.d = w1.shape
        self.S = S
        dev = torch.device(device)
        self.host = []   # pinned host copies [E][...]
        self.slots = []  # device slots [S][...]
        for t in (w1, b1, w2, b2):
            if t is None:
                self.host.append(None)
                self.slots.append(None)
                continue
            hcopy = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            hcopy.copy_(t)
            self.host.append(hcopy)
            self.slots.append(torch.empty((S,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev))
        self.state = np.zeros(N.moe_cache_state_bytes(self.E, S), np.uint8)
        N.moe_cache_init(self.state, self.E, S)
        self.slot_of = torch.empty((self.E,), dtype=torch.int32, device=dev)
        self.phase_of = torch.empty((self.E,), dtype=torch.int32, device=dev)
        self.copy_stream = torch.cuda.Stream(dev)  # default priority
        self.loaded = 0

    def step(self, counts_host, stream):
        """Plan one step and enqueue the misses' copies; returns an event the
        compute stream waits on before the misses' FFN."""
        pairs = [(h, s) for h, s in zip(self.host, self.slots) if h is not None]
        # the slots being refilled may still be read by the previous step
        self.copy_stream.wait_stream(stream)
        self.loaded = N.moe_cache_step(self.state, counts_host, [p[0] for p in pairs],
                                       [p[1] for p in pairs], self.slot_of, self.phase_of,
                                       stream, self.copy_stream)
        ev = torch.cuda.Event()
        ev.record(self.copy_stream)
        return ev


def moe_layer_forward_cached(x, w_gate, gate_bias, cache: ExpertCache, k, renorm=True,
                             capacity=-1, residual=False, want_logits=False,
                             bufs: MoEBuffers | None = None, stream=None,
                             out_dtype=torch.float32) -> MoEBuffers:
    """Token-choice layer over host-resident experts: route and permute, read
    the counts back (one synchronisation), load the missing experts on the
    copy stream while the resident ones run, then run the loaded ones."""
    T, d = x.shape
    E = w_gate.shape[0]
    h = cache.h
    if bufs is None:
        bufs = MoEBuffers(T, d, h, E, k, x.dtype, x.device, out_dtype)
    b = bufs
    s = torch.cuda.current_stream() if stream is None else stream
    N.moe_router_topk(x, w_gate, gate_bias, E, k, renorm, b.logits if want_logits else None,
                      b.topk_idx, b.topk_gate, b.prob_sum, b.ws_router, s)
    N.moe_permute(b.topk_idx, T, k, E, capacity, b.counts, b.offsets, b.dest_row,
                  b.sorted_token, b.ws_permute, s)
    with torch.cuda.stream(s):
        counts = b.counts.cpu().numpy()
    ready = cache.step(counts, s)
    w1s, b1s, w2s, b2s = cache.slots
    for phase in (0, 1):
        if phase == 1:
            s.wait_event(ready)
        N.moe_grouped_ffn_cached(x, T, d, h, E, k, b.offsets, b.sorted_token, cache.slot_of,
                                 cache.phase_of, phase, w1s, b1s, w2s, b2s, b.y_perm, b.ws_ffn, s)
    N.moe_combine(b.y_perm, x.dtype, b.dest_row, b.topk_gate, T, k, d, x if residual else None,
                  b.out, s)
    N.moe_aux_loss(b.prob_sum, b.counts, T, E, b.f, b.P, b.loss, s)
    return b


@dataclasses.dataclass
class MoEGrads:
    """Gradients and scratch of one token-choice layer backward."""
    T: int
    d: int
    h: int
    E: int
    k: int
    dtype: torch.dtype
    device: torch.device
    has_b1: bool = True
    has_b2: bool = True
    has_gate_bias: bool = False
    slots: int = 0  # gate slots per token (0: k; Expert Choice: E)

    def __post_init__(self):
        T, d, h, E, k = self.T, self.d, self.h, self.E, self.k
        dev, dt, f32 = self.device, self.dtype, torch.float32
        self.dy_perm = torch.empty((T * k, d), dtype=dt, device=dev)
        self.dgate = torch.empty((T, self.slots or k), dtype=f32, device=dev)
        self.dlogits = torch.empty((T, E), dtype=f32, device=dev)
        self.dx_perm = torch.empty((T * k, d), dtype=dt, device=dev)
        self.dx = torch.empty((T, d), dtype=dt, device=dev)
        self.dw_gate = torch.empty((E, d), dtype=dt, device=dev)
        self.dgate_bias = torch.empty((E,), dtype=f32, device=dev) if self.has_gate_bias else None
        self.dw1 = torch.empty((E, h, d), dtype=dt, device=dev)
        self.db1 = torch.empty((E, h), dtype=dt, device=dev) if self.has_b1 else None
        self.dw2 = torch.empty((E, d, h), dtype=dt, device=dev)
        self.db2 = torch.empty((E, d), dtype=dt, device=dev) if self.has_b2 else None

        def ws(op):
            n = N.moe_workspace_size(op, T, d, h, E, k)
            return torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)

        self.ws_ffn = ws(N.MOE_OP_FFN_BWD)
        self.ws_router = ws(N.MOE_OP_ROUTER_BWD)


def moe_layer_backward(fwd: MoEBuffers, x, w_gate, gate_bias, w1, b1, w2, b2, dout, renorm=True,
                       residual=False, daux=0.0, grads: MoEGrads | None = None,
                       stream=None) -> MoEGrads:
    """Enqueue the backward of a token-choice layer whose forward ran with
    want_logits=True into ``fwd`` (with train=True the backward reuses the
    forward's pre-activations instead of recomputing them). dout [T][d] in
    the layer dtype; daux is
    the weight of the aux loss in the differentiated scalar. Returns the
    gradient buffers (valid once the stream runs):
      moe_combine_backward -> moe_router_backward -> moe_grouped_ffn_backward
      -> moe_gather_backward -> moe_router_weight_backward
    """
    T, d = x.shape
    E = w_gate.shape[0]
    h = w1.shape[1]
    k = fwd.k
    if grads is None:
        grads = MoEGrads(T, d, h, E, k, x.dtype, x.device, b1 is not None, b2 is not None,
                         gate_bias is not None)
    g = grads
    N.moe_combine_backward(fwd.y_perm, fwd.dest_row, fwd.topk_gate, T, k, d, dout, g.dy_perm,
                           g.dgate, stream)
    N.moe_router_backward(fwd.logits, fwd.topk_idx, fwd.topk_gate, g.dgate, fwd.counts, T, E, k,
                          renorm, daux, g.dlogits, stream)
    N.moe_grouped_ffn_backward(x, T, d, h, E, k, fwd.offsets, fwd.sorted_token, w1, b1, w2,
                               g.dy_perm, fwd.z_perm, fwd.h_perm, g.dx_perm, g.dw1, g.db1, g.dw2,
                               g.db2, g.ws_ffn, stream)
    N.moe_gather_backward(g.dx_perm, fwd.dest_row, T, k, d, dout if residual else None, g.dlogits,
                          w_gate, E, g.dx, stream)
    N.moe_router_weight_backward(x, T, d, E, g.dlogits, g.dw_gate, g.dgate_bias, g.ws_router,
                                 stream)
    return g


def moe_layer_backward_ec(fwd: ECBuffers, x, w_gate, gate_bias, w1, b1, w2, b2, dout,
                          residual=False, grads: MoEGrads | None = None,
                          stream=None) -> MoEGrads:
    """Enqueue the backward of an Expert Choice layer whose forward ran into
    ``fwd`` (train=True keeps Z and H). The same five calls as token choice,
    with one gate slot per expert: the combine and gather run with k = E,
    the router with no index table (slot j is expert j) and renorm = 0,
    since a chosen pair's gate is its probability; no aux loss.
    """
    T, d = x.shape
    E = w_gate.shape[0]
    h = w1.shape[1]
    k = fwd.k_ffn
    if grads is None:
        grads = MoEGrads(T, d, h, E, k, x.dtype, x.device, b1 is not None, b2 is not None,
                         gate_bias is not None, slots=E)
    g = grads
    N.moe_combine_backward(fwd.y_perm, fwd.dest_row, fwd.gate, T, E, d, dout, g.dy_perm, g.dgate,
                           stream)
    N.moe_router_backward(fwd.logits, None, fwd.gate, g.dgate, None, T, E, E, False, 0.0,
                          g.dlogits, stream)
    N.moe_grouped_ffn_backward(x, T, d, h, E, k, fwd.offsets, fwd.sorted_token, w1, b1, w2,
                               g.dy_perm, fwd.z_perm, fwd.h_perm, g.dx_perm, g.dw1, g.db1, g.dw2,
                               g.db2, g.ws_ffn, stream)
    N.moe_gather_backward(g.dx_perm, fwd.dest_row, T, E, d, dout if residual else None,
                          g.dlogits, w_gate, E, g.dx, stream)
    N.moe_router_weight_backward(x, T, d, E, g.dlogits, g.dw_gate, g.dgate_bias, g.ws_router,
                                 stream)
    return g

"""Thin ctypes binding of libmoe.so.

The five calls keep the C names and argument order of ``include/moe.h``;
this module only turns torch tensors into device pointers, picks the current
HIP stream and raises ``MoEError`` on a non-zero status. Every step of the
layer runs in the library's HIP kernels; nothing here computes.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_LAUNCH, MOE_ERR_WORKSPACE = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_OP_ROUTER, MOE_OP_PERMUTE, MOE_OP_FFN, MOE_OP_FFN_BWD, MOE_OP_ROUTER_BWD = 0, 1, 2, 3, 4

_DTYPE = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


class MoEError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def use_library(path):
    """Route every call of this module through the library at `path` (for
    instance the debug build, libmoe_debug.so); returns the one it replaces
    (None if none was loaded yet), which use_library(old) puts back."""
    global _lib
    old, _lib = _lib, (None if path is None else (path if isinstance(path, ctypes.CDLL)
                                                    else load(path)))
    return old


def load(path):
    """ctypes handle of a build of libmoe with every argument type set."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m top_routing_expert_topk_amd.build`")
    L = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.moe_check_permutation.argtypes = [P, I, P, P, I, I]
    L.moe_check_permutation.restype = I
    L.moe_debug_checks.argtypes = []
    L.moe_debug_checks.restype = I
    L.moe_status_string.argtypes = [I]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_version.argtypes = []
    L.moe_version.restype = I
    L.moe_expert_output_bytes.argtypes = [I, I, I]
    L.moe_expert_output_bytes.restype = Z
    L.moe_workspace_size.argtypes = [I, I, I, I, I, I]
    L.moe_workspace_size.restype = Z
    L.moe_router_topk.argtypes = [P, I, I, I, P, P, I, I, I, P, P, P, P, P, Z, P]
    L.moe_permute.argtypes = [P, I, I, I, I, P, P, P, P, P, Z, P]
    L.moe_permute_noalloc.argtypes = [P, I, I, I, I, P, P, P, P, P]
    L.moe_grouped_ffn.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P]
    L.moe_combine.argtypes = [P, I, P, P, I, I, I, P, P, I, P]
    L.moe_aux_loss.argtypes = [P, P, I, I, P, P, P, P]
    L.moe_expert_choice.argtypes = [P, I, I, I, P, P, P, P, P, P]
    L.moe_cache_state_bytes.argtypes = [I, I]
    L.moe_cache_state_bytes.restype = Z
    L.moe_cache_init.argtypes = [P, I, I]
    L.moe_cache_step.argtypes = [P, P, I, P, P, P, P, P, P, P, P]
    L.moe_cache_slot_of.argtypes = [P, P, P]
    L.moe_grouped_ffn_cached.argtypes = [P, I, I, I, I, I, I, P, P, P, P, I, P, P, P, P, P,
                                         P, Z, P]
    F = ctypes.c_float
    L.moe_combine_backward.argtypes = [P, I, P, P, I, I, I, P, P, P, P]
    L.moe_router_backward.argtypes = [P, P, P, P, P, I, I, I, I, F, P, P]
    L.moe_grouped_ffn_backward.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P,
                                           P, P, P, P, P, Z, P]
    L.moe_grouped_ffn_train.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, Z,
                                        P]
    L.moe_gather_backward.argtypes = [P, I, P, I, I, I, P, P, P, I, P, P]
    L.moe_router_weight_backward.argtypes = [P, I, I, I, I, P, P, P, P, Z, P]
    for f in ("moe_router_topk", "moe_permute", "moe_permute_noalloc", "moe_grouped_ffn",
              "moe_combine",
              "moe_aux_loss", "moe_expert_choice", "moe_cache_init", "moe_cache_step",
              "moe_cache_slot_of", "moe_grouped_ffn_cached", "moe_combine_backward",
              "moe_router_backward", "moe_grouped_ffn_backward", "moe_gather_backward",
              "moe_router_weight_backward", "moe_grouped_ffn_train"):
        getattr(L, f).restype = I
    return L


def declared_functions() -> list:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def version() -> int:
    return lib().moe_version()


def moe_workspace_size(op: int, T: int, d: int, h: int, E: int, k: int) -> int:
    return int(lib().moe_workspace_size(op, T, d, h, E, k))


def moe_expert_output_bytes(dtype, rows: int, d: int) -> int:
    """Bytes of `rows` rows of y_perm for a layer of torch dtype `dtype`."""
    return int(lib().moe_expert_output_bytes(_DTYPE[dtype], rows, d))


def expert_output_buffer(dtype, rows: int, d: int, device):
    """A y_perm buffer: fp32 [rows][d] for fp32 layers; for bf16 layers
    [rows][row bytes] uint8 holding the block fixed point."""
    if dtype == torch.float32:
        return torch.empty((rows, d), dtype=torch.float32, device=device)
    rb = moe_expert_output_bytes(dtype, 1, d)
    if rb == 0:
        raise ValueError(f"no expert-output layout for {dtype} with d = {d}")
    return torch.empty((rows, rb), dtype=torch.uint8, device=device)


def moe_check_permutation(offsets, E, sorted_token, dest_row, T, k) -> int:
    """The host-side permutation check on host int32 arrays (numpy or CPU
    tensors, or None); returns the status (0 ok, 1 invalid)."""
    def host(a):
        if a is None:
            return None, None
        if isinstance(a, torch.Tensor):
            if a.is_cuda:
                raise ValueError("moe_check_permutation takes host arrays")
            a = a.numpy()
        import numpy as np
        a = np.ascontiguousarray(a, dtype=np.int32)
        return a, ctypes.c_void_p(a.ctypes.data)
    keep = [host(a) for a in (offsets, sorted_token, dest_row)]
    return int(lib().moe_check_permutation(keep[0][1], E, keep[1][1], keep[2][1], T, k))


def debug_checks() -> bool:
    """True in the debug build (host-side permutation checks before launches)."""
    return bool(lib().moe_debug_checks())


def _p(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _check(call, status):
    if status != MOE_OK:
        raise MoEError(call, status)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_router_topk(x, w_gate, gate_bias, E, k, renorm, logits_out, topk_idx, topk_gate,
                    prob_sum, ws, stream=None):
    T, d = x.shape
    _check("moe_router_topk", lib().moe_router_topk(
        _p(x), _dt(x), T, d, _p(w_gate), _p(gate_bias), E, k, int(bool(renorm)), _p(logits_out),
        _p(topk_idx), _p(topk_gate), _p(prob_sum), _p(ws), _nbytes(ws), _stream(stream)))


def moe_permute(topk_idx, T, k, E, capacity, counts, offsets, dest_row, sorted_token, ws,
                stream=None):
    _check("moe_permute", lib().moe_permute(
        _p(topk_idx), T, k, E, int(capacity), _p(counts), _p(offsets), _p(dest_row),
        _p(sorted_token), _p(ws), _nbytes(ws), _stream(stream)))


def moe_permute_noalloc(topk_idx, T, k, E, capacity, counts, offsets, dest_row, sorted_token,
                        stream=None):
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        _p(topk_idx), T, k, E, int(capacity), _p(counts), _p(offsets), _p(dest_row),
        _p(sorted_token), _stream(stream)))


def moe_grouped_ffn(x, T, d, h, E, k, offsets, sorted_token, w1, b1, w2, b2, y_perm, ws,
                    stream=None):
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _p(x), _dt(x), T, d, h, E, k, _p(offsets), _p(sorted_token), _p(w1), _p(b1), _p(w2),
        _p(b2), _p(y_perm), _p(ws), _nbytes(ws), _stream(stream)))


def moe_combine(y_perm, dtype, dest_row, topk_gate, T, k, d, residual, out, stream=None):
    """y_perm: fp32 expert outputs; dtype: the layer's torch dtype (that of
    x and of residual)."""
    _check("moe_combine", lib().moe_combine(
        _p(y_perm), _DTYPE[dtype], _p(dest_row), _p(topk_gate), T, k, d, _p(residual), _p(out),
        _dt(out), _stream(stream)))


def moe_aux_loss(prob_sum, counts, T, E, f, P, loss, stream=None):
    _check("moe_aux_loss", lib().moe_aux_loss(
        _p(prob_sum), _p(counts), T, E, _p(f), _p(P), _p(loss), _stream(stream)))


def moe_expert_choice(logits, T, E, C, scores, offsets, sorted_token, dest_row, gate,
                      stream=None):
    _check("moe_expert_choice", lib().moe_expert_choice(
        _p(logits), T, E, int(C), _p(scores), _p(offsets), _p(sorted_token), _p(dest_row),
        _p(gate), _stream(stream)))


# ------------------------------------------------------------ expert cache ----
# The cache state and the per-step counts live in host memory (numpy arrays).

def _host_ptr(a):
    import numpy as np
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "host arrays must be contiguous"
    return a.ctypes.data


def moe_cache_state_bytes(E, S) -> int:
    return int(lib().moe_cache_state_bytes(E, S))


def moe_cache_init(state, E, S):
    _check("moe_cache_init", lib().moe_cache_init(_host_ptr(state), E, S))


def moe_cache_step(state, counts, host_tensors, dev_tensors, slot_of_dev, phase_of_dev,
                   compute_stream=None, copy_stream=None) -> int:
    """host_tensors / dev_tensors: per-expert-major tensors ([E][...] pinned host, [S][...]
    device); returns the number of experts copied."""
    import numpy as np
    n = len(host_tensors)
    assert len(dev_tensors) == n
    hb = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in host_tensors])
    db = (ctypes.c_void_p * max(n, 1))(*[_p(t) for t in dev_tensors])
    nb = (ctypes.c_size_t * max(n, 1))(*[t[0].numel() * t.element_size() for t in host_tensors])
    for t in host_tensors:
        if t.is_cuda or not t.is_pinned():
            raise ValueError("host expert tensors must be pinned host memory")
    loaded = ctypes.c_int(0)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    _check("moe_cache_step", lib().moe_cache_step(
        _host_ptr(state), _host_ptr(counts), n, hb if n else None, db if n else None,
        nb if n else None, _p(slot_of_dev), _p(phase_of_dev), ctypes.byref(loaded),
        _stream(compute_stream), _stream(copy_stream)))
    return loaded.value


def moe_cache_slot_of(state, E):
    import numpy as np
    slot = np.empty(E, np.int32)
    phase = np.empty(E, np.int32)
    _check("moe_cache_slot_of", lib().moe_cache_slot_of(_host_ptr(state), _host_ptr(slot),
                                                        _host_ptr(phase)))
    return slot, phase


def moe_grouped_ffn_cached(x, T, d, h, E, k, offsets, sorted_token, slot_of, phase_of, phase,
                           w1, b1, w2, b2, y_perm, ws, stream=None):
    _check("moe_grouped_ffn_cached", lib().moe_grouped_ffn_cached(
        _p(x), _dt(x), T, d, h, E, k, _p(offsets), _p(sorted_token), _p(slot_of), _p(phase_of),
        int(phase), _p(w1), _p(b1), _p(w2), _p(b2), _p(y_perm), _p(ws), _nbytes(ws),
        _stream(stream)))


# ---------------------------------------------------------------- backward ----

def moe_combine_backward(y_perm, dest_row, topk_gate, T, k, d, dout, dy_perm, dgate,
                         stream=None):
    _check("moe_combine_backward", lib().moe_combine_backward(
        _p(y_perm), _dt(dout), _p(dest_row), _p(topk_gate), T, k, d, _p(dout), _p(dy_perm),
        _p(dgate), _stream(stream)))


def moe_router_backward(logits, topk_idx, topk_gate, dgate, counts, T, E, k, renorm, daux,
                        dlogits, stream=None):
    _check("moe_router_backward", lib().moe_router_backward(
        _p(logits), _p(topk_idx), _p(topk_gate), _p(dgate), _p(counts), T, E, k,
        int(bool(renorm)), float(daux), _p(dlogits), _stream(stream)))


def moe_grouped_ffn_backward(x, T, d, h, E, k, offsets, sorted_token, w1, b1, w2, dy_perm,
                             z_perm, h_perm, dx_perm, dw1, db1, dw2, db2, ws, stream=None):
    _check("moe_grouped_ffn_backward", lib().moe_grouped_ffn_backward(
        _p(x), _dt(w1), T, d, h, E, k, _p(offsets), _p(sorted_token), _p(w1), _p(b1), _p(w2),
        _p(dy_perm), _p(z_perm), _p(h_perm), _p(dx_perm), _p(dw1), _p(db1), _p(dw2), _p(db2),
        _p(ws), _nbytes(ws), _stream(stream)))


def moe_grouped_ffn_train(x, T, d, h, E, k, offsets, sorted_token, w1, b1, w2, b2, y_perm,
                          z_perm, h_perm, ws, stream=None):
    _check("moe_grouped_ffn_train", lib().moe_grouped_ffn_train(
        _p(x), _dt(x), T, d, h, E, k, _p(offsets), _p(sorted_token), _p(w1), _p(b1), _p(w2),
        _p(b2), _p(y_perm), _p(z_perm), _p(h_perm), _p(ws), _nbytes(ws), _stream(stream)))


def moe_gather_backward(dx_perm, dest_row, T, k, d, dout_residual, dlogits, w_gate, E, dx,
                        stream=None):
    _check("moe_gather_backward", lib().moe_gather_backward(
        _p(dx_perm), _dt(dx), _p(dest_row), T, k, d, _p(dout_residual), _p(dlogits),
        _p(w_gate), E, _p(dx), _stream(stream)))


def moe_router_weight_backward(x, T, d, E, dlogits, dw_gate, dgate_bias, ws, stream=None):
    _check("moe_router_weight_backward", lib().moe_router_weight_backward(
        _p(x), _dt(dw_gate), T, d, E, _p(dlogits), _p(dw_gate), _p(dgate_bias), _p(ws),
        _nbytes(ws), _stream(stream)))

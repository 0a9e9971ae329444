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
MOE_OP_ROUTER, MOE_OP_PERMUTE, MOE_OP_FFN = 0, 1, 2

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
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m top_routing_expert_topk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_status_string.argtypes = [I]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        L.moe_version.restype = I
        L.moe_workspace_size.argtypes = [I, I, I, I, I, I]
        L.moe_workspace_size.restype = Z
        L.moe_router_topk.argtypes = [P, I, I, I, P, P, I, I, I, P, P, P, P, P, Z, P]
        L.moe_permute.argtypes = [P, I, I, I, I, P, P, P, P, P, Z, P]
        L.moe_grouped_ffn.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P]
        L.moe_combine.argtypes = [P, I, P, P, I, I, I, P, P, I, P]
        L.moe_aux_loss.argtypes = [P, P, I, I, P, P, P, P]
        L.moe_expert_choice.argtypes = [P, I, I, I, P, P, P, P, P, P]
        for f in ("moe_router_topk", "moe_permute", "moe_grouped_ffn", "moe_combine",
                  "moe_aux_loss", "moe_expert_choice"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


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


def moe_grouped_ffn(x, T, d, h, E, k, offsets, sorted_token, w1, b1, w2, b2, y_perm, ws,
                    stream=None):
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _p(x), _dt(x), T, d, h, E, k, _p(offsets), _p(sorted_token), _p(w1), _p(b1), _p(w2),
        _p(b2), _p(y_perm), _p(ws), _nbytes(ws), _stream(stream)))


def moe_combine(y_perm, dest_row, topk_gate, T, k, d, residual, out, stream=None):
    _check("moe_combine", lib().moe_combine(
        _p(y_perm), _dt(y_perm), _p(dest_row), _p(topk_gate), T, k, d, _p(residual), _p(out),
        _dt(out), _stream(stream)))


def moe_aux_loss(prob_sum, counts, T, E, f, P, loss, stream=None):
    _check("moe_aux_loss", lib().moe_aux_loss(
        _p(prob_sum), _p(counts), T, E, _p(f), _p(P), _p(loss), _stream(stream)))


def moe_expert_choice(logits, T, E, C, scores, offsets, sorted_token, dest_row, gate,
                      stream=None):
    _check("moe_expert_choice", lib().moe_expert_choice(
        _p(logits), T, E, int(C), _p(scores), _p(offsets), _p(sorted_token), _p(dest_row),
        _p(gate), _stream(stream)))

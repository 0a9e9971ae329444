"""The C-ABI boundary on the host: the library loads, exports what the header
declares, and rejects bad arguments with status codes before any launch.
No call here reaches a kernel launch, so these run without a GPU."""
import ctypes
import subprocess

import pytest

from top_routing_expert_topk_amd import native as N

BAD = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_library_exports_every_declared_symbol():
    lib = N.lib()
    declared = N.declared_functions()
    assert {"moe_router_topk", "moe_permute", "moe_grouped_ffn", "moe_combine",
            "moe_aux_loss", "moe_workspace_size", "moe_status_string", "moe_version"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported


def test_status_strings_and_version():
    assert N.status_string(0) == "ok"
    assert "workspace" in N.status_string(4)
    assert N.status_string(99) == "unknown status"
    assert N.version() >= 100


def test_workspace_sizes():
    assert N.moe_workspace_size(N.MOE_OP_ROUTER, 4096, 4096, 14336, 8, 2) >= 128 * 8 * 4
    assert N.moe_workspace_size(N.MOE_OP_PERMUTE, 8192, 7168, 2048, 256, 8) >= 2 * 256 * 64 * 4
    ffn = N.moe_workspace_size(N.MOE_OP_FFN, 4096, 4096, 14336, 8, 2)
    assert ffn >= 4096 * 2 * 14336 * 2
    assert N.moe_workspace_size(7, 10, 10, 10, 4, 2) == 0
    assert N.moe_workspace_size(N.MOE_OP_FFN, 10, 0, 10, 4, 2) == 0
    # more experts than any call takes (the host-sanitized build found the
    # router's plan dividing by a zero-row token tile there)
    for op in range(5):
        assert N.moe_workspace_size(op, 0, 64, 128, 513, 2) == 0
        assert N.moe_workspace_size(op, 100, 64, 128, 513, 2) == 0
        assert N.moe_workspace_size(op, 100, 64, 128, 512, 2) > 0


def _ceil(a, b):
    return -(-a // b)


@pytest.mark.parametrize("T,d,h,E,k", [(4096, 4096, 14336, 8, 2), (8192, 7168, 2048, 256, 8),
                                       (8192, 768, 3072, 128, 1), (32, 4096, 4096, 64, 2),
                                       (256, 128, 256, 8, 2), (300, 512, 1024, 8, 2),
                                       (1, 256, 256, 512, 16), (6000, 512, 1536, 64, 1)])
def test_ffn_workspace_holds_the_tile_path_layout(T, d, h, E, k):
    """The FFN workspace must hold, for 128- and 256-row tiles alike: two
    32-byte work entries per tile and per split unit of both GEMMs, a token
    table of every row block (padded to the tile height), the hidden
    activations (4 bytes per element at most) and 256 fp32 partial tiles of
    up to 288 rows x 256 features. Restated here from the layout, independently of the C++ sizing."""
    rows = T * k
    need_plan = 0
    for bm in (128, 256):
        mslots = _ceil(rows, bm) + min(rows, E)
        lists = 256 + sum(_ceil(mslots * (n // 256) + 256, 8) * 8 for n in (h, d)) * 32
        table = mslots * bm * 4
        need_plan = max(need_plan, _ceil(lists, 256) * 256 + _ceil(table, 256) * 256)
    need = need_plan + rows * h * 4 + 256 * 288 * 256 * 4
    assert N.moe_workspace_size(N.MOE_OP_FFN, T, d, h, E, k) >= need


def _router(**kw):
    a = dict(x=BAD, dtype=1, T=64, d=64, w=BAD, gb=None, E=8, k=2, renorm=1, lg=None, idx=BAD,
             gate=BAD, ps=None, ws=BAD, wsb=1 << 20, s=None)
    a.update(kw)
    return N.lib().moe_router_topk(a["x"], a["dtype"], a["T"], a["d"], a["w"], a["gb"], a["E"],
                                   a["k"], a["renorm"], a["lg"], a["idx"], a["gate"], a["ps"],
                                   a["ws"], a["wsb"], a["s"])


def test_router_rejects_bad_arguments():
    assert _router(T=-1) == N.MOE_ERR_INVALID
    assert _router(k=0) == N.MOE_ERR_INVALID
    assert _router(k=9) == N.MOE_ERR_INVALID
    assert _router(dtype=5) == N.MOE_ERR_INVALID
    assert _router(renorm=2) == N.MOE_ERR_INVALID
    assert _router(E=600, k=2) == N.MOE_ERR_UNSUPPORTED
    assert _router(E=64, k=17) == N.MOE_ERR_UNSUPPORTED
    assert _router(d=60) == N.MOE_ERR_UNSUPPORTED
    assert _router(x=None) == N.MOE_ERR_INVALID
    assert _router(idx=None) == N.MOE_ERR_INVALID
    assert _router(gate=None) == N.MOE_ERR_INVALID
    # logits only (no idx, gate or prob_sum) needs logits_out
    assert _router(idx=None, gate=None, ps=None, lg=None) == N.MOE_ERR_INVALID
    assert _router(idx=None, gate=None, ps=BAD, lg=BAD) == N.MOE_ERR_INVALID
    assert _router(wsb=16) == N.MOE_ERR_WORKSPACE
    assert _router(ws=None) == N.MOE_ERR_WORKSPACE


def test_permute_rejects_bad_arguments():
    L = N.lib()
    assert L.moe_permute(BAD, -1, 2, 8, -1, BAD, BAD, BAD, BAD, BAD, 1 << 20, None) == 1
    assert L.moe_permute(BAD, 10, 9, 8, -1, BAD, BAD, BAD, BAD, BAD, 1 << 20, None) == 1
    assert L.moe_permute(BAD, 10, 2, 513, -1, BAD, BAD, BAD, BAD, BAD, 1 << 20, None) == 2
    assert L.moe_permute(BAD, 10, 2, 8, -1, None, BAD, BAD, BAD, BAD, 1 << 20, None) == 1
    assert L.moe_permute(BAD, 10, 2, 8, -1, BAD, BAD, None, BAD, BAD, 1 << 20, None) == 1
    assert L.moe_permute(BAD, 10, 2, 8, -1, BAD, BAD, BAD, BAD, BAD, 4, None) == 4


def test_noalloc_permute_rejects_bad_arguments_and_sizes_beyond_its_array():
    L = N.lib()
    assert L.moe_permute_noalloc(BAD, -1, 2, 8, -1, BAD, BAD, BAD, BAD, None) == 1
    assert L.moe_permute_noalloc(BAD, 10, 9, 8, -1, BAD, BAD, BAD, BAD, None) == 1
    assert L.moe_permute_noalloc(BAD, 10, 2, 513, -1, BAD, BAD, BAD, BAD, None) == 2
    assert L.moe_permute_noalloc(BAD, 10, 2, 8, -1, None, BAD, BAD, BAD, None) == 1
    # MOE_PERMUTE_NOALLOC_MAX_ASSIGN = 2^20 assignments, refused beyond
    header = open(N.HEADER).read()
    assert "#define MOE_PERMUTE_NOALLOC_MAX_ASSIGN (1L << 20)" in header
    assert L.moe_permute_noalloc(BAD, (1 << 17) + 1, 8, 512, -1, BAD, BAD, BAD, BAD, None) == 2
    assert L.moe_permute_noalloc(BAD, 1 << 19, 4, 512, -1, BAD, BAD, BAD, BAD, None) == 2


def test_ffn_rejects_bad_arguments():
    L = N.lib()

    def ffn(dtype=1, T=10, d=128, h=256, E=8, k=2, wsb=1 << 30, w1=BAD, ws=BAD):
        return L.moe_grouped_ffn(BAD, dtype, T, d, h, E, k, BAD, BAD, w1, None, BAD, None, BAD,
                                 ws, wsb, None)
    assert ffn(T=-1) == 1
    assert ffn(dtype=3) == 1
    assert ffn(k=9) == 1
    assert ffn(d=100) == 2   # bf16 needs multiples of 64
    assert ffn(h=96) == 2
    assert ffn(E=1000, k=2) == 2
    assert ffn(w1=None) == 1
    assert ffn(wsb=100) == 4
    assert ffn(ws=None) == 4


def test_combine_and_aux_reject_bad_arguments():
    L = N.lib()
    assert L.moe_combine(BAD, 1, BAD, BAD, -1, 2, 64, None, BAD, 0, None) == 1
    assert L.moe_combine(BAD, 2, BAD, BAD, 4, 2, 64, None, BAD, 0, None) == 1
    assert L.moe_combine(BAD, 1, BAD, BAD, 4, 2, 64, None, BAD, 5, None) == 1
    assert L.moe_combine(BAD, 0, BAD, BAD, 4, 2, 64, None, BAD, 1, None) == 2
    assert L.moe_combine(BAD, 1, BAD, BAD, 4, 513, 64, None, BAD, 0, None) == 2
    assert L.moe_combine(BAD, 1, BAD, BAD, 4, 2, 60, None, BAD, 0, None) == 2
    assert L.moe_combine(None, 1, BAD, BAD, 4, 2, 64, None, BAD, 0, None) == 1
    assert L.moe_aux_loss(BAD, BAD, 0, 8, None, None, BAD, None) == 1
    assert L.moe_aux_loss(BAD, BAD, 4, 600, None, None, BAD, None) == 2
    assert L.moe_aux_loss(BAD, BAD, 4, 8, None, None, None, None) == 1


def test_expert_choice_rejects_bad_arguments():
    L = N.lib()

    def call(T=64, E=8, C=4, logits=BAD, scores=BAD, offsets=BAD, st=BAD, dest=BAD, gate=BAD):
        return L.moe_expert_choice(logits, T, E, C, scores, offsets, st, dest, gate, None)
    assert call(T=-1) == N.MOE_ERR_INVALID
    assert call(E=0) == N.MOE_ERR_INVALID
    assert call(C=-1) == N.MOE_ERR_INVALID
    assert call(E=513) == N.MOE_ERR_UNSUPPORTED
    assert call(T=1 << 23, E=512) == N.MOE_ERR_UNSUPPORTED  # T*E >= 2^31
    assert call(offsets=None) == N.MOE_ERR_INVALID
    assert call(logits=None) == N.MOE_ERR_INVALID
    assert call(dest=None) == N.MOE_ERR_INVALID
    assert call(st=None) == N.MOE_ERR_INVALID
    assert call(scores=None) == N.MOE_ERR_INVALID


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    y = torch.zeros(4, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        N.moe_combine(y, x.dtype, x, x, 4, 1, 64, None, x)


def test_backward_workspace_sizes():
    """FFN backward: the forward plan, the weight-gradient work lists, Z and
    dZ (4 B each), the tail partials and the gathered input rows; router
    weight backward: fp32 partials over up to 64 token ranges (about 4096
    blocks of 64 x 64 tiles, at least 16 tokens per range)."""
    for T, d, h, E, k in [(4096, 4096, 14336, 8, 2), (8192, 7168, 2048, 256, 8),
                          (256, 128, 256, 8, 2), (1, 256, 256, 512, 16)]:
        rows = T * k
        need = (N.moe_workspace_size(N.MOE_OP_FFN, T, d, h, E, k) - rows * h * 4
                - 256 * 288 * 256 * 4)  # the plan part of the forward workspace
        zr = 256 + _ceil((_ceil(rows, 256) + min(rows, E)) * (h // 256) + 256, 8) * 8 * 32
        need += (4 * E * (d // 256) * (h // 256) * 32 + zr + 2 * rows * h * 4
                 + 256 * 288 * 256 * 4 + rows * d * 2)
        assert N.moe_workspace_size(N.MOE_OP_FFN_BWD, T, d, h, E, k) >= need
        tiles = _ceil(E, 64) * _ceil(d, 64)
        s = max(1, min(_ceil(4096, tiles), 64, T // 16))
        assert N.moe_workspace_size(N.MOE_OP_ROUTER_BWD, T, d, h, E, k) >= s * E * d * 4
    assert N.moe_workspace_size(N.MOE_OP_FFN_BWD, 10, 256, 256, 600, 2) == 0


def test_backward_calls_reject_bad_arguments():
    L = N.lib()
    # combine backward
    assert L.moe_combine_backward(BAD, 1, BAD, BAD, -1, 2, 64, BAD, BAD, BAD, None) == 1
    assert L.moe_combine_backward(BAD, 2, BAD, BAD, 4, 2, 64, BAD, BAD, BAD, None) == 1
    assert L.moe_combine_backward(BAD, 1, BAD, BAD, 4, 513, 64, BAD, BAD, BAD, None) == 2
    assert L.moe_combine_backward(BAD, 1, BAD, BAD, 4, 2, 64, None, BAD, BAD, None) == 1
    assert L.moe_combine_backward(None, 1, BAD, BAD, 0, 2, 64, None, None, None, None) == 0
    # router backward
    F = ctypes.c_float
    assert L.moe_router_backward(BAD, BAD, BAD, BAD, BAD, 4, 8, 9, 1, F(0), BAD, None) == 1
    assert L.moe_router_backward(BAD, BAD, BAD, BAD, BAD, 4, 600, 2, 1, F(0), BAD, None) == 2
    assert L.moe_router_backward(BAD, BAD, BAD, BAD, None, 4, 8, 2, 1, F(0.5), BAD, None) == 1
    assert L.moe_router_backward(BAD, BAD, BAD, None, BAD, 4, 8, 2, 1, F(0), BAD, None) == 1
    assert L.moe_router_backward(BAD, None, BAD, BAD, None, 4, 8, 2, 0, F(0), BAD, None) == 1  # no table: k = E

    # grouped FFN backward
    def ffn(dtype=1, T=10, d=256, h=512, E=8, k=2, w1=BAD, dy=BAD, z=None, hh=None, ws=BAD,
            wsb=1 << 40):
        return L.moe_grouped_ffn_backward(BAD, dtype, T, d, h, E, k, BAD, BAD, w1, None, BAD, dy,
                                          z, hh, BAD, BAD, None, BAD, None, ws, wsb, None)
    assert ffn(T=-1) == 1
    assert ffn(dtype=3) == 1
    assert ffn(k=9) == 1
    assert ffn(E=600, k=2) == 2
    assert ffn(w1=None) == 1
    assert ffn(dy=None) == 1
    assert ffn(wsb=100) == 4
    assert ffn(ws=None) == 4
    assert ffn(d=192) == 2   # bf16 tiles need multiples of 256
    assert ffn(h=320) == 2
    assert ffn(z=BAD) == 1   # the kept pre-activations come with the hidden rows
    assert ffn(hh=BAD) == 1

    # training forward: as moe_grouped_ffn, plus both kept arrays
    def train(z=BAD, hh=BAD, d=128, wsb=1 << 40):
        return L.moe_grouped_ffn_train(BAD, 1, 10, d, 256, 8, 2, BAD, BAD, BAD, None, BAD, None,
                                       BAD, z, hh, BAD, wsb, None)
    assert train(z=None) == 1
    assert train(hh=None) == 1
    assert train(d=100) == 2
    assert train(wsb=16) == 4

    # gather backward
    assert L.moe_gather_backward(BAD, 1, BAD, -1, 2, 64, None, None, None, 8, BAD, None) == 1
    assert L.moe_gather_backward(BAD, 1, BAD, 4, 2, 64, None, BAD, None, 8, BAD, None) == 1
    assert L.moe_gather_backward(BAD, 1, BAD, 4, 2, 64, None, None, None, 600, BAD, None) == 2
    assert L.moe_gather_backward(None, 1, BAD, 4, 2, 64, None, None, None, 8, BAD, None) == 1
    # router weight backward
    assert L.moe_router_weight_backward(BAD, 1, -1, 64, 8, BAD, BAD, None, BAD, 1 << 30, None) == 1
    assert L.moe_router_weight_backward(BAD, 1, 64, 64, 600, BAD, BAD, None, BAD, 1 << 30, None) == 2
    assert L.moe_router_weight_backward(BAD, 1, 64, 64, 8, None, BAD, None, BAD, 1 << 30, None) == 1
    assert L.moe_router_weight_backward(BAD, 1, 64, 64, 8, BAD, BAD, None, BAD, 16, None) == 4

"""moe_permute_noalloc (the permute call that allocates nothing: its
histograms live in a static device array) against moe_permute, through the
C-ABI: every output bit for bit, on calls in a row whose sizes shrink (the
array keeps the last call's contents), with and without capacity drops, at
the array's largest size, and the refusal beyond it."""
import pytest
import torch

from top_routing_expert_topk_amd import native as N

pytestmark = pytest.mark.gpu

MAX_ASSIGN = 1 << 20  # MOE_PERMUTE_NOALLOC_MAX_ASSIGN


def _topk(T, k, E, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.topk(torch.rand(T, E, generator=g), k, dim=1).indices.to(torch.int32).cuda()


def _run(idx, E, cap, noalloc):
    T, k = idx.shape
    fill = dict(dtype=torch.int32, device="cuda")
    counts = torch.full((E,), -7, **fill)
    offsets = torch.full((E + 1,), -7, **fill)
    dest = torch.full((T * k,), -7, **fill)
    st = torch.full((T * k,), -7, **fill)
    torch.cuda.synchronize()
    if noalloc:
        before = torch.cuda.memory_allocated()
        N.moe_permute_noalloc(idx, T, k, E, cap, counts, offsets, dest, st)
        assert torch.cuda.memory_allocated() == before
    else:
        ws = torch.empty(max(1, N.moe_workspace_size(N.MOE_OP_PERMUTE, T, 1, 1, E, k)),
                         dtype=torch.uint8, device="cuda")
        N.moe_permute(idx, T, k, E, cap, counts, offsets, dest, st, ws)
    torch.cuda.synchronize()
    R = int(offsets[-1])
    return counts.cpu(), offsets.cpu(), dest.cpu(), st[:R].cpu()


def _same(idx, E, cap):
    want = _run(idx, E, cap, noalloc=False)
    got = _run(idx, E, cap, noalloc=True)
    for name, a, b in zip(("counts", "offsets", "dest_row", "sorted_token"), want, got):
        assert torch.equal(a, b), name
    return want


def test_noalloc_permute_equals_the_workspace_one_on_shrinking_calls():
    print("[noalloc] T=8192 k=8 E=256 no cap, then T=1000 k=2 E=64 cap 20, then T=37 k=3 E=5",
          flush=True)
    c, o, d, s = _same(_topk(8192, 8, 256, 1), 256, -1)
    assert int(o[-1]) == 8192 * 8
    c, o, d, s = _same(_topk(1000, 2, 64, 2), 64, 20)
    assert (d < 0).any() and int(o[-1]) < 2000
    _same(_topk(37, 3, 5, 3), 5, 4)


def test_noalloc_permute_at_the_largest_size_and_beyond():
    print("[noalloc] T*k = 2^20 (E=512), then 2^20 + 8 refused", flush=True)
    _same(_topk(MAX_ASSIGN // 8, 8, 512, 4), 512, -1)
    idx = _topk(MAX_ASSIGN // 8 + 1, 8, 512, 5)
    with pytest.raises(N.MoEError) as err:
        _run(idx, 512, -1, noalloc=True)
    assert err.value.status == N.MOE_ERR_UNSUPPORTED


def test_noalloc_permute_empty_batch():
    print("[noalloc] T=0", flush=True)
    fill = dict(dtype=torch.int32, device="cuda")
    counts = torch.full((8,), -7, **fill)
    offsets = torch.full((9,), -7, **fill)
    N.moe_permute_noalloc(None, 0, 2, 8, -1, counts, offsets, None, None)
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0

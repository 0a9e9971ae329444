"""moe_check_permutation (host pointers, no GPU) against permutations the
oracle builds: it accepts the oracle's token-choice permutations (with and
without capacity drops) and Expert Choice layouts, and refuses each kind of
corruption that would send a kernel outside its arrays or to the wrong row."""
import numpy as np
import pytest

from oracle import oracle as orc
from top_routing_expert_topk_amd import native as N


def _token_choice(seed, T, E, k, cap):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E))
    idx, _, _ = orc.route(lg, k, True)
    counts, offsets, dest, st = orc.permute(idx, E, cap)
    return offsets, st, dest


CASES = [(1, 50, 8, 2, -1), (2, 300, 16, 4, 20), (3, 7, 5, 5, -1), (4, 64, 4, 1, 0),
         (5, 1, 3, 2, 1), (6, 200, 64, 8, 11)]


@pytest.mark.parametrize("seed,T,E,k,cap", CASES)
def test_accepts_the_oracles_permutations(seed, T, E, k, cap):
    off, st, dest = _token_choice(seed, T, E, k, cap)
    assert N.moe_check_permutation(off, E, st, dest, T, k) == 0
    assert N.moe_check_permutation(off, E, st, None, T, k) == 0
    assert N.moe_check_permutation(None, E, None, dest, T, k) == 0


@pytest.mark.parametrize("T,E,C", [(40, 6, 9), (10, 4, 10), (25, 30, 1), (8, 3, 0)])
def test_accepts_expert_choice_layouts(T, E, C):
    rng = np.random.default_rng(T + E + C)
    off, st, dest, _ = orc.expert_choice(orc.ec_scores(rng.standard_normal((T, E))), C)
    assert N.moe_check_permutation(off, E, st, dest.ravel(), T, E) == 0


@pytest.mark.parametrize("seed,T,E,k,cap", CASES[:3] + CASES[5:])
def test_refuses_corrupted_permutations(seed, T, E, k, cap):
    off, st, dest = _token_choice(seed, T, E, k, cap)
    R = int(off[-1])
    assert R > 1

    def bad(o=off, s=st, d=dest):
        return N.moe_check_permutation(o, E, s, d, T, k) == 1
    o = off.copy(); o[0] = 1
    assert bad(o=o)
    o = off.copy(); o[E] = T * k + 1
    assert bad(o=o, s=np.zeros(T * k + 1, np.int32))
    e = int(np.argmax(np.diff(off)))
    o = off.copy(); o[e] = o[e + 1] + 1
    assert bad(o=o)
    for v in (T, -1):
        s = st.copy(); s[R // 2] = v
        assert bad(s=s)
    s = st.copy(); r = int(dest[dest >= 0][0]); s[r] = (s[r] + 1) % T
    assert bad(s=s)  # a row holding another token
    for v in (R, -2):
        d = dest.copy(); d[0] = v
        assert bad(d=d)
    kept = np.nonzero(dest >= 0)[0]
    d = dest.copy(); d[kept[1]] = d[kept[0]]
    assert bad(d=d)  # two slots, one row
    d = dest.copy(); d[kept[0]] = -1
    assert bad(d=d)  # a row nobody owns
    assert N.moe_check_permutation(None, E, st, None, T, k) == 1  # length unknown


def test_refuses_bad_sizes():
    assert N.moe_check_permutation(None, 4, None, None, -1, 2) == 1
    assert N.moe_check_permutation(None, 0, None, None, 4, 2) == 1
    assert N.moe_check_permutation(None, 4, None, None, 4, 0) == 1
    assert N.moe_check_permutation(None, 4, None, None, 0, 2) == 0

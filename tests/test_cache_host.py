"""The expert cache's slot policy on the host (no device memory, no copies).

moe_cache_step decides, per step, which needed experts are hits, which slot
each miss takes (the least recently used one the step does not need, empty
slots first) and what it evicts. These tests drive it through the C-ABI with
no tensors to copy and compare every decision with a small Python model of
that policy, over random sequences of steps.
"""
import ctypes

import numpy as np
import pytest

from top_routing_expert_topk_amd import native as N


def _step(state, counts):
    L = N.lib()
    loaded = ctypes.c_int(-1)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    st = L.moe_cache_step(state.ctypes.data, counts.ctypes.data, 0, None, None, None, None, None,
                          ctypes.byref(loaded), None, None)
    return st, loaded.value


class Model:
    """Least-recently-used slots; hits refresh their slot first, then misses in expert order."""

    def __init__(self, E, S):
        self.E, self.S = E, S
        self.slot_of = [-1] * E
        self.expert_in = [-1] * S
        self.last = [-1] * S
        self.clock = 0

    def step(self, counts):
        need = [e for e in range(self.E) if counts[e] > 0]
        if len(need) > self.S:
            return None
        self.clock += 1
        phase = [-1] * self.E
        for e in need:
            if self.slot_of[e] >= 0:
                phase[e] = 0
                self.last[self.slot_of[e]] = self.clock
        loaded = 0
        for e in need:
            if self.slot_of[e] >= 0:
                continue
            free = [s for s in range(self.S) if self.last[s] < self.clock]
            victim = min(free, key=lambda s: (self.last[s], s))
            if self.expert_in[victim] >= 0:
                self.slot_of[self.expert_in[victim]] = -1
            self.expert_in[victim] = e
            self.slot_of[e] = victim
            self.last[victim] = self.clock
            phase[e] = 1
            loaded += 1
        return loaded, list(self.slot_of), phase


@pytest.mark.parametrize("E,S,k", [(8, 8, 2), (16, 6, 2), (64, 48, 2), (128, 20, 1), (512, 40, 16)])
def test_policy_matches_the_model(E, S, k):
    state = np.zeros(N.moe_cache_state_bytes(E, S), np.uint8)
    N.moe_cache_init(state, E, S)
    model = Model(E, S)
    rng = np.random.default_rng(E * 31 + S)
    for it in range(60):
        counts = np.zeros(E, np.int32)
        # a hot set plus random experts, so hits, misses and evictions all occur
        hot = rng.choice(min(E, S), size=min(k, S), replace=False)
        cold = rng.choice(E, size=rng.integers(0, S - len(hot) + 1), replace=False)
        counts[hot] += 1
        counts[cold] += rng.integers(1, 4, size=cold.size)
        want = model.step(counts)
        st, loaded = _step(state, counts)
        assert st == 0 and want is not None
        slot, phase = N.moe_cache_slot_of(state, E)
        assert loaded == want[0], f"step {it}"
        assert slot.tolist() == want[1], f"step {it}"
        assert phase.tolist() == want[2], f"step {it}"
        # every needed expert sits in a distinct slot
        live = slot[counts > 0]
        assert np.all(live >= 0) and len(set(live.tolist())) == live.size


def test_more_experts_than_slots_is_refused():
    E, S = 10, 3
    state = np.zeros(N.moe_cache_state_bytes(E, S), np.uint8)
    N.moe_cache_init(state, E, S)
    st, _ = _step(state, np.array([1, 1, 1, 1] + [0] * 6))
    assert st == N.MOE_ERR_UNSUPPORTED
    st, loaded = _step(state, np.array([1, 1, 1] + [0] * 7))
    assert st == 0 and loaded == 3
    st, loaded = _step(state, np.array([1, 1, 1] + [0] * 7))
    assert st == 0 and loaded == 0  # all hits


def test_arguments_are_checked():
    L = N.lib()
    assert N.moe_cache_state_bytes(0, 4) == 0
    assert N.moe_cache_state_bytes(600, 4) == 0
    assert L.moe_cache_init(None, 4, 4) == N.MOE_ERR_INVALID
    state = np.zeros(N.moe_cache_state_bytes(4, 4), np.uint8)
    assert L.moe_cache_init(state.ctypes.data, 4, 0) == N.MOE_ERR_INVALID
    assert L.moe_cache_step(None, None, 0, None, None, None, None, None, None, None,
                            None) == N.MOE_ERR_INVALID
    N.moe_cache_init(state, 4, 4)
    counts = np.ones(4, np.int32)
    # tensors to copy but no pointer arrays
    assert L.moe_cache_step(state.ctypes.data, counts.ctypes.data, 2, None, None, None, None, None,
                            None, None, None) == N.MOE_ERR_INVALID

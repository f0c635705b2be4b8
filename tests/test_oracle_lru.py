"""Pins for the oracle's LRU slot cache (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class _IdKeyedLRU:
    """A second, id-keyed statement of the same policy, for cross-checking."""

    def __init__(self, L, E, S):
        self.E, self.S = E, S
        self.res = {}          # id -> [slot, last_use]
        self.free = list(range(S))
        self.clock = 0

    def resolve(self, layer, idx):
        self.clock += 1
        want = sorted({layer * self.E + int(e) for e in np.asarray(idx).reshape(-1)})
        for i in want:
            if i in self.res:
                self.res[i][1] = self.clock
        misses = []
        for i in want:
            if i in self.res:
                continue
            if self.free:
                s = min(self.free)
                self.free.remove(s)
            else:
                cands = [(lu, sl, ident) for ident, (sl, lu) in self.res.items() if lu < self.clock]
                if not cands:
                    raise oracle.CapacityError("full")
                _lu, s, old = min(cands)
                del self.res[old]
            self.res[i] = [s, self.clock]
            misses.append((i, s))
        return misses


def test_hand_trace():
    g = json.load(open(os.path.join(GOLDEN, "lru_trace.json")))
    c = oracle.LRUCache(g["n_layers"], g["n_experts"], g["n_slots"])
    for call in g["calls"]:
        if call.get("capacity_error"):
            with pytest.raises(oracle.CapacityError):
                c.resolve(0, np.array(call["idx"]))
            continue
        slots, misses = c.resolve(0, np.array(call["idx"]))
        assert [list(m) for m in misses] == call["misses"]
        assert c.stamp.tolist() == call["stamp"]
        assert c.id_of.tolist() == call["id_of"]
        for i, s in enumerate(c.id_of):
            if s >= 0:
                assert c.slot_of[s] == i
        assert np.array_equal(slots, np.vectorize(lambda e: c.slot_of[e])(np.array(call["idx"])))
    # the failing call changed nothing: state, clock and counts are call 4's
    last = g["calls"][3]
    assert c.stamp.tolist() == last["stamp"] and c.id_of.tolist() == last["id_of"] and c.clock == 4
    assert c.lookups == g["lookups_after_4"] and c.hits == g["hits_after_4"]


@pytest.mark.parametrize("S", [12, 16, 40, 64])
def test_against_id_keyed_simulator(S):
    L, E, k = 3, 32, 4
    rng = np.random.default_rng(S)
    a = oracle.LRUCache(L, E, S)
    b = _IdKeyedLRU(L, E, S)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    for step in range(300):
        layer = step % L
        T = int(rng.integers(1, 3))
        idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)])
        _, m1 = a.resolve(layer, idx)
        m2 = b.resolve(layer, idx)
        assert m1 == m2
    assert a.hits + a.misses == a.lookups


def test_compulsory_misses_only_when_everything_fits():
    L, E = 2, 16
    c = oracle.LRUCache(L, E, L * E - 1)  # capped by one, but the run touches fewer ids
    rng = np.random.default_rng(0)
    seen = set()
    for step in range(100):
        layer = step % L
        idx = rng.choice(12, (2, 3))
        idx = np.array([rng.choice(12, 3, replace=False) for _ in range(2)])
        c.resolve(layer, idx)
        seen |= {layer * E + int(e) for e in idx.reshape(-1)}
    assert c.misses == len(seen)


def test_cyclic_access_always_misses():
    S = 5
    c = oracle.LRUCache(1, S + 1, S)
    for rep in range(4):
        for e in range(S + 1):
            c.resolve(0, np.array([[e]]))
    assert c.hits == 0 and c.misses == 4 * (S + 1)


def test_reset_fills_slots_in_order():
    S = 6
    c = oracle.LRUCache(1, 20, S)
    c.resolve(0, np.array([[3, 9]]))
    c.reset()
    order = []
    for e in [7, 2, 11, 5, 0, 19]:
        _, m = c.resolve(0, np.array([[e]]))
        order.append(m[0][1])
    assert order == list(range(S))


def test_identity_mode():
    c = oracle.LRUCache(2, 8, 16)
    slots, misses = c.resolve(1, np.array([[3, 5], [5, 0]]))
    assert misses == [] and slots.tolist() == [[11, 13], [13, 8]]
    assert c.lookups == 3 and c.hits == 3


def test_slots_touched_this_call_are_never_evicted():
    S = 4
    c = oracle.LRUCache(1, 10, S)
    c.resolve(0, np.array([[0, 1, 2, 3]]))
    # one call touching 2 resident ids and 2 new ids: the new ones may only
    # take the slots of the two ids not touched now
    slots, m = c.resolve(0, np.array([[2, 3, 7, 8]]))
    assert sorted(s for _, s in m) == [0, 1]
    assert slots.tolist() == [[2, 3, 0, 1]]

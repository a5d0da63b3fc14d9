"""Pins of the oracle's batch-LRU slot bookkeeping.

(i) a move-to-front recency list that implements the same rules with no keys,
(ii) closed forms, (iii) invariants, (iv) inclusion in S, (v) the optimal
(hindsight) miss count as a lower bound, (vi) a trace worked out by hand.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import SlotState

GOLD = os.path.join(os.path.dirname(__file__), "golden", "lru_hand_trace.json")


class MoveToFront:
    """Recency list from least to most recent; empty slots are used lowest id first.
    Pinned experts sit in the first slots, outside the recency list."""

    def __init__(self, E, S, preload=False, pins=()):
        self.E, self.S = E, S
        self.slot_of = {}
        self.expert_in = [-1] * S
        self.recency = []          # unpinned experts, LRU first
        self.pinned = list(pins)
        for s, e in enumerate(self.pinned):
            self.slot_of[e] = s
            self.expert_in[s] = e
        if preload:
            for s in range(S):
                self.slot_of[s] = s
                self.expert_in[s] = s
                self.recency.append(s)   # equal clocks: lower slot is older

    def step(self, ids):
        P = [int(e) for e in np.asarray(ids).reshape(-1)]
        M = np.asarray(ids).shape[0]
        U = list(dict.fromkeys(P))
        free = self.S - len(self.pinned)
        if M > 16 or len([e for e in U if e not in self.pinned]) > free:
            return True, []
        hits = {e for e in U if e in self.slot_of}
        victims = [s for s in range(len(self.pinned), self.S) if self.expert_in[s] < 0]
        victims += [self.slot_of[e] for e in self.recency if e not in hits]
        events = []
        for i, e in enumerate([e for e in U if e not in hits]):
            s = victims[i]
            old = self.expert_in[s]
            if old >= 0:
                del self.slot_of[old]
                self.recency.remove(old)
            self.slot_of[e] = s
            self.expert_in[s] = e
            events.append((e, s, old))
        last = {e: p for p, e in enumerate(P)}
        for e in U:
            if e in self.recency:
                self.recency.remove(e)
        self.recency += sorted([e for e in U if e not in self.pinned], key=lambda e: last[e])
        return False, events


def _random_ids(rng, E, k, M):
    return np.array([rng.choice(E, size=k, replace=False) for _ in range(M)])


@pytest.mark.parametrize("E,S,k", [(4, 1, 1), (6, 2, 1), (8, 3, 2), (8, 4, 3), (5, 5, 2), (7, 4, 2)])
@pytest.mark.parametrize("preload", [False, True])
def test_matches_move_to_front(E, S, k, preload):
    rng = np.random.default_rng(E * 100 + S * 10 + k + preload)
    st = SlotState(E, S, k)
    mtf = MoveToFront(E, S, preload)
    if preload:
        st.preload()
    for t in range(2500):
        M = int(rng.choice([1, 1, 1, 2, 3, 17]))
        ids = _random_ids(rng, E, k, M)
        rec = st.step(ids)
        bypass, events = mtf.step(ids)
        assert rec.bypass == bypass
        assert rec.events == events, (t, ids)
        st.check_invariants()
        if not rec.bypass:
            for e in rec.uniques:
                assert st.e2s[e] >= 0
    assert st.t == 2500


@pytest.mark.parametrize("E,S,k,npin", [(6, 3, 1, 1), (8, 4, 2, 2), (9, 5, 2, 3), (8, 4, 3, 4), (10, 6, 2, 5)])
def test_pinned_slots_match_move_to_front(E, S, k, npin):
    """Hybrid policy: npin experts pinned in the first slots, LRU over the rest,
    against the key-free recency list (bypass decisions and every event)."""
    rng = np.random.default_rng(E * 31 + S * 7 + npin)
    pins = [int(e) for e in rng.choice(E, size=npin, replace=False)]
    st = SlotState(E, S, k)
    st.pin(pins)
    mtf = MoveToFront(E, S, pins=pins)
    for t in range(2500):
        M = int(rng.choice([1, 1, 1, 2, 3, 17]))
        ids = _random_ids(rng, E, k, M)
        rec = st.step(ids)
        bypass, events = mtf.step(ids)
        assert rec.bypass == bypass, t
        assert rec.events == events, (t, ids)
        st.check_invariants()
        assert [st.s2e[s] for s in range(npin)] == pins      # pinned slots never change
        if not rec.bypass:
            for e in rec.uniques:
                assert st.e2s[e] >= 0


def test_all_slots_pinned_is_the_static_pin():
    """P = S: a step is cached exactly when all its experts are pinned, nothing
    is ever filled, and the resident fraction of all lookups (hits on cached
    steps plus residents of bypass steps, whose host bytes exclude them) equals
    the static-pin hit rate of the same pinned set."""
    from oracle import static_pin, static_pin_hit_rate
    rng = np.random.default_rng(21)
    E, S, k, B = 12, 5, 2, 1000
    trace = [_random_ids(rng, E, k, int(rng.choice([1, 1, 2, 3]))) for _ in range(1500)]
    uniques = [list(dict.fromkeys(int(e) for e in ids.reshape(-1))) for ids in trace]
    pin = static_pin(uniques, E, S)
    st = SlotState(E, S, k, blob_bytes=B)
    st.pin(pin)
    for ids, u in zip(trace, uniques):
        rec = st.step(ids)
        assert rec.bypass == (not set(u) <= set(pin))
        assert rec.events == []
    c = st.counters
    total = sum(len(u) for u in uniques)
    resident = c.hits + sum(len(u) for u in uniques) - c.lookups - c.bypass_bytes // B
    assert c.misses == 0 and c.bytes_filled == 0
    assert resident / total == pytest.approx(static_pin_hit_rate(uniques, E, S), abs=0)


def test_bypass_reads_only_non_resident_experts():
    """A bypass step's host bytes count its non-resident unique experts only."""
    st = SlotState(4, 2, 2, blob_bytes=10)
    st.step(np.array([[0, 1]]))                 # fills slots with 0, 1
    rec = st.step(np.array([[0, 2], [3, 1]]))   # U = 0,2,3,1 > S: bypass; 0 and 1 resident
    assert rec.bypass
    assert st.counters.bypass_bytes == 2 * 10


def test_victim_has_the_minimum_key():
    rng = np.random.default_rng(7)
    st = SlotState(10, 4, 2)
    for _ in range(3000):
        ids = _random_ids(rng, 10, 2, int(rng.integers(1, 3)))
        before_key, before_s2e = list(st.key), list(st.s2e)
        rec = st.step(ids)
        if rec.bypass:
            continue
        hit = {e for e, h in zip(rec.uniques, rec.hit) if h}
        cand = sorted((before_key[s], s) for s in range(4) if before_s2e[s] not in hit)
        assert [s for _, s in cand[:len(rec.events)]] == [s for _, s, _ in rec.events]


def test_closed_form_enough_slots():
    rng = np.random.default_rng(3)
    E, k = 9, 3
    st = SlotState(E, E, k)
    seen = set()
    for _ in range(400):
        ids = _random_ids(rng, E, k, int(rng.integers(1, 4)))
        seen |= set(int(e) for e in ids.reshape(-1))
        st.step(ids)
    assert st.counters.misses == len(seen)
    assert st.counters.evictions == 0


def test_closed_form_one_slot_top1():
    rng = np.random.default_rng(4)
    ids = rng.integers(0, 3, size=5000)
    st = SlotState(3, 1, 1)
    for e in ids:
        st.step(np.array([[e]]))
    changes = int(np.sum(ids[1:] != ids[:-1]))
    assert st.counters.misses == 1 + changes
    assert st.counters.evictions == changes


def test_inclusion_hits_grow_with_slots():
    rng = np.random.default_rng(5)
    E, k = 12, 2
    trace = [_random_ids(rng, E, k, int(rng.integers(1, 3))) for _ in range(3000)]
    maxu = max(len(set(t.reshape(-1))) for t in trace)
    prev = -1
    contents_prev = None
    for S in range(maxu, E + 1):
        st = SlotState(E, S, k)
        contents = []
        for ids in trace:
            st.step(ids)
            contents.append({e for e in range(E) if st.e2s[e] >= 0})
        assert st.counters.bypass_steps == 0
        assert st.counters.hits >= prev
        if contents_prev is not None:
            assert all(a <= b for a, b in zip(contents_prev, contents))
        prev, contents_prev = st.counters.hits, contents


def _optimal_misses(trace, E, S):
    """Fewest misses any demand-fill policy can reach (dynamic programming over cache contents)."""
    states = {frozenset(): 0}
    for ids in trace:
        U = frozenset(int(e) for e in ids.reshape(-1))
        nxt = {}
        for c, cost in states.items():
            miss = len(U - c)
            keep_pool = sorted(c - U)
            room = S - len(U)
            for r in range(0, min(room, len(keep_pool)) + 1):
                for keep in itertools.combinations(keep_pool, r):
                    n = U | frozenset(keep)
                    if cost + miss < nxt.get(n, 1 << 60):
                        nxt[n] = cost + miss
        states = nxt
    return min(states.values())


def test_lru_never_beats_the_optimum():
    rng = np.random.default_rng(6)
    for trial in range(30):
        E, S, k = 6, int(rng.integers(2, 4)), int(rng.integers(1, 3))
        trace = [_random_ids(rng, E, k, 1) for _ in range(10)]
        st = SlotState(E, S, k)
        for ids in trace:
            st.step(ids)
        opt = _optimal_misses(trace, E, S)
        assert st.counters.misses >= opt
        if S >= E:
            assert st.counters.misses == opt


def test_hand_worked_trace():
    g = json.load(open(GOLD))
    st = SlotState(g["n_experts"], g["n_slots"], g["top_k"])
    for s in g["steps"]:
        rec = st.step(np.array(s["ids"]))
        assert rec.bypass == s["bypass"]
        assert [list(e) for e in rec.events] == s["events"]
    f = g["final"]
    assert st.e2s == f["e2s"] and st.s2e == f["s2e"] and st.key == f["key"] and st.t == f["t"]
    for name, v in f["counters"].items():
        assert getattr(st.counters, name) == v, name


def test_bad_ids_raise():
    st = SlotState(4, 2, 1)
    with pytest.raises(ValueError):
        st.step(np.array([[4]]))
    with pytest.raises(ValueError):
        SlotState(4, 5, 1)

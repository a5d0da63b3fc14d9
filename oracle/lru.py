"""Per-layer slot bookkeeping: batch LRU over S HBM slots (test infrastructure).

Pages: each MoE layer owns S fixed HBM slots; router ids are mapped to slot ids
on the device before the single expert launch; a missing expert is copied into
the least-recently-used victim slot and the map is updated (page "GLM 5.3
Testing: HBM Expert Allocation", sections "What the slot cache is" and the
shelf analogy after it).  Occupancy follows a running LRU clock and the per-layer
slot map only sets the capacity (page "GB300 GLM 5.3 Testing", section "Expert
allocation vs a cache").  Batches of more than 16 rows bypass the cache and read
experts directly (same section on the HBM allocation page).

Readings taken where the pages are silent (one launch maps a whole step, so the
bookkeeping is per step, not per pick):
  * P = the M*k picks flattened in (row, rank) order, positions p = 0..M*k-1.
  * U = unique experts of P in first-occurrence order; hits H = resident ones;
    misses = U minus H, in first-occurrence order.
  * A step bypasses (state untouched, step counter still advances) when M > 16
    or when its unique experts do not fit: |U| > S.  A bypass step reads only
    its non-resident experts from the host store; resident ones are read from
    their slots (page "GB300 GLM 5.3 Testing", section on sizing the context
    window: the bypass path fetches only experts that are not resident), so
    its host bytes are (non-resident unique experts) * B_e.
  * Pinned slots (the hybrid policy; page "GB300 GLM 5.3 Testing", section
    "Expert allocation vs a cache", compares pins with LRU): the first P slots
    hold a fixed expert each and are never victims; LRU runs over the other
    S - P.  The fit rule becomes |U| - (pinned hits) > S - P, which for P = 0
    is |U| > S.
  * Victim candidates = slots whose resident is not a hit, sorted by
    (key, slot id); empty slots carry key -1 and so come first, in slot order.
    The i-th miss takes the i-th candidate; a resident there is evicted.
  * After the step every e in U gets key = t*(16*k) + (last position of e in P),
    t being the step counter before the increment.
  * Counters count unique lookups; picks are counted alongside.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

BYPASS_ROWS = 16


@dataclass
class Counters:
    steps: int = 0
    bypass_steps: int = 0
    picks: int = 0
    lookups: int = 0
    hits: int = 0
    misses: int = 0
    evictions: int = 0
    bytes_filled: int = 0
    bypass_bytes: int = 0


@dataclass
class StepRecord:
    step: int
    bypass: bool
    uniques: List[int]
    hit: List[bool]
    events: List[Tuple[int, int, int]]      # (expert, slot, evicted expert or -1), miss order
    slot_of_unique: List[int]                # slot per unique expert (-1 on bypass)
    unique_of_pick: List[int]


class SlotState:
    def __init__(self, n_experts: int, n_slots: int, top_k: int, blob_bytes: int = 0):
        if not 1 <= n_slots <= n_experts:
            raise ValueError("need 1 <= S <= E")
        self.E, self.S, self.k = n_experts, n_slots, top_k
        self.blob_bytes = blob_bytes
        self.e2s = [-1] * n_experts
        self.s2e = [-1] * n_slots
        self.key = [-1] * n_slots
        self.P = 0                  # pinned slots [0, P)
        self.t = 0
        self.counters = Counters()

    def preload(self):
        """Warm start: slot s holds expert s (s < S), all keys -1, no pins."""
        self.P = 0
        self.e2s = [-1] * self.E
        for s in range(self.S):
            self.s2e[s] = s
            self.e2s[s] = s
            self.key[s] = -1

    def pin(self, experts):
        """Slot i holds experts[i] for good (i < P = len(experts) <= S); the other
        slots are emptied; all keys -1.  Counters and the step counter are kept."""
        experts = [int(e) for e in experts]
        if len(experts) > self.S or len(set(experts)) != len(experts):
            raise ValueError("need at most S distinct experts")
        if any(not 0 <= e < self.E for e in experts):
            raise ValueError("expert id out of range")
        self.P = len(experts)
        self.e2s = [-1] * self.E
        self.s2e = [-1] * self.S
        self.key = [-1] * self.S
        for s, e in enumerate(experts):
            self.s2e[s] = e
            self.e2s[e] = s

    def step(self, ids) -> StepRecord:
        ids = np.asarray(ids)
        M, k = ids.shape
        if k != self.k:
            raise ValueError("top_k mismatch")
        P = [int(e) for e in ids.reshape(-1)]
        for e in P:
            if not 0 <= e < self.E:
                raise ValueError("expert id out of range")
        uniques, first_pos, last_pos = [], {}, {}
        for p, e in enumerate(P):
            if e not in first_pos:
                first_pos[e] = p
                uniques.append(e)
            last_pos[e] = p
        u_index = {e: i for i, e in enumerate(uniques)}
        unique_of_pick = [u_index[e] for e in P]
        t = self.t
        self.t += 1
        c = self.counters
        c.steps += 1
        resident = [self.e2s[e] >= 0 for e in uniques]
        pinned_hits = sum(1 for e in uniques if 0 <= self.e2s[e] < self.P)
        if M > BYPASS_ROWS or len(uniques) - pinned_hits > self.S - self.P:
            c.bypass_steps += 1
            c.bypass_bytes += (len(uniques) - sum(resident)) * self.blob_bytes
            return StepRecord(t, True, uniques, [False] * len(uniques), [], [-1] * len(uniques),
                              unique_of_pick)
        hit = resident
        hit_set = {e for e, h in zip(uniques, hit) if h}
        misses = [e for e, h in zip(uniques, hit) if not h]
        cands = self._victim_order([s for s in range(self.P, self.S) if self.s2e[s] not in hit_set])
        events = []
        for i, e in enumerate(misses):
            s = cands[i]
            old = self.s2e[s]
            if old >= 0:
                self.e2s[old] = -1
                c.evictions += 1
            self.e2s[e] = s
            self.s2e[s] = e
            events.append((e, s, old))
        for e in uniques:
            self.key[self.e2s[e]] = t * (BYPASS_ROWS * self.k) + last_pos[e]
        c.picks += len(P)
        c.lookups += len(uniques)
        c.hits += len(uniques) - len(misses)
        c.misses += len(misses)
        c.bytes_filled += len(misses) * self.blob_bytes
        return StepRecord(t, False, uniques, hit, events, [self.e2s[e] for e in uniques],
                          unique_of_pick)

    def _victim_order(self, cands):
        """Least recently used first: ascending (key, slot id)."""
        return sorted(cands, key=lambda s: (self.key[s], s))

    def check_invariants(self):
        res = [e for e in range(self.E) if self.e2s[e] >= 0]
        assert len(res) <= self.S
        for e in res:
            assert self.s2e[self.e2s[e]] == e
        for s in range(self.S):
            if self.s2e[s] >= 0:
                assert self.e2s[self.s2e[s]] == s
            else:
                assert self.key[s] == -1   # a slot is empty only before its first fill

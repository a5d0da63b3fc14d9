"""Slot-budget and placement policies over routing traces (test infrastructure).

Page "GB300 GLM 5.3 Testing": a per-layer slot count is a capacity, occupancy
follows an LRU clock, and a hindsight static pin is the comparator (section
"Expert allocation vs a cache"); the slot map should come from the routing
traces by transfer bytes saved per HBM byte, with fewer slots for flat layers
(page "GLM 5.3 Testing: HBM Expert Allocation", section "What's next, in
order"); and decode speed follows a closed-form token model (same page,
section "What the physics says to expect").

  lru_hit_curve   hits of the batch LRU at every S, for one-row steps
  allocate_slots  per-layer S maximising total hits under a total budget
  hybrid_curve    hits with P pinned hottest experts + LRU, for every P
  token_rate      the pages' token model with our measured step costs
"""
import numpy as np

from .lru import SlotState
from .static_pin import static_pin


def lru_hit_curve(unique_sets, n_experts: int):
    """hits[S] for S = 0..E of the batch LRU, cold start, for one-row steps
    (every step looks up its k distinct experts, first-occurrence order).

    The cache always holds the S experts with the newest keys among those seen
    (the inclusion argument), so a lookup hits at S exactly when fewer than S
    seen experts have a newer key than the looked-up one before the step.  For
    S < k every step bypasses (|U| = k > S), so those entries are 0."""
    E = n_experts
    k = len(unique_sets[0]) if unique_sets else 0
    if any(len(u) != k or len(set(u)) != k for u in unique_sets):
        raise ValueError("one-row steps: every step has the same number k of distinct experts")
    key = np.full(E, -1, dtype=np.int64)        # -1: never seen
    rank_hist = np.zeros(E + 1, dtype=np.int64)
    for t, u in enumerate(unique_sets):
        for e in u:
            if key[e] >= 0:
                rank_hist[int(np.sum(key > key[e]))] += 1
        for j, e in enumerate(u):
            key[e] = t * (E + 1) + j            # pick order within the step, newer than any earlier step
    hits = np.concatenate([[0], np.cumsum(rank_hist)[:E]]).astype(np.int64)
    hits[:k] = 0
    return hits


def lru_hits_by_simulation(unique_sets, n_experts: int, n_slots: int) -> int:
    """Hits of the batch LRU at one S, stepping the slot state (one row per step)."""
    if n_slots < 1:
        return 0
    k = len(unique_sets[0])
    st = SlotState(n_experts, n_slots, k)
    for u in unique_sets:
        st.step(np.array([list(u)]))
    return st.counters.hits


def allocate_slots(curves, total: int, s_min: int = 0, s_max=None):
    """Per-layer slot counts S_l (s_min <= S_l <= s_max, sum S_l = total)
    maximising sum_l curves[l][S_l]: an exact max-plus dynamic programme over
    layers.  Returns (S list, total hits)."""
    L = len(curves)
    caps = [len(c) - 1 if s_max is None else min(s_max, len(c) - 1) for c in curves]
    NEG = np.iinfo(np.int64).min // 4
    best = np.full(total + 1, NEG, dtype=np.int64)
    best[0] = 0
    choice = []
    for l in range(L):
        c = np.asarray(curves[l], dtype=np.int64)
        nxt = np.full(total + 1, NEG, dtype=np.int64)
        arg = np.full(total + 1, -1, dtype=np.int64)
        for s in range(s_min, caps[l] + 1):
            if s > total:
                break
            cand = np.full(total + 1, NEG, dtype=np.int64)
            cand[s:] = best[: total + 1 - s] + c[s]
            better = cand > nxt
            nxt[better] = cand[better]
            arg[better] = s
        best = nxt
        choice.append(arg)
    if best[total] <= NEG // 2:
        raise ValueError("budget cannot be met within the bounds")
    S = [0] * L
    b = total
    for l in range(L - 1, -1, -1):
        s = int(choice[l][b])
        S[l] = s
        b -= s
    return S, int(best[total])


def hybrid_curve(unique_sets, n_experts: int, n_slots: int):
    """Resident lookups (hits of cached steps + resident experts of bypass
    steps, which read those from their slots) with the P hottest experts
    pinned and LRU over the other S - P slots, for P = 0..S; one-row steps.
    The pinned set of size P is the hindsight static pin."""
    k = len(unique_sets[0])
    out = []
    for p in range(n_slots + 1):
        st = SlotState(n_experts, n_slots, k)
        st.pin(static_pin(unique_sets, n_experts, p) if p else [])
        res = 0
        for u in unique_sets:
            resident = sum(1 for e in u if st.e2s[e] >= 0)
            rec = st.step(np.array([list(u)]))
            res += resident if rec.bypass else sum(rec.hit)
        out.append(res)
    return out


def token_rate(n_layers: int, t_hit_us: float, misses_per_layer_step: float, t_miss_us: float,
               t_other_ms: float) -> float:
    """Tokens per second of the pages' decode model: every token runs each MoE
    layer once, paying the all-hit step time plus the misses' host-link time,
    plus the rest of the model."""
    ms = n_layers * (t_hit_us + misses_per_layer_step * t_miss_us) / 1000.0 + t_other_ms
    return 1000.0 / ms

"""Pins of the oracle's slot-budget and placement policies.

LRU hit curves against step-by-step replays at every S; the budget split
against exhaustive search; the hybrid policy's end points against plain LRU
and the static pin; the token model against the page's worked example."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import (SlotState, allocate_slots, hybrid_curve, lru_hit_curve, lru_hits_by_simulation,
                    static_pin_hit_rate, token_rate)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "token_model.json")


def _one_row_trace(rng, E, k, T, skew=0.0):
    p = np.exp(-skew * np.arange(E)) if skew else np.ones(E)
    p = p / p.sum()
    return [list(int(e) for e in rng.choice(E, size=k, replace=False, p=p)) for _ in range(T)]


@pytest.mark.parametrize("E,k,skew", [(6, 1, 0.0), (10, 2, 0.3), (16, 3, 0.2), (12, 4, 0.0), (20, 2, 0.5)])
def test_lru_hit_curve_equals_replay_at_every_S(E, k, skew):
    rng = np.random.default_rng(E * 7 + k)
    us = _one_row_trace(rng, E, k, 500, skew)
    curve = lru_hit_curve(us, E)
    assert [int(v) for v in curve] == [lru_hits_by_simulation(us, E, S) for S in range(E + 1)]
    assert all(curve[S] <= curve[S + 1] for S in range(E))          # inclusion
    assert curve[E] == 500 * k - len({e for u in us for e in u})    # S = E: every repeat hits


def test_allocate_slots_is_the_exhaustive_optimum():
    rng = np.random.default_rng(5)
    for _ in range(30):
        L, Smax = 3, 6
        curves = [np.concatenate([[0], np.cumsum(rng.integers(0, 9, size=Smax))]) for _ in range(L)]
        for total in range(0, L * Smax + 1, 2):
            S, hits = allocate_slots(curves, total)
            assert sum(S) == total and hits == sum(int(curves[l][S[l]]) for l in range(L))
            best = max(sum(int(curves[l][s[l]]) for l in range(L))
                       for s in itertools.product(range(Smax + 1), repeat=L) if sum(s) == total)
            assert hits == best


def test_allocate_slots_respects_bounds():
    curves = [np.arange(9) * 3, np.arange(9), np.arange(9) * 2]
    S, _ = allocate_slots(curves, 12, s_min=2, s_max=6)
    assert S == [6, 2, 4]
    with pytest.raises(ValueError):
        allocate_slots(curves, 30, s_min=2, s_max=6)


def test_hybrid_curve_end_points():
    rng = np.random.default_rng(8)
    E, k, S = 14, 2, 6
    us = _one_row_trace(rng, E, k, 600, 0.25)
    h = hybrid_curve(us, E, S)
    assert h[0] == lru_hits_by_simulation(us, E, S)                           # no pins: plain LRU
    assert h[S] == round(static_pin_hit_rate(us, E, S) * sum(len(u) for u in us))   # all pinned: static pin


def test_token_model_reproduces_the_page():
    g = json.load(open(GOLD))
    for c in g["cases"]:
        misses = g["top_k"] * (1.0 - c["hit_rate"])
        r = token_rate(g["n_layers"], g["t_hit_ms"] * 1e3, misses, g["t_miss_ms"] * 1e3, g["t_other_ms"])
        assert abs(r - c["tok_per_s_about"]) < 1.0, (c, r)

"""Hindsight static pin, the comparator the pages replay against LRU (test infrastructure).

Page "GB300 GLM 5.3 Testing", sections on the September 13 verdict and "Expert
allocation vs a cache": a hindsight-optimal static pin of the S experts a layer
uses most, compared with LRU at the same slot budget.  For a fixed pinned set the
hit count is the sum over steps of |U_t intersect pin|, which is maximised by
the S experts that appear in the most steps (ties: lower expert id).
"""
import numpy as np


def _step_unique_counts(unique_sets, n_experts: int) -> np.ndarray:
    counts = np.zeros(n_experts, dtype=np.int64)
    for u in unique_sets:
        for e in set(u):
            counts[e] += 1
    return counts


def static_pin(unique_sets, n_experts: int, n_slots: int):
    counts = _step_unique_counts(unique_sets, n_experts)
    order = sorted(range(n_experts), key=lambda e: (-counts[e], e))
    return sorted(order[:n_slots])


def static_pin_hit_rate(unique_sets, n_experts: int, n_slots: int) -> float:
    pin = set(static_pin(unique_sets, n_experts, n_slots))
    tot = sum(len(set(u)) for u in unique_sets)
    hits = sum(len(set(u) & pin) for u in unique_sets)
    return hits / tot if tot else 0.0

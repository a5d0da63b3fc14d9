"""The pages' invariant on the oracle: the cached layer's output equals the
all-resident layer's output bit for bit under churn; plus negative controls."""
import numpy as np
import pytest

from oracle import OracleLayer
from oracle.lru import SlotState
from synth import CONFIGS, activations, expert_blobs, global_scales, routing_trace


def _tiny_layer(gs_mode="unit", S=None):
    cfg = CONFIGS["tiny"]
    backing = expert_blobs(cfg, 0)
    gs = global_scales(cfg, 0, gs_mode)
    lay = OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, S or cfg.slots,
                      lambda e: backing[e], gs)
    return cfg, lay, backing


@pytest.mark.parametrize("gs_mode", ["unit", "uniform"])
def test_cached_equals_all_resident_under_churn(gs_mode):
    cfg, lay, _ = _tiny_layer(gs_mode)
    logits, rows = routing_trace(cfg, 0)
    misses = 0
    for t in range(cfg.steps):
        x = activations(cfg, 0, t, int(rows[t]))
        y, rec, ids, w = lay.decode(logits[t, :rows[t]], x)
        ref = lay.all_resident_output(logits[t, :rows[t]], x)
        assert np.array_equal(y, ref), t
        misses += len(rec.events)
        lay.state.check_invariants()
    assert misses > cfg.slots            # the run churns: more fills than slots
    assert lay.state.counters.evictions > 0


def test_corrupt_slot_byte_breaks_the_invariant():
    cfg, lay, backing = _tiny_layer()
    logits, rows = routing_trace(cfg, 0)
    for t in range(8):
        lay.decode(logits[t, :1], activations(cfg, 0, t, 1))
    e = next(e for e in range(cfg.n_experts) if lay.state.e2s[e] >= 0)
    lay.slot_bytes[lay.state.e2s[e]][5] ^= 0x11          # a resident copy goes stale
    z = np.full((1, cfg.n_experts), -5.0, dtype=np.float32)
    z[0, e] = 5.0
    x = activations(cfg, 0, 99, 1)
    y, rec, _, _ = lay.decode(z, x)
    assert rec.hit[rec.uniques.index(e)]
    assert not np.array_equal(y, lay.all_resident_output(z, x))


class _WrongVictim(SlotState):
    """Mutant: evicts the most recently used candidate."""

    def _victim_order(self, cands):
        return sorted(cands, key=lambda s: (-self.key[s], s))


def test_wrong_victim_order_is_detected():
    cfg = CONFIGS["tiny"]
    logits, rows = routing_trace(cfg, 0)
    from oracle import route
    good, bad = SlotState(16, 8, 2), _WrongVictim(16, 8, 2)
    diverged = False
    for t in range(cfg.steps):
        ids, _ = route(logits[t, :1], 2)
        if good.step(ids).events != bad.step(ids).events:
            diverged = True
            break
    assert diverged

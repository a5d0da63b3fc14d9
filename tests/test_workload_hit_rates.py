"""Oracle-only report on the synthetic routing: LRU vs hindsight static pin at the
workloads' slot budgets (the comparison the pages replay on their frozen trace,
page "GB300 GLM 5.3 Testing", September 13 verdict).  The magnitudes are not
pinned to the pages (their traces are not available); the checks are orderings
that hold for any trace: more slots never lose hits, and the static pin is the
best fixed set."""
import numpy as np

from oracle import route, static_pin_hit_rate
from oracle.lru import SlotState
from synth import CONFIGS, routing_trace


def _lru_and_pin(cfg, layer, steps, S):
    logits, rows = routing_trace(cfg, layer, steps=steps)
    st = SlotState(cfg.n_experts, S, cfg.top_k)
    us = []
    for t in range(steps):
        ids, _ = route(logits[t, :rows[t]], cfg.top_k)
        rec = st.step(ids)
        us.append(rec.uniques)
    c = st.counters
    return c.hits / c.lookups, static_pin_hit_rate(us, cfg.n_experts, S), us


def test_glm_layer_lru_vs_static_pin():
    cfg = CONFIGS["glm"]
    lru, pin, _ = _lru_and_pin(cfg, 0, cfg.steps, cfg.slots)
    print("GLM layer, 300 steps, S=128: LRU %.4f, static pin %.4f" % (lru, pin))
    assert 0.5 < lru < 1.0 and 0.5 < pin < 1.0
    lru_small, pin_small, _ = _lru_and_pin(cfg, 0, cfg.steps, 32)
    assert lru_small <= lru and pin_small <= pin


def test_flash_layers_lru_vs_static_pin():
    cfg = CONFIGS["flash"]
    rates = [_lru_and_pin(cfg, l, 256, cfg.slots)[:2] for l in range(3)]
    lru = float(np.mean([r[0] for r in rates]))
    pin = float(np.mean([r[1] for r in rates]))
    print("Flash layers 0-2, 256 steps, M=8, S=54: LRU %.4f, static pin %.4f" % (lru, pin))
    assert 0.2 < lru < 1.0 and 0.2 < pin < 1.0

"""One cached MoE layer: routing, slot bookkeeping, miss fills and the expert math (test infrastructure).

Pages: the miss handler copies the missing expert's weight row and scale row
into the LRU victim slot before the expert launch, and the expert launch then
reads the same bytes it would read if every expert were resident -- only the
index changes (page "GLM 5.3 Testing: HBM Expert Allocation", section "What the
slot cache is").  A step with more than 16 rows reads the backing store
directly.  The cached layer's output therefore equals the all-resident layer's
output bit for bit under churn (same page, section "The build").
"""
import numpy as np

from .blob import blob_size
from .expert import layer_output
from .lru import SlotState, BYPASS_ROWS
from .routing import route


class OracleLayer:
    def __init__(self, H, I, E, k, S, backing, gs, keep_slot_bytes=True):
        """backing(e) -> uint8 blob of expert e (the pinned host copy)."""
        self.H, self.I, self.E, self.k, self.S = H, I, E, k, S
        self.backing = backing
        self.gs = np.asarray(gs, dtype=np.float32)
        self.state = SlotState(E, S, k, blob_size(H, I))
        self.keep = keep_slot_bytes
        self.slot_bytes = [None] * S

    def preload(self):
        self.state.preload()
        if self.keep:
            for s in range(self.S):
                self.slot_bytes[s] = np.array(self.backing(s), dtype=np.uint8, copy=True)

    def _slot_fetch(self, e):
        s = self.state.e2s[e]
        if s < 0 or self.slot_bytes[s] is None:
            raise RuntimeError("expert %d is not resident" % e)
        return self.slot_bytes[s]

    def decode(self, logits, x_bits, with_output=True):
        """One step.  Returns (y or None, record, ids, weights)."""
        logits = np.asarray(logits, dtype=np.float32)
        ids, w = route(logits, self.k)
        rec = self.state.step(ids)
        if not rec.bypass and self.keep:
            for e, s, _old in rec.events:
                self.slot_bytes[s] = np.array(self.backing(e), dtype=np.uint8, copy=True)
        y = None
        if with_output:
            if rec.bypass or not self.keep:
                fetch = self.backing
            else:
                fetch = self._slot_fetch
            y = layer_output(ids, w, x_bits, fetch, self.gs, self.H, self.I)
        return y, rec, ids, w

    def all_resident_output(self, logits, x_bits):
        """The same step with every expert read from the backing store."""
        ids, w = route(np.asarray(logits, dtype=np.float32), self.k)
        return layer_output(ids, w, x_bits, self.backing, self.gs, self.H, self.I)

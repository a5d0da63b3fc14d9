"""SlotCache: owns the torch device buffers a libslotcache handle is bound to.

PyTorch supplies device memory and streams only; every step of the decode
path runs in the library's HIP kernels (moe_layer_decode).
"""
import ctypes

import numpy as np

from . import binding as B


class SlotCache:
    """prefill_stage: experts a prefill chunk (more than 16 rows) stages into
    HBM per group before computing them (0: read them in place from the
    pinned host store).  64 is the group size of the pages' prefill-groups
    knob; the staging area costs prefill_stage * blob_bytes of workspace.

    overlap_fill: on one-row steps, compute the resident experts' gate/up
    while the misses are copied (SC_FLAG_OVERLAP_FILL); same output bits."""

    def __init__(self, n_layers, hidden, inter, n_experts, top_k, slots, max_rows,
                 n_banks=1, event_capacity=0, device="cuda", batch_invariant=False, prefill_stage=64,
                 overlap_fill=False):
        import torch

        self.torch = torch
        if isinstance(slots, int):
            slots = [slots] * n_layers
        self.slots = [int(s) for s in slots]
        self.n_layers, self.hidden, self.inter = n_layers, hidden, inter
        self.n_experts, self.top_k, self.max_rows, self.n_banks = n_experts, top_k, max_rows, n_banks
        self.cfg = B.make_config(n_layers, hidden, inter, n_experts, top_k, self.slots, max_rows,
                                 n_banks, event_capacity,
                                 flags=((B.SC_FLAG_BATCH_INVARIANT if batch_invariant else 0)
                                        | (B.SC_FLAG_OVERLAP_FILL if overlap_fill else 0)),
                                 prefill_stage=prefill_stage)
        self.sizes = B.slotcache_query_sizes(self.cfg)
        self.blob_bytes = self.sizes.blob_bytes
        self.device = torch.device(device)
        u8 = torch.uint8
        self.pool = torch.empty(max(self.sizes.slot_pool_bytes, 256), dtype=u8, device=self.device)
        self.state = torch.empty(self.sizes.state_bytes, dtype=u8, device=self.device)
        self.workspace = torch.empty(self.sizes.workspace_bytes, dtype=u8, device=self.device)
        torch.cuda.synchronize(self.device)
        self.h = B.slotcache_init(self.cfg, self.pool.data_ptr(), self.state.data_ptr(),
                                  self.workspace.data_ptr())

    # ---- backing store -----------------------------------------------------
    def backing(self, bank):
        """numpy uint8 view [E, B_e] of the pinned host bank."""
        ptr, n = B.slotcache_backing(self.h, bank)
        arr = np.ctypeslib.as_array((ctypes.c_uint8 * n).from_address(ptr))
        return arr.reshape(self.n_experts, self.blob_bytes)

    def set_global_scales(self, bank, gs):
        gs = np.ascontiguousarray(gs, dtype=np.float32).reshape(self.n_experts, 2)
        B.slotcache_set_global_scales(self.h, bank, gs.ctypes.data)

    def preload(self, layer):
        B.slotcache_preload(self.h, layer)

    def pin(self, layer, experts):
        """Pin `experts` to the first len(experts) slots of `layer` (hybrid policy)."""
        arr = np.ascontiguousarray(experts, dtype=np.int32)
        B.slotcache_pin(self.h, layer, arr.ctypes.data if arr.size else None, int(arr.size))

    # ---- the step ------------------------------------------------------------
    def decode(self, layer, logits, x, y, stream=None, events=None):
        """logits fp32 [M, E], x bf16 bits (int16/uint16/bfloat16) [M, H], y fp32 [M, H]; all on device."""
        M = int(logits.shape[0])
        if stream is None:
            stream = self.torch.cuda.current_stream(self.device)
        s = ctypes.c_void_p(stream.cuda_stream)
        if events is None:
            B.moe_layer_decode(self.h, layer, logits.data_ptr(), x.data_ptr(), M, y.data_ptr(), s)
        else:
            handles = [ev.cuda_event for ev in events]
            if len(handles) != B.SC_N_EVENTS or not all(handles):
                raise ValueError("need %d recorded (created) events" % B.SC_N_EVENTS)
            arr = (ctypes.c_void_p * B.SC_N_EVENTS)(*handles)
            B.moe_layer_decode_ev(self.h, layer, logits.data_ptr(), x.data_ptr(), M, y.data_ptr(), s,
                                  ctypes.cast(arr, ctypes.c_void_p))

    # ---- readback --------------------------------------------------------------
    def kernel_spans(self):
        """Execution spans (us) of the kernels of the last timed step (decode with events)."""
        return B.slotcache_read_kernel_spans(self.h)

    def stats(self, layer):
        st = B.slotcache_stats(self.h, layer)
        return {name: int(getattr(st, name)) for name, _ in B.sc_stats._fields_ if name != "reserved"}

    def read_state(self, layer):
        S = self.slots[layer]
        e2s = np.empty(self.n_experts, np.int32)
        s2e = np.empty(S, np.int32)
        key = np.empty(S, np.int64)
        step = np.empty(1, np.int64)
        B.slotcache_read_state(self.h, layer, e2s.ctypes.data, s2e.ctypes.data, key.ctypes.data,
                               step.ctypes.data)
        return e2s, s2e, key, int(step[0])

    def write_state(self, layer, e2s, s2e, key, step):
        e2s = np.ascontiguousarray(e2s, np.int32)
        s2e = np.ascontiguousarray(s2e, np.int32)
        key = np.ascontiguousarray(key, np.int64)
        B.slotcache_write_state(self.h, layer, e2s.ctypes.data, s2e.ctypes.data, key.ctypes.data, int(step))

    def read_events(self, layer, cap=1 << 16):
        buf = (B.sc_event * cap)()
        n, total = B.slotcache_read_events(self.h, layer, ctypes.cast(buf, ctypes.c_void_p), cap)
        return [(int(buf[i].step), int(buf[i].expert), int(buf[i].slot), int(buf[i].evicted))
                for i in range(n)], total

    def read_routing(self):
        P = self.max_rows * self.top_k
        ids = np.empty(P, np.int32)
        w = np.empty(P, np.float32)
        M, byp = B.slotcache_read_routing(self.h, ids.ctypes.data, w.ctypes.data)
        return ids[:M * self.top_k].reshape(M, self.top_k), w[:M * self.top_k].reshape(M, self.top_k), bool(byp)

    def close(self):
        if getattr(self, "h", None) is not None:
            B.slotcache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

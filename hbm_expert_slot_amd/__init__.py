"""hbm_expert_slot_amd: the expert-slot MoE decode step for MI355X (gfx950).

libslotcache.so (HIP, built in-tree by hbm_expert_slot_amd.build) does all of
the work; `binding` is its ctypes binding and `SlotCache` binds torch device
buffers to a handle.
"""
from . import binding
from .binding import SlotCacheError

__all__ = ["binding", "SlotCacheError", "SlotCache"]


def __getattr__(name):
    if name == "SlotCache":
        from .cache import SlotCache
        return SlotCache
    raise AttributeError(name)

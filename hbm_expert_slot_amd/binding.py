"""ctypes binding of libslotcache (include/slotcache.h): argument marshalling only.

Every function keeps the C name and raises SlotCacheError on a non-OK status.
The library is loaded from this package directory; if it is missing the
import of a call fails loudly -- there is no fallback implementation.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libslotcache.so")

SC_OK = 0
SC_E_ARG = -1
SC_E_HOST_OOM = -2
SC_E_HIP = -3
SC_E_STATE = -4
SC_E_DEVICE = -5
SC_E_UNSUPPORTED = -6
SC_BYPASS_ROWS = 16
SC_FLAG_BATCH_INVARIANT = 1
SC_FLAG_OVERLAP_FILL = 2
SC_MFMA_MIN_ROWS_GATEUP = 5
SC_MFMA_MIN_ROWS_DOWN = 5
SC_N_KERNELS = 5
SC_N_EVENTS = 2 * SC_N_KERNELS
SC_STATIC_SCRATCH_BYTES = 16777216

EXPORTED = (
    "slotcache_query_sizes", "slotcache_init", "slotcache_backing", "slotcache_set_global_scales",
    "slotcache_preload", "moe_layer_decode", "moe_layer_decode_ev", "slotcache_stats",
    "slotcache_read_state", "slotcache_write_state", "slotcache_read_events",
    "slotcache_read_routing", "slotcache_read_kernel_spans", "slotcache_pin", "slotcache_last_error",
    "slotcache_destroy", "moe_layer_decode_static",
)


class SlotCacheError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("slotcache status %d: %s" % (status, message))
        self.status = status


class sc_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("slots_per_layer", ctypes.POINTER(ctypes.c_int32)), ("max_rows", ctypes.c_int32),
        ("n_banks", ctypes.c_int32), ("event_capacity", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("prefill_stage", ctypes.c_int32),
    ]


class sc_sizes(ctypes.Structure):
    _fields_ = [
        ("blob_bytes", ctypes.c_size_t), ("slot_pool_bytes", ctypes.c_size_t),
        ("state_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
        ("backing_bytes_per_bank", ctypes.c_size_t),
    ]


class sc_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "steps", "bypass_steps", "picks", "lookups", "hits", "misses", "evictions",
        "bytes_filled", "bypass_bytes")] + [("device_error", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class sc_event(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("expert", ctypes.c_int32), ("slot", ctypes.c_int32),
                ("evicted", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libslotcache.so is not built; run python -m hbm_expert_slot_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "slotcache_query_sizes": [ctypes.POINTER(sc_config), ctypes.POINTER(sc_sizes)],
            "slotcache_init": [ctypes.POINTER(sc_config), P, P, P, ctypes.POINTER(P)],
            "slotcache_backing": [P, i32, ctypes.POINTER(P), ctypes.POINTER(sz)],
            "slotcache_set_global_scales": [P, i32, P],
            "slotcache_preload": [P, i32],
            "moe_layer_decode": [P, i32, P, P, i32, P, P],
            "moe_layer_decode_ev": [P, i32, P, P, i32, P, P, P],
            "moe_layer_decode_static": [P, i32, P, P, i32, P, P],
            "slotcache_stats": [P, i32, ctypes.POINTER(sc_stats)],
            "slotcache_read_state": [P, i32, P, P, P, P],
            "slotcache_write_state": [P, i32, P, P, P, i64],
            "slotcache_read_events": [P, i32, P, sz, ctypes.POINTER(sz), ctypes.POINTER(ctypes.c_uint64)],
            "slotcache_read_routing": [P, P, P, ctypes.POINTER(i32), ctypes.POINTER(i32)],
            "slotcache_read_kernel_spans": [P, ctypes.POINTER(ctypes.c_double)],
            "slotcache_pin": [P, i32, P, i32],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.slotcache_last_error.argtypes = []
        L.slotcache_last_error.restype = ctypes.c_char_p
        L.slotcache_destroy.argtypes = [P]
        L.slotcache_destroy.restype = None
        _lib = L
    return _lib


def _check(st):
    if st != SC_OK:
        raise SlotCacheError(st, lib().slotcache_last_error().decode())


def make_config(n_layers, hidden, inter, n_experts, top_k, slots_per_layer, max_rows,
                n_banks=1, event_capacity=0, flags=0, prefill_stage=0):
    arr = (ctypes.c_int32 * n_layers)(*[int(s) for s in slots_per_layer])
    cfg = sc_config(n_layers, hidden, inter, n_experts, top_k,
                    ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), max_rows, n_banks,
                    event_capacity, flags, prefill_stage)
    cfg._keep = arr
    return cfg


def slotcache_query_sizes(cfg):
    out = sc_sizes()
    _check(lib().slotcache_query_sizes(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def slotcache_init(cfg, d_slot_pool, d_state, d_workspace):
    h = ctypes.c_void_p()
    _check(lib().slotcache_init(ctypes.byref(cfg), d_slot_pool, d_state, d_workspace, ctypes.byref(h)))
    return h


def slotcache_backing(h, bank):
    p, n = ctypes.c_void_p(), ctypes.c_size_t()
    _check(lib().slotcache_backing(h, bank, ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value


def slotcache_set_global_scales(h, bank, h_gs_ptr):
    _check(lib().slotcache_set_global_scales(h, bank, h_gs_ptr))


def slotcache_preload(h, layer):
    _check(lib().slotcache_preload(h, layer))


def moe_layer_decode(h, layer, d_logits, d_x, M, d_y, stream):
    _check(lib().moe_layer_decode(h, layer, d_logits, d_x, M, d_y, stream))


def moe_layer_decode_static(h, layer, d_logits, d_x, M, d_y, stream):
    _check(lib().moe_layer_decode_static(h, layer, d_logits, d_x, M, d_y, stream))


def moe_layer_decode_ev(h, layer, d_logits, d_x, M, d_y, stream, events):
    _check(lib().moe_layer_decode_ev(h, layer, d_logits, d_x, M, d_y, stream, events))


def slotcache_stats(h, layer):
    out = sc_stats()
    _check(lib().slotcache_stats(h, layer, ctypes.byref(out)))
    return out


def slotcache_read_state(h, layer, e2s_ptr, s2e_ptr, key_ptr, step_ptr):
    _check(lib().slotcache_read_state(h, layer, e2s_ptr, s2e_ptr, key_ptr, step_ptr))


def slotcache_write_state(h, layer, e2s_ptr, s2e_ptr, key_ptr, step):
    _check(lib().slotcache_write_state(h, layer, e2s_ptr, s2e_ptr, key_ptr, step))


def slotcache_read_events(h, layer, buf_ptr, cap):
    n, tot = ctypes.c_size_t(), ctypes.c_uint64()
    _check(lib().slotcache_read_events(h, layer, buf_ptr, cap, ctypes.byref(n), ctypes.byref(tot)))
    return n.value, tot.value


def slotcache_read_routing(h, ids_ptr, w_ptr):
    M, byp = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().slotcache_read_routing(h, ids_ptr, w_ptr, ctypes.byref(M), ctypes.byref(byp)))
    return M.value, byp.value


def slotcache_pin(h, layer, experts_ptr, n):
    _check(lib().slotcache_pin(h, layer, experts_ptr, n))


def slotcache_read_kernel_spans(h):
    """Execution spans (us) of the kernels of the last timed step."""
    out = (ctypes.c_double * SC_N_KERNELS)()
    _check(lib().slotcache_read_kernel_spans(h, out))
    return list(out)


def slotcache_last_error():
    return lib().slotcache_last_error().decode()


def slotcache_destroy(h):
    lib().slotcache_destroy(h)

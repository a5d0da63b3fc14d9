"""The C-ABI library loads and exports every declared entry point; host-side
configuration checks (no GPU needed: these calls do not touch the device)."""
import os
import re

import pytest

from hbm_expert_slot_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            src = open(os.path.join(inc, f)).read()
            names |= set(re.findall(r"^SC_API\s+[\w\s\*]+?\b(\w+)\s*\(", src, re.M))
    return names


def test_every_declared_symbol_is_exported():
    decl = _declared()
    assert len(decl) >= 14
    L = B.lib()
    for n in decl:
        assert hasattr(L, n), n
    assert decl == set(B.EXPORTED)


def _cfg(**kw):
    d = dict(n_layers=1, hidden=6144, inter=2048, n_experts=256, top_k=8, slots_per_layer=[128],
             max_rows=64, n_banks=1)
    d.update(kw)
    return B.make_config(**d)


def test_sizes_for_the_glm_layer():
    s = B.slotcache_query_sizes(_cfg())
    assert s.blob_bytes == 21_233_664
    assert s.slot_pool_bytes == 128 * 21_233_664
    assert s.backing_bytes_per_bank == 256 * 21_233_664     # exact size, no rounding
    # workspace holds h [P, I] and per-pick down outputs [P, H] in fp32
    assert s.workspace_bytes >= 64 * 8 * (2048 + 6144) * 4
    s2 = B.slotcache_query_sizes(_cfg(n_layers=3, slots_per_layer=[8, 16, 256], n_banks=2))
    assert s2.slot_pool_bytes == (8 + 16 + 256) * 21_233_664


def test_prefill_staging_area_is_part_of_the_workspace():
    """G staged blobs are added to the workspace when prefill chunks (more than 16 rows) can occur."""
    base = B.slotcache_query_sizes(_cfg(prefill_stage=0)).workspace_bytes
    for G in (1, 64, 1024):
        ws = B.slotcache_query_sizes(_cfg(prefill_stage=G)).workspace_bytes
        assert G * 21_233_664 <= ws - base < G * 21_233_664 + 256
    # no prefill chunk can occur at max_rows <= 16: no staging area
    assert (B.slotcache_query_sizes(_cfg(max_rows=16, prefill_stage=64)).workspace_bytes
            == B.slotcache_query_sizes(_cfg(max_rows=16, prefill_stage=0)).workspace_bytes)


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=0), B.SC_E_ARG),
    (dict(top_k=33), B.SC_E_ARG),
    (dict(n_experts=4), B.SC_E_ARG),
    (dict(slots_per_layer=[0]), B.SC_E_ARG),
    (dict(slots_per_layer=[257]), B.SC_E_ARG),
    (dict(max_rows=0), B.SC_E_ARG),
    (dict(max_rows=257), B.SC_E_ARG),
    (dict(max_rows=256, top_k=16), B.SC_E_ARG),
    (dict(n_banks=2), B.SC_E_ARG),
    (dict(hidden=6000), B.SC_E_ARG),
    (dict(hidden=3072), B.SC_E_UNSUPPORTED),
    (dict(inter=64), B.SC_E_UNSUPPORTED),
    (dict(flags=4), B.SC_E_ARG),
    (dict(prefill_stage=-1), B.SC_E_ARG),
    (dict(prefill_stage=1025), B.SC_E_ARG),
])
def test_invalid_configs_are_rejected(kw, code):
    with pytest.raises(B.SlotCacheError) as ei:
        B.slotcache_query_sizes(_cfg(**kw))
    assert ei.value.status == code
    assert B.slotcache_last_error()


def test_binding_constants_match_the_header():
    """Every integer #define of include/slotcache.h that the binding mirrors has the same value."""
    src = open(os.path.join(ROOT, "include", "slotcache.h")).read()
    defs = dict(re.findall(r"^#define\s+(SC_\w+)\s+(\d+)u?\s*$", src, re.M))
    mirrored = [n for n in defs if hasattr(B, n)]
    assert {"SC_BYPASS_ROWS", "SC_FLAG_BATCH_INVARIANT", "SC_MFMA_MIN_ROWS_GATEUP",
            "SC_MFMA_MIN_ROWS_DOWN", "SC_N_KERNELS"} <= set(mirrored)
    for n in mirrored:
        assert getattr(B, n) == int(defs[n]), n


def test_defined_flags_are_accepted_and_need_no_memory():
    """Both defined flags, alone and together, pass the configuration checks
    and leave every buffer size unchanged (the overlapped fill and the
    batch-invariant rows reuse the plain path's buffers)."""
    base = B.slotcache_query_sizes(_cfg())
    for flags in (B.SC_FLAG_BATCH_INVARIANT, B.SC_FLAG_OVERLAP_FILL,
                  B.SC_FLAG_BATCH_INVARIANT | B.SC_FLAG_OVERLAP_FILL):
        s = B.slotcache_query_sizes(_cfg(flags=flags))
        for f in ("blob_bytes", "slot_pool_bytes", "state_bytes", "workspace_bytes", "backing_bytes_per_bank"):
            assert getattr(s, f) == getattr(base, f), (flags, f)

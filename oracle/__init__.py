"""CPU oracle of the expert-slot MoE decode step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct reference written from the pages
("GLM 5.3 Testing: HBM Expert Allocation", sections "What the slot cache is" and
"The build, measured on a synthetic GLM-shaped layer"; "GB300 GLM 5.3 Testing",
section "Expert allocation vs a cache"; "TensorFold GLM-5.3 explained") and from
the OCP FP4/FP8 format definitions.  It works in float64 and Python integers.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import it.  The HIP library never imports, links or calls anything here, and
nothing here imports the library: the two share only the seeded input
generators in synth/.

Parity pins: every function is pinned by tests under tests/test_oracle_*.py
(exhaustive codec checks against torch's float8/bfloat16 decoders and the OCP
tables, brute-force routing and LRU replays, exact rational expert math, closed
forms and invariants).  No function here is "parity unpinned".
"""
from .formats import E2M1_TABLE, e2m1_value, e4m3_value, bf16_value, decode_e2m1, decode_e4m3, decode_bf16
from .blob import part_layout, blob_size, dequant_expert
from .routing import route
from .lru import SlotState, StepRecord, Counters
from .static_pin import static_pin, static_pin_hit_rate
from .policy import lru_hit_curve, lru_hits_by_simulation, allocate_slots, hybrid_curve, token_rate
from .expert import silu, expert_apply, layer_output
from .layer import OracleLayer

__all__ = [
    "E2M1_TABLE", "e2m1_value", "e4m3_value", "bf16_value", "decode_e2m1", "decode_e4m3",
    "decode_bf16", "part_layout", "blob_size", "dequant_expert", "route", "SlotState",
    "StepRecord", "Counters", "static_pin", "static_pin_hit_rate", "lru_hit_curve", "lru_hits_by_simulation",
    "allocate_slots", "hybrid_curve", "token_rate", "silu", "expert_apply",
    "layer_output", "OracleLayer",
]

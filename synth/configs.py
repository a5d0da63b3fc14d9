"""Workload table: the layer shapes and run lengths of the five synthetic workloads.

Shapes follow the pages: the GLM-5.3 layer ("GLM 5.3 Testing: HBM Expert
Allocation", section "What the slot cache is": 256 routed experts per layer,
top-8, 21.234 MB per expert row incl. block scales) and the GLM-5.3-Flash layer
("glm53 - GLM-5.3-Flash (NVFP4)", section "How it fits": 42 MoE layers, top-8 of
288, about 13.5 MiB per expert).
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    slots: int
    rows: int            # rows per step (the largest, when the schedule varies)
    steps: int
    n_layers: int = 1
    routing: str = "zipf"   # "normal" (i.i.d. N(0,1) logits) or "zipf"
    drafted: bool = False   # rows 1..M-1 share picks with row 0
    schedule: str = "fixed"  # "fixed" or "draft_verify_prefill"
    seed: int = 0
    description: str = ""


CONFIGS = {
    "tiny": WorkloadConfig(
        name="tiny", hidden=256, inter=128, n_experts=16, top_k=2, slots=8, rows=1,
        steps=64, routing="normal", seed=11,
        description="tiny MoE layer: H256 I128, 16 experts, top-2, 8 slots, M=1, 64 steps"),
    "glm": WorkloadConfig(
        name="glm", hidden=6144, inter=2048, n_experts=256, top_k=8, slots=128, rows=1,
        steps=300, routing="zipf", seed=22,
        description="GLM-shaped MoE layer: H6144 I2048, 256 experts, top-8, 128 slots, M=1, 300 steps"),
    "glm_draft": WorkloadConfig(
        name="glm_draft", hidden=6144, inter=2048, n_experts=256, top_k=8, slots=128, rows=64,
        steps=200, routing="zipf", drafted=True, schedule="draft_verify_prefill", seed=33,
        description="GLM layer, drafted rounds: M=4 (1 token + 3 drafts), M=16 verify, M=64 prefill bypass; 200 steps"),
    "glm_stack": WorkloadConfig(
        name="glm_stack", hidden=6144, inter=2048, n_experts=256, top_k=8, slots=128, rows=1,
        steps=512, n_layers=75, routing="zipf", seed=44,
        description="75-layer GLM-shaped MoE stack, 128 slots per layer, M=1, 512 steps"),
    "flash": WorkloadConfig(
        name="flash", hidden=4096, inter=2048, n_experts=288, top_k=8, slots=54, rows=8,
        steps=512, n_layers=42, routing="zipf", seed=55,
        description="Flash-shaped stack: 42 layers H4096 I2048, 288 experts, top-8, 54 slots, M=8, 512 steps"),
}


def rows_at_step(cfg: WorkloadConfig, t: int) -> int:
    """Rows M at step t.  The drafted workload mixes M=4 draft rounds, M=16 verify
    batches (every 10th step) and M=64 prefill chunks (every 50th step)."""
    if cfg.schedule == "draft_verify_prefill":
        if t % 50 == 49:
            return 64
        if t % 10 == 9:
            return 16
        return 4
    return cfg.rows


def blob_parts(hidden: int, inter: int) -> Tuple[Tuple[str, int], ...]:
    """Byte sizes of the four parts of one expert blob, in blob order."""
    return (
        ("w13_codes", 2 * inter * hidden // 2),
        ("w13_scales", 2 * inter * hidden // 16),
        ("w2_codes", hidden * inter // 2),
        ("w2_scales", hidden * inter // 16),
    )


def blob_bytes(hidden: int, inter: int) -> int:
    return sum(n for _, n in blob_parts(hidden, inter))

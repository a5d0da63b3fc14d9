"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package holds input synthesis only (random expert blobs, router logits,
activations, and the workload table).  It computes none of the decode step:
no routing, no slot bookkeeping, no dequantisation, no expert products.
"""
from .configs import CONFIGS, WorkloadConfig, blob_parts, blob_bytes, rows_at_step
from .gen import (
    bf16_bits_from_f32,
    e4m3_bits_rne,
    expert_blob,
    expert_blobs,
    probe_blob,
    probe_column,
    global_scales,
    activations,
    routing_trace,
)

__all__ = [
    "CONFIGS", "WorkloadConfig", "blob_parts", "blob_bytes", "rows_at_step",
    "bf16_bits_from_f32", "e4m3_bits_rne", "expert_blob", "expert_blobs",
    "global_scales", "activations", "routing_trace", "probe_blob", "probe_column",
]

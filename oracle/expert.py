"""Routed expert products and the weighted top-k combine, in float64 (test infrastructure).

Pages: each routed expert is three NVFP4 matrices (page "TensorFold GLM-5.3
explained", expert sizes paragraph), stored as the fused gate/up weight "w13"
and the down weight "w2" (page "GB300 GLM 5.3 Testing", section "E1 v2"); the
routed outputs are combined in fp32 and reduced once (page "GLM 5.3 Testing:
HBM Expert Allocation", section "A correction first"; page "glm53 -
GLM-5.3-Flash (NVFP4)", prefill-groups knob).  The activation is SiLU on the
gate times the up projection (the standard gated MoE expert; the pages name
SiLU only through the workload definition).

For one row x and pick j with expert e:  h = silu(G_e x) * (U_e x),
y += w_j * (D_e h), summed over j = 0..k-1 in rank order.
"""
import numpy as np

from .blob import dequant_expert
from .formats import decode_bf16


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_apply(G, U, D, x):
    """One expert on one row: D @ (silu(G x) * (U x)); also returns h."""
    x = np.asarray(x, dtype=np.float64)
    h = silu(G @ x) * (U @ x)
    return D @ h, h


def layer_output(ids, w, x_bits, fetch, gs, H: int, I: int):
    """y [M, H] float64 for routed picks (ids, w) and bf16 rows x_bits [M, H].

    fetch(e) returns the blob bytes the step reads for expert e (a slot copy on
    the cached path, the backing store on the all-resident and bypass paths).
    gs is the [E, 2] table of fp32 global scales (w13, w2).
    """
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    x = decode_bf16(x_bits)
    M, k = ids.shape
    mats = {}
    for e in dict.fromkeys(int(v) for v in ids.reshape(-1)):
        mats[e] = dequant_expert(fetch(e), H, I, gs[e][0], gs[e][1])
    y = np.zeros((M, H), dtype=np.float64)
    for m in range(M):
        for j in range(k):
            G, U, D = mats[int(ids[m, j])]
            out, _ = expert_apply(G, U, D, x[m])
            y[m] += w[m, j] * out
    return y

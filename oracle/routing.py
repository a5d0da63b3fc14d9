"""Router top-k selection and routing weights (test infrastructure).

Pages: the router picks the top 8 of 256 experts per row before the expert
kernel runs (page "GLM 5.3 Testing: HBM Expert Allocation", section "What the
slot cache is"); router ties break by a stable expert order (page "TensorFold
GLM-5.3 explained", exact-decoding rule); routing weights by rank sum to one
(page "glm53 - GLM-5.3-Flash (NVFP4)", section "Why 25 tok/s is unreachable").

Reading where the pages are silent: select on the raw fp32 logits, ordered by
(logit descending, expert id ascending), NaN below -inf and -0 equal to +0; the
weights are the softmax over the k selected logits only, in float64.  Limits for
non-finite picks: NaN counts as -inf; if any pick is +inf the +inf picks share
the weight equally; if every pick is -inf the k picks share it equally.
"""
import math

import numpy as np


def _order_key(z: float, e: int):
    if math.isnan(z):
        return (1, 0.0, e)
    return (0, -z, e)


def route(logits, k: int):
    """logits float32 [M, E] -> (ids int64 [M, k], weights float64 [M, k])."""
    z = np.asarray(logits, dtype=np.float32)
    M, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("top_k out of range")
    ids = np.empty((M, k), dtype=np.int64)
    w = np.empty((M, k), dtype=np.float64)
    for m in range(M):
        row = [float(v) for v in z[m]]
        order = sorted(range(E), key=lambda e: _order_key(row[e], e))
        chosen = order[:k]
        ids[m] = chosen
        zs = [row[e] for e in chosen]
        zs = [-math.inf if math.isnan(v) else v for v in zs]
        n_pinf = sum(1 for v in zs if v == math.inf)
        zmax = max(zs)
        if n_pinf:
            w[m] = [1.0 / n_pinf if v == math.inf else 0.0 for v in zs]
        elif zmax == -math.inf:
            w[m] = [1.0 / k] * k
        else:
            ex = [math.exp(v - zmax) for v in zs]
            s = sum(ex)
            w[m] = [v / s for v in ex]
    return ids, w

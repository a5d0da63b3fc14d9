"""Pins of the oracle's expert math: exact rational / 50-digit evaluation on tiny shapes."""
from fractions import Fraction

import mpmath
import numpy as np

from oracle import blob, formats, layer_output, route, silu
from synth import CONFIGS, activations, expert_blob, global_scales, routing_trace

mpmath.mp.dps = 50


def _exact_step(cfg, ids, w, x_bits, blobs, gs):
    H, I = cfg.hidden, cfg.inter
    x = [Fraction(float(v)) for v in formats.decode_bf16(x_bits[0])]
    y = [mpmath.mpf(0)] * H
    for j, e in enumerate(ids[0]):
        G, U, D = blob.dequant_expert(blobs[int(e)], H, I, gs[e][0], gs[e][1])
        h = []
        for r in range(I):
            g = sum(Fraction(float(G[r, c])) * x[c] for c in range(H) if G[r, c] != 0)
            u = sum(Fraction(float(U[r, c])) * x[c] for c in range(H) if U[r, c] != 0)
            gm = mpmath.mpf(g.numerator) / g.denominator
            um = mpmath.mpf(u.numerator) / u.denominator
            h.append(gm / (1 + mpmath.exp(-gm)) * um)
        wj = mpmath.mpf(Fraction(float(w[0, j])).numerator) / Fraction(float(w[0, j])).denominator
        for r in range(H):
            acc = mpmath.mpf(0)
            for c in range(I):
                if D[r, c] != 0:
                    acc += mpmath.mpf(float(D[r, c])) * h[c]
            y[r] += wj * acc
    return np.array([float(v) for v in y])


def test_fp64_oracle_matches_exact_arithmetic():
    cfg = CONFIGS["tiny"]
    gs = global_scales(cfg, 0, "uniform")
    logits, _ = routing_trace(cfg, 0, steps=2)
    for t in range(2):
        ids, w = route(logits[t, :1], cfg.top_k)
        blobs = {int(e): expert_blob(cfg, 0, int(e)) for e in ids[0]}
        x_bits = activations(cfg, 0, t, 1)
        y = layer_output(ids, w, x_bits, lambda e: blobs[e], gs, cfg.hidden, cfg.inter)[0]
        ref = _exact_step(cfg, ids, w, x_bits, blobs, gs)
        scale = np.max(np.abs(ref))
        assert scale > 0
        assert np.max(np.abs(y - ref)) <= 1e-12 * scale


def test_silu_special_values():
    assert silu(0.0) == 0.0
    assert abs(silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert silu(-800.0) == 0.0 and silu(800.0) == 800.0
    # silu(g) + silu(-g) == g  (sigma(g) + sigma(-g) = 1)
    g = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(silu(g) - silu(-g), g, rtol=0, atol=1e-13)

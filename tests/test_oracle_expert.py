"""Pins of the oracle's expert math: exact rational / 50-digit evaluation on tiny shapes."""
from fractions import Fraction

import pytest

import mpmath
import numpy as np

from oracle import OracleLayer, blob, formats, layer_output, route, silu
from synth import CONFIGS, WorkloadConfig, activations, expert_blob, global_scales, routing_trace

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


# ---- multi-row steps --------------------------------------------------------------
# The exact evaluation below is organised differently from the oracle: it walks the
# step's unique experts, evaluates each expert once per row that picked it, and
# finds that row's weight by searching the row's picks.  An index slip in the
# oracle's row/rank loops (a row's x or weight taken from another row, a rank
# order mix-up) makes the two disagree.
MINI = WorkloadConfig("mini", hidden=64, inter=32, n_experts=8, top_k=3, slots=4, rows=6, steps=8,
                      routing="normal", seed=7)


def _exact_rows(cfg, ids, w, x_bits, blobs, gs):
    H, I = cfg.hidden, cfg.inter
    M = ids.shape[0]
    xs = [[Fraction(float(v)) for v in formats.decode_bf16(x_bits[m])] for m in range(M)]
    y = [[mpmath.mpf(0)] * H for _ in range(M)]
    uniq = sorted(set(int(e) for e in ids.reshape(-1)))
    for e in uniq:
        G, U, D = blob.dequant_expert(blobs[e], H, I, gs[e][0], gs[e][1])
        Gq = [[Fraction(float(v)) for v in row] for row in G]
        Uq = [[Fraction(float(v)) for v in row] for row in U]
        for m in range(M):
            hits = [j for j in range(ids.shape[1]) if int(ids[m, j]) == e]
            if not hits:
                continue
            assert len(hits) == 1          # top-k picks of one row are distinct experts
            wf = Fraction(float(w[m, hits[0]]))
            wm = mpmath.mpf(wf.numerator) / wf.denominator
            h = []
            for r in range(I):
                g = sum(Gq[r][c] * xs[m][c] for c in range(H))
                u = sum(Uq[r][c] * xs[m][c] for c in range(H))
                gm = mpmath.mpf(g.numerator) / g.denominator
                um = mpmath.mpf(u.numerator) / u.denominator
                h.append(gm / (1 + mpmath.exp(-gm)) * um)
            for r in range(H):
                acc = mpmath.mpf(0)
                for c in range(I):
                    acc += mpmath.mpf(float(D[r, c])) * h[c]
                y[m][r] += wm * acc
    return np.array([[float(v) for v in row] for row in y])


def _shared_pick_logits(cfg, M, seed):
    """M rows whose top-k picks overlap: two favourites shared by every row, the rest differ."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, cfg.n_experts)).astype(np.float32)
    z[:, 1] += 3.0
    z[:, 5] += 2.5
    return z


@pytest.mark.parametrize("M", [2, 3, 4])
def test_multi_row_layer_output_matches_exact_arithmetic(M):
    cfg = MINI
    gs = global_scales(cfg, 0, "uniform")
    z = _shared_pick_logits(cfg, M, 100 + M)
    ids, w = route(z, cfg.top_k)
    # the rows share experts but pick them at different ranks with different weights
    assert len(set(int(e) for e in ids.reshape(-1))) < M * cfg.top_k
    assert not np.allclose(w[0], w[1])
    blobs = {int(e): expert_blob(cfg, 0, int(e)) for e in set(ids.reshape(-1))}
    x_bits = activations(cfg, 0, M, M)
    y = layer_output(ids, w, x_bits, lambda e: blobs[e], gs, cfg.hidden, cfg.inter)
    ref = _exact_rows(cfg, ids, w, x_bits, blobs, gs)
    for m in range(M):
        scale = np.max(np.abs(ref[m]))
        assert scale > 0
        assert np.max(np.abs(y[m] - ref[m])) <= 1e-12 * scale, m
    # sensitivity: the same step with row 0's weights used for every row (a plausible
    # indexing slip) is far from the exact result
    slip = layer_output(ids, np.repeat(w[:1], M, axis=0), x_bits, lambda e: blobs[e], gs,
                        cfg.hidden, cfg.inter)
    assert np.max(np.abs(slip[1:] - ref[1:])) > 1e-6 * np.max(np.abs(ref[1:]))


def test_each_row_equals_its_one_row_step():
    """Rows do not interact: row m of an M-row step is the one-row step of row m, bit for bit."""
    cfg = CONFIGS["tiny"]
    gs = global_scales(cfg, 0, "uniform")
    for M, seed in ((3, 1), (6, 2), (17, 3)):
        z = _shared_pick_logits(cfg, M, seed)
        ids, w = route(z, cfg.top_k)
        blobs = {int(e): expert_blob(cfg, 0, int(e)) for e in set(ids.reshape(-1))}
        x_bits = activations(cfg, 0, 500 + M, M)
        y = layer_output(ids, w, x_bits, lambda e: blobs[e], gs, cfg.hidden, cfg.inter)
        for m in range(M):
            one = layer_output(ids[m:m + 1], w[m:m + 1], x_bits[m:m + 1], lambda e: blobs[e], gs,
                               cfg.hidden, cfg.inter)
            assert np.array_equal(y[m], one[0]), (M, m)


def test_bypass_step_output_matches_exact_arithmetic():
    """A step of more than 16 rows bypasses the cache and reads the backing store; its
    output is still the exact routed product of every row."""
    cfg = MINI
    gs = global_scales(cfg, 0, "unit")
    backing = {e: expert_blob(cfg, 0, e) for e in range(cfg.n_experts)}
    orc = OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, lambda e: backing[e], gs)
    M = 17
    z = _shared_pick_logits(cfg, M, 9)
    x_bits = activations(cfg, 0, 77, M)
    y, rec, ids, w = orc.decode(z, x_bits)
    assert rec.bypass
    ref = _exact_rows(cfg, ids, w, x_bits, backing, gs)
    for m in range(M):
        assert np.max(np.abs(y[m] - ref[m])) <= 1e-12 * np.max(np.abs(ref[m])), m

"""GPU parity on structured expert blobs that expose single weights.

A whole-output relative L2 of 1e-3 can hide a mistake confined to one block
scale, one K chunk or one row group: such a mistake moves a long dot product by
far less than the bar.  These tests give the layer blobs whose structure makes
the step's output show individual values, and compare those element by element
with the oracle's fp64 values (the expert products of the page "GLM 5.3
Testing: HBM Expert Allocation", section "What the slot cache is", with the
fp32 combine of its section "A correction first"):

* select_h: the down matrix is a selection matrix (row r holds 1.0 at column
  r mod I), one pick per row, unit down scale: output element r is the
  intermediate value h[r mod I] = SiLU(g) * u, so every gate/up row sum is
  checked on its own.
* one_column: every up row but one is zero, so h is zero except at one index
  c0 and the output is column c0 of the down matrix times h[c0]: every code and
  block scale of that column is checked on its own.

Layer: GLM shapes (H 6144, I 2048), 8 experts, top-1, 5 slots (misses go
through the fill; steps with more unique experts than slots read the others
from the host store), steps of 1 to 16 rows, so the one-row, shared-operand
streaming and matrix-core kernels all run.
"""
import numpy as np
import pytest

from oracle import OracleLayer, dequant_expert, expert_apply, route, silu
from synth import WorkloadConfig, activations, global_scales, probe_blob, probe_column

from gpu_util import GpuStepper, log, torch_cuda

pytestmark = pytest.mark.gpu

PROBE = WorkloadConfig("probe", hidden=6144, inter=2048, n_experts=8, top_k=1, slots=5, rows=16, steps=12,
                       routing="normal", seed=66)
ROWS = [1, 1, 2, 1, 4, 16, 3, 1, 8, 2, 16, 1]


def _logits(t, M):
    return np.random.default_rng((PROBE.seed, 7100, t)).standard_normal((M, PROBE.n_experts)).astype(np.float32)


# fp32 accumulation error of a row sum, as a multiple of the sum of its absolute terms:
# 64 roundings of 2^-24 (the streaming kernels add at most about 30 times in sequence,
# the matrix-core kernels' running sums stay far below this in practice)
ACC = 64 * 2.0 ** -24


def _h_tolerance(G, U, x, h, split):
    """Bound on |h_gpu - h|: the accumulation error of g = G x and u = U x (ACC times
    the sums of absolute terms) propagated through SiLU(g) * u (|SiLU'| <= 1.1), plus
    a few roundings of h itself, or the bf16 pair (about 2^-17 relative) that carries h
    into the matrix-core down product when `split`."""
    ax = np.abs(x)
    Ag = np.abs(G) @ ax
    Au = np.abs(U) @ ax
    g, u = G @ x, U @ x
    rel = 2.0 ** -16 if split else 1e-6
    return ACC * (1.2 * np.abs(u) * Ag + np.abs(silu(g)) * Au) + rel * np.abs(h)


def _split(M):
    from hbm_expert_slot_amd.binding import SC_MFMA_MIN_ROWS_DOWN
    return M >= SC_MFMA_MIN_ROWS_DOWN


class _Blobs:
    def __init__(self, mode, gs):
        self.mode, self.gs = mode, gs
        self.blob = {e: probe_blob(PROBE, 0, e, mode) for e in range(PROBE.n_experts)}
        self.mats = {}

    def __call__(self, e):
        return self.blob[int(e)]

    def matrices(self, e):
        if e not in self.mats:
            self.mats[e] = dequant_expert(self.blob[e], PROBE.hidden, PROBE.inter, self.gs[e][0], self.gs[e][1])
        return self.mats[e]


def _setup(mode):
    from hbm_expert_slot_amd.cache import SlotCache
    cfg = PROBE
    gs = global_scales(cfg, 0, "uniform").copy()
    if mode == "select_h":
        gs[:, 1] = 1.0            # the selection matrix must pass h through unscaled
    blobs = _Blobs(mode, gs)
    sc = SlotCache(1, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, cfg.rows)
    bk = sc.backing(0)
    for e in range(cfg.n_experts):
        bk[e] = blobs(e)
    sc.set_global_scales(0, gs)
    orc = OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, blobs, gs, keep_slot_bytes=False)
    return sc, orc, blobs


def _run(mode, check_row):
    torch_cuda()
    sc, orc, blobs = _setup(mode)
    g = GpuStepper(sc)
    worst = 0.0
    for t, M in enumerate(ROWS):
        z = _logits(t, M)
        x_bits = activations(PROBE, 0, t, M)
        log("%s: step %d, M=%d" % (mode, t, M))
        y, ids, w, byp = g.step(z, x_bits)
        _, rec, ids_o, w_o = orc.decode(z, x_bits, with_output=False)
        assert np.array_equal(ids, ids_o), t
        assert np.all(w == 1.0), t          # one pick per row: weight exactly 1
        assert byp == rec.bypass, t         # more unique experts than slots: read from the host store
        ev = g.new_events()
        assert [tuple(e[1:]) for e in ev] == rec.events, t
        x = orc_x(x_bits)
        for m in range(M):
            worst = max(worst, check_row(blobs, int(ids[m, 0]), x[m], y[m], _split(M), (t, M, m)))
    log("%s: worst error / tolerance %.3g" % (mode, worst))
    st = sc.stats(0)
    assert st["misses"] > PROBE.slots and st["bypass_steps"] > 0 and st["device_error"] == 0
    sc.close()


def orc_x(x_bits):
    from oracle import decode_bf16
    return decode_bf16(x_bits)


def test_select_h_exposes_every_intermediate_value():
    H, I = PROBE.hidden, PROBE.inter

    def check(blobs, e, x, y, split, ctx):
        G, U, D = blobs.matrices(e)
        _, h = expert_apply(G, U, D, x)
        tol = _h_tolerance(G, U, x, h, split)
        y = np.asarray(y, np.float64)
        # the three copies of h in the output row are the same bits
        for c in range(1, H // I):
            assert np.array_equal(y[c * I:(c + 1) * I], y[:I]), ctx
        err = np.abs(y[:I] - h)
        bad = np.nonzero(err > tol)[0]
        assert bad.size == 0, (ctx, "h elements off", bad[:8], err[bad[:8]], tol[bad[:8]])
        return float(np.max(err / tol))

    _run("select_h", check)


def test_one_column_exposes_every_down_weight_of_a_column():
    def check(blobs, e, x, y, split, ctx):
        G, U, D = blobs.matrices(e)
        c0 = probe_column(PROBE, e)
        _, h = expert_apply(G, U, D, x)
        assert np.count_nonzero(h) <= 1 and h[c0] != 0.0, ctx
        tol = _h_tolerance(G, U, x, h, split)[c0]
        col = D[:, c0]
        y = np.asarray(y, np.float64)
        zero = col == 0.0
        assert np.all(y[zero] == 0.0), (ctx, "nonzero output where the column is zero")
        q = y[~zero] / col[~zero]                   # each should be h[c0] as the GPU computed it
        q0 = np.median(q)
        spread = np.abs(q / q0 - 1.0)
        bad = np.nonzero(spread > 1e-6)[0]
        assert bad.size == 0, (ctx, "column elements off", np.nonzero(~zero)[0][bad[:8]], spread[bad[:8]])
        assert abs(q0 - h[c0]) <= tol, (ctx, q0, h[c0], tol)
        assert (~zero).sum() > PROBE.hidden // 2, ctx
        return max(float(np.max(spread)) / 1e-6, abs(q0 - h[c0]) / tol)

    _run("one_column", check)

"""GPU parity of the overlapped miss fill (SC_FLAG_OVERLAP_FILL): on one-row
steps the copy of the misses shares a launch with the resident experts'
gate/up products and the copied experts' gate/up runs after it.  Against the
oracle (bookkeeping bit for bit, outputs to relative L2 1e-3) and against the
same steps without the flag (outputs, slot bytes and state bit for bit)."""
import numpy as np
import pytest

from synth import CONFIGS, WorkloadConfig, activations, routing_trace

from gpu_util import GpuStepper, check_output, log, make_cache, torch_cuda
from test_gpu_parity import (Y_TOL, _check_counters, _check_slots_hold_their_experts, _check_state,
                             _check_step, _oracle_layer)

pytestmark = pytest.mark.gpu


def _shape(name):
    if name == "glm48":
        g = CONFIGS["glm"]
        return WorkloadConfig("glm48", g.hidden, g.inter, 48, g.top_k, 30, rows=17, steps=40, seed=g.seed)
    if name == "h1024_i512":
        return WorkloadConfig("h1024_i512", 1024, 512, 32, 4, 12, rows=17, steps=40, seed=71)
    if name == "tiny_s6":
        # top-2 of 16 experts in 6 slots: one-row steps miss often, four-row
        # steps can exceed the slots (bypass)
        t = CONFIGS["tiny"]
        return WorkloadConfig("tiny_s6", t.hidden, t.inter, t.n_experts, t.top_k, 6, rows=17, steps=40,
                              seed=t.seed)
    if name == "tiny_k4_pin":
        # top-4 of 16 in 6 slots, 3 of them pinned: a one-row step whose picks
        # miss every pinned expert exceeds the 3 LRU slots and bypasses
        t = CONFIGS["tiny"]
        return WorkloadConfig("tiny_k4_pin", t.hidden, t.inter, t.n_experts, 4, 6, rows=17, steps=40,
                              seed=t.seed)
    return CONFIGS["tiny"]

PINS = {"tiny_k4_pin": [10, 9, 8]}


def _logits(cfg, steps, seed):
    rng = np.random.default_rng(seed)
    zs = []
    for _ in range(steps):
        z = rng.standard_normal((17, cfg.n_experts)).astype(np.float32)
        z[:, : max(2, cfg.top_k // 2)] += 1.5      # a few favourites: hits as well as misses
        zs.append(z)
    return zs


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", ["tiny", "tiny_s6", "tiny_k4_pin", "h1024_i512", "glm48"])
def test_overlap_fill_against_the_oracle_and_the_plain_path(shape):
    """Mostly one-row steps (the overlapped path) with multi-row and prefill
    steps (the plain path) in between; every step against the oracle's
    bookkeeping and bitwise against a cache without the flag."""
    cfg = _shape(shape)
    steps = 36
    Ms = [1, 1, 1, 4, 1, 1, 2, 1, 17, 1, 1, 1]
    log("overlapped fill vs oracle and plain path: %s (H %d, I %d, E %d, k %d, S %d), %d steps"
        % (shape, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, steps))
    ov = make_cache(cfg, max_rows=17, overlap_fill=True, gs_mode="uniform")
    pl = make_cache(cfg, max_rows=17, gs_mode="uniform")
    orc = _oracle_layer(cfg, cfg.slots, gs_mode="uniform")
    zs = _logits(cfg, steps, 11)
    pins = PINS.get(shape, [])
    if pins:
        for z in zs:
            z[:, pins] += 0.75
        ov.pin(0, pins)
        pl.pin(0, pins)
        orc.state.pin(pins)
    go, gp = GpuStepper(ov), GpuStepper(pl)
    sample = None if cfg.hidden <= 1024 else {0, 1, 2, 4, 9, 13}
    worst = 0.0
    for t in range(steps):
        M = Ms[t % len(Ms)]
        z = zs[t][:M]
        x = activations(cfg, 0, t, M)
        y, ids, w, byp = go.step(z, x)
        yp, idsp, _, bypp = gp.step(z, x)
        assert np.isfinite(y).all(), t
        assert np.array_equal(y, yp), (t, M)                  # same bits as without the flag
        assert np.array_equal(ids, idsp) and byp == bypp, t
        ev = go.new_events()
        gp.new_events()
        want_y = sample is None or t in sample
        o = orc.decode(z, x, with_output=want_y)
        r = _check_step(t, (y, ids, w, byp, ev), o, None, want_y)
        if r is not None:
            worst = max(worst, r)
        _check_state(ov, 0, orc.state)
    _check_counters(ov, 0, orc.state)
    for u, v in zip(ov.read_state(0), pl.read_state(0)):
        assert np.array_equal(u, v)
    n = _check_slots_hold_their_experts(ov)
    st = ov.stats(0)
    log("%s: misses %d, bypass %d, %d occupied slots verified, worst rel L2 %.3g"
        % (shape, st["misses"], st["bypass_steps"], n, worst))
    assert st["misses"] > 0
    if shape in ("tiny_s6", "tiny_k4_pin"):
        assert st["bypass_steps"] > 0
    ov.close()
    pl.close()


def test_overlap_fill_timed_entry_point():
    """With events the shared launch and the copied experts' gate/up still
    compute the plain step; the fill and gate/up spans are those of the shared
    launch's copy and product blocks."""
    torch = torch_cuda()
    from hbm_expert_slot_amd import binding as B
    cfg = CONFIGS["tiny"]
    log("overlapped fill, timed entry point: tiny, 24 steps")
    a, b = make_cache(cfg, overlap_fill=True), make_cache(cfg, overlap_fill=True)
    logits, _ = routing_trace(cfg, 0)
    for t in range(24):
        z = torch.from_numpy(logits[t, :1]).cuda()
        x = torch.from_numpy(activations(cfg, 0, t, 1).view(np.int16)).cuda()
        ya = torch.empty((1, cfg.hidden), dtype=torch.float32, device="cuda")
        yb = torch.empty_like(ya)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(B.SC_N_EVENTS)]
        for ev in evs:
            ev.record()
        a.decode(0, z, x, ya)
        b.decode(0, z, x, yb, events=evs)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), t
        ev_ms = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(B.SC_N_KERNELS)]
        assert all(v >= 0 for v in ev_ms)
        spans = b.kernel_spans()
        assert all(0 < s_us for s_us in spans), (t, spans)
        # gate/up's stamps lie inside its events (the shared launch); the fill's
        # events are recorded around that launch
        assert spans[2] <= 1e3 * ev_ms[2] + 1.0 and spans[1] <= 1e3 * ev_ms[1] + 1.0, (t, spans, ev_ms)
    for u, v in zip(a.read_state(0), b.read_state(0)):
        assert np.array_equal(u, v)
    assert a.stats(0)["misses"] > 0
    a.close()
    b.close()


def test_overlap_fill_graph_replay_under_churn():
    """A captured one-row step with the flag, replayed with new inputs, eager
    work and synchronisations in between, against the oracle."""
    torch = torch_cuda()
    cfg = CONFIGS["tiny"]
    log("overlapped fill, graph capture + replay under churn: tiny")
    sc = make_cache(cfg, overlap_fill=True)
    orc = _oracle_layer(cfg, cfg.slots)
    logits, _ = routing_trace(cfg, 0)
    z = torch.zeros((1, cfg.n_experts), dtype=torch.float32, device="cuda")
    x = torch.zeros((1, cfg.hidden), dtype=torch.int16, device="cuda")
    y = torch.zeros((1, cfg.hidden), dtype=torch.float32, device="cuda")
    z.copy_(torch.from_numpy(logits[0, :1]))
    x.copy_(torch.from_numpy(activations(cfg, 0, 0, 1).view(np.int16)))
    sc.decode(0, z, x, y)
    orc.decode(logits[0, :1], activations(cfg, 0, 0, 1), with_output=False)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.capture_begin()
        sc.decode(0, z, x, y, stream=s)
        g.capture_end()
    torch.cuda.synchronize()
    stepper = GpuStepper(sc)
    stepper.n_events = sc.read_events(0)[1]
    for t in range(1, 40):
        xb = activations(cfg, 0, t, 1)
        z.copy_(torch.from_numpy(logits[t, :1]))
        x.copy_(torch.from_numpy(xb.view(np.int16)))
        g.replay()
        torch.cuda.synchronize()
        y_o, rec, ids_o, w_o = orc.decode(logits[t, :1], xb)
        check_output(y.cpu().numpy(), y_o, t)
        assert [tuple(e[1:]) for e in stepper.new_events()] == rec.events, t
        _check_state(sc, 0, orc.state)
        _ = (y * 2).sum().item()
    _check_counters(sc, 0, orc.state)
    assert sc.stats(0)["misses"] > 0
    sc.close()


@pytest.mark.timeout(600)
def test_overlap_fill_random_layers():
    """Twelve seeded random layers (1-40 experts, top-1..8, 1..E slots, pins
    on some, prefill staging on some), mostly one-row steps, with the flag:
    every step's bookkeeping against the oracle and outputs bitwise against
    the same layer without the flag."""
    torch_cuda()
    from test_gpu_parity import _random_layer
    rng = np.random.default_rng(4048)
    for i in range(12):
        H, I, E, k, S, npin, max_rows, Ms, stage = _random_layer(rng, i)
        Ms = [1 if rng.random() < 0.7 else m for m in Ms]
        log("overlapped fill, random layer %d: H=%d I=%d E=%d k=%d S=%d pins=%d max_rows=%d stage=%d M=%s"
            % (i, H, I, E, k, S, npin, max_rows, stage, Ms))
        cfg = WorkloadConfig("ovrand%d" % i, H, I, E, k, S, rows=max_rows, steps=len(Ms), seed=500 + i)
        ov = make_cache(cfg, max_rows=max_rows, gs_mode="uniform", prefill_stage=stage, overlap_fill=True)
        pl = make_cache(cfg, max_rows=max_rows, gs_mode="uniform", prefill_stage=stage)
        orc = _oracle_layer(cfg, S, "uniform")
        if npin:
            pins = [int(e) for e in rng.permutation(E)[:npin]]
            ov.pin(0, pins)
            pl.pin(0, pins)
            orc.state.pin(pins)
        zs = [rng.standard_normal((max_rows, E)).astype(np.float32) for _ in Ms]
        for z in zs:
            z[:, : max(1, E // 6)] += 1.0
        go, gp = GpuStepper(ov), GpuStepper(pl)
        worst = 0.0
        for t, M in enumerate(Ms):
            z = zs[t][:M]
            x = activations(cfg, 0, t, M)
            y, ids, w, byp = go.step(z, x)
            yp, _, _, _ = gp.step(z, x)
            assert np.array_equal(y, yp), (i, t, M)
            ev = go.new_events()
            gp.new_events()
            r = _check_step(t, (y, ids, w, byp, ev), orc.decode(z, x), None)
            worst = max(worst, r)
            _check_state(ov, 0, orc.state)
        _check_counters(ov, 0, orc.state)
        log("overlapped fill, random layer %d: worst rel L2 %.3g, stats %s" % (i, worst, ov.stats(0)))
        ov.close()
        pl.close()


def test_overlap_fill_multi_layer_banks():
    """Four layers of one handle with 3, 5, 8 and 16 slots over two host
    backing banks (layer l reads bank l mod 2), one-row steps taken layer by
    layer: every layer's bookkeeping against its own oracle, outputs against
    the oracle and bitwise against a handle without the flag."""
    torch_cuda()
    from oracle import OracleLayer
    from gpu_util import OracleBlobs
    from synth import global_scales
    cfg = CONFIGS["tiny"]
    slots, n_banks, steps = [3, 5, 8, 16], 2, 40
    log("overlapped fill, 4 layers (slots %s) over %d banks, %d steps each" % (slots, n_banks, steps))
    ov = make_cache(cfg, n_layers=4, slots=slots, max_rows=1, n_banks=n_banks, gs_mode="uniform", overlap_fill=True)
    pl = make_cache(cfg, n_layers=4, slots=slots, max_rows=1, n_banks=n_banks, gs_mode="uniform")
    E = cfg.n_experts
    orcs = [OracleLayer(cfg.hidden, cfg.inter, E, cfg.top_k, S, OracleBlobs(cfg, l % n_banks),
                        global_scales(cfg, l % n_banks, "uniform")[:E], keep_slot_bytes=False)
            for l, S in enumerate(slots)]
    go = [GpuStepper(ov, l) for l in range(4)]
    gp = [GpuStepper(pl, l) for l in range(4)]
    rng = np.random.default_rng(77)
    worst = 0.0
    for t in range(steps):
        for l in range(4):
            z = rng.standard_normal((1, E)).astype(np.float32)
            z[:, :3] += 1.0
            x = activations(cfg, 0, 4 * t + l, 1)
            y, ids, w, byp = go[l].step(z, x)
            yp, _, _, _ = gp[l].step(z, x)
            assert np.array_equal(y, yp), (t, l)
            ev = go[l].new_events()
            gp[l].new_events()
            r = _check_step(t, (y, ids, w, byp, ev), orcs[l].decode(z, x), None)
            worst = max(worst, r)
    for l in range(4):
        _check_state(ov, l, orcs[l].state)
        _check_counters(ov, l, orcs[l].state)
    log("4 layers: worst rel L2 %.3g, misses per layer %s" % (worst, [ov.stats(l)["misses"] for l in range(4)]))
    assert ov.stats(0)["evictions"] > 0
    ov.close()
    pl.close()

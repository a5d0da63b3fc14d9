"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs.  Slot bookkeeping (routing ids, miss/eviction events, slot maps,
LRU keys, counters) must match bit for bit; routing weights to 1e-6 relative;
outputs to relative L2 <= 1e-3 (fp32 accumulation against fp64)."""
import json
import os

import numpy as np
import pytest

from oracle import OracleLayer, route
from synth import CONFIGS, WorkloadConfig, activations, global_scales, routing_trace

from gpu_util import Y_TOL, GpuStepper, OracleBlobs, check_output, log, make_cache, torch_cuda

pytestmark = pytest.mark.gpu

W_TOL = 1e-6
GOLD = os.path.join(os.path.dirname(__file__), "golden", "lru_hand_trace.json")


def _oracle_layer(cfg, S, gs_mode="unit", E=None):
    E = E or cfg.n_experts
    return OracleLayer(cfg.hidden, cfg.inter, E, cfg.top_k, S, OracleBlobs(cfg),
                       global_scales(cfg, 0, gs_mode)[:E], keep_slot_bytes=False)


def _check_step(t, gpu_out, orc, rec_events, want_y=True):
    y_gpu, ids_gpu, w_gpu, byp_gpu, ev_gpu = gpu_out
    y_o, rec, ids_o, w_o = orc
    assert np.array_equal(ids_gpu, ids_o), (t, ids_gpu, ids_o)
    np.testing.assert_allclose(w_gpu, w_o, rtol=W_TOL, atol=1e-7, err_msg="step %d" % t)
    assert byp_gpu == rec.bypass, t
    assert [tuple(e[1:]) for e in ev_gpu] == rec.events, (t, ev_gpu, rec.events)
    assert all(e[0] == rec.step for e in ev_gpu)
    if want_y:
        return check_output(y_gpu, y_o, t)
    return None


def _check_state(sc, layer, st):
    e2s, s2e, key, step = sc.read_state(layer)
    assert list(e2s) == st.e2s
    assert list(s2e) == st.s2e
    assert list(key) == st.key
    assert step == st.t


def _check_counters(sc, layer, st):
    c = sc.stats(layer)
    oc = st.counters
    for name in ("steps", "bypass_steps", "picks", "lookups", "hits", "misses", "evictions",
                 "bytes_filled", "bypass_bytes"):
        assert c[name] == getattr(oc, name), name
    assert c["device_error"] == 0


def _run_trace(cfg, sc, orc, steps, rows_fn, logits_fn, y_steps=None, state_every=1):
    g = GpuStepper(sc)
    worst = 0.0
    for t in range(steps):
        M = rows_fn(t)
        z = logits_fn(t)[:M]
        x = activations(cfg, 0, t, M)
        want_y = y_steps is None or t in y_steps
        y, ids, w, byp = g.step(z, x)
        assert np.isfinite(y).all(), t          # every step, also those whose output is not compared
        ev = g.new_events()
        o = orc.decode(z, x, with_output=want_y)
        r = _check_step(t, (y, ids, w, byp, ev), o, None, want_y)
        if r is not None:
            worst = max(worst, r)
        if state_every and t % state_every == 0:
            _check_state(sc, 0, orc.state)
    _check_state(sc, 0, orc.state)
    _check_counters(sc, 0, orc.state)
    return worst


@pytest.mark.parametrize("gs_mode", ["unit", "uniform"])
def test_tiny_layer_all_steps(gs_mode):
    cfg = CONFIGS["tiny"]
    log("tiny parity gs=%s: 64 steps, H256 I128 E16 k2 S8" % gs_mode)
    sc = make_cache(cfg, gs_mode=gs_mode)
    orc = _oracle_layer(cfg, cfg.slots, gs_mode)
    logits, rows = routing_trace(cfg, 0)
    worst = _run_trace(cfg, sc, orc, cfg.steps, lambda t: 1, lambda t: logits[t])
    log("tiny worst rel L2 %.3g, counters %s" % (worst, sc.stats(0)))
    assert sc.stats(0)["evictions"] > 0
    sc.close()


def test_tiny_multi_row_steps():
    """M in {2, 3, 4, 8, 16, 17, 32}: shared picks (union fetch), U > S bypass, M > 16 bypass."""
    cfg = CONFIGS["tiny"]
    log("tiny multi-row parity: M mix up to 32, S8")
    sc = make_cache(cfg, max_rows=32)
    orc = _oracle_layer(cfg, cfg.slots)
    rng = np.random.default_rng(123)
    Ms = [2, 3, 4, 8, 16, 17, 32, 1, 4, 2]
    zs = [rng.standard_normal((32, cfg.n_experts)).astype(np.float32) for _ in range(40)]
    for t in range(40):
        zs[t][:, :4] += 1.5          # shared favourites
    worst = _run_trace(cfg, sc, orc, 40, lambda t: Ms[t % len(Ms)], lambda t: zs[t])
    st = sc.stats(0)
    log("multi-row worst rel L2 %.3g, stats %s" % (worst, st))
    assert st["bypass_steps"] > 0 and st["misses"] > 0
    sc.close()


def test_hand_worked_trace_on_gpu():
    g = json.load(open(GOLD))
    base = CONFIGS["tiny"]
    cfg = WorkloadConfig("hand", base.hidden, base.inter, g["n_experts"], g["top_k"], g["n_slots"],
                         rows=2, steps=len(g["steps"]), seed=base.seed)
    log("hand trace on GPU: E4 S2 k2")
    sc = make_cache(cfg)
    stepper = GpuStepper(sc)
    for t, s in enumerate(g["steps"]):
        ids = np.array(s["ids"])
        z = np.zeros((ids.shape[0], g["n_experts"]), np.float32)
        for m in range(ids.shape[0]):
            for j, e in enumerate(ids[m]):
                z[m, e] = 10.0 - j
        y, gids, w, byp = stepper.step(z, activations(cfg, 0, t, ids.shape[0]))
        assert np.array_equal(gids, ids)
        assert byp == s["bypass"]
        assert [list(e[1:]) for e in stepper.new_events()] == s["events"], t
    e2s, s2e, key, step = sc.read_state(0)
    f = g["final"]
    assert list(e2s) == f["e2s"] and list(s2e) == f["s2e"] and list(key) == f["key"] and step == f["t"]
    c = sc.stats(0)
    for name, v in f["counters"].items():
        assert c[name] == v, name
    sc.close()


def test_nonfinite_logits_route_like_the_oracle():
    cfg = CONFIGS["tiny"]
    log("non-finite logits routing")
    sc = make_cache(cfg, max_rows=8)
    orc = _oracle_layer(cfg, cfg.slots)
    E = cfg.n_experts
    rows = [
        [np.nan] * 3 + [-np.inf] * 2 + [0.5] + [np.nan] * (E - 6),
        [np.inf, 1.0, np.inf] + [0.0] * (E - 3),
        [-np.inf] * (E - 1) + [np.nan],
        [-0.0, 0.0] + [-1.0] * (E - 2),
        [3.0] * E,
    ]
    z = np.array(rows, np.float32)
    x = activations(cfg, 0, 0, len(rows))
    y, ids, w, byp = GpuStepper(sc).step(z, x)
    ids_o, w_o = route(z, cfg.top_k)
    assert np.array_equal(ids, ids_o)
    np.testing.assert_allclose(w, w_o, rtol=W_TOL, atol=0)
    sc.close()


def test_argument_errors_enqueue_nothing():
    from hbm_expert_slot_amd import binding as B
    torch = torch_cuda()
    cfg = CONFIGS["tiny"]
    log("argument errors")
    sc = make_cache(cfg, max_rows=4)
    z = torch.zeros((8, cfg.n_experts), dtype=torch.float32, device="cuda")
    x = torch.zeros((8, cfg.hidden), dtype=torch.int16, device="cuda")
    y = torch.zeros((8, cfg.hidden), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for layer, M, zp in ((0, 0, z.data_ptr()), (0, 5, z.data_ptr()), (1, 1, z.data_ptr()),
                         (-1, 1, z.data_ptr()), (0, 1, None)):
        with pytest.raises(B.SlotCacheError) as ei:
            B.moe_layer_decode(sc.h, layer, zp, x.data_ptr(), M, y.data_ptr(), s)
        assert ei.value.status == B.SC_E_ARG
    assert sc.stats(0)["steps"] == 0
    with pytest.raises(B.SlotCacheError):
        sc.write_state(0, np.full(cfg.n_experts, -1), np.array([0] + [-1] * 7), np.full(8, -1), 0)
    sc.close()


def test_cached_layer_equals_all_resident_layer_bitwise():
    """The pages' invariant, on the GPU: a churning 8-slot layer and a 16-slot
    preloaded (all-resident) layer give bit-identical outputs on every step."""
    torch = torch_cuda()
    cfg = CONFIGS["tiny"]
    log("cached vs all-resident bitwise: tiny, 2 layers (S=8, S=16 preloaded)")
    sc = make_cache(cfg, n_layers=2, slots=[8, 16], max_rows=4, gs_mode="uniform")
    sc.preload(1)
    rng = np.random.default_rng(5)
    for t in range(96):
        M = 1 if t < 64 else 4
        z = torch.from_numpy(rng.standard_normal((M, cfg.n_experts)).astype(np.float32)).cuda()
        x = torch.from_numpy(activations(cfg, 0, t, M).view(np.int16)).cuda()
        y0 = torch.empty((M, cfg.hidden), dtype=torch.float32, device="cuda")
        y1 = torch.empty_like(y0)
        sc.decode(0, z, x, y0)
        sc.decode(1, z, x, y1)
        assert torch.equal(y0, y1), t
    s0, s1 = sc.stats(0), sc.stats(1)
    log("cached layer stats %s / all-resident %s" % (s0, s1))
    assert s0["evictions"] > 0 and s1["misses"] == 0
    sc.close()


def test_graph_replay_under_churn():
    """One captured step replayed with new inputs each time (fixed addresses and
    shapes), eager work and synchronisations in between, checked against the oracle."""
    torch = torch_cuda()
    cfg = CONFIGS["tiny"]
    log("graph capture + replay under churn: tiny")
    sc = make_cache(cfg)
    orc = _oracle_layer(cfg, cfg.slots)
    logits, _ = routing_trace(cfg, 0)
    z = torch.zeros((1, cfg.n_experts), dtype=torch.float32, device="cuda")
    x = torch.zeros((1, cfg.hidden), dtype=torch.int16, device="cuda")
    y = torch.zeros((1, cfg.hidden), dtype=torch.float32, device="cuda")
    # warm-up step outside the graph (also the first oracle step)
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
        _ = (y * 2).sum().item()     # unrelated eager work between replays
    _check_counters(sc, 0, orc.state)
    sc.close()


def test_checkpoint_resume_matches_a_continuous_run():
    torch = torch_cuda()
    cfg = CONFIGS["tiny"]
    log("checkpoint / resume: tiny")
    a = make_cache(cfg)
    logits, _ = routing_trace(cfg, 0)
    ga = GpuStepper(a)
    for t in range(20):
        ga.step(logits[t, :1], activations(cfg, 0, t, 1))
    e2s, s2e, key, step = a.read_state(0)
    b = make_cache(cfg)
    b.write_state(0, e2s, s2e, key, step)
    gb = GpuStepper(b)
    for t in range(20, 50):
        x = activations(cfg, 0, t, 1)
        ya, ia, _, _ = ga.step(logits[t, :1], x)
        yb, ib, _, _ = gb.step(logits[t, :1], x)
        assert np.array_equal(ya, yb) and np.array_equal(ia, ib), t
    for u, v in zip(a.read_state(0), b.read_state(0)):
        assert np.array_equal(u, v)
    a.close()
    b.close()


def test_write_state_rejects_keys_the_layer_cannot_have_stamped():
    """Occupied slots' keys must lie in [-1, step*16*k) and the step in [0, 2^40): the remap
    orders victims by packing (key + 2) above the slot index, so keys outside that range
    would reorder victims against the oracle's signed (key, slot) order.  A rejected
    state changes nothing."""
    from hbm_expert_slot_amd import binding as B
    torch_cuda()
    cfg = CONFIGS["tiny"]
    log("write_state key checks: tiny")
    sc = make_cache(cfg)
    logits, _ = routing_trace(cfg, 0)
    g = GpuStepper(sc)
    for t in range(10):
        g.step(logits[t, :1], activations(cfg, 0, t, 1))
    e2s, s2e, key, step = sc.read_state(0)
    occ = int(np.nonzero(s2e >= 0)[0][0])
    end = step * 16 * cfg.top_k
    for bad_key, bad_step in ((-2, step), (end, step), (1 << 62, step), (-(1 << 62), step), (0, 1 << 40),
                              (0, -1)):
        k2 = key.copy()
        k2[occ] = bad_key
        with pytest.raises(B.SlotCacheError) as ei:
            sc.write_state(0, e2s, s2e, k2, bad_step)
        assert ei.value.status == B.SC_E_ARG, (bad_key, bad_step)
        for u, v in zip(sc.read_state(0), (e2s, s2e, key, step)):
            assert np.array_equal(u, v)
    # the limits themselves are accepted
    for ok_key in (-1, end - 1):
        k2 = key.copy()
        k2[occ] = ok_key
        sc.write_state(0, e2s, s2e, k2, step)
    sc.close()


@pytest.mark.timeout(600)
def test_glm_layer_300_steps():
    """GLM-shaped layer at full size (H6144 I2048, 256 experts, top-8, S=128):
    bookkeeping on all 300 steps, outputs on sampled steps (and every step's
    output is checked for finiteness)."""
    cfg = CONFIGS["glm"]
    log("GLM parity: filling 256 x 21.2 MB backing")
    sc = make_cache(cfg)
    orc = _oracle_layer(cfg, cfg.slots)
    logits, _ = routing_trace(cfg, 0)
    sample = {0, 1, 2, 17, 128, 299}
    log("GLM parity: 300 steps, y sampled at %s" % sorted(sample))
    worst = _run_trace(cfg, sc, orc, cfg.steps, lambda t: 1, lambda t: logits[t], y_steps=sample,
                       state_every=10)
    st = sc.stats(0)
    log("GLM worst rel L2 %.3g; hit rate %.3f; stats %s" % (worst, st["hits"] / st["lookups"], st))
    sc.close()


@pytest.mark.timeout(900)
def test_glm_drafted_rounds_and_prefill_bypass():
    """M=4 draft rounds, M=16 verify batches and M=64 prefill bypass on the GLM layer."""
    cfg = CONFIGS["glm_draft"]
    steps = cfg.steps
    log("GLM drafted parity: filling backing; %d steps with M in {4, 16, 64}" % steps)
    sc = make_cache(cfg)
    orc = _oracle_layer(cfg, cfg.slots)
    logits, rows = routing_trace(cfg, 0, steps=steps)
    sample = {0, 9, 48, 49, 159, 198}     # M=4, M=16, M=4, M=64 (bypass), M=16, M=4
    worst = _run_trace(cfg, sc, orc, steps, lambda t: int(rows[t]), lambda t: logits[t], y_steps=sample,
                       state_every=5)
    st = sc.stats(0)
    log("GLM drafted worst rel L2 %.3g; stats %s" % (worst, st))
    assert st["bypass_steps"] == 4
    sc.close()


def test_timed_entry_point_matches_the_plain_one():
    """moe_layer_decode_ev (per-kernel start/stop events and execution stamps) computes the same step,
    on one-row and four-row (matrix-core) steps."""
    torch = torch_cuda()
    from hbm_expert_slot_amd import binding as B
    cfg = CONFIGS["tiny"]
    log("timed entry point vs plain: tiny, 24 steps of 1 and 4 rows")
    a, b = make_cache(cfg, max_rows=4), make_cache(cfg, max_rows=4)
    logits, _ = routing_trace(cfg, 0)
    rng = np.random.default_rng(5)
    for t in range(24):
        M = 4 if t % 3 == 2 else 1
        zt = logits[t, :1] if M == 1 else rng.standard_normal((M, cfg.n_experts)).astype(np.float32)
        z = torch.from_numpy(np.ascontiguousarray(zt)).cuda()
        x = torch.from_numpy(activations(cfg, 0, t, M).view(np.int16)).cuda()
        ya = torch.empty((M, cfg.hidden), dtype=torch.float32, device="cuda")
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
        # the kernels' own start/end stamps: positive, and inside the event brackets
        spans = b.kernel_spans()
        assert all(0 < s_us <= 1e3 * e_ms + 1.0 for s_us, e_ms in zip(spans, ev_ms)), (M, spans, ev_ms)
    with pytest.raises(B.SlotCacheError):
        a.kernel_spans()          # a's steps were not timed
    for u, v in zip(a.read_state(0), b.read_state(0)):
        assert np.array_equal(u, v)
    a.close()
    b.close()


def _check_slots_hold_their_experts(sc, layer=0):
    """Every occupied slot holds its expert's blob byte for byte (single-layer pools)."""
    e2s, s2e, key, step = sc.read_state(layer)
    pool = sc.pool[: sc.slots[layer] * sc.blob_bytes].cpu().numpy().reshape(sc.slots[layer], sc.blob_bytes)
    back = sc.backing(layer % sc.n_banks)
    filled = 0
    for s, e in enumerate(s2e):
        if e >= 0:
            assert np.array_equal(pool[s], back[e]), (s, e)
            filled += 1
    return filled


@pytest.mark.parametrize("shape", ["tiny", "glm48"])
def test_misses_fill_their_slots_exactly(shape):
    """After a churning mix of one-row, multi-row (experts with several picks)
    and matrix-core steps, every occupied slot equals its expert's blob byte
    for byte: the fill copied each miss whole into its victim slot."""
    cfg = CONFIGS["tiny"]
    if shape == "glm48":
        g = CONFIGS["glm"]
        cfg = WorkloadConfig("glm48", g.hidden, g.inter, 48, g.top_k, 30, rows=16, steps=40, seed=g.seed)
    log("slot contents after churn: %s, M in {1, 2, 3, 4, 8, 12, 16}" % shape)
    sc = make_cache(cfg, max_rows=16)
    orc = _oracle_layer(cfg, cfg.slots)
    rng = np.random.default_rng(9)
    Ms = [1, 4, 2, 16, 1, 3, 12, 8, 1, 4]
    E = cfg.n_experts
    zs = []
    for t in range(30):
        z = rng.standard_normal((16, E)).astype(np.float32)
        z[:, : max(2, cfg.top_k // 2)] += 2.0      # shared favourites: several picks per expert
        zs.append(z)
    sample = None if shape == "tiny" else {0, 1, 6, 9}     # M = 1, 4, 12, 4 (fp64 oracle cost at GLM shapes)
    worst = _run_trace(cfg, sc, orc, 30, lambda t: Ms[t % len(Ms)], lambda t: zs[t], y_steps=sample,
                       state_every=5)
    st = sc.stats(0)
    n = _check_slots_hold_their_experts(sc)
    log("%s: %d occupied slots verified; misses %d, bypass %d, worst rel L2 %.3g" % (shape, n, st["misses"],
                                                                                   st["bypass_steps"], worst))
    assert st["misses"] > 0 and n > 0
    sc.close()


def _rows_vs_single(cfg, sc_multi, sc_single, Ms, seed, drafted=True, identical=False):
    """Max number of rows whose output differs (bitwise) from the same row run as a one-row step."""
    torch = torch_cuda()
    rng = np.random.default_rng(seed)
    E, H = cfg.n_experts, cfg.hidden
    bad = {}
    for t, M in enumerate(Ms):
        z = rng.standard_normal((M, E)).astype(np.float32)
        if identical:                 # every row routes alike: each expert gets M picks
            z[:] = z[0]
        elif drafted:                 # later rows share picks with row 0 (draft / verify rounds)
            top = np.argsort(-z[0])[:cfg.top_k]
            for m in range(1, M):
                z[m, rng.choice(top, min(3, len(top)), replace=False)] += 20.0
        x = activations(cfg, 0, 1000 + t, M)
        zd = torch.from_numpy(z).cuda()
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        y = torch.empty((M, H), dtype=torch.float32, device="cuda")
        sc_multi.decode(0, zd, xd, y)
        ym = y.cpu().numpy()
        n = 0
        for m in range(M):
            y1 = torch.empty((1, H), dtype=torch.float32, device="cuda")
            sc_single.decode(0, zd[m:m + 1].contiguous(), xd[m:m + 1].contiguous(), y1)
            n += int(not np.array_equal(ym[m], y1.cpu().numpy()[0]))
        bad[M] = max(bad.get(M, 0), n)
    return bad


@pytest.mark.parametrize("shape", ["tiny", "glm32", "h1024_i512"])
def test_batch_invariant_rows(shape):
    """SC_FLAG_BATCH_INVARIANT: every row of an M-row step (drafted rows sharing
    picks, M up to 16, and a prefill-sized bypass step) is bit-equal to the
    same row decoded alone.  Without the flag the steps that run only the
    streaming kernels (M below both matrix-core thresholds) are invariant too;
    the matrix-core kernels need not be."""
    cfg = CONFIGS["tiny"]
    if shape == "glm32":
        g = CONFIGS["glm"]
        cfg = WorkloadConfig("glm32", g.hidden, g.inter, 32, g.top_k, 32, rows=24, steps=1, seed=g.seed)
    elif shape == "h1024_i512":
        # 16- and 32-lane row groups: the multi-row down kernels sum eight values per row group
        cfg = WorkloadConfig("h1024_i512", 1024, 512, 32, 4, 32, rows=24, steps=1, seed=71)
    log("batch invariance: %s" % shape)
    E = cfg.n_experts
    inv = make_cache(cfg, n_layers=1, slots=[E], max_rows=24, batch_invariant=True)
    dflt = make_cache(cfg, n_layers=1, slots=[E], max_rows=24)
    one = make_cache(cfg, n_layers=1, slots=[E], max_rows=1)
    for sc in (inv, dflt, one):
        sc.preload(0)
    Ms = [2, 3, 4, 8, 11, 12, 16, 24]
    bad_inv = _rows_vs_single(cfg, inv, one, Ms, seed=3)
    from hbm_expert_slot_amd import binding as B
    m_stream = min(B.SC_MFMA_MIN_ROWS_GATEUP, B.SC_MFMA_MIN_ROWS_DOWN)
    bad_dflt = _rows_vs_single(cfg, dflt, one, [M for M in Ms if M < m_stream], seed=3)
    log("rows differing from their one-row result: invariant %s; default (M < %d) %s" % (bad_inv, m_stream, bad_dflt))
    assert all(v == 0 for v in bad_inv.values()), bad_inv
    assert all(v == 0 for v in bad_dflt.values()), bad_dflt
    assert inv.stats(0)["bypass_steps"] == 1      # M = 24 > 16
    for sc in (inv, dflt, one):
        sc.close()


def test_identical_rows_fill_every_pick_column():
    """Steps whose rows all route alike give each picked expert as many picks as
    the step has rows: 4 on the shared-operand streaming kernels, 8 and 16 on
    the matrix-core kernels, whose pick columns are then all live.  Outputs
    match the oracle; at 4 rows (streaming) and, with SC_FLAG_BATCH_INVARIANT,
    at 8 and 16 rows every row is bit-equal to the same row decoded alone."""
    g = CONFIGS["glm"]
    cfg = WorkloadConfig("glm32", g.hidden, g.inter, 32, g.top_k, 32, rows=16, steps=9, seed=g.seed)
    E = cfg.n_experts
    log("identical rows: glm32, M in 4, 8, 16")
    sc = make_cache(cfg, max_rows=16)
    orc = _oracle_layer(cfg, cfg.slots)
    rng = np.random.default_rng(29)
    Ms = [4, 8, 16, 16, 8, 4, 16, 4, 8]
    zs = [np.repeat(rng.standard_normal((1, E)).astype(np.float32), 16, axis=0) for _ in Ms]
    worst = _run_trace(cfg, sc, orc, len(Ms), lambda t: Ms[t], lambda t: zs[t])
    st = sc.stats(0)
    log("identical rows: worst rel L2 %.3g, stats %s" % (worst, st))
    assert st["bypass_steps"] == 0 and st["picks"] == sum(M * cfg.top_k for M in Ms)
    assert st["lookups"] == len(Ms) * cfg.top_k          # one lookup per unique expert
    sc.close()

    from hbm_expert_slot_amd import binding as B
    m_stream = min(B.SC_MFMA_MIN_ROWS_GATEUP, B.SC_MFMA_MIN_ROWS_DOWN)
    dflt = make_cache(cfg, n_layers=1, slots=[E], max_rows=16)
    inv = make_cache(cfg, n_layers=1, slots=[E], max_rows=16, batch_invariant=True)
    one = make_cache(cfg, n_layers=1, slots=[E], max_rows=1)
    for c in (dflt, inv, one):
        c.preload(0)
    bad_dflt = _rows_vs_single(cfg, dflt, one, [M for M in (2, 3, 4) if M < m_stream], seed=5, identical=True)
    bad_inv = _rows_vs_single(cfg, inv, one, [4, 8, 16], seed=5, identical=True)
    log("identical rows differing from one-row results: default %s, invariant %s" % (bad_dflt, bad_inv))
    assert all(v == 0 for v in bad_dflt.values()), bad_dflt
    assert all(v == 0 for v in bad_inv.values()), bad_inv
    for c in (dflt, inv, one):
        c.close()


@pytest.mark.parametrize("shape", ["tiny", "glm32"])
def test_pinned_slots_against_the_oracle(shape):
    """Hybrid policy (slotcache_pin): a few experts pinned in the first slots, LRU
    over the rest, under one-row, multi-row, matrix-core and bypass steps: every
    event, the slot map, keys and counters (bypass host bytes included) match
    the oracle; pinned slots keep their experts; slot bytes stay exact."""
    cfg = CONFIGS["tiny"]
    npin, Ms = 3, [1, 2, 1, 3, 4, 1, 8, 17, 1, 2]
    if shape == "glm32":
        g = CONFIGS["glm"]
        cfg = WorkloadConfig("glm32", g.hidden, g.inter, 32, g.top_k, 16, rows=17, steps=30, seed=g.seed)
        npin, Ms = 6, [1, 1, 2, 12, 1, 4, 17, 1, 1, 3]
    log("pinned slots vs oracle: %s, %d pinned of %d" % (shape, npin, cfg.slots))
    E = cfg.n_experts
    sc = make_cache(cfg, max_rows=17)
    orc = _oracle_layer(cfg, cfg.slots)
    rng = np.random.default_rng(17)
    zs = []
    for t in range(30):
        z = rng.standard_normal((17, E)).astype(np.float32)
        z[:, : cfg.top_k] += 1.0           # a few favourites, pinned below
        zs.append(z)
    pins = list(range(npin))[::-1]          # pinned in reverse id order: slot i holds npin-1-i
    sc.pin(0, pins)
    orc.state.pin(pins)
    sample = None if shape == "tiny" else {0, 3, 6}
    worst = _run_trace(cfg, sc, orc, 30, lambda t: Ms[t % len(Ms)], lambda t: zs[t], y_steps=sample)
    e2s, s2e, key, step = sc.read_state(0)
    assert list(s2e[:npin]) == pins
    st = sc.stats(0)
    n = _check_slots_hold_their_experts(sc)
    log("pinned %s: worst rel L2 %.3g, stats %s, %d slots verified" % (shape, worst, st, n))
    assert st["bypass_steps"] > 0 and st["misses"] > 0
    bad_s2e = np.array(s2e)
    bad_s2e[[0, 1]] = bad_s2e[[1, 0]]
    bad_e2s = np.array(e2s)
    bad_e2s[bad_s2e[0]], bad_e2s[bad_s2e[1]] = 0, 1
    from hbm_expert_slot_amd import binding as B
    with pytest.raises(B.SlotCacheError):
        sc.write_state(0, bad_e2s, bad_s2e, key, step)      # pinned slots must keep their experts
    sc.close()


@pytest.mark.parametrize("shape", ["tiny", "glm32"])
def test_prefill_groups_match_in_place_reads(shape):
    """Prefill chunks (M > 16) with their non-resident experts staged into HBM G
    at a time (G = 1, a ragged G and 64) produce the same bits as the in-place
    host reads (G = 0), with the same bookkeeping; the staged run also matches
    the oracle.  Cached steps in between keep some experts resident, so the
    first group mixes slot-resident and staged experts.  A timed staged step
    computes the same bits as well."""
    torch = torch_cuda()
    from hbm_expert_slot_amd import binding as B
    cfg = CONFIGS["tiny"]
    Ms, Gs, steps = [1, 2, 17, 4, 32, 1, 24, 3, 32, 1], [0, 1, 3, 64], 30
    if shape == "glm32":
        g = CONFIGS["glm"]
        cfg = WorkloadConfig("glm32", g.hidden, g.inter, 32, g.top_k, 12, rows=24, steps=12, seed=g.seed)
        Ms, Gs, steps = [1, 2, 24, 1, 17, 4, 24, 1, 20, 1, 24, 2], [0, 5, 64], 12
    maxM = max(Ms)
    log("prefill groups vs in-place reads: %s, G in %s, %d steps" % (shape, Gs, steps))
    E = cfg.n_experts
    caches = {G: make_cache(cfg, max_rows=maxM, prefill_stage=G) for G in Gs}
    orc = _oracle_layer(cfg, cfg.slots)
    rng = np.random.default_rng(29)
    sample = None if shape == "tiny" else {2, 4, 6}
    worst = 0.0
    for t in range(steps):
        M = Ms[t % len(Ms)]
        z = rng.standard_normal((M, E)).astype(np.float32)
        z[:, : cfg.top_k] += 0.8
        x = activations(cfg, 0, 500 + t, M)
        zd = torch.from_numpy(z).cuda()
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        ys = {}
        for G, sc in caches.items():
            y = torch.empty((M, cfg.hidden), dtype=torch.float32, device="cuda")
            if G == Gs[-1] and M > 16:
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(B.SC_N_EVENTS)]
                for ev in evs:
                    ev.record()
                sc.decode(0, zd, xd, y, events=evs)
                torch.cuda.synchronize()
                assert all(v > 0 for v in sc.kernel_spans())
            else:
                sc.decode(0, zd, xd, y)
            ys[G] = y.cpu().numpy()
        for G in Gs[1:]:
            assert np.array_equal(ys[G], ys[0]), (t, M, G)
        want_y = sample is None or t in sample
        y_o, rec, ids_o, w_o = orc.decode(z, x, with_output=want_y)
        if M > 16:
            assert rec.bypass
        if want_y:
            r = check_output(ys[Gs[-1]], y_o, (t, M))
            worst = max(worst, r)
    for G, sc in caches.items():
        _check_state(sc, 0, orc.state)
        _check_counters(sc, 0, orc.state)
    st = caches[0].stats(0)
    log("prefill groups %s: worst rel L2 %.3g, stats %s" % (shape, worst, st))
    assert st["bypass_steps"] > 0 and st["bypass_bytes"] > 0 and st["hits"] > 0
    for sc in caches.values():
        sc.close()


LIMIT_SHAPES = {
    # the library's largest top-k, expert count, slot count and picks per step (max_rows * k = 2048)
    "max": dict(E=1024, k=32, S=1024, Ms=[1, 2, 16, 1, 64, 16, 3, 64, 1], max_rows=64),
    # one expert, one slot, top-1: every step after the first is a hit
    "one_expert": dict(E=1, k=1, S=1, Ms=[1, 1, 4, 17, 1, 2], max_rows=17),
    # every expert picked every step (k = E)
    "k_eq_E": dict(E=8, k=8, S=8, Ms=[1, 2, 1, 17, 1], max_rows=17),
    # one slot for two picks per row: every step bypasses
    "one_slot": dict(E=16, k=2, S=1, Ms=[1, 1, 3, 1, 17], max_rows=17),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", list(LIMIT_SHAPES))
def test_limit_shapes_against_the_oracle(shape):
    """The compiled limits (E = 1024, k = 32, S = 1024, 2048 picks per step,
    a 64-row step staged in 16 groups) and degenerate layers (one expert;
    k = E; one slot for two picks) match the oracle's bookkeeping bit for bit
    and its outputs to the tolerance."""
    p = LIMIT_SHAPES[shape]
    E, k, S, Ms = p["E"], p["k"], p["S"], p["Ms"]
    cfg = WorkloadConfig("limit_" + shape, 256, 128, E, k, S, rows=p["max_rows"], steps=len(Ms), seed=41)
    log("limit shapes: %s (E=%d k=%d S=%d, M in %s)" % (shape, E, k, S, Ms))
    sc = make_cache(cfg, max_rows=p["max_rows"], gs_mode="uniform")
    orc = _oracle_layer(cfg, S, "uniform")
    rng = np.random.default_rng(43)
    zs = [rng.standard_normal((max(Ms), E)).astype(np.float32) for _ in Ms]
    for z in zs:
        z[:, : max(1, E // 8)] += 1.0      # favourites, so that later steps hit
    worst = _run_trace(cfg, sc, orc, len(Ms), lambda t: Ms[t], lambda t: zs[t])
    st = sc.stats(0)
    log("limit %s: worst rel L2 %.3g, stats %s" % (shape, worst, st))
    if shape == "max":
        assert st["misses"] > 512 and st["bypass_steps"] == 2
    if shape == "one_slot":
        assert st["bypass_steps"] == len(Ms)
    if shape == "one_expert":
        assert st["misses"] == 1 and st["hits"] == sum(1 for M in Ms if M <= 16) - 1
    sc.close()


# Layer shapes beyond the tiny, Flash and GLM ones: each gives the GEMVs other
# row-group widths (lanes per row: 8, 16, 32 or 64 for K = 256, 512, 1024,
# >= 2048), so every step of the cross-lane row sums, the matrix-core kernels
# at other K and a ragged split of rows over wavefronts are exercised.
OTHER_SHAPES = {"h512_i256": (512, 256), "h1024_i512": (1024, 512), "h2048_i1024": (2048, 1024),
                "h8192_i256": (8192, 256)}


@pytest.mark.timeout(600)
def test_one_row_runs_longer_than_32_row_steps():
    """A one-row step whose gate/up wavefronts each compute more than 32 row
    steps (H 2048, I 4096, 32 picks: 42 or 43 per wavefront), so the kernel
    writes the SiLU outputs of a run in more than one batch: bookkeeping bit
    for bit and every output against the oracle."""
    H, I, E, k, S = 2048, 4096, 32, 32, 32
    cfg = WorkloadConfig("long_runs", H, I, E, k, S, rows=1, steps=3, seed=67)
    log("long runs: H=%d I=%d E=%d k=%d S=%d, 3 one-row steps" % (H, I, E, k, S))
    sc = make_cache(cfg, max_rows=1, gs_mode="uniform")
    orc = _oracle_layer(cfg, S, "uniform")
    rng = np.random.default_rng(71)
    zs = [rng.standard_normal((1, E)).astype(np.float32) for _ in range(3)]
    worst = _run_trace(cfg, sc, orc, 3, lambda t: 1, lambda t: zs[t])
    st = sc.stats(0)
    log("long runs: worst rel L2 %.3g, stats %s" % (worst, st))
    assert st["misses"] == E and st["hits"] == 2 * E
    sc.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", list(OTHER_SHAPES))
def test_other_layer_shapes_against_the_oracle(shape):
    """One-row, two-row (streaming), matrix-core and bypass steps on layer
    shapes with other H and I: bookkeeping bit for bit, outputs to the
    tolerance, every step's output checked."""
    H, I = OTHER_SHAPES[shape]
    E, k, S = 12, 3, 6
    Ms = [1, 1, 2, 3, 1, 4, 17, 1, 2, 1, 5, 1]
    cfg = WorkloadConfig("shape_" + shape, H, I, E, k, S, rows=17, steps=len(Ms), seed=53)
    log("layer shape %s: H=%d I=%d (E=%d k=%d S=%d, M in %s)" % (shape, H, I, E, k, S, Ms))
    sc = make_cache(cfg, max_rows=17, gs_mode="uniform", prefill_stage=2)
    orc = _oracle_layer(cfg, S, "uniform")
    rng = np.random.default_rng(59)
    zs = [rng.standard_normal((17, E)).astype(np.float32) for _ in Ms]
    for z in zs:
        z[:, :2] += 1.0
    worst = _run_trace(cfg, sc, orc, len(Ms), lambda t: Ms[t], lambda t: zs[t])
    st = sc.stats(0)
    log("shape %s: worst rel L2 %.3g, stats %s" % (shape, worst, st))
    assert st["misses"] > 0 and st["bypass_steps"] >= 1
    sc.close()


# Layers aimed at the routing kernel's paths: one-row steps on one wavefront
# (experts and slots over 64, 256 and 512, so several values per lane; up to
# 16 picks; k equal to the unpinned slot count), the four-wavefront kernel on
# a one-row step that can bypass, and steps of at most 64 picks (bookkeeping
# on one wavefront, with bypasses) next to a step of 128 picks.
ROUTE_CASES = {
    "one_e300_k16_s200": dict(E=300, k=16, S=200, npin=5, Ms=[1] * 40),
    "one_e1000_k16_s260": dict(E=1000, k=16, S=260, npin=0, Ms=[1] * 40),
    "one_e100_k6_s50": dict(E=100, k=6, S=50, npin=0, Ms=[1] * 24),
    "one_k_fills_unpinned": dict(E=300, k=12, S=16, npin=4, Ms=[1] * 16),
    "one_row_may_bypass": dict(E=300, k=12, S=15, npin=4, Ms=[1] * 16),
    "small_steps": dict(E=200, k=8, S=40, npin=3, Ms=[2, 3, 4, 8, 5, 1, 8, 7, 2, 6, 16, 4, 8, 3]),
}


@pytest.mark.parametrize("case", sorted(ROUTE_CASES))
def test_route_paths_against_the_oracle(case):
    """Every step's ids, weights, events, slot map, keys and counters bit for
    bit, and outputs to the tolerance, on layers that send steps down each
    path of the routing kernel; the popular experts shift every few steps, so
    the cached paths take misses, evictions and victim searches."""
    p = ROUTE_CASES[case]
    E, k, S, npin, Ms = p["E"], p["k"], p["S"], p["npin"], p["Ms"]
    maxM = max(Ms)
    log("route paths: %s (E=%d k=%d S=%d pins=%d M=%s)" % (case, E, k, S, npin, Ms))
    cfg = WorkloadConfig("route_" + case, 256, 128, E, k, S, rows=maxM, steps=len(Ms), seed=91)
    sc = make_cache(cfg, max_rows=maxM, gs_mode="uniform")
    orc = _oracle_layer(cfg, S, "uniform")
    rng = np.random.default_rng(37)
    if npin:
        pins = [int(e) for e in rng.permutation(E)[:npin]]
        sc.pin(0, pins)
        orc.state.pin(pins)
    zs = []
    for t in range(len(Ms)):
        if t % 4 == 0:
            hot = rng.permutation(E)[: max(k, E // 5)]
        z = rng.standard_normal((maxM, E)).astype(np.float32)
        z[:, hot] += 2.0
        zs.append(z)
    worst = _run_trace(cfg, sc, orc, len(Ms), lambda t: Ms[t], lambda t: zs[t])
    st = sc.stats(0)
    log("route paths %s: worst rel L2 %.3g, stats %s" % (case, worst, st))
    assert st["misses"] > 0
    if case == "one_row_may_bypass" or case == "small_steps":
        assert st["bypass_steps"] > 0
    else:
        assert st["bypass_steps"] == 0 and st["evictions"] > 0
    sc.close()


def _random_layer(rng, i):
    """A small random layer: expert count, top-k, slots, pins, row mix, staging."""
    H, I = [(256, 128), (512, 256), (256, 256), (1024, 128)][i % 4]
    E = int(rng.integers(1, 41))
    k = int(rng.integers(1, min(E, 8) + 1))
    S = int(rng.integers(1, E + 1))
    npin = int(rng.integers(0, S + 1)) if rng.random() < 0.3 else 0
    max_rows = int(rng.choice([1, 4, 17, 24]))
    Ms = [int(rng.integers(1, max_rows + 1)) for _ in range(14)]
    stage = int(rng.integers(1, 6)) if rng.random() < 0.5 else 0
    return H, I, E, k, S, npin, max_rows, Ms, stage


@pytest.mark.timeout(600)
def test_random_layers_against_the_oracle():
    """Twelve seeded random layers (1-40 experts, top-1..8, 1..E slots, pins on
    some, row mixes up to 24 with and without prefill staging, four H x I
    shapes): every step's bookkeeping bit for bit and output to the tolerance."""
    torch_cuda()
    rng = np.random.default_rng(2024)
    for i in range(12):
        H, I, E, k, S, npin, max_rows, Ms, stage = _random_layer(rng, i)
        log("random layer %d: H=%d I=%d E=%d k=%d S=%d pins=%d max_rows=%d stage=%d M=%s"
            % (i, H, I, E, k, S, npin, max_rows, stage, Ms))
        cfg = WorkloadConfig("rand%d" % i, H, I, E, k, S, rows=max_rows, steps=len(Ms), seed=300 + i)
        sc = make_cache(cfg, max_rows=max_rows, gs_mode="uniform", prefill_stage=stage)
        orc = _oracle_layer(cfg, S, "uniform")
        if npin:
            pins = [int(e) for e in rng.permutation(E)[:npin]]
            sc.pin(0, pins)
            orc.state.pin(pins)
        zs = [rng.standard_normal((max_rows, E)).astype(np.float32) for _ in Ms]
        for z in zs:
            z[:, : max(1, E // 6)] += 1.0
        worst = _run_trace(cfg, sc, orc, len(Ms), lambda t: Ms[t], lambda t: zs[t])
        log("random layer %d: worst rel L2 %.3g, stats %s" % (i, worst, sc.stats(0)))
        sc.close()


def test_graph_replay_of_multi_row_and_staged_prefill_steps():
    """Captured steps of 4 rows (streaming gate/up, matrix-core down), 8 rows
    (matrix cores for both) and 24 rows (a prefill chunk staged 3 experts per
    group: several fill / gate/up / down launches in one step), replayed in
    turn with new inputs and eager work in between, against the oracle."""
    torch = torch_cuda()
    cfg = CONFIGS["tiny"]
    Ms = (4, 8, 24)
    log("graph capture + replay: tiny, M in %s, prefill staged 3 per group" % (Ms,))
    sc = make_cache(cfg, max_rows=max(Ms), prefill_stage=3)
    orc = _oracle_layer(cfg, cfg.slots)
    rng = np.random.default_rng(61)
    E, H = cfg.n_experts, cfg.hidden
    bufs = {M: (torch.zeros((M, E), dtype=torch.float32, device="cuda"),
                torch.zeros((M, H), dtype=torch.int16, device="cuda"),
                torch.zeros((M, H), dtype=torch.float32, device="cuda")) for M in Ms}
    s = torch.cuda.Stream()
    graphs = {}
    torch.cuda.synchronize()
    for M in Ms:
        z, x, y = bufs[M]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            g.capture_begin()
            sc.decode(0, z, x, y, stream=s)
            g.capture_end()
        graphs[M] = g
    torch.cuda.synchronize()
    stepper = GpuStepper(sc)
    for t in range(30):
        M = Ms[t % len(Ms)]
        z, x, y = bufs[M]
        zh = rng.standard_normal((M, E)).astype(np.float32)
        zh[:, :3] += 1.0
        xh = activations(cfg, 0, 700 + t, M)
        z.copy_(torch.from_numpy(zh))
        x.copy_(torch.from_numpy(xh.view(np.int16)))
        graphs[M].replay()
        torch.cuda.synchronize()
        y_o, rec, ids_o, w_o = orc.decode(zh, xh)
        check_output(y.cpu().numpy(), y_o, (t, M))
        if M > 16:
            assert rec.bypass
        assert [tuple(e[1:]) for e in stepper.new_events()] == rec.events, (t, M)
        _check_state(sc, 0, orc.state)
        _ = (y * 2).sum().item()     # unrelated eager work between replays
    _check_counters(sc, 0, orc.state)
    st = sc.stats(0)
    log("graph multi-row: stats %s" % st)
    assert st["bypass_steps"] >= 10 and st["misses"] > 0
    sc.close()

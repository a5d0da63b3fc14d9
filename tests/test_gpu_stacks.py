"""GPU parity on the multi-layer workloads: the 75-layer GLM-shaped stack (M=1,
128 slots per layer) and the 42-layer Flash-shaped stack (M=8 streams, 54 slots
per layer).  Every layer's miss/eviction log and final slot map must equal the
oracle's replay of the same routing; outputs are checked on sampled
layer-steps.  Host backing banks are shared round-robin by the layers (layer l
reads bank l mod n_banks), which changes weight values but not bytes moved or
bookkeeping."""
import time

import numpy as np
import pytest

from oracle import OracleLayer, route, static_pin_hit_rate
from oracle.lru import SlotState
from synth import CONFIGS, activations, global_scales, routing_trace

from gpu_util import OracleBlobs, check_output, log, make_cache, torch_cuda

pytestmark = pytest.mark.gpu


def _oracle_replay(cfg, logits_l, rows):
    st = SlotState(cfg.n_experts, cfg.slots, cfg.top_k)
    events, uniques = [], []
    for t in range(logits_l.shape[0]):
        ids, _ = route(logits_l[t, :rows], cfg.top_k)
        rec = st.step(ids)
        events += [(rec.step, e, s, old) for e, s, old in rec.events]
        uniques.append(rec.uniques)
    return st, events, uniques


def _run_stack(cfg, n_layers, n_banks, steps, samples, event_capacity=0):
    import gc
    torch = torch_cuda()
    gc.collect()
    torch.cuda.empty_cache()      # the stack's slot pool is one large allocation
    M = cfg.rows
    t0 = time.time()
    sc = make_cache(cfg, n_layers=n_layers, slots=cfg.slots, max_rows=M, n_banks=n_banks,
                    event_capacity=event_capacity)
    log("%s: %d layers x %d slots bound, %d banks filled in %.1f s" % (cfg.name, n_layers, cfg.slots, n_banks,
                                                                       time.time() - t0))
    traces = [routing_trace(cfg, l, steps=steps)[0][:, :M] for l in range(n_layers)]
    d_logits = torch.from_numpy(np.stack(traces)).cuda()                      # [L, T, M, E]
    xs = np.stack([activations(cfg, 0, t, M) for t in range(steps)])          # shared by the layers
    d_x = torch.from_numpy(xs.view(np.int16)).cuda()
    y = torch.empty((M, cfg.hidden), dtype=torch.float32, device="cuda")
    kept = {}
    for t in range(steps):
        for l in range(n_layers):
            sc.decode(l, d_logits[l, t], d_x[t], y)
            if (l, t) in samples:
                kept[(l, t)] = y.cpu().numpy()
        if t % 16 == 15:
            torch.cuda.synchronize()
            log("  step %d/%d (%.1f s)" % (t + 1, steps, time.time() - t0))
    torch.cuda.synchronize()
    return sc, traces, xs, kept


def _check_layers(cfg, sc, traces, n_layers, keep_uniques=None):
    M = cfg.rows
    hits = lookups = 0
    for l in range(n_layers):
        st, events, uniques = _oracle_replay(cfg, traces[l], M)
        if keep_uniques is not None:
            keep_uniques.append(uniques)
        ev_gpu, total = sc.read_events(l)
        assert total == len(events) and len(ev_gpu) == total, (l, total, len(events))   # the ring did not wrap
        assert ev_gpu == events, l
        e2s, s2e, key, step = sc.read_state(l)
        assert list(e2s) == st.e2s and list(s2e) == st.s2e and list(key) == st.key and step == st.t, l
        c = sc.stats(l)
        assert c["misses"] == st.counters.misses and c["hits"] == st.counters.hits, l
        assert c["bypass_steps"] == st.counters.bypass_steps and c["device_error"] == 0, l
        hits += c["hits"]
        lookups += c["lookups"]
    return hits / lookups


def _check_samples(cfg, kept, traces, xs, n_banks):
    worst = 0.0
    for (l, t), y in kept.items():
        bank = l % n_banks
        orc = OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots,
                          OracleBlobs(cfg, bank=bank), global_scales(cfg, bank, "unit"), keep_slot_bytes=False)
        y_o = orc.all_resident_output(traces[l][t], xs[t])
        r = check_output(y, y_o, (l, t))
        worst = max(worst, r)
    return worst


@pytest.mark.timeout(1200)
def test_glm_75_layer_stack():
    cfg = CONFIGS["glm_stack"]
    L, banks, steps = cfg.n_layers, 4, cfg.steps
    log("GLM stack: %d layers, S=%d, M=1, %d steps, %d host banks" % (L, cfg.slots, steps, banks))
    samples = {(0, 3), (37, 100), (74, steps - 1)}
    sc, traces, xs, kept = _run_stack(cfg, L, banks, steps, samples)
    hit = _check_layers(cfg, sc, traces, L)
    worst = _check_samples(cfg, kept, traces, xs, banks)
    log("GLM stack: bookkeeping exact on %d layer-steps, LRU hit %.4f, worst rel L2 %.2e" % (L * steps, hit, worst))
    sc.close()


@pytest.mark.timeout(1200)
def test_flash_stack_m8():
    cfg = CONFIGS["flash"]
    L, banks, steps = cfg.n_layers, 4, cfg.steps
    log("Flash stack: %d layers, S=%d, M=%d, %d steps, %d host banks" % (L, cfg.slots, cfg.rows, steps, banks))
    samples = {(0, 5), (20, 257), (41, steps - 1)}
    # about 18 misses per layer-step: the event ring holds the whole run
    sc, traces, xs, kept = _run_stack(cfg, L, banks, steps, samples, event_capacity=16384)
    uniq = []
    hit = _check_layers(cfg, sc, traces, L, uniq)
    worst = _check_samples(cfg, kept, traces, xs, banks)
    # the pages' comparator: a hindsight-optimal static pin of S experts per layer
    pin = np.mean([static_pin_hit_rate(uniq[l], cfg.n_experts, cfg.slots) for l in range(L)])
    log("Flash stack: bookkeeping exact on %d layer-steps, LRU hit %.4f (static pin %.4f), worst rel L2 %.2e"
        % (L * steps, hit, pin, worst))
    sc.close()

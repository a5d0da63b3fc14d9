"""Benchmark: microseconds per MoE layer-step of the expert-slot decode path on one MI355X.

Headline (`value`): the GLM-shaped MoE layer -- H 6144, I 2048, 256 experts,
top-8, 128 HBM slots, M=1 decode rows, NVFP4 weights, Zipf(1.1)-skewed routing
with AR(1) drift -- at its LRU hit rate, misses and their host-link fills
included.  A step is one moe_layer_decode call: routing + remap/LRU, miss fills
from the pinned host store, gate/up and down FP4 GEMVs, combine.  After a
32-step cache warm-up and `--warmup` untimed steps the layer state is
snapshotted; an eager pass over the `--steps` timed steps gives the per-step
spread and per-kernel spans; then the state is restored and a HIP-graph replay
of the same steps, each after a 512 MiB read sweep that evicts the 256 MiB
Infinity Cache, minus a replay of the sweeps alone, gives the mean.  The replay
takes exactly the eager pass's misses (checked).

Beside it: an all-hit block (every expert resident, S = E; the gate/up and
down GEMV rooflines over at least 100 launches), the host link's measured DMA
ceiling, the drafted-rows workload, and the oracle on a bounded CPU sample.
`--config glm_stack` / `--config flash` time the 75- and 42-layer stacks
instead.  Prints one JSON line per workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MoE layer-step (M=1) + achieved HBM GB/s vs peak; LRU hit rate"
HBM_PEAK_GBS = 8000.0
PHASES = ("route_remap", "fill", "gateup", "down", "combine")
# kernels of a one-row GLM step, as rocprofv3 names them (template arguments included)
KERNEL_NAMES = {"route_remap": "k_route_one<4, 4>", "fill": "k_fill(", "gateup": "k_gemv<6144, 1, 1, true, true>",
                "down": "k_gemv<2048, 1, 4, false, true>", "combine": "k_combine("}
CACHE_WARMUP = 32          # steps that fill the cache before anything is measured
ALL_HIT_WARM = 4           # untimed all-hit steps before the timed ones
ALL_HIT_MIN = 100          # timed all-hit launches, at least


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's own length: 300 for glm, 64 for tiny, "
                         "512 for the stacks)")
    ap.add_argument("--warmup", type=int, default=32,
                    help="untimed steps after the 32-step cache warm-up")
    ap.add_argument("--config", default="glm", choices=("glm", "tiny", "glm_stack", "flash"))
    ap.add_argument("--reps", type=int, default=3, help="timed graph replays of the headline (state restored each)")
    ap.add_argument("--no-flush", action="store_true", help="back-to-back steps (Infinity Cache may serve repeats)")
    ap.add_argument("--cpu-baseline-steps", type=int, default=10,
                    help="consecutive one-row GLM steps the oracle's full math is timed on (about 1 s each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-hit", action="store_true", help="skip the all-hit block")
    ap.add_argument("--no-drafted", action="store_true",
                    help="skip the drafted-rows workload (GLM layer, M = 4 / 16 / 64 schedule) in the default run")
    ap.add_argument("--no-link", action="store_true", help="skip the host-link DMA ceiling measurement")
    ap.add_argument("--no-overlap-compare", action="store_true",
                    help="skip the second pass of the churning workload with the overlapped miss fill "
                         "(SC_FLAG_OVERLAP_FILL) in the default run")
    ap.add_argument("--banks", type=int, default=4, help="host backing banks of the stack workloads")
    ap.add_argument("--no-static", action="store_true", help="stack workloads: skip the static-pin comparator pass")
    ap.add_argument("--sweep-rows", default="",
                    help="comma-separated M values: all-hit GLM layer (every expert resident), drafted rows; "
                         "prints one JSON line per M instead of the headline line")
    ap.add_argument("--prefill", action="store_true",
                    help="only time M=64 prefill chunks on the GLM layer (128 slots warmed by 64 one-row steps), "
                         "staged 64 experts at a time and read in place; prints one JSON line")
    ap.add_argument("--link-ceiling", action="store_true",
                    help="only measure the host link: DMA copies between pinned host memory and HBM on a side "
                         "stream, and the fill kernel's zero-copy reads on steps that miss every expert")
    ap.add_argument("--overlap-fill", action="store_true",
                    help="one-row steps copy their misses while the resident experts' gate/up runs in the same "
                         "launch (SC_FLAG_OVERLAP_FILL); the roofline is then that shared launch's product blocks. "
                         "Applies to the default M=1 workload (the flag changes nothing for steps of several rows)")
    ap.add_argument("--dump-steps", default="",
                    help="write the all-hit block's launch counts and per-launch spans to this JSON file "
                         "(input of --trace-summary)")
    ap.add_argument("--pmc-summary", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/pmc_gateup_glm_m1.json and pmc_down_glm_m1.json from the rocprofv3 "
                         "--pmc counter files of a bench run and of the --calibrate-copy run")
    ap.add_argument("--trace-summary", nargs=3, metavar=("KERNEL_TRACE_CSV", "KERNEL_STATS_CSV", "STEPS_JSON"),
                    help="only summarize a rocprofv3 kernel trace of this bench: each kernel's duration over "
                         "the all-hit block's timed launches listed by --dump-steps (written to "
                         "profiles/dur_allhit_glm_m1.json), and the run's kernel statistics (written to "
                         "profiles/glm_m1_decode_step_kernels.md)")
    ap.add_argument("--sweep-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "SWEEP_OUTPUT"),
                    help="only summarize a rocprofv3 kernel trace of a --sweep-rows run (its JSON lines in "
                         "SWEEP_OUTPUT): each kernel's duration per M, written to "
                         "profiles/glm_drafted_rows_kernels.md")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (counter calibration)")
    a = ap.parse_args()
    if a.steps is None:
        a.steps = {"glm": 300, "tiny": 64, "glm_stack": 512, "flash": 512}[a.config]
    return a


DUR_FILE = os.path.join(ROOT, "profiles", "dur_allhit_glm_m1.json")


def rocprof_duration(src_hash):
    """rocprofv3 durations of the all-hit block's timed launches of a profiled bench run, if
    it was taken on the current kernel source; else None."""
    try:
        d = json.load(open(DUR_FILE))
    except Exception:
        return None
    return d if d.get("source_sha256") == src_hash else None


def pmc_traffic(kernel_key, src_hash):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_%s.json" % kernel_key)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("source_sha256") != src_hash:
        return None
    return d.get("bytes_per_launch")


def code_text(src):
    """Source text with comments and whitespace runs removed: edits to comments do not
    change it, edits to code do."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash():
    """Hash of the GEMV kernels' code, the key of the committed counter and duration summaries."""
    import hashlib
    h = hashlib.sha256()
    for f in ("expert_gemv.hip", "internal.h"):
        h.update(code_text(open(os.path.join(ROOT, "hbm_expert_slot_amd", "csrc", f)).read()).encode())
    return h.hexdigest()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


def cpu_baseline(glm_logits, glm_xs, start, nsteps):
    """The oracle, as it stands, on bounded samples of the workloads' own inputs.

    value: full fp64 step (routing, LRU, dequant, expert math) on `nsteps`
    consecutive one-row GLM steps.  Beside it: the tiny layer's full step on all
    its 64 steps, the Flash stack's expert math on one fixed layer-step, and bookkeeping alone (routing + slot bookkeeping) per
    layer-step on every workload (the stacks on a sample of layers)."""
    from oracle import OracleLayer, route
    from oracle.lru import SlotState
    from synth import CONFIGS, activations, expert_blob, expert_blobs, global_scales, routing_trace
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = 1
    glm = CONFIGS["glm"]
    # input generation (blob bytes) is not oracle work: stage them first
    need = set()
    for t in range(start, start + nsteps):
        ids, _ = route(glm_logits[t, :1], glm.top_k)
        need |= set(int(e) for e in ids.reshape(-1))
    blobs = {e: expert_blob(glm, 0, e) for e in sorted(need)}
    orc = OracleLayer(glm.hidden, glm.inter, glm.n_experts, glm.top_k, glm.slots, lambda e: blobs[e],
                      global_scales(glm, 0, "unit"), keep_slot_bytes=False)
    t0 = time.perf_counter()
    for t in range(start, start + nsteps):
        orc.decode(glm_logits[t, :1], glm_xs[t])
    full = (time.perf_counter() - t0) / nsteps

    tiny = CONFIGS["tiny"]
    tb = expert_blobs(tiny, 0)
    tl, tr = routing_trace(tiny, 0)
    to = OracleLayer(tiny.hidden, tiny.inter, tiny.n_experts, tiny.top_k, tiny.slots, lambda e: tb[e],
                     global_scales(tiny, 0, "unit"), keep_slot_bytes=False)
    txs = [activations(tiny, 0, t, 1) for t in range(tiny.steps)]
    t0 = time.perf_counter()
    for t in range(tiny.steps):
        to.decode(tl[t, :1], txs[t])
    tiny_full = (time.perf_counter() - t0) / tiny.steps

    def bookkeeping(cfg, layers, steps):
        traces = [routing_trace(cfg, l, steps=steps) for l in range(layers)]
        t0 = time.perf_counter()
        n = 0
        for lg, rows in traces:
            st = SlotState(cfg.n_experts, cfg.slots, cfg.top_k)
            for t in range(steps):
                ids, _ = route(lg[t, :rows[t]], cfg.top_k)
                st.step(ids)
                n += 1
        return {"us_per_layer_step": round((time.perf_counter() - t0) / n * 1e6, 1), "layer_steps": n,
                "sample": "%d of %d layers x %d steps" % (layers, cfg.n_layers, steps) if cfg.n_layers > 1
                          else "all %d steps" % steps}

    # the Flash stack's expert math (M = 8) on a fixed sample: step 63 of layer 0
    from oracle.expert import layer_output
    fl = CONFIGS["flash"]
    fl_us = []
    for layer in (0,):
        lg, rows = routing_trace(fl, layer, steps=64)
        M = int(rows[63])
        ids, w = route(lg[63, :M], fl.top_k)
        fb = {e: expert_blob(fl, layer, e) for e in sorted(set(int(v) for v in ids.reshape(-1)))}
        xb = activations(fl, layer, 63, M)
        gsf = global_scales(fl, layer, "unit")
        t0 = time.perf_counter()
        layer_output(ids, w, xb, lambda e: fb[e], gsf, fl.hidden, fl.inter)
        fl_us.append((time.perf_counter() - t0) * 1e6)

    bk = {"tiny": bookkeeping(tiny, 1, tiny.steps), "glm": bookkeeping(glm, 1, glm.steps),
          "glm_draft": bookkeeping(CONFIGS["glm_draft"], 1, CONFIGS["glm_draft"].steps),
          "glm_stack": bookkeeping(CONFIGS["glm_stack"], 4, CONFIGS["glm_stack"].steps),
          "flash": bookkeeping(CONFIGS["flash"], 2, CONFIGS["flash"].steps)}
    return {
        "value": round(full * 1e6, 1), "unit": "us/layer-step", "cores": int(threads), "kind": "oracle",
        "sample": "%d consecutive M=1 steps of the GLM trace after its warm-up (full fp64 step: routing, LRU, "
                  "dequant, expert math); blob generation excluded" % nsteps,
        "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
        "tiny_full_step_us": {"us_per_layer_step": round(tiny_full * 1e6, 1), "sample": "all 64 steps"},
        "flash_expert_math_us": {"us_per_layer_step": round(float(np.mean(fl_us)), 1),
                                 "sample": "step 63 of layer 0 (M = 8): dequant and expert math of the "
                                           "step's unique experts, blob generation excluded; the GLM stack's "
                                           "layers have the GLM layer's shape, whose full step is `value`"},
        "bookkeeping_only": bk,
    }


def _sweep(torch, dev):
    """A 512 MiB read-only sweep whose result lands in one float: it evicts the 256 MiB
    Infinity Cache between steps (clean lines, nothing written back)."""
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    return lambda: sink.copy_(flush.amax())


def _graph_us(torch, dev, step_fns, sweep, no_flush):
    """Capture the steps (each after the sweep) and the sweeps alone into two HIP graphs;
    returns a function that replays both once and gives (steps_ms, sweeps_ms)."""
    gstream = torch.cuda.Stream(dev)
    g_steps, g_sweeps = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(gstream):
        g_steps.capture_begin()
        for fn in step_fns:
            if not no_flush:
                sweep()
            fn(gstream)
        g_steps.capture_end()
        g_sweeps.capture_begin()
        for _ in step_fns:
            if not no_flush:
                sweep()
        g_sweeps.capture_end()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def timed(g):
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ga.record(stream)
        g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        return ga.elapsed_time(gb)

    def run():
        sw = timed(g_sweeps) if not no_flush else 0.0
        return timed(g_steps), sw

    return run, g_steps, g_sweeps


def _eager_timed(torch, dev, sc, steps, sweep, no_flush):
    """Eager pass, one step at a time after the sweep: per step, the step time from HIP
    events (routing kernel start to combine end), each kernel's event-pair time and its
    execution span from the kernels' own device-clock stamps."""
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(PHASES))]
    for ev in evs:          # torch creates the HIP event on first record
        ev.record(stream)
    torch.cuda.synchronize()
    step_us, ev_us, spans = [], [], []
    for fn in steps:
        if not no_flush:
            sweep()
        fn(stream, evs)
        spans.append(sc.kernel_spans())       # synchronizes: one step at a time
        step_us.append(evs[0].elapsed_time(evs[-1]) * 1e3)
        ev_us.append([evs[2 * j].elapsed_time(evs[2 * j + 1]) * 1e3 for j in range(len(PHASES))])
    return np.array(step_us), np.array(ev_us), np.array(spans)


def _stats_delta(s1, s0):
    return {n: s1[n] - s0[n] for n in ("steps", "bypass_steps", "lookups", "hits", "misses", "bytes_filled",
                                       "bypass_bytes")}


def _pct(v):
    v = np.asarray(v, dtype=np.float64)
    return {"mean": round(float(np.mean(v)), 3), "p10": round(float(np.percentile(v, 10)), 3),
            "p50": round(float(np.percentile(v, 50)), 3), "p90": round(float(np.percentile(v, 90)), 3)}


def all_hit_block(a, torch, env):
    """Every expert of the GLM layer resident (S = E, preloaded): the one-row step and its
    GEMVs at HBM speed, over at least 100 launches on the same routing trace.  Each
    step follows the cache sweep (the Infinity Cache holds a whole 170 MB step)."""
    SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace = env
    cfg = CONFIGS["glm"]
    dev = torch.device("cuda:0")
    N = max(ALL_HIT_MIN, a.steps if a.config == "glm" else 0)
    Wa = ALL_HIT_WARM
    sc = SlotCache(1, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_experts, 1,
                   overlap_fill=a.overlap_fill)
    expert_blobs(cfg, 0, out=sc.backing(0))
    sc.set_global_scales(0, global_scales(cfg, 0, "unit"))
    sc.preload(0)
    logits, _ = routing_trace(cfg, 0, steps=Wa + N)
    xs = np.stack([activations(cfg, 0, t, 1) for t in range(Wa + N)])
    d_l = torch.from_numpy(logits[:, :1].copy()).to(dev)
    d_x = torch.from_numpy(xs.view(np.int16)).to(dev)
    d_y = torch.empty((Wa + N, 1, cfg.hidden), dtype=torch.float32, device=dev)
    sweep = _sweep(torch, dev)
    for t in range(Wa):
        sc.decode(0, d_l[t], d_x[t], d_y[t])
    torch.cuda.synchronize()
    st0 = sc.stats(0)
    step_us, ev_us, spans = _eager_timed(
        torch, dev, sc,
        [(lambda s, e, t=t: sc.decode(0, d_l[t], d_x[t], d_y[t], stream=s, events=e)) for t in range(Wa, Wa + N)],
        sweep, a.no_flush)
    st1 = sc.stats(0)
    d = _stats_delta(st1, st0)
    assert d["misses"] == 0 and d["hits"] == d["lookups"] == N * cfg.top_k, d
    run, _, _ = _graph_us(torch, dev, [(lambda s, t=t: sc.decode(0, d_l[t], d_x[t], d_y[t], stream=s))
                                       for t in range(Wa, Wa + N)], sweep, a.no_flush)
    run()                     # the first replay uploads the graphs
    reps = [run() for _ in range(3)]
    graph_us = sorted((st - sw) * 1e3 / N for st, sw in reps)[1]
    sc.close()
    kus = {p: float(np.mean(spans[:, j])) for j, p in enumerate(PHASES)}
    gb, db = gemv_bytes(cfg)
    src = source_hash()
    dur = None if a.overlap_fill else rocprof_duration(src)
    if a.dump_steps:
        json.dump({"all_hit_warm": Wa, "all_hit_timed": N, "kernel_names": KERNEL_NAMES,
                   "spans_us": {p: [float(v) for v in spans[:, j]] for j, p in enumerate(PHASES)},
                   "events_us": {p: [float(v) for v in ev_us[:, j]] for j, p in enumerate(PHASES)}},
                  open(a.dump_steps, "w"))

    def roof(bytes_, us_live, kernel, rp_us):
        # frac follows the committed rocprofv3 durations of this kernel source when they exist (the
        # dispatch window includes the wave launch and retirement that the kernels' own stamps do
        # not); otherwise the live device-clock spans
        us = rp_us if rp_us else us_live
        return {"kernel": kernel, "bound": "hbm",
                "achieved": round(bytes_ / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(bytes_ / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": bytes_, "avg_launch_us": round(us, 3),
                "duration": ("rocprofv3 dispatch duration over the all-hit block's %d timed launches (%s)"
                             % (dur["timed_launches"], os.path.relpath(DUR_FILE, ROOT))) if rp_us else
                            "mean of the kernel's own execution spans over %d all-hit launches (device wall "
                            "clock, first block start to last wavefront end)" % N,
                "live_spans_us": round(us_live, 3), "live_spans_frac": round(bytes_ / (us_live * 1e-6) / 1e9 /
                                                                              HBM_PEAK_GBS, 4)}

    rp = (dur or {}).get("rocprof_avg_us", {})
    gu_k = ("k_fill_gateup<%d> (product blocks)" % cfg.hidden) if a.overlap_fill else KERNEL_NAMES["gateup"]
    roof_gu = roof(gb, kus["gateup"], gu_k, rp.get("gateup"))
    roof_gu["traffic"] = None if a.overlap_fill else pmc_traffic("gateup_glm_m1", src)
    roof_dn = roof(db, kus["down"], KERNEL_NAMES["down"], rp.get("down"))
    roof_dn["traffic"] = None if a.overlap_fill else pmc_traffic("down_glm_m1", src)
    pair_us = roof_gu["avg_launch_us"] + roof_dn["avg_launch_us"]
    out = {
        "workload": "GLM-shaped MoE layer, every expert resident (S = E = 256, preloaded), M=1, %d steps of the "
                    "same routing trace after %d untimed ones, each after the cache sweep" % (N, Wa),
        "us_per_layer_step_graph": round(graph_us, 3),
        "graph_reps_us": [round((st - sw) * 1e3 / N, 3) for st, sw in reps],
        "step_us_eager": _pct(step_us),
        "kernels_us": {p: round(v, 3) for p, v in kus.items()},
        "kernels_us_events": {p: round(float(np.mean(ev_us[:, j])), 3) for j, p in enumerate(PHASES)},
        "kernels_us_rocprof": rp or None,
        "gateup": roof_gu, "down": roof_dn,
        "gemv_pair": {"bytes": gb + db, "us": round(pair_us, 3),
                      "achieved_GBs": round((gb + db) / (pair_us * 1e-6) / 1e9, 1),
                      "frac": round((gb + db) / (pair_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "target_us": round((gb + db) / (0.7 * HBM_PEAK_GBS * 1e9) * 1e6, 2)},
        "step_frac": round(169_869_312 / (graph_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }
    return out


def churn_headline(a, torch, env):
    """The configured workload at its LRU hit rate (see the module docstring)."""
    SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace = env
    cfg = CONFIGS[a.config]
    dev = torch.device("cuda:0")
    CW, W, K = CACHE_WARMUP, a.warmup, a.steps
    T0 = CW + W
    sc = SlotCache(1, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, 1, overlap_fill=a.overlap_fill)
    t0 = time.time()
    expert_blobs(cfg, 0, out=sc.backing(0))
    sc.set_global_scales(0, global_scales(cfg, 0, "unit"))
    print("bench: backing filled in %.1f s" % (time.time() - t0), file=sys.stderr, flush=True)
    logits, _ = routing_trace(cfg, 0, steps=T0 + K)
    xs = np.stack([activations(cfg, 0, t, 1) for t in range(T0 + K)])
    d_l = torch.from_numpy(logits[:, :1].copy()).to(dev)
    d_x = torch.from_numpy(xs.view(np.int16)).to(dev)
    d_y = torch.empty((T0 + K, 1, cfg.hidden), dtype=torch.float32, device=dev)
    sweep = _sweep(torch, dev)
    for t in range(T0):
        sc.decode(0, d_l[t], d_x[t], d_y[t])
    torch.cuda.synchronize()
    snap = sc.read_state(0)
    st0 = sc.stats(0)
    ev0 = sc.read_events(0)[1]
    # eager pass over the timed steps: per-step spread and per-kernel spans
    wall0 = time.perf_counter()
    step_us, ev_us, spans = _eager_timed(
        torch, dev, sc,
        [(lambda s, e, t=t: sc.decode(0, d_l[t], d_x[t], d_y[t], stream=s, events=e)) for t in range(T0, T0 + K)],
        sweep, a.no_flush)
    wall = time.perf_counter() - wall0
    st1 = sc.stats(0)
    eager = _stats_delta(st1, st0)
    events, total = sc.read_events(0)
    miss_steps = set(e[0] for e in events[len(events) - (total - ev0):]) if total > ev0 else set()
    miss_idx = [i for i in range(K) if T0 + i in miss_steps]
    # graph replay of the same steps from the same state: the same misses
    run, _, _ = _graph_us(torch, dev, [(lambda s, t=t: sc.decode(0, d_l[t], d_x[t], d_y[t], stream=s))
                                       for t in range(T0, T0 + K)], sweep, a.no_flush)

    def restore():
        sc.write_state(0, *snap)
        torch.cuda.synchronize()

    restore()
    run()                      # the first replay uploads the graphs
    reps = []
    for _ in range(max(1, a.reps)):
        restore()
        s0 = sc.stats(0)
        st_ms, sw_ms = run()
        g = _stats_delta(sc.stats(0), s0)
        for n in ("lookups", "hits", "misses", "bytes_filled", "bypass_steps"):
            if g[n] != eager[n]:
                raise SystemExit("graph replay diverged from the eager pass: %s %d against %d" % (n, g[n], eager[n]))
        reps.append((st_ms - sw_ms) * 1e3 / K)
    value = float(np.median(reps))
    sc.close()
    fill = spans[:, PHASES.index("fill")]
    fill_us_miss = float(np.sum(fill[miss_idx])) if miss_idx else 0.0
    hit_idx = [i for i in range(K) if i not in set(miss_idx)]
    return {
        "value": value, "reps_us": [round(v, 3) for v in reps], "wall_s_eager": wall,
        "lru": {"hit_rate": round(eager["hits"] / eager["lookups"], 4) if eager["lookups"] else None,
                "misses_per_step": eager["misses"] / K, "lookups": eager["lookups"], "hits": eager["hits"],
                "misses": eager["misses"], "miss_steps": len(miss_idx), "all_hit_steps": len(hit_idx),
                "graph_replay_misses": eager["misses"]},
        "step_us_eager": _pct(step_us),
        "step_us_eager_all_hit_steps": _pct(step_us[hit_idx]) if hit_idx else None,
        "step_us_eager_miss_steps": _pct(step_us[miss_idx]) if miss_idx else None,
        "kernels_us": {p: round(float(np.mean(spans[:, j])), 3) for j, p in enumerate(PHASES)},
        "fill": {"bytes_filled": eager["bytes_filled"], "fill_us_on_miss_steps": round(fill_us_miss, 1),
                 "achieved_GBs": round(eager["bytes_filled"] / (fill_us_miss * 1e-6) / 1e9, 2)
                 if fill_us_miss > 0 else None},
        "cfg": cfg,
    }


def link_ceiling(torch, nbytes=1 << 30, reps=5):
    """The host link's DMA ceiling: hipMemcpyAsync between pinned host memory (hipHostMalloc,
    through torch's pinned allocator) and HBM on a side stream, 1 GiB per copy."""
    dev = torch.device("cuda:0")
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    host.fill_(7)
    devbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream(dev)
    out = {}
    for name, dst, src in (("h2d", devbuf, host), ("d2h", host, devbuf)):
        times = []
        with torch.cuda.stream(s):
            dst.copy_(src, non_blocking=True)
            s.synchronize()
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                dst.copy_(src, non_blocking=True)
                e1.record(s)
                s.synchronize()
                times.append(e0.elapsed_time(e1))
        out[name + "_GBs"] = round(nbytes / (float(np.median(times)) * 1e-3) / 1e9, 2)
    del host, devbuf
    out["method"] = ("hipMemcpyAsync of 1 GiB between pinned host memory and HBM on a side stream, median of "
                     "%d copies after one untimed" % reps)
    return out


def zero_copy_fill(torch, env, steps=12):
    """The fill kernel's host-link rate on steps that miss all eight experts: 8 slots, and
    each step's picks are eight experts no slot holds (168 MB over the link per step)."""
    SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace = env
    cfg = CONFIGS["glm"]
    dev = torch.device("cuda:0")
    k = cfg.top_k
    sc = SlotCache(1, cfg.hidden, cfg.inter, cfg.n_experts, k, k, 1)
    expert_blobs(cfg, 0, range(cfg.n_experts), out=sc.backing(0))
    z = np.full((steps, 1, cfg.n_experts), -10.0, dtype=np.float32)
    for t in range(steps):
        z[t, 0, (np.arange(k) + t * k) % cfg.n_experts] = 10.0 - np.arange(k)
    d_l = torch.from_numpy(z).to(dev)
    d_x = torch.from_numpy(activations(cfg, 0, 0, 1).view(np.int16)).to(dev)
    y = torch.empty((1, cfg.hidden), dtype=torch.float32, device=dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(PHASES))]
    stream = torch.cuda.current_stream(dev)
    for ev in evs:
        ev.record(stream)
    fills = []
    for t in range(steps):
        sc.decode(0, d_l[t], d_x, y, events=evs)
        fills.append(sc.kernel_spans()[PHASES.index("fill")])
    st = sc.stats(0)
    sc.close()
    assert st["misses"] == steps * k, st
    us = float(np.median(fills[2:]))
    return {"GBs": round(k * sc.blob_bytes / (us * 1e-6) / 1e9, 2), "fill_us_per_step": round(us, 1),
            "bytes_per_step": k * sc.blob_bytes,
            "method": "fill kernel span (device clock) on one-row GLM steps that miss all %d experts; median of "
                      "%d steps after 2" % (k, steps - 2)}


def stack_workload(a, torch, env):
    """The 75-layer GLM stack (M=1) or the 42-layer Flash stack (M=8): every layer of a step
    in order, eager (the launches queue ahead of the GPU), timed from the first layer of the
    first timed step to the last layer of the last.  Rotating over the layers keeps any
    expert's two uses gigabytes apart, so no sweep is needed (Infinity Cache cold).  For
    the Flash stack the same steps are then replayed with the hindsight-optimal static pin
    (each layer's S experts that appear in the most steps of the whole run, pinned in every
    slot) and the GPU's counters give its resident fraction."""
    SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace = env
    import gc
    cfg = CONFIGS[a.config]
    dev = torch.device("cuda:0")
    L, M, banks = cfg.n_layers, cfg.rows, max(1, min(a.banks, cfg.n_layers))
    CW, W, K = CACHE_WARMUP, a.warmup, a.steps
    T = CW + W + K
    gc.collect()
    torch.cuda.empty_cache()
    t0 = time.time()
    sc = SlotCache(L, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, M, banks, event_capacity=64)
    for b in range(banks):
        expert_blobs(cfg, b, out=sc.backing(b))
        sc.set_global_scales(b, global_scales(cfg, b, "unit"))
    print("bench: %s bound (%d layers, %.1f GB of slots), %d banks filled in %.1f s"
          % (a.config, L, L * cfg.slots * sc.blob_bytes / 1e9, banks, time.time() - t0), file=sys.stderr, flush=True)
    traces = [routing_trace(cfg, l, steps=T)[0][:, :M] for l in range(L)]
    d_l = torch.from_numpy(np.stack(traces)).to(dev)                 # [L, T, M, E]
    d_x = torch.from_numpy(np.stack([activations(cfg, 0, t, M) for t in range(T)]).view(np.int16)).to(dev)
    y = torch.empty((M, cfg.hidden), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(t_lo, t_hi):
        for t in range(t_lo, t_hi):
            for l in range(L):
                sc.decode(l, d_l[l, t], d_x[t], y)
            if t % 16 == 15:
                torch.cuda.synchronize()
                print("bench:   step %d/%d" % (t + 1, T), file=sys.stderr, flush=True)

    def counters():
        tot = {}
        for l in range(L):
            for n, v in sc.stats(l).items():
                tot[n] = tot.get(n, 0) + v
        return tot

    run(0, CW + W)
    torch.cuda.synchronize()
    c0 = counters()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(CW + W, T)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    c1 = counters()
    d = _stats_delta(c1, c0)
    assert c1["device_error"] == 0
    n_ls = K * L
    out = {
        "workload": cfg.description,
        "us_per_layer_step": round(ms * 1e3 / n_ls, 2), "timed_layer_steps": n_ls,
        "untimed": "%d cache warm-up + %d warmup steps, every layer" % (CW, W),
        "hit_rate": round(d["hits"] / d["lookups"], 4) if d["lookups"] else None,
        "misses_per_layer_step": round(d["misses"] / n_ls, 3),
        "unique_experts_per_layer_step": round(d["lookups"] / max(1, n_ls - d["bypass_steps"]), 2),
        "bypass_layer_steps": d["bypass_steps"],
        "host_GB_per_layer_step": round((d["bytes_filled"] + d["bypass_bytes"]) / n_ls / 1e9, 4),
        "host_GBs": round((d["bytes_filled"] + d["bypass_bytes"]) / (ms * 1e-3) / 1e9, 2),
        "host_banks": "%d banks of %d experts, layer l reads bank l mod %d (weight values alias; bytes moved and "
                      "bookkeeping do not change)" % (banks, cfg.n_experts, banks),
        "timing": "eager, all layers of a step in order, HIP events around the %d timed steps" % K,
    }
    if a.config == "flash" and not a.no_static:
        # hindsight-optimal static pin over the whole run: per layer, the S experts that appear in the
        # most steps (ties to the lower id); every slot pinned, so a step whose experts are not all
        # pinned reads the others from the host store
        lookups_all = c1["lookups"]
        assert c1["bypass_steps"] == 0, "the LRU pass bypassed; its lookups do not cover every step"
        k = cfg.top_k
        for l in range(L):
            z = traces[l]
            order = np.argsort(-z, axis=-1, kind="stable")[..., :k]       # [T, M, k], ties -> lower id
            cnt = np.zeros(cfg.n_experts, np.int64)
            for t in range(T):
                cnt[np.unique(order[t])] += 1
            pins = np.lexsort((np.arange(cfg.n_experts), -cnt))[:cfg.slots]
            sc.pin(l, pins.astype(np.int32))
        s0 = counters()
        e0.record(stream)
        run(0, T)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_pin = e0.elapsed_time(e1)
        s1 = counters()
        dp = _stats_delta(s1, s0)
        nonres = dp["bypass_bytes"] // sc.blob_bytes
        lru_all = c1["hits"] / c1["lookups"]
        out["lru_vs_static_pin"] = {
            "steps": T, "lru_hit_rate": round(lru_all, 4),
            "static_pin_resident_fraction": round((lookups_all - nonres - dp["misses"]) / lookups_all, 4),
            "static_us_per_layer_step": round(ms_pin * 1e3 / (T * L), 2),
            "static_bypass_layer_steps": dp["bypass_steps"],
            "note": "both over all %d steps (cache warm-up included); the static pin is chosen in hindsight from "
                    "the same run's picks" % T}
    sc.close()
    return out


def sweep_rows(a, torch, SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace):
    """All-hit GLM layer (S = E, preloaded) at several M, drafted rows; graph replay, cache swept."""
    import dataclasses
    base = CONFIGS["glm_draft"]
    Ms = [int(v) for v in a.sweep_rows.split(",")]
    Mmax = max(Ms)
    dev = torch.device("cuda:0")
    sc = SlotCache(1, base.hidden, base.inter, base.n_experts, base.top_k, base.n_experts, Mmax)
    expert_blobs(base, 0, out=sc.backing(0))
    sc.set_global_scales(0, global_scales(base, 0, "unit"))
    sc.preload(0)
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    gstream = torch.cuda.Stream(dev)
    K = a.steps
    for M in Ms:
        cfg = dataclasses.replace(base, rows=M, schedule="fixed", drafted=M <= 16)
        logits, _ = routing_trace(cfg, 0, steps=K)
        xs = np.stack([activations(cfg, 0, t, M) for t in range(K)])
        d_l = torch.from_numpy(logits).to(dev)
        d_x = torch.from_numpy(xs.view(np.int16)).to(dev)
        d_y = torch.empty((K, M, cfg.hidden), dtype=torch.float32, device=dev)
        for t in range(min(K, 4)):
            sc.decode(0, d_l[t], d_x[t], d_y[t])
        torch.cuda.synchronize()
        st0 = sc.stats(0)
        graphs = []
        for with_steps in (True, False):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(gstream):
                g.capture_begin()
                for t in range(K):
                    sink.copy_(flush.amax())
                    if with_steps:
                        sc.decode(0, d_l[t], d_x[t], d_y[t], stream=gstream)
                g.capture_end()
            graphs.append(g)
        torch.cuda.synchronize()
        times = []
        for g in graphs:
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        st1 = sc.stats(0)
        us = (times[0] - times[1]) * 1e3 / K
        uniq = (st1["lookups"] - st0["lookups"]) / max(1, st1["steps"] - st0["steps"])
        byts = uniq * sc.blob_bytes
        # eager pass over the same steps: each kernel's execution span
        spans = []
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(PHASES))]
        for ev in evs:           # torch creates the HIP event on first record
            ev.record(stream)
        for t in range(K):
            sink.copy_(flush.amax())
            sc.decode(0, d_l[t], d_x[t], d_y[t], stream=stream, events=evs)
            spans.append(sc.kernel_spans())
        kus = np.mean(np.array(spans), axis=0)
        print(json.dumps({"sweep": "all-hit GLM layer, drafted rows", "M": M, "us_per_step": round(us, 2),
                          "unique_experts_per_step": round(uniq, 2), "weight_GBs": round(byts / (us * 1e-6) / 1e9, 1),
                          "kernels_us": {n: round(float(v), 2) for n, v in zip(PHASES, kus)}}), flush=True)
    sc.close()


def gemv_bytes(cfg):
    """Algorithmic bytes of the one-row gate/up and down launches: the U = k
    experts' weight codes and scales, the activation row, h written (gate/up)
    and read (down), the per-pick down outputs."""
    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    U = k  # M=1: the k picks are distinct experts
    gateup = U * (2 * I * H // 2 + 2 * I * H // 16) + H * 2 + k * I * 4
    down = U * (H * I // 2 + H * I // 16) + k * I * 4 + k * H * 4
    return gateup, down


PMC_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/gpurun_out/pmc_fetch "
    "-o run -- python3 -u $REPO/bench.py --steps 20 --warmup 4 --no-cpu-baseline",
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/gpurun_out/pmc_write "
    "-o run -- python3 -u $REPO/bench.py --steps 20 --warmup 4 --no-cpu-baseline",
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/gpurun_out/pmc_fetch_copy "
    "-o run -- python3 -u $REPO/bench.py --calibrate-copy",
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/gpurun_out/pmc_write_copy "
    "-o run -- python3 -u $REPO/bench.py --calibrate-copy",
    "cd $REPO && python3 bench.py --pmc-summary gpurun_out/pmc_fetch/run_counter_collection.csv "
    "gpurun_out/pmc_write/run_counter_collection.csv gpurun_out/pmc_fetch_copy/run_counter_collection.csv "
    "gpurun_out/pmc_write_copy/run_counter_collection.csv",
]


def pmc_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per launch of the one-row GEMVs from rocprofv3 counters.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the counter's
    instances) come from separate runs; each is scaled by what the same
    counter reads for a plain 1 GiB device copy (--calibrate-copy), and the
    median over a kernel's dispatches is kept.  The result carries the sha256
    of the kernel source so that the bench reports it only for that source."""
    import csv
    import statistics

    def per_dispatch(path, counter, name_part):
        by, full = {}, None
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                by[r["Dispatch_Id"]] = by.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
                full = full or r["Kernel_Name"]
        return list(by.values()), full

    gib = 1 << 30
    cf = max(per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")[0])
    cw = max(per_dispatch(copy_write_csv, "WRITE_SIZE", "copyBuffer")[0])
    ff, wf = cf * 1024 / gib, cw * 1024 / gib
    from synth import CONFIGS
    gb, db = gemv_bytes(CONFIGS["glm"])
    src = source_hash()
    table = []
    for key, name, algo in (("gateup_glm_m1", KERNEL_NAMES["gateup"], gb), ("down_glm_m1", KERNEL_NAMES["down"], db)):
        f, full = per_dispatch(fetch_csv, "FETCH_SIZE", name)
        w, _ = per_dispatch(write_csv, "WRITE_SIZE", name)
        if not f or not w:
            raise SystemExit("no %s dispatches of %s in the counter files" % ("FETCH_SIZE" if not f else "WRITE_SIZE", name))
        fm, wm = statistics.median(f), statistics.median(w)
        bpl = int(round(fm * 1024 / ff + wm * 1024 / wf))
        out = {"kernel": (full.split(">(")[0] + ">") if ">(" in full else full,
               "workload": "GLM-shaped MoE layer, H6144 I2048, 256 experts, top-8, 128 slots, M=1 "
                           "(bench.py --steps 20 --warmup 4)",
               "source_sha256": src, "fetch_size_kib_median": fm, "write_size_kib_median": wm, "dispatches": len(f),
               "calibration": {"kernel": "__amd_rocclr_copyBuffer (torch copy_ of 1 GiB)", "bytes_read": gib,
                               "bytes_written": gib, "fetch_size_kib": cf, "write_size_kib": cw,
                               "fetch_factor": ff, "write_factor": wf},
               "bytes_per_launch": bpl, "algorithmic_bytes_per_launch": algo,
               "traffic_over_algorithmic": bpl / algo, "commands": PMC_COMMANDS}
        with open(os.path.join(ROOT, "profiles", "pmc_%s.json" % key), "w") as fh:
            json.dump(out, fh, indent=1)
        print(key, out["kernel"], "bytes/launch", bpl, "ratio", round(bpl / algo, 4), "dispatches", len(f))
        table.append("| `%s` | %.1f | %.1f | %d | %d | %.4f |" % (kernel_label(full), fm, wm, bpl, algo, bpl / algo))
    L = ["# HBM traffic of the FP4 GEMV kernels (rocprofv3 counters), GLM layer M=1\n",
         "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, TCC) were taken in separate runs, then scaled by what the same "
         "counters read for a plain 1 GiB device copy (torch `copy_`, kernel `__amd_rocclr_copyBuffer`): FETCH_SIZE "
         "reads %.4f of the bytes read, WRITE_SIZE %.4f of the bytes written.  Medians over each kernel's one-row "
         "dispatches (%d per kernel) of a `bench.py --steps 20 --warmup 4` run.\n" % (ff, wf, len(f)),
         "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) | algorithmic bytes | ratio |",
         "|---|---|---|---|---|---|"] + table + [
         "", "`bench.py` reports these bytes as `roofline.traffic` while the GEMV source hash recorded in "
         "`pmc_gateup_glm_m1.json` / `pmc_down_glm_m1.json` matches.\n",
         "Commands (`$REPO` = repository root on the GPU host):\n", "```"] + PMC_COMMANDS + ["```"]
    with open(os.path.join(ROOT, "profiles", "pmc_gemv_glm_m1.md"), "w") as fh:
        fh.write("\n".join(L) + "\n")


def prefill(a, torch, SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace):
    """M=64 prefill chunks on the GLM layer (128 slots warmed by 64 one-row steps): resident
    experts come from their slots, the others are staged into HBM 64 at a time (the default)
    or read in place from pinned host memory (prefill_stage=0).  One JSON line."""
    cfg = CONFIGS["glm"]
    dev = torch.device("cuda:0")
    W, K, M = 64, min(a.steps, 20), 64
    logits, _ = routing_trace(cfg, 0, steps=W + K * M)
    d_l = torch.from_numpy(logits[:, :1].copy()).to(dev)          # [T, 1, E]
    x1 = torch.from_numpy(np.stack([activations(cfg, 0, t, 1) for t in range(W)]).view(np.int16)).to(dev)
    # a prefill chunk: the next 64 positions of the same routing stream, one row each
    chunks = [torch.from_numpy(logits[W + i * M:W + (i + 1) * M, 0].copy()).to(dev) for i in range(K)]
    xs = torch.from_numpy(activations(cfg, 0, 10_000, M).view(np.int16)).to(dev)
    out = {"prefill": "GLM layer, 128 slots warmed by %d one-row steps, then %d chunks of M=%d rows" % (W, K, M),
           "steps": K}
    ys = {}
    for G in (64, 0):
        sc = SlotCache(1, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, M, prefill_stage=G)
        expert_blobs(cfg, 0, out=sc.backing(0))
        sc.set_global_scales(0, global_scales(cfg, 0, "unit"))
        y = torch.empty((M, cfg.hidden), dtype=torch.float32, device=dev)
        for t in range(W):
            sc.decode(0, d_l[t], x1[t], y[:1])
        sc.decode(0, chunks[0], xs, y)      # untimed first chunk
        torch.cuda.synchronize()
        st0 = sc.stats(0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(1, K):
            sc.decode(0, chunks[i], xs, y)
        e1.record()
        torch.cuda.synchronize()
        st1 = sc.stats(0)
        ys[G] = y.clone()
        us = e0.elapsed_time(e1) * 1e3 / (K - 1)
        host = (st1["bypass_bytes"] - st0["bypass_bytes"]) / (K - 1)
        out["staged_64" if G else "in_place"] = {
            "us_per_step": round(us, 1), "host_experts_per_step": round(host / sc.blob_bytes, 2),
            "host_GBs": round(host / (us * 1e-6) / 1e9, 2),
            "tok_per_s_one_layer": round(M / (us * 1e-6), 1)}
        sc.close()
    out["speedup"] = round(out["in_place"]["us_per_step"] / out["staged_64"]["us_per_step"], 3)
    out["bit_equal"] = bool(torch.equal(ys[64], ys[0]))
    print(json.dumps(out), flush=True)


def drafted_workload(torch, SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace, no_flush):
    """The drafted-rows workload on the GLM layer with 128 slots: 4-row draft rounds, a 16-row verify
    step every 10th step and a 64-row prefill chunk (staged, 64 experts per group) every 50th; after 32
    warm-up steps, one HIP-graph replay of the next 200 steps (each after the cache sweep) minus a replay
    of the sweeps alone."""
    cfg = CONFIGS["glm_draft"]
    dev = torch.device("cuda:0")
    W, K = 32, 200
    logits, rows = routing_trace(cfg, 0, steps=W + K)
    rows = [int(r) for r in rows]
    Mmax = max(rows)
    sc = SlotCache(1, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, Mmax)
    expert_blobs(cfg, 0, out=sc.backing(0))
    sc.set_global_scales(0, global_scales(cfg, 0, "unit"))
    d_l = [torch.from_numpy(logits[t, :rows[t]].copy()).to(dev) for t in range(W + K)]
    d_x = [torch.from_numpy(activations(cfg, 0, t, rows[t]).view(np.int16)).to(dev) for t in range(W + K)]
    y = torch.empty((Mmax, cfg.hidden), dtype=torch.float32, device=dev)
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    for t in range(W):
        sc.decode(0, d_l[t], d_x[t], y[:rows[t]])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    gstream = torch.cuda.Stream(dev)
    graphs = []
    for with_steps in (True, False):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gstream):
            g.capture_begin()
            for t in range(W, W + K):
                if not no_flush:
                    sink.copy_(flush.amax())
                if with_steps:
                    sc.decode(0, d_l[t], d_x[t], y[:rows[t]], stream=gstream)
            g.capture_end()
        graphs.append(g)
    torch.cuda.synchronize()
    graphs[1].replay()
    torch.cuda.synchronize()
    ms = []
    st0 = sc.stats(0)
    for g in graphs:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    st1 = sc.stats(0)
    sc.close()
    d = {n: st1[n] - st0[n] for n in ("steps", "bypass_steps", "lookups", "hits", "misses", "bypass_bytes")}
    counts = {str(m): rows[W:].count(m) for m in sorted(set(rows[W:]))}
    return {"workload": "GLM layer, 128 slots, drafted rows: M per step %s over %d steps after %d warm-up steps"
                        % (counts, K, W),
            "us_per_layer_step": round((ms[0] - (0.0 if no_flush else ms[1])) * 1e3 / K, 2),
            "hit_rate_cached_steps": round(d["hits"] / d["lookups"], 4) if d["lookups"] else None,
            "misses": d["misses"], "bypass_steps": d["bypass_steps"],
            "bypass_host_GB": round(d["bypass_bytes"] / 1e9, 3),
            "timing": "one HIP-graph replay of the steps (each after the cache sweep) minus a replay of the sweeps alone"}


def kernel_label(name):
    """A rocprofv3 kernel name without the anonymous-namespace qualifier and the argument list."""
    n = name.replace("(anonymous namespace)::", "").split("(")[0].strip()
    if "reduce_kernel" in n:
        return "at::native::reduce_kernel (the read sweep between steps)"
    if "rocclr_copyBuffer" in n:
        return "__amd_rocclr_copyBuffer (bench plumbing: inputs, state restore)"
    if "rocclr_fillBuffer" in n:
        return "__amd_rocclr_fillBufferAligned (bench plumbing)"
    if "elementwise" in n:
        return "at::native elementwise (setup)"
    return n.replace("void ", "")


def trace_markdown(stats_csv, dur):
    """profiles/glm_m1_decode_step_kernels.md: the run's per-kernel statistics and the all-hit
    block's timed launches by rocprofv3, the kernels' own spans and their event pairs."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    L = ["# Kernel durations: GLM-shaped MoE layer decode step, M=1 (rocprofv3 kernel trace)\n",
         "Workload: H 6144, I 2048, 256 experts, top-8, NVFP4, Zipf(1.1)-skewed routing.  One `bench.py` process: "
         "first the all-hit block (every expert resident, %d untimed + %d timed one-row steps, each after a "
         "512 MiB read sweep, then graph replays), then the churning 128-slot layer (32 cache warm-up + 5 warmup + "
         "20 timed eager steps, then graph replays of the 20 steps from the restored state), then the drafted-rows "
         "workload (M = 4 / 16 / 64).\n" % (dur["all_hit_warm"], dur["timed_launches"]),
         "Commands (`$REPO` = repository root on the GPU host):\n", "```"] + dur["commands"] + ["```\n",
         "| kernel | calls | avg us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:16]:
        L.append("| `%s` | %s | %.2f | %.2f | %.2f | %.2f |" % (kernel_label(r["Name"]), r["Calls"],
                 float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                 float(r["TotalDurationNs"]) / 1e6))
    L += ["", "## The all-hit block's timed launches (the roofline kernels)\n",
          "Each kernel of the one-row step over the %d timed all-hit launches (the block's launches come first in "
          "the process, so launch `%d + j` of each kernel is timed step `j`):\n" % (dur["timed_launches"],
                                                                                    dur["all_hit_warm"]),
          "| kernel | rocprofv3 dispatch avg us | own device-clock spans avg us | hipExtLaunchKernelGGL event pair avg us |",
          "|---|---|---|---|"]
    for p in ("route_remap", "fill", "gateup", "down", "combine"):
        L.append("| `%s` (%s) | %.3f | %.3f | %.3f |" % (dur["kernel_names"][p].rstrip("("), p,
                 dur["rocprof_avg_us"][p], dur["spans_avg_us"][p], dur["events_avg_us"][p]))
    gu, dn = gemv_bytes(CONFIGS_GLM())
    g, d = dur["rocprof_avg_us"]["gateup"], dur["rocprof_avg_us"]["down"]
    L += ["", "At the rocprofv3 durations: gate/up %d B / %.3f us = %.1f GB/s = %.4f of 8 TB/s; down %d B / %.3f us = "
          "%.1f GB/s = %.4f; the pair %d B / %.3f us = %.4f (0.70 of peak is %.2f us for the pair)."
          % (gu, g, gu / g / 1e3, gu / g / 1e3 / 8000, dn, d, dn / d / 1e3, dn / d / 1e3 / 8000, gu + dn, g + d,
             (gu + dn) / (g + d) / 1e3 / 8000, (gu + dn) / (0.7 * 8e12) * 1e6),
          "The dispatch window includes the wave launch before the first block starts and the end-of-kernel signal "
          "after the last wavefront, which the kernels' own stamps do not; the event pairs' stop lands a few "
          "microseconds after the dispatch end.  `bench.py` takes `frac` from `dur_allhit_glm_m1.json` while the "
          "GEMV source hash recorded there matches."]
    path = os.path.join(ROOT, "profiles", "glm_m1_decode_step_kernels.md")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")


SWEEP_PROFILE_COMMAND = (
    "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
    "-d $REPO/gpurun_out/prof_sweep -o run -- python3 -u $REPO/bench.py --sweep-rows 2,3,4,8,16 --steps 40 "
    "> $REPO/gpurun_out/prof_sweep.out")


def sweep_summary(trace_csv, sweep_out):
    """Per-M dispatch durations of a profiled --sweep-rows run.  Each M runs
    min(steps, 4) + 3 * steps steps (warm-up, two graph replays, an eager
    pass), in M order, and each step starts with one routing launch, so the
    trace's launches are grouped by M by counting routing launches."""
    import csv
    lines = [json.loads(l) for l in open(sweep_out) if l.startswith("{")]
    Ms = [d["M"] for d in lines]
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    n_route = sum("k_route_" in r["Kernel_Name"] for r in rows)
    per = n_route // len(Ms)
    if per * len(Ms) != n_route:
        raise SystemExit("%d routing launches for %d values of M" % (n_route, len(Ms)))

    def role(name):
        n = name.replace("(anonymous namespace)::", "")
        if "k_route_" in n:
            return "route"
        if "k_fill" in n:
            return "fill"
        if "k_combine" in n:
            return "combine"
        if "k_gemv" in n:
            k0 = int(n.split("<")[1].split(",")[0])
            return "gateup" if k0 == 6144 else "down"
        return None

    acc, names, step = {}, {}, -1
    for r in rows:
        k = role(r["Kernel_Name"])
        if k is None:
            continue
        step += k == "route"
        if step < 0:
            continue
        M = Ms[min(step // per, len(Ms) - 1)]
        acc.setdefault((M, k), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        names.setdefault((M, k), kernel_label(r["Kernel_Name"]).replace("sc::", ""))
    GU, DN = 14155776, 7077888     # weight bytes of one expert's gate/up and down (GLM layer)
    L = ["# Kernel durations: all-hit GLM-shaped layer with drafted rows, M = %s (rocprofv3 kernel trace)\n"
         % ", ".join(str(m) for m in Ms),
         "Workload: H 6144, I 2048, 256 experts, top-8, every expert resident (S = E, preloaded), drafted rows: "
         "rows 1..M-1 add +20 to three of row 0's top-8 logits, so about half their picks are shared; Zipf(1.1) "
         "routing.  Per M: warm-up steps, two HIP-graph replays of the timed steps (each after a 512 MiB read "
         "sweep, not shown) and an eager pass of the same steps: %d launches of each kernel per M.  `bench.py "
         "--sweep-summary` groups the trace's launches by M by counting routing launches.\n" % per,
         "Commands (`$REPO` = repository root on the GPU host):\n", "```", SWEEP_PROFILE_COMMAND,
         "cd $REPO && python3 bench.py --sweep-summary gpurun_out/prof_sweep/run_kernel_trace.csv "
         "gpurun_out/prof_sweep.out", "```\n",
         "Mean (min) dispatch duration in us; weight bytes per launch are U x %d B (gate/up) and U x %d B (down), "
         "over the mean duration in GB/s and as a fraction of 8 TB/s:\n" % (GU, DN),
         "| M | unique experts U | route + remap | fill (exits: all hit) | gate/up | gate/up GB/s = frac | down | "
         "down GB/s = frac | combine | graph step us (same run) |", "|---|---|---|---|---|---|---|---|---|---|"]
    for d in lines:
        M, U = d["M"], d["unique_experts_per_step"]
        mm = {k: (float(np.mean(acc[(M, k)])), float(np.min(acc[(M, k)]))) for k in
              ("route", "fill", "gateup", "down", "combine")}
        g, dn = mm["gateup"][0], mm["down"][0]
        L.append("| %d | %.2f | %.2f | %.2f | %.2f (%.2f) | %.0f = %.2f | %.2f (%.2f) | %.0f = %.2f | %.2f | %.2f |"
                 % (M, U, mm["route"][0], mm["fill"][0], g, mm["gateup"][1], U * GU / g / 1e3,
                    U * GU / g / 1e6 / 8, dn, mm["down"][1], U * DN / dn / 1e3, U * DN / dn / 1e6 / 8,
                    mm["combine"][0], d["us_per_step"]))
    L += ["", "Kernels by M:"]
    for d in lines:
        L.append("- M = %d: gate/up `%s`, down `%s`" % (d["M"], names[(d["M"], "gateup")], names[(d["M"], "down")]))
    path = os.path.join(ROOT, "profiles", "glm_drafted_rows_kernels.md")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")
    print("\n".join(L))


def CONFIGS_GLM():
    from synth import CONFIGS
    return CONFIGS["glm"]


def trace_summary(trace_csv, stats_csv, steps_json):
    """rocprofv3 dispatch durations of each kernel over the all-hit block's timed launches.

    The all-hit block runs first in a default bench process: its kernels' first
    all_hit_warm + all_hit_timed launches (in start order) are that block's, the
    last all_hit_timed of them the timed ones.  Written to the committed
    summary that the bench quotes while the kernel source hash matches."""
    import csv
    st = json.load(open(steps_json))
    rows = list(csv.DictReader(open(trace_csv)))
    Wa, N = st["all_hit_warm"], st["all_hit_timed"]
    out = {"rocprof_avg_us": {}, "spans_avg_us": {}, "events_avg_us": {}, "launches_in_trace": {}}
    for p, name in st["kernel_names"].items():
        rs = sorted((r for r in rows if name in r.get("Kernel_Name", "")), key=lambda r: int(r["Start_Timestamp"]))
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        if len(dur) < Wa + N:
            raise SystemExit("%s: %d launches in the trace, the all-hit block alone has %d" % (name, len(dur), Wa + N))
        out["rocprof_avg_us"][p] = round(float(np.mean(dur[Wa:Wa + N])), 3)
        out["spans_avg_us"][p] = round(float(np.mean(st["spans_us"][p])), 3)
        out["events_avg_us"][p] = round(float(np.mean(st["events_us"][p])), 3)
        out["launches_in_trace"][p] = len(dur)
    out["timed_launches"] = N
    out["all_hit_warm"] = Wa
    out["kernel_names"] = st["kernel_names"]
    out["source_sha256"] = source_hash()
    out["commands"] = [
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
        "-d $REPO/gpurun_out/prof_bench -o run -- python3 -u $REPO/bench.py --steps 20 --warmup 5 "
        "--no-cpu-baseline --dump-steps $REPO/gpurun_out/steps_prof.json",
        "cd $REPO && python3 bench.py --trace-summary gpurun_out/prof_bench/run_kernel_trace.csv "
        "gpurun_out/prof_bench/run_kernel_stats.csv gpurun_out/steps_prof.json"]
    print(json.dumps(out))
    with open(DUR_FILE, "w") as f:
        json.dump(out, f, indent=1)
    trace_markdown(stats_csv, out)


def main():
    a = parse()
    if a.trace_summary:
        trace_summary(*a.trace_summary)
        return
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
        return
    if a.sweep_summary:
        sweep_summary(*a.sweep_summary)
        return
    if a.gpus != 1:
        print("bench.py measures one GPU: the decode path runs on a single MI355X "
              "(no collectives); --gpus %d is not supported" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if a.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "launches": 3}))
        return
    from hbm_expert_slot_amd.cache import SlotCache
    from synth import CONFIGS, activations, expert_blobs, global_scales, routing_trace
    env = (SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace)

    if a.sweep_rows:
        sweep_rows(a, torch, SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace)
        return
    if a.prefill:
        prefill(a, torch, SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace)
        return
    if a.link_ceiling:
        print(json.dumps({"host_link": dict(dma=link_ceiling(torch), zero_copy_fill=zero_copy_fill(torch, env))}))
        return
    if a.config in ("glm_stack", "flash"):
        cfg = CONFIGS[a.config]
        print("bench: %s, %d cache warm-up + %d warmup + %d timed steps" % (cfg.description, CACHE_WARMUP,
                                                                            a.warmup, a.steps),
              file=sys.stderr, flush=True)
        r = stack_workload(a, torch, env)
        line = {"metric": METRIC, "value": r["us_per_layer_step"], "unit": "us/layer-step", "n_gpus": 1,
                "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(r["us_per_layer_step"] * cfg.n_layers / 1e3, 4),
                "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "fp4e2m1*bf16->fp32",
                "data": "synthetic", "config": {"workload": cfg.description}}
        line.update(r)
        print(json.dumps(line), flush=True)
        return

    cfg = CONFIGS[a.config]
    W, K = a.warmup, a.steps
    print("bench: %s, %d cache warm-up + %d warmup + %d timed steps" % (cfg.description, CACHE_WARMUP, W, K),
          file=sys.stderr, flush=True)
    all_hit = None
    if not a.no_all_hit:
        # first in the process: a profiled run finds this block's launches first in the trace
        print("bench: all-hit block (S = E, preloaded)", file=sys.stderr, flush=True)
        all_hit = all_hit_block(a, torch, env)
    print("bench: churning workload", file=sys.stderr, flush=True)
    ch = churn_headline(a, torch, env)
    link = None
    if not a.no_link:
        print("bench: host-link DMA ceiling", file=sys.stderr, flush=True)
        link = link_ceiling(torch)
    value = ch["value"]
    fill = ch["fill"]
    if link and fill["achieved_GBs"]:
        fill["dma_ceiling_GBs"] = link["h2d_GBs"]
        fill["frac_of_dma_ceiling"] = round(fill["achieved_GBs"] / link["h2d_GBs"], 3)
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(value / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1*bf16->fp32",
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "routing": "Zipf(1.1) popularity, AR(0.99) drift, Gumbel top-k (seeded)" if cfg.routing == "zipf"
                       else "i.i.d. N(0,1) logits (seeded)",
            "miss_fill": "overlapped: copy blocks share the resident experts' gate/up launch" if a.overlap_fill
                         else "copy kernel, then the products",
            "infinity_cache": "flushed between steps (512 MiB read sweep, not timed)" if not a.no_flush
                              else "not flushed (back-to-back steps; repeats may hit the 256 MiB cache)",
            "timing": "value: median over %d HIP-graph replays of the %d timed steps (each after the cache sweep), "
                      "each from the layer state snapshotted after %d cache warm-up + %d warmup steps, minus a "
                      "replay of the sweeps alone, divided by %d; misses included (the replay's lookups, hits and "
                      "misses equal the eager pass's)" % (max(1, a.reps), K, CACHE_WARMUP, W, K),
        },
        "lru": ch["lru"],
        "graph_reps_us": ch["reps_us"],
        "step_us_eager": ch["step_us_eager"],
        "step_us_eager_all_hit_steps": ch["step_us_eager_all_hit_steps"],
        "step_us_eager_miss_steps": ch["step_us_eager_miss_steps"],
        "kernels_us": ch["kernels_us"],
        "wall_s_timed_eager_pass": round(ch["wall_s_eager"], 3),
    }
    if all_hit:
        result["roofline"] = all_hit["gateup"]
        result["roofline_gemv_pair"] = dict(all_hit["gemv_pair"], down=all_hit["down"])
        result["all_hit"] = {k: v for k, v in all_hit.items() if k not in ("gateup", "down", "gemv_pair")}
    result["host_link"] = dict(fill, dma=link)
    if not a.overlap_fill and not a.no_overlap_compare and a.config == "glm":
        # the same steps from the same warmed state with the opt-in overlapped miss fill
        print("bench: churning workload with the overlapped miss fill", file=sys.stderr, flush=True)
        import copy
        a_ov = copy.copy(a)
        a_ov.overlap_fill = True
        ov = churn_headline(a_ov, torch, env)
        result["overlap_fill_workload"] = {
            "flag": "SC_FLAG_OVERLAP_FILL",
            "value": round(ov["value"], 3), "graph_reps_us": ov["reps_us"],
            "vs_plain": round(ov["value"] / value, 4),
            "hit_rate": ov["lru"]["hit_rate"], "misses": ov["lru"]["misses"],
            "step_us_eager_all_hit_steps": ov["step_us_eager_all_hit_steps"],
            "step_us_eager_miss_steps": ov["step_us_eager_miss_steps"],
            "fill_GBs": ov["fill"]["achieved_GBs"],
            "timing": "as value, same trace and warm-up, the misses copied while the resident experts' gate/up runs",
        }
    # the pages' decode token model ("GLM 5.3 Testing: HBM Expert Allocation", section "What the physics says
    # to expect"): every token runs each of the 75 MoE layers once, plus about 3 ms of non-MoE work
    result["token_model"] = {"n_moe_layers": 75, "us_per_layer_step": round(value, 3), "other_ms": 3.0,
                             "hit_rate": ch["lru"]["hit_rate"],
                             "tok_per_s": round(1000.0 / (75 * value / 1000.0 + 3.0), 2)}
    if not a.no_drafted and a.config == "glm":
        print("bench: drafted-rows workload (M = 4 / 16 / 64 schedule)", file=sys.stderr, flush=True)
        result["drafted_workload"] = drafted_workload(torch, SlotCache, CONFIGS, activations, expert_blobs,
                                                      global_scales, routing_trace, a.no_flush)
    if not a.no_cpu_baseline and a.config == "glm":
        print("bench: timing the oracle on bounded CPU samples", file=sys.stderr, flush=True)
        T0 = CACHE_WARMUP + W
        logits, _ = routing_trace(cfg, 0, steps=T0 + a.cpu_baseline_steps)
        xs = [activations(cfg, 0, t, 1) for t in range(T0 + a.cpu_baseline_steps)]
        result["cpu_baseline"] = cpu_baseline(logits, xs, T0, a.cpu_baseline_steps)
    print(json.dumps(result))


if __name__ == "__main__":
    main()

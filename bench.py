"""Benchmark: microseconds per MoE layer-step of the expert-slot decode path on one MI355X.

Workload (default): the GLM-shaped MoE layer -- H 6144, I 2048, 256 experts,
top-8, 128 HBM slots, M=1 decode rows, NVFP4 weights, Zipf(1.1)-skewed routing
with AR(1) drift -- for `--steps` timed steps after `--warmup` untimed ones.
A step is one moe_layer_decode call: routing + remap/LRU, miss fills from the
pinned host store, gate/up and down FP4 GEMVs, combine.  Inputs are resident in
HBM before the timed region.  Between steps a 512 MiB buffer is read so
that the 256 MiB Infinity Cache cannot serve slot bytes from the previous step
(in a real stack 74 other layers read their weights in between).  The reported
mean is a HIP-graph replay of the timed steps minus a replay of the sweeps
alone; an eager pass over the same steps with per-kernel HIP events gives the
per-step spread, the per-kernel times and the GEMV roofline.  Prints one JSON
line.
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
PCIE_PEAK_GBS = 64.0       # PCIe Gen5 x16, per direction
PHASES = ("route_remap", "fill", "gateup", "down", "combine")
KERNEL_NAMES = {"gateup": "k_gemv<6144, 1, 1, true, true>", "down": "k_gemv<2048, 1, 4, false, true>"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--config", default="glm")
    ap.add_argument("--no-flush", action="store_true", help="back-to-back steps (Infinity Cache may serve repeats)")
    ap.add_argument("--cpu-baseline-steps", type=int, default=10,
                    help="consecutive one-row steps the oracle is timed on (about 1 s each on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-rows", default="",
                    help="comma-separated M values: all-hit GLM layer (every expert resident), drafted rows; "
                         "prints one JSON line per M instead of the headline line")
    ap.add_argument("--no-drafted", action="store_true",
                    help="skip the drafted-rows workload (GLM layer, M = 4 / 16 / 64 schedule) in the default run")
    ap.add_argument("--prefill", action="store_true",
                    help="only time M=64 prefill chunks on the GLM layer (128 slots warmed by 64 one-row steps), "
                         "staged 64 experts at a time and read in place; prints one JSON line")
    ap.add_argument("--overlap-fill", action="store_true",
                    help="one-row steps copy their misses while the resident experts' gate/up runs in the same "
                         "launch (SC_FLAG_OVERLAP_FILL); the roofline is then that shared launch's product blocks. "
                         "Applies to the default M=1 workload (the flag changes nothing for steps of several rows)")
    ap.add_argument("--dump-steps", default="",
                    help="write the timed steps' all-hit indices and gate/up event durations to this JSON file")
    ap.add_argument("--pmc-summary", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/pmc_gateup_glm_m1.json and pmc_down_glm_m1.json from the rocprofv3 "
                         "--pmc counter files of a bench run and of the --calibrate-copy run")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "STEPS_JSON"),
                    help="only summarize a rocprofv3 kernel trace of this bench: gate/up durations over the "
                         "all-hit timed launches listed by --dump-steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (counter calibration)")
    return ap.parse_args()


def rocprof_duration(src_hash):
    """The gate/up kernel's rocprofv3 duration over the all-hit timed launches of a
    profiled bench run, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "dur_gateup_glm_m1.json")
    try:
        d = json.load(open(path))
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


def cpu_baseline(cfg, logits, x_rows, start, nsteps):
    """The oracle, as it stands, on `nsteps` steps of the same trace (bounded sample)."""
    from oracle import OracleLayer, route
    from synth import expert_blob, global_scales
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = 1
    # input generation (blob bytes) is not oracle work: stage them first
    need = set()
    for t in range(start, start + nsteps):
        ids, _ = route(logits[t, :1], cfg.top_k)
        need |= set(int(e) for e in ids.reshape(-1))
    blobs = {e: expert_blob(cfg, 0, e) for e in sorted(need)}
    gs = global_scales(cfg, 0, "unit")
    orc = OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, lambda e: blobs[e], gs,
                      keep_slot_bytes=False)
    t0 = time.perf_counter()
    for t in range(start, start + nsteps):
        orc.decode(logits[t, :1], x_rows[t])
    dt = time.perf_counter() - t0
    # bookkeeping alone (routing + slot bookkeeping) over the whole trace
    from oracle.lru import SlotState
    st = SlotState(cfg.n_experts, cfg.slots, cfg.top_k)
    t1 = time.perf_counter()
    for t in range(logits.shape[0]):
        ids, _ = route(logits[t, :1], cfg.top_k)
        st.step(ids)
    bk = (time.perf_counter() - t1) / logits.shape[0]
    return {
        "value": dt / nsteps * 1e6, "unit": "us/layer-step", "cores": int(threads), "kind": "oracle",
        "sample": "%d consecutive M=1 steps of the same GLM trace (full fp64 step: routing, LRU, dequant, "
                  "expert math); blob generation excluded" % nsteps,
        "bookkeeping_us_per_step": bk * 1e6,
        "host_cpus": os.cpu_count(),
    }


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


def trace_summary(trace_csv, steps_json):
    """Average rocprofv3 duration of the gate/up kernel over the all-hit timed launches.

    The bench launches the gate/up kernel once per step: `warmup` eager steps,
    then the `timed` eager steps (the ones --dump-steps lists), then graph
    replays; launch j of the timed pass is dispatch warmup + j in the trace."""
    import csv
    st = json.load(open(steps_json))
    rows = [r for r in csv.DictReader(open(trace_csv)) if "k_gemv<6144, 1, 1, true" in r.get("Kernel_Name", "")]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    W, K = st["warmup"], st["timed"]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    timed = dur[W:W + K]
    hit = [timed[i] for i in st["all_hit_timed_steps"]]
    ev = st["gateup_us_events"]
    sp = st["gateup_us_spans"]
    out = {"spans_avg_us_all_hit": round(float(np.mean([sp[i] for i in st["all_hit_timed_steps"]])), 3),
           "gateup_launches_in_trace": len(dur), "timed_launches": len(timed),
           "all_hit_launches": len(hit),
           "rocprof_avg_us_all_hit": round(float(np.mean(hit)), 3),
           "events_avg_us_all_hit": round(float(np.mean([ev[i] for i in st["all_hit_timed_steps"]])), 3),
           "rocprof_avg_us_all_launches": round(float(np.mean(dur)), 3)}
    print(json.dumps(out))
    # kept beside the counters: the bench line quotes the rocprofv3 duration of the same
    # kernel source next to its own measurement
    rec = dict(out, kernel=KERNEL_NAMES["gateup"], source_sha256=source_hash(),
               command="rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_bench -o run -- "
                       "python3 -u bench.py --no-cpu-baseline --dump-steps gpurun_out/steps_prof.json; "
                       "python3 bench.py --trace-summary gpurun_out/prof_bench/run_kernel_trace.csv "
                       "gpurun_out/steps_prof.json")
    with open(os.path.join(ROOT, "profiles", "dur_gateup_glm_m1.json"), "w") as f:
        json.dump(rec, f, indent=1)


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


def main():
    a = parse()
    if a.trace_summary:
        trace_summary(*a.trace_summary)
        return
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
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

    if a.sweep_rows:
        sweep_rows(a, torch, SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace)
        return
    if a.prefill:
        prefill(a, torch, SlotCache, CONFIGS, activations, expert_blobs, global_scales, routing_trace)
        return
    cfg = CONFIGS[a.config]
    if cfg.rows != 1 or cfg.n_layers != 1:
        print("bench.py times the single-layer M=1 workloads (tiny, glm)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    W, K = a.warmup, a.steps
    T = W + K
    print("bench: %s, %d warmup + %d timed steps" % (cfg.description, W, K), file=sys.stderr, flush=True)
    sc = SlotCache(1, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.slots, 1, overlap_fill=a.overlap_fill)
    t0 = time.time()
    expert_blobs(cfg, 0, out=sc.backing(0))
    sc.set_global_scales(0, global_scales(cfg, 0, "unit"))
    print("bench: backing filled in %.1f s" % (time.time() - t0), file=sys.stderr, flush=True)
    logits, _ = routing_trace(cfg, 0, steps=T)
    xs = np.stack([activations(cfg, 0, t, 1) for t in range(T)])
    d_logits = torch.from_numpy(logits[:, :1].copy()).to(dev)
    d_x = torch.from_numpy(xs.view(np.int16)).to(dev)
    d_y = torch.empty((T, 1, cfg.hidden), dtype=torch.float32, device=dev)
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    for t in range(W):
        sc.decode(0, d_logits[t], d_x[t], d_y[t])
    torch.cuda.synchronize()
    st0 = sc.stats(0)
    ev0 = sc.read_events(0)[1]

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(PHASES))] for _ in range(K)]
    for row in evs:          # torch creates the HIP event on first record
        for ev in row:
            ev.record(stream)
    torch.cuda.synchronize()
    spans = []
    wall0 = time.perf_counter()
    for i in range(K):
        if not a.no_flush:
            flush_sink.copy_(flush.amax())     # read-only sweep: evicts clean, writes nothing back
        sc.decode(0, d_logits[W + i], d_x[W + i], d_y[W + i], stream=stream, events=evs[i])
        spans.append(sc.kernel_spans())       # synchronizes: one step at a time
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    span_us = {p: np.array([spans[i][j] for i in range(K)]) for j, p in enumerate(PHASES)}

    # step: start of the routing kernel to the end of the combine; kernels: own start/end stamps
    step_us = np.array([evs[i][0].elapsed_time(evs[i][-1]) * 1e3 for i in range(K)])
    phase_us = {p: np.array([evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) * 1e3 for i in range(K)])
                for j, p in enumerate(PHASES)}
    st1 = sc.stats(0)
    events, total = sc.read_events(0)
    miss_steps = set(e[0] for e in events[len(events) - (total - ev0):]) if total > ev0 else set()
    step_ids = [W + i for i in range(K)]   # the layer's step counter during timed step i
    allhit = np.array([step_us[i] for i in range(K) if step_ids[i] not in miss_steps])
    lookups = st1["lookups"] - st0["lookups"]
    hits = st1["hits"] - st0["hits"]
    misses = st1["misses"] - st0["misses"]
    filled = st1["bytes_filled"] - st0["bytes_filled"]
    gu_us = span_us["gateup"]
    hit_idx = [i for i in range(K) if step_ids[i] not in miss_steps]
    fill_us = span_us["fill"]
    fill_time_miss = float(np.sum([fill_us[i] for i in range(K) if step_ids[i] in miss_steps]))

    # ---- graph replay: the same K steps captured in one HIP graph -------------
    # Mean step time = (graph of K steps each preceded by the cache sweep
    #                  - graph of the K sweeps alone) / K.
    gstream = torch.cuda.Stream(dev)
    g_steps, g_sweeps = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(gstream):
        g_steps.capture_begin()
        for i in range(K):
            if not a.no_flush:
                flush_sink.copy_(flush.amax())
            sc.decode(0, d_logits[W + i], d_x[W + i], d_y[W + i], stream=gstream)
        g_steps.capture_end()
        g_sweeps.capture_begin()
        for i in range(K):
            if not a.no_flush:
                flush_sink.copy_(flush.amax())
        g_sweeps.capture_end()
    torch.cuda.synchronize()
    g_sweeps.replay()
    g_steps.replay()          # first replay uploads the graph (and runs the trace once more)
    torch.cuda.synchronize()
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record(stream)
    g_sweeps.replay()
    gb.record(stream)
    torch.cuda.synchronize()
    sweeps_ms = ga.elapsed_time(gb)
    st_g0 = sc.stats(0)
    ga.record(stream)
    g_steps.replay()
    gb.record(stream)
    torch.cuda.synchronize()
    steps_ms = ga.elapsed_time(gb)
    st_g1 = sc.stats(0)
    graph_us = (steps_ms - (0.0 if a.no_flush else sweeps_ms)) * 1e3 / K
    g_lookups = st_g1["lookups"] - st_g0["lookups"]
    g_hits = st_g1["hits"] - st_g0["hits"]

    B = sc.blob_bytes
    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    gateup_bytes, down_bytes = gemv_bytes(cfg)
    # roofline: the gate/up kernel on the timed steps without a miss (a miss step's slot was just
    # written by the fill, so part of it can come from the Infinity Cache)
    gu = float(np.mean(gu_us[hit_idx])) if hit_idx else float("nan")
    dn = float(np.mean(span_us["down"][hit_idx])) if hit_idx else float("nan")
    if a.dump_steps:
        with open(a.dump_steps, "w") as f:
            json.dump({"warmup": W, "timed": K, "all_hit_timed_steps": hit_idx,
                       "gateup_us_spans": [float(v) for v in gu_us],
                       "gateup_us_events": [float(v) for v in phase_us["gateup"]]}, f)
    src_hash = source_hash()
    # the committed counters were taken on the plain gate/up kernel
    traffic = None if a.overlap_fill else pmc_traffic("gateup_glm_m1", src_hash)
    gu_kernel = ("k_fill_gateup<%d> (product blocks)" % H) if a.overlap_fill else KERNEL_NAMES["gateup"]
    dur = None if a.overlap_fill else rocprof_duration(src_hash)
    # the same launches in a rocprofv3 trace of this kernel source: its dispatch windows include
    # the wave launch before the first block starts and the kernel's end after the last
    # wavefront, which the kernel's own stamps do not
    duration_check = None if dur is None else {
        "rocprof_avg_us": dur["rocprof_avg_us_all_hit"], "own_stamps_avg_us": dur["spans_avg_us_all_hit"],
        "launches": dur["all_hit_launches"],
        "frac_at_rocprof_duration": round(gateup_bytes / (dur["rocprof_avg_us_all_hit"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "source": "profiles/dur_gateup_glm_m1.json"}
    result = {
        "metric": METRIC,
        "value": round(graph_us, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(graph_us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1*bf16->fp32",
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "routing": "Zipf(1.1) popularity, AR(0.99) drift, Gumbel top-k (seeded)",
            "miss_fill": "overlapped: copy blocks share the resident experts' gate/up launch" if a.overlap_fill
                         else "copy kernel, then the products",
            "infinity_cache": "flushed between steps (512 MiB read sweep, not timed)" if not a.no_flush
                              else "not flushed (back-to-back steps; repeats may hit the 256 MiB cache)",
            "timing": "value: one HIP-graph replay of the K steps (each after the cache sweep) minus a replay of "
                      "the K sweeps alone, divided by K; eager pass over the same steps, one step at a time: step_us "
                      "from HIP events (routing kernel start to combine end), kernels_us from the kernels' own "
                      "start/end stamps on the device wall clock (slotcache_read_kernel_spans)",
        },
        "graph": {"us_per_step": graph_us, "replay_ms": steps_ms, "sweeps_ms": sweeps_ms,
                  "hit_rate": g_hits / g_lookups if g_lookups else None},
        "step_us": {"mean": float(np.mean(step_us)), "p10": float(np.percentile(step_us, 10)),
                    "p50": float(np.percentile(step_us, 50)), "p90": float(np.percentile(step_us, 90)),
                    "all_hit_mean": float(np.mean(allhit)) if allhit.size else None,
                    "all_hit_steps": int(allhit.size)},
        "kernels_us": {p: float(np.mean(v)) for p, v in span_us.items()},
        "kernels_us_all_hit_steps": {p: float(np.mean(v[hit_idx])) for p, v in span_us.items()} if hit_idx else None,
        "lru": {"hit_rate": hits / lookups if lookups else None, "misses_per_step": misses / K,
                "lookups": lookups, "hits": hits, "misses": misses},
        "roofline": {
            "kernel": gu_kernel, "bound": "hbm",
            "achieved": round(gateup_bytes / (gu * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gateup_bytes / (gu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": gateup_bytes, "avg_launch_us": gu,
            "launches": "gate/up kernel on the %d all-hit timed steps" % len(hit_idx),
            "duration": "mean of the kernel's own execution spans (first block start to last wavefront end, "
                        "device wall clock)",
            "rocprof_check": duration_check,
        },
        "down_gemv": {"kernel": KERNEL_NAMES["down"], "achieved_GBs": round(down_bytes / (dn * 1e-6) / 1e9, 1),
                      "avg_launch_us": dn, "algorithmic_bytes_per_launch": down_bytes},
        "host_link": {"bytes_filled": filled, "fill_us_on_miss_steps": fill_time_miss,
                      "achieved_GBs": round(filled / (fill_time_miss * 1e-6) / 1e9, 2) if fill_time_miss > 0 else None,
                      "peak_GBs": PCIE_PEAK_GBS},
        "wall_s_timed_region": wall,
        # the pages' decode token model ("GLM 5.3 Testing: HBM Expert Allocation", section "What the physics
        # says to expect"): every token runs each of the 75 MoE layers once, plus ~3 ms of non-MoE work
        "token_model": {"n_moe_layers": 75, "us_per_layer_step": round(graph_us, 3), "other_ms": 3.0,
                        "tok_per_s": round(1000.0 / (75 * graph_us / 1000.0 + 3.0), 2)},
    }
    sc.close()
    if not a.no_drafted and a.config == "glm":
        print("bench: drafted-rows workload (M = 4 / 16 / 64 schedule)", file=sys.stderr, flush=True)
        result["drafted_workload"] = drafted_workload(torch, SlotCache, CONFIGS, activations, expert_blobs,
                                                      global_scales, routing_trace, a.no_flush)
    if not a.no_cpu_baseline:
        print("bench: timing the oracle on a bounded CPU sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, logits, xs, W, a.cpu_baseline_steps)
    print(json.dumps(result))


if __name__ == "__main__":
    main()

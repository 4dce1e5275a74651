#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X, with the roofline of the dominant kernel
and the CPU oracle timed beside it.

Default workload (--workload prefill_mxfp4): 4096-token prefill layers of the
MXFP4 shape (hidden 4096, 256 routed experts, top-6, expert intermediate 2048,
E2M1 weights with an E8M0 scale per 32-element block, bf16 activations), N(0,1)
logits so that every expert is active with about 96 tokens.  A step is one
4096-token chunk through 43 layers: every layer's 3.42 GB of expert weights come
from pinned host memory into one of two HBM banks while the previous layer runs
the whole path (top-k, permutation, grouped GEMM gate_up + down, combine).  The
line's roofline is the grouped GEMM gate_up kernel against the bf16 MFMA peak.
The same run then measures the MXFP4 decode stack (43 layers, every expert
resident, batches of 64, 1 and 8 tokens) and reports it under "decode_mxfp4"
with its own HBM roofline (--no-decode-leg skips it).

Other workloads, each printing one JSON line of the same form:
  decode_mxfp4       the MXFP4 decode stack alone (headline batch 64).
  decode_bf16        16 stacked bf16 decode layers (hidden 2048, 256 routed
                     experts + 1 shared, top-8, intermediate 512), batches 16, 1, 4.
  cached_trace_bf16  1000 single-token steps through 48 bf16 layers with a cold
                     global-LRU slot cache holding 37% of the experts.
  hostbw             pinned host -> HBM copy bandwidth at the fill sizes.

CPU baseline: the oracle (plain fp64 C, test infrastructure) on a bounded
sample of the same workload, once on one thread and once with its per-expert
calls spread over every host core allotted to the process (a thread pool over
experts; each call is the unmodified oracle routine; rows are combined per token
in a fixed order).
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0  # dense; the scaled FP4 x FP8 MFMA runs at the FP8 rate
METRIC = "MoE-layer tokens/s at 1 MI355X; % HBM BW (decode), % MFMA peak (prefill)"
# HBM byte counters of each workload's dominant kernel (rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs summarised by --summarize-counters), valid while the FFN
# sources hash to the value recorded in the file.
COUNTERS = {
    "decode_bf16": ("gate_up_mfma_bf16_decode_T16_counters.txt", "gate_up_mfma"),
    "decode_mxfp4": ("gate_up_mfma_mxfp4_decode_T64_counters.txt", "gate_up_mfma"),
    "prefill_mxfp4": ("grouped_gate_up_mxfp4_T4096_counters.txt", "grouped_gate_up"),
    "prefill_mxfp4_a8": ("grouped_gate_up_native_fp4_T8192_counters.txt", "grouped_gate_up"),
}
FFN_SOURCES = [os.path.join(ROOT, "routed_expert_ffn_layer_amd", "csrc", f)
               for f in ("ffn.hip", "ffn_prefill.hip", "ffn_common.hpp", "common.hpp")]
WORKLOADS = ("decode_bf16", "decode_mxfp4", "prefill_mxfp4", "prefill_mxfp4_a8", "cached_trace_bf16", "hostbw")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=WORKLOADS, default="prefill_mxfp4")
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default depends on the workload)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default depends on the workload)")
    ap.add_argument("--tokens", type=int, default=None, help="tokens per layer of the headline batch")
    ap.add_argument("--layers", type=int, default=None, help="stacked layers")
    ap.add_argument("--extra-batches", default=None, help="other decode batches to report")
    ap.add_argument("--host-layers", type=int, default=None,
                    help="distinct layers kept in pinned host memory (layer l reads host layer l mod this)")
    ap.add_argument("--distinct-experts", type=int, default=512,
                    help="decode_mxfp4: distinct generated experts copied into the 11,008 slots")
    ap.add_argument("--eager", action="store_true",
                    help="decode workloads: launch every call from Python each step (default: one captured HIP "
                         "graph per step, replayed)")
    ap.add_argument("--split-waves", action="store_true",
                    help="cached_trace_bf16: compute each wave's hits while its misses fill (default: after all fills)")
    ap.add_argument("--fill-fraction", default=None, metavar="NUM/DEN",
                    help="cached_trace_bf16: miss split; of each step's misses floor(m*NUM/DEN + 1/2) are filled, the "
                         "rest computed in place from pinned host memory (default: every miss filled)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of each oracle CPU baseline leg (one thread, all cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-leg", action="store_true",
                    help="prefill_mxfp4: skip the MXFP4 decode stack measured after the prefill line")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="threads of the all-core CPU baseline (default: the cores allotted to this process)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--summarize-pmc", metavar="PROF_DIR", default=None,
                    help="print per-kernel averages of every counter in rocprofv3 --pmc runs (no GPU)")
    ap.add_argument("--summarize-counters", metavar="PROF_DIR", default=None,
                    help="print per-kernel HBM bytes per dispatch from rocprofv3 FETCH_SIZE/WRITE_SIZE runs (no GPU)")
    return ap.parse_args()


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ffn_source_hash():
    """Hash of the FFN kernel sources with comments and whitespace removed (a
    comment edit does not change the kernels the counters describe)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        src = open(f).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel from the committed
    counter summary (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by the same counters
    on a copy of known size), or None if there is none or the kernel sources
    changed since the counters were taken."""
    if workload not in COUNTERS:
        return None
    path = os.path.join(ROOT, "profiles", COUNTERS[workload][0])
    if not os.path.exists(path):
        return None
    d = json.loads("\n".join(l for l in open(path).read().splitlines() if not l.startswith("#")))
    if d.get("ffn_source_sha256") != ffn_source_hash():
        return None
    k = d.get("kernels", {}).get(COUNTERS[workload][1])
    return None if k is None else k.get("hbm_bytes_per_launch")


def summarize_counters(prof_dir):
    """Per-kernel HBM bytes per dispatch from rocprofv3 --pmc runs laid out as
    prof_dir/{FETCH_SIZE,WRITE_SIZE}/**.csv (the workload) and
    prof_dir/{FETCH_SIZE,WRITE_SIZE}_copy/**.csv (bench.py --calibrate-copy).
    Counters are KiB per dispatch; each is scaled by bytes/KiB read on the copy."""
    import csv
    import glob
    import re

    def load(sub):
        per = {}
        for f in glob.glob(os.path.join(prof_dir, sub, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name = re.sub(r"^void ", "", r["Kernel_Name"]).split("(")[0].split("<")[0].split("::")[-1]
                d = per.setdefault(name, {"sum": 0.0, "dispatches": set()})
                d["sum"] += float(r["Counter_Value"])
                d["dispatches"].add(r.get("Dispatch_Id", r.get("Correlation_Id")))
        return {k: (v["sum"] / len(v["dispatches"]), len(v["dispatches"])) for k, v in per.items()}

    n_copy = 256 << 20
    fc = load("FETCH_SIZE_copy")
    wc = load("WRITE_SIZE_copy")
    copy_kernel = max(fc, key=lambda k: fc[k][0])
    f_factor = n_copy / (fc[copy_kernel][0] * 1024.0)
    w_factor = n_copy / (wc[copy_kernel][0] * 1024.0)
    fk, wk = load("FETCH_SIZE"), load("WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fk) & set(wk)):
        fb = fk[k][0] * 1024.0 * f_factor
        wb = wk[k][0] * 1024.0 * w_factor
        kernels[k] = {"fetch_kib_raw": round(fk[k][0], 1), "write_kib_raw": round(wk[k][0], 1),
                      "fetch_bytes": int(fb), "write_bytes": int(wb), "hbm_bytes_per_launch": int(fb + wb),
                      "dispatches": fk[k][1]}
    return {"ffn_source_sha256": ffn_source_hash(),
            "copy_calibration": {"copy_kernel": copy_kernel, "copy_bytes": n_copy,
                                 "fetch_kib_raw": round(fc[copy_kernel][0], 1),
                                 "write_kib_raw": round(wc[copy_kernel][0], 1),
                                 "fetch_factor": round(f_factor / 1.0, 6), "write_factor": round(w_factor, 6)},
            "kernels": kernels}


def summarize_pmc(prof_dir):
    """Per-kernel averages per dispatch of every counter in rocprofv3 --pmc runs
    under prof_dir (rows of one dispatch and counter are summed first), plus the
    MFMA busy fraction SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 256 CUs
    * 4 SIMDs) where both counters were collected in the same run (both arrive
    summed over the GPU's instances: GRBM_GUI_ACTIVE once per XCD, the MFMA busy
    cycles once per SIMD).  Where a run also traced kernels (--kernel-trace), the
    median core clock of the kernel's dispatches (GRBM_GUI_ACTIVE per XCD over the
    dispatch's duration) and that clock over the 2.4 GHz of the spec peaks."""
    import csv
    import glob
    import re
    per = {}
    for f in glob.glob(os.path.join(prof_dir, "**", "*counter_collection.csv"), recursive=True):
        run = os.path.relpath(os.path.dirname(f), prof_dir).split(os.sep)[0]
        for r in csv.DictReader(open(f)):
            name = re.sub(r"^void ", "", r["Kernel_Name"]).split("(")[0].split("<")[0].split("::")[-1]
            key = (run, name, r["Counter_Name"])
            disp = r.get("Dispatch_Id", r.get("Correlation_Id"))
            per.setdefault(key, {}).setdefault(disp, 0.0)
            per[key][disp] += float(r["Counter_Value"])
    # kernel-trace durations of the same runs (when the pass also traced kernels)
    dur = {}
    for f in glob.glob(os.path.join(prof_dir, "**", "*kernel_trace.csv"), recursive=True):
        run = os.path.relpath(os.path.dirname(f), prof_dir).split(os.sep)[0]
        for r in csv.DictReader(open(f)):
            dur[(run, r.get("Dispatch_Id", r.get("Correlation_Id")))] = (
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    out = {}
    for (run, name, ctr), d in sorted(per.items()):
        out.setdefault(name, {}).setdefault(run, {})[ctr] = {"per_dispatch": sum(d.values()) / len(d),
                                                             "dispatches": len(d)}
    for name, runs in out.items():
        for run, ctrs in runs.items():
            if "SQ_VALU_MFMA_BUSY_CYCLES" in ctrs and "GRBM_GUI_ACTIVE" in ctrs:
                ctrs["mfma_busy_frac"] = (ctrs["SQ_VALU_MFMA_BUSY_CYCLES"]["per_dispatch"] /
                                          (ctrs["GRBM_GUI_ACTIVE"]["per_dispatch"] / 8 * 256 * 4))
            grbm = per.get((run, name, "GRBM_GUI_ACTIVE"))
            if grbm:
                # core clock of each dispatch: its GUI-active cycles per XCD over its
                # traced duration; the spec peaks assume 2.4 GHz
                # (only dispatches of 300 us or more: the counter window adds cycles
                # outside the traced kernel, which short dispatches overstate)
                clk = sorted(v / 8 / dur[(run, disp)] / 1e9 for disp, v in grbm.items()
                             if (run, disp) in dur and dur[(run, disp)] >= 300e-6)
                ds = sorted(dur[(run, disp)] for disp in grbm if (run, disp) in dur)
                if clk:
                    ctrs["median_duration_us"] = ds[len(ds) // 2] * 1e6
                    ctrs["clock_ghz_median"] = clk[len(clk) // 2]
                    ctrs["clock_limited_peak_frac"] = clk[len(clk) // 2] / 2.4
    return out


def calibrate_copy():
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def out_line(value, unit, steps, warmup, ms_per_step, dtype, data, config, roofline, cpu, **extra):
    d = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
         "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
         "dtype": dtype, "data": data, "config": config, "roofline": roofline}
    d.update(extra)
    d["cpu_baseline"] = cpu
    return d


def time_back_to_back(fn, n_calls, passes):
    """Average duration of fn(i) for i < n_calls, launched back to back on the
    current stream; one event pair around each whole pass."""
    import torch
    for i in range(n_calls):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(passes):
        for i in range(n_calls):
            fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (passes * n_calls)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores.

def host_cores():
    """Cores allotted to this process (capped by OMP_NUM_THREADS when it is set,
    the host share that goes with one GPU) and the CPU model name."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def expert_jobs(ids, E):
    """(expert, its tokens ascending) for every expert the routing selects, by id."""
    jobs = []
    for e in range(E):
        tok = np.nonzero((ids == e).any(axis=1))[0].astype(np.int32)
        if tok.size:
            jobs.append((e, tok))
    return jobs


def run_jobs(jobs, work, threads, seconds=None):
    """work(e, tokens) over the jobs in order on `threads` threads (the oracle's C
    routines release the GIL while they run).  New jobs stop being started once
    `seconds` have passed (None: run them all).  Returns (results in job order,
    token pairs done, seconds)."""
    import concurrent.futures as cf
    t0 = time.perf_counter()
    out, pairs = [], 0
    if threads <= 1:
        for e, tok in jobs:
            out.append(work(e, tok))
            pairs += tok.size
            if seconds is not None and time.perf_counter() - t0 >= seconds:
                break
        return out, pairs, time.perf_counter() - t0
    res = {}
    with cf.ThreadPoolExecutor(threads) as ex:
        pending, nxt = {}, 0
        while nxt < len(jobs) and len(pending) < threads:
            pending[ex.submit(work, *jobs[nxt])] = nxt
            nxt += 1
        while pending:
            done, _ = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
            for f in done:
                i = pending.pop(f)
                res[i] = f.result()
                pairs += jobs[i][1].size
            while nxt < len(jobs) and len(pending) < threads and (
                    seconds is None or time.perf_counter() - t0 < seconds):
                pending[ex.submit(work, *jobs[nxt])] = nxt
                nxt += 1
    n = 0
    while n in res:
        n += 1
    return [res[i] for i in range(n)], pairs, time.perf_counter() - t0


def oracle_layer_threads(dtype, experts, x, logits, k, H, I, threads):
    """One whole layer with the oracle's routines: top-k, then every selected
    expert's rows (one oracle call per expert, spread over `threads` threads),
    then y = sum_j w_tj * row(t, j) per token in increasing j (oracle combine)."""
    import oracle
    ids, _, w64 = oracle.route_topk(logits, k)
    T = logits.shape[0]
    jobs = expert_jobs(ids, logits.shape[1])
    rows, _, _ = run_jobs(jobs, lambda e, tok: oracle.expert_rows(dtype, experts[e], H, I, x, tok), threads)
    where = {}
    for (e, tok), r in zip(jobs, rows):
        for i, t in enumerate(tok):
            where[(int(t), e)] = r[i]
    gathered = np.array([[where[(t, int(ids[t, j]))] for j in range(k)] for t in range(T)])
    return oracle.combine(gathered.reshape(T * k, H), w64)


def cpu_threads(args):
    """(threads of the all-core leg, CPU model)."""
    n, model = host_cores()
    return (args.cpu_threads or n), model


def cpu_baseline_entry(single, multi, threads, model, unit):
    """The cpu_baseline object: the all-core figure as the value, the single-thread
    figure beside it."""
    return dict(value=multi["value"], unit=unit, cores=threads, kind="oracle", sample=multi["sample"],
                cpu_model=model, cores_allotted=len(os.sched_getaffinity(0)),
                single_thread={"value": single["value"], "cores": 1, "sample": single["sample"]})


# ---------------------------------------------------------------------------
# Algorithmic work.

def w13_bytes(wdt, H, I):
    """Bytes of the gate/up half of an expert slot (codes and, for MXFP4, scales)."""
    import synth
    o = synth.slot_offsets(wdt, H, I)
    if wdt == synth.MXFP4:
        return (o["w2"] - o["w13"]) + (o["s2"] - o["s13"])
    return o["w2"] - o["w13"]


def gate_up_bytes(wdt, n_experts_active, has_shared, T, k, H, I):
    """Algorithmic HBM bytes of one gate_up launch: each active expert's W13 once,
    the T token rows of x, the SwiGLU intermediate written (bf16)."""
    experts = n_experts_active + (1 if has_shared else 0)
    rows = T * k + (T if has_shared else 0)
    return experts * w13_bytes(wdt, H, I) + T * H * 2 + rows * I * 2


def layer_bytes(wdt, n_experts_active, has_shared, T, k, E, H, I):
    """Algorithmic HBM bytes of the whole layer: every active expert's weights once,
    logits, x, the intermediate (write + read), expert output rows (write + read),
    gate weights and the bf16 layer output."""
    import synth
    experts = n_experts_active + (1 if has_shared else 0)
    rows = T * k + (T if has_shared else 0)
    w = experts * synth.expert_bytes(wdt, H, I)
    act = T * E * 4 + T * H * 2 + 2 * rows * I * 2 + 2 * rows * H * 4 + T * k * 4 + T * H * 2
    return w + act


# ---------------------------------------------------------------------------
# decode_bf16 (the headline workload).

def replay_step(step, eager):
    """The step as given (eager), or captured once into a HIP graph and replayed:
    a decode step over resident experts has no host synchronisation, so its
    launches are recorded once (after one eager run that loads the kernels)."""
    if eager:
        return step
    import torch
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    return graph.replay


def run_decode_bf16(T, n_layers, steps, warmup, time_kernel=True, eager=False):
    import torch
    import synth
    from routed_expert_ffn_layer_amd import layer as L
    from routed_expert_ffn_layer_amd import moe

    c = synth.CONFIGS["decode_bf16"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    dev = torch.device("cuda:0")
    stride = moe.moe_expert_bytes(moe.MOE_BF16, H, I)
    pools = [synth.torch_bf16_expert_pool(E + 1, H, I, seed=c["seed"] * 100 + l, device=dev) for l in range(n_layers)]
    bufs = [L.LayerBuffers(T, E, k, H, I, moe.MOE_BF16, I_shared=I) for _ in range(n_layers)]
    logits = [torch.from_numpy(synth.normal_logits(c["seed"], T, E, 7, l)).to(dev) for l in range(n_layers)]
    xs = [torch.from_numpy(synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], T, H, 7, l))
                           .view(np.int16)).to(dev) for l in range(n_layers)]
    slots = L.identity_slots(E, dev)

    def gate_up(l):
        b = bufs[l]
        moe.moe_grouped_ffn_gate_up(b.wdt, pools[l][:E], stride, slots, pools[l][E], I, xs[l], b.offsets,
                                    b.sorted_rows, T, k, E, H, I, b.out_rows, b.shared_out, b.workspace)

    def step():
        for l in range(n_layers):
            b = bufs[l]
            L.route(b, logits[l])
            gate_up(l)
            moe.moe_grouped_ffn_down(b.wdt, pools[l][:E], stride, slots, pools[l][E], I, xs[l], b.offsets,
                                     b.sorted_rows, T, k, E, H, I, b.out_rows, b.shared_out, b.workspace)
            L.combine(b, True)

    run = replay_step(step, eager)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    active = [int((b.counts > 0).sum().item()) for b in bufs]
    res = dict(T=T, layers=n_layers, steps=steps, seconds=elapsed, ms_per_step=1e3 * elapsed / steps,
               layer_tokens_per_s=T * n_layers * steps / elapsed, active_experts_mean=float(np.mean(active)))
    step_bytes = sum(layer_bytes(synth.BF16, a, True, T, k, E, H, I) for a in active)
    res["layer_hbm_gbs"] = step_bytes * steps / elapsed / 1e9
    if time_kernel:
        # The dominant kernel, timed live on its launch stream: the same layers'
        # gate_up launches back to back (same inputs, same routing as the timed
        # steps), one event pair around each pass of n_layers launches, so the
        # events add no gap between launches and their own cost spreads over the pass.
        passes = max(4, steps // 4)
        per_launch = time_back_to_back(gate_up, n_layers, passes)
        gb = float(np.mean([gate_up_bytes(synth.BF16, a, True, T, k, H, I) for a in active]))
        res["gate_up_avg_us"] = per_launch * 1e6
        res["gate_up_bytes_avg"] = gb
        res["gate_up_gbs"] = gb / per_launch / 1e9
        res["gate_up_launches_timed"] = passes * n_layers
    del pools
    torch.cuda.empty_cache()
    return res


def cpu_decode_bf16(seconds, threads, model):
    """The oracle on a bounded sample of the same workload: decode layers of 16
    tokens with the same shapes, whole layers until the budget is spent, on one
    thread and on `threads` threads."""
    import synth
    import oracle
    c = synth.CONFIGS["decode_bf16"]
    H, I, E, k, T = c["H"], c["I"], c["E"], c["k"], 16
    g = synth.rng(c["seed"], 99)
    logits = synth.normal_logits(c["seed"], T, E, 99)
    ids, _, _ = oracle.route_topk(logits, k)
    used = sorted(set(ids.ravel().tolist()))
    # only the experts the sample routes to are generated; the rest are never read
    experts = [None] * E
    for e in used:
        experts[e] = synth.random_expert(synth.BF16, H, I, synth.rng(c["seed"], 98, e))
    blank = np.zeros(synth.expert_bytes(synth.BF16, H, I), np.uint8)
    experts = [blank if v is None else v for v in experts]
    shared = synth.random_expert(synth.BF16, H, I, g)
    x = synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], T, H, 99))
    legs = {}
    for nthr in (1, threads):
        n = 0
        t0 = time.perf_counter()
        while True:
            if nthr == 1:
                oracle.layer(synth.BF16, experts, x, logits, k, H, I, shared=shared, I_shared=I)
            else:
                oracle_layer_threads(synth.BF16, experts, x, logits, k, H, I, nthr)
                oracle.expert_rows(synth.BF16, shared, H, I, x, np.arange(T, dtype=np.int32))
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds or n >= 50:
                break
        legs[nthr] = dict(value=T * n / el,
                          sample=f"{n} decode layers of {T} tokens (H={H}, I={I}, {E} experts + shared, top-{k}) "
                                 f"on {nthr} thread(s), {el:.1f} s")
    return cpu_baseline_entry(legs[1], legs[threads], threads, model, "layer-tokens/s")


def workload_decode_bf16(args):
    T = args.tokens or 16
    n_layers = args.layers or 16
    steps, warmup = args.steps or 50, 5 if args.warmup is None else args.warmup
    extra = [int(v) for v in ("1,4" if args.extra_batches is None else args.extra_batches).split(",") if v.strip()]
    main_res = run_decode_bf16(T, n_layers, steps, warmup, eager=args.eager)
    keys = ("layer_tokens_per_s", "ms_per_step", "layer_hbm_gbs", "gate_up_gbs", "gate_up_avg_us",
            "active_experts_mean")
    by_batch = {str(T): {k: main_res[k] for k in keys}}
    for tb in extra:
        if tb == T:
            continue
        r = run_decode_bf16(tb, n_layers, max(10, steps // 2), 2, eager=args.eager)
        by_batch[str(tb)] = {k: r[k] for k in keys}
    cpu = None if args.no_cpu_baseline else cpu_decode_bf16(args.cpu_seconds, *cpu_threads(args))
    achieved = main_res["gate_up_gbs"]
    return out_line(
        main_res["layer_tokens_per_s"], "layer-tokens/s", steps, warmup, main_res["ms_per_step"], "bf16",
        "synthetic (seeded N(0,0.02) weights, N(0,1) logits and activations)",
        {"workload": "decode layer bf16: hidden 2048, 256 routed experts + 1 shared, top-8, intermediate 512",
         "tokens_per_layer": T, "stacked_layers": n_layers,
         "weights_in_hbm_gb": round(n_layers * 257 * 6291456 / 1e9, 2), "slots": "all resident",
         "launch": "eager" if args.eager else "one HIP graph per step"},
        {"kernel": "gate_up_mfma<bf16> (moe_grouped_ffn_gate_up)", "bound": "hbm", "achieved": achieved,
         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("decode_bf16"),
         "avg_launch_us": main_res["gate_up_avg_us"], "algorithmic_bytes_per_launch": main_res["gate_up_bytes_avg"],
         "launches_timed": main_res["gate_up_launches_timed"],
         "timing": "events around back-to-back passes of the timed layers' gate_up launches"},
        cpu, layer_hbm_frac=main_res["layer_hbm_gbs"] / HBM_PEAK_GBS, by_batch=by_batch)


# ---------------------------------------------------------------------------
# decode_mxfp4: 43 stacked layers, every expert resident.

def mxfp4_resident_stack(c, n_layers, n_distinct, dev):
    """[n_layers * E][expert_bytes] uint8 in HBM.  n_distinct experts are generated
    (N(0, 0.02) -> MXFP4) and copied into the slots, slot s of layer l taking
    distinct expert (7 s + 131 l) mod n_distinct: every slot is its own address,
    so the bytes a layer streams are its own."""
    import torch
    import synth
    H, I, E = c["H"], c["I"], c["E"]
    eb = synth.expert_bytes(synth.MXFP4, H, I)
    distinct = torch.empty((n_distinct, eb), dtype=torch.uint8, device=dev)
    for j in range(0, n_distinct, 256):
        n = min(256, n_distinct - j)
        distinct[j:j + n].copy_(synth.torch_mxfp4_expert_pool(n, H, I, seed=c["seed"] * 100 + j // 256, device=dev))
        progress(f"generated {j + n}/{n_distinct} distinct MXFP4 experts")
    stack = torch.empty((n_layers * E, eb), dtype=torch.uint8, device=dev)
    for l in range(n_layers):
        idx = (torch.arange(E, device=dev) * 7 + 131 * l) % n_distinct
        torch.index_select(distinct, 0, idx, out=stack[l * E:(l + 1) * E])
        if l % 8 == 7 or l == n_layers - 1:
            torch.cuda.synchronize()
            progress(f"filled {l + 1}/{n_layers} resident layers")
    return stack, distinct


def run_decode_mxfp4(stack, c, T, n_layers, steps, warmup, n_batches=4, eager=False):
    import torch
    import synth
    from routed_expert_ffn_layer_amd import layer as L
    from routed_expert_ffn_layer_amd import moe
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    dev = stack.device
    eb = synth.expert_bytes(synth.MXFP4, H, I)
    bufs = [L.LayerBuffers(T, E, k, H, I, moe.MOE_MXFP4) for _ in range(n_layers)]
    logits = [[torch.from_numpy(synth.zipf_noise_logits(c["seed"], T, E, l, c["zipf_s"], batch=bi)).to(dev)
               for bi in range(n_batches)] for l in range(n_layers)]
    xs = [torch.from_numpy(synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], T, H, 7, bi))
                           .view(np.int16)).to(dev) for bi in range(n_batches)]
    slots = L.identity_slots(E, dev)
    pools = [stack[l * E:(l + 1) * E] for l in range(n_layers)]

    def step(j):
        bi = j % n_batches
        for l in range(n_layers):
            L.forward(bufs[l], logits[l][bi], xs[bi], pools[l], eb, slots)

    # one captured step per batch (the batches are different input buffers)
    runs = [replay_step(lambda bi=bi: step(bi), eager) for bi in range(n_batches)]
    for j in range(warmup):
        runs[j % n_batches]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(steps):
        runs[j % n_batches]()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # routing of every (layer, batch), for the algorithmic bytes of the timed steps
    active = np.zeros((n_layers, n_batches))
    for bi in range(n_batches):
        for l in range(n_layers):
            L.route(bufs[l], logits[l][bi])
            active[l, bi] = int((bufs[l].counts > 0).sum().item())
    step_bytes = [sum(layer_bytes(synth.MXFP4, active[l, bi], False, T, k, E, H, I) for l in range(n_layers))
                  for bi in range(n_batches)]
    total_bytes = sum(step_bytes[j % n_batches] for j in range(steps))

    # the FFN kernels of every layer on batch 0's routing, back to back
    for l in range(n_layers):
        L.route(bufs[l], logits[l][0])

    def gate_up(l):
        b = bufs[l]
        moe.moe_grouped_ffn_gate_up(b.wdt, pools[l], eb, slots, None, 0, xs[0], b.offsets, b.sorted_rows,
                                    T, k, E, H, I, b.out_rows, None, b.workspace)

    def down(l):
        b = bufs[l]
        moe.moe_grouped_ffn_down(b.wdt, pools[l], eb, slots, None, 0, xs[0], b.offsets, b.sorted_rows,
                                 T, k, E, H, I, b.out_rows, None, b.workspace)

    passes = 4
    gu = time_back_to_back(gate_up, n_layers, passes)
    dn = time_back_to_back(down, n_layers, passes)
    gub = float(np.mean([gate_up_bytes(synth.MXFP4, active[l, 0], False, T, k, H, I) for l in range(n_layers)]))
    w2b = eb - w13_bytes(synth.MXFP4, H, I)
    dnb = float(np.mean([active[l, 0] * w2b + T * k * I * 2 + T * k * H * 4 for l in range(n_layers)]))
    return dict(T=T, layers=n_layers, steps=steps, seconds=elapsed, ms_per_step=1e3 * elapsed / steps,
                layer_tokens_per_s=T * n_layers * steps / elapsed, stack_tokens_per_s=T * steps / elapsed,
                layer_hbm_gbs=total_bytes / elapsed / 1e9, active_experts_mean=float(active.mean()),
                gate_up_avg_us=gu * 1e6, gate_up_bytes_avg=gub, gate_up_gbs=gub / gu / 1e9,
                down_avg_us=dn * 1e6, down_gbs=dnb / dn / 1e9, gate_up_launches_timed=passes * n_layers)


def cpu_decode_mxfp4(stack, c, T, seconds, threads, model):
    """The oracle on a bounded sample: MXFP4 decode layers of T tokens (layer 0's
    experts, copied from HBM), whole layers until the budget is spent, on one
    thread (the plain oracle layer) and on `threads` threads (its routines, one
    call per expert)."""
    import synth
    import oracle
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    logits = synth.zipf_noise_logits(c["seed"], T, E, 0, c["zipf_s"], batch=0)
    ids, _, _ = oracle.route_topk(logits, k)
    used = sorted(set(ids.ravel().tolist()))
    eb = synth.expert_bytes(synth.MXFP4, H, I)
    blank = np.zeros(eb, np.uint8)
    experts = [blank] * E
    for e in used:
        experts[e] = stack[e].cpu().numpy()
    x = synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], T, H, 7, 0))
    legs = {}
    for nthr in (1, threads):
        n = 0
        t0 = time.perf_counter()
        while True:
            if nthr == 1:
                oracle.layer(synth.MXFP4, experts, x, logits, k, H, I)
            else:
                oracle_layer_threads(synth.MXFP4, experts, x, logits, k, H, I, nthr)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds or n >= 20:
                break
        legs[nthr] = dict(value=T * n / el,
                          sample=f"{n} MXFP4 decode layers of {T} tokens ({len(used)} active experts of {E}, H={H}, "
                                 f"I={I}, top-{k}) on {nthr} thread(s), {el:.1f} s")
    return cpu_baseline_entry(legs[1], legs[threads], threads, model, "layer-tokens/s")


def workload_decode_mxfp4(args):
    import torch
    import synth
    c = synth.CONFIGS["decode_mxfp4"]
    n_layers = args.layers or c["layers"]
    steps, warmup = args.steps or 10, 2 if args.warmup is None else args.warmup
    T = args.tokens or 64
    extra = "1,8" if args.extra_batches is None else args.extra_batches
    batches = [T] + [int(v) for v in extra.split(",") if v.strip() and int(v) != T]
    dev = torch.device("cuda:0")
    stack, distinct = mxfp4_resident_stack(c, n_layers, args.distinct_experts, dev)
    del distinct
    torch.cuda.empty_cache()
    res = {}
    for tb in batches:
        progress(f"decode_mxfp4: T={tb}")
        res[tb] = run_decode_mxfp4(stack, c, tb, n_layers, steps if tb == T else max(4, steps // 2), warmup,
                                   eager=args.eager)
    cpu = None if args.no_cpu_baseline else cpu_decode_mxfp4(stack, c, 8, args.cpu_seconds, *cpu_threads(args))
    m = res[T]
    keys = ("layer_tokens_per_s", "stack_tokens_per_s", "ms_per_step", "layer_hbm_gbs", "gate_up_gbs",
            "gate_up_avg_us", "down_gbs", "down_avg_us", "active_experts_mean")
    return out_line(
        m["layer_tokens_per_s"], "layer-tokens/s", steps, warmup, m["ms_per_step"], "bf16 (MXFP4 weights)",
        f"synthetic (seeded N(0,0.02) weights quantized to MXFP4, {args.distinct_experts} distinct experts copied "
        "into every slot; Zipf(1.1) popularity + N(0,1) logits, 4 batches per layer cycled; N(0,1) activations)",
        {"workload": "decode layer MXFP4: hidden 4096, 256 routed experts, top-6, intermediate 2048",
         "tokens_per_layer": T, "stacked_layers": n_layers,
         "weights_in_hbm_gb": round(stack.numel() / 1e9, 2), "slots": "all resident",
         "launch": "eager" if args.eager else "one HIP graph per step"},
        {"kernel": "gate_up_mfma<mxfp4> (moe_grouped_ffn_gate_up)", "bound": "hbm", "achieved": m["gate_up_gbs"],
         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": m["gate_up_gbs"] / HBM_PEAK_GBS,
         "traffic": measured_traffic("decode_mxfp4"),
         "avg_launch_us": m["gate_up_avg_us"], "algorithmic_bytes_per_launch": m["gate_up_bytes_avg"],
         "launches_timed": m["gate_up_launches_timed"],
         "timing": "events around back-to-back passes of the stack's gate_up launches"},
        cpu, layer_hbm_frac=m["layer_hbm_gbs"] / HBM_PEAK_GBS,
        by_batch={str(tb): {k: r[k] for k in keys} for tb, r in res.items()})


# ---------------------------------------------------------------------------
# hostbw: pinned host -> HBM copies.

def host_to_device_gbs(nbytes, reps=None):
    """GB/s of hipMemcpyAsync from pinned host memory into HBM (torch copy_ with
    non_blocking on a side stream), reps copies back to back."""
    import torch
    reps = reps or max(3, min(50, int(2e9 // nbytes)))
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    src.fill_(3)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dst.copy_(src, non_blocking=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3
    del src, dst
    return nbytes * reps / sec / 1e9


def workload_hostbw(args):
    import synth
    sizes = {"bf16_expert": synth.expert_bytes(synth.BF16, 2048, 512),
             "mxfp4_expert": synth.expert_bytes(synth.MXFP4, 4096, 2048),
             "mxfp4_layer": 256 * synth.expert_bytes(synth.MXFP4, 4096, 2048)}
    res = {}
    for name, n in sizes.items():
        res[name] = {"bytes": n, "gbs": host_to_device_gbs(n)}
        progress(f"hostbw {name}: {res[name]['gbs']:.1f} GB/s")
    big = res["mxfp4_layer"]["gbs"]
    return out_line(big, "GB/s", 1, 1, None, "u8", "synthetic (constant bytes)",
                    {"workload": "pinned host -> HBM hipMemcpyAsync at the fill sizes"},
                    None, None, by_size=res)


# ---------------------------------------------------------------------------
# prefill_mxfp4: double-buffered layer streaming around 4096-token layers.

def workload_prefill_mxfp4(args, native=False):
    import torch
    import synth
    from routed_expert_ffn_layer_amd import layer as L
    from routed_expert_ffn_layer_amd import moe
    c = synth.CONFIGS["prefill_mxfp4"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    T = args.tokens or (8192 if native else c["T"])
    wdt = moe.MOE_MXFP4_A8 if native else moe.MOE_MXFP4
    n_layers = args.layers or c["layers"]
    n_host = args.host_layers or 2
    steps, warmup = args.steps or 2, 1 if args.warmup is None else args.warmup
    dev = torch.device("cuda:0")
    eb = synth.expert_bytes(synth.MXFP4, H, I)
    lb = E * eb
    # pinned host layers (layer l streams host layer l mod n_host)
    host = []
    for j in range(n_host):
        h = torch.empty((E, eb), dtype=torch.uint8, pin_memory=True)
        h.copy_(synth.torch_mxfp4_expert_pool(E, H, I, seed=c["seed"] * 100 + j, device=dev).cpu())
        host.append(h)
        progress(f"host layer {j + 1}/{n_host} ready ({lb / 1e9:.2f} GB pinned)")
    banks = [torch.empty((E, eb), dtype=torch.uint8, device=dev) for _ in range(2)]
    ptrs = (ctypes.c_void_p * n_layers)(*[host[l % n_host].data_ptr() for l in range(n_layers)])
    fill_stream = torch.cuda.Stream()
    ls = moe.LayerStream(n_layers, lb, banks[0], banks[1], fill_stream, host_layer_ptrs=ptrs)
    b = L.LayerBuffers(T, E, k, H, I, wdt)
    n_x = 4
    logits = [torch.from_numpy(synth.normal_logits(c["seed"], T, E, 7, l)).to(dev) for l in range(n_layers)]
    xs = [torch.from_numpy(synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], T, H, 7, j))
                           .view(np.int16)).to(dev) for j in range(n_x)]
    slots = L.identity_slots(E, dev)
    comp = torch.cuda.current_stream()

    def compute(l, bank):
        L.forward(b, logits[l], xs[l % n_x], banks[bank], eb, slots)

    def pipelined():
        ls.fill(0, 0)
        for l in range(n_layers):
            if l + 1 < n_layers:
                ls.fill(l + 1, (l + 1) % 2)
            ls.acquire(l % 2, comp)
            compute(l, l % 2)
            ls.release(l % 2, comp)
        torch.cuda.synchronize()

    for _ in range(warmup):
        pipelined()
    progress("prefill: pipelined warm")
    t0 = time.perf_counter()
    for _ in range(steps):
        pipelined()
    t_pipe = (time.perf_counter() - t0) / steps
    progress(f"prefill: pipelined {t_pipe * 1e3:.1f} ms per {n_layers} layers")
    # fills alone
    t0 = time.perf_counter()
    for l in range(n_layers):
        ls.fill(l, l % 2)
    torch.cuda.synchronize()
    t_fill = time.perf_counter() - t0
    # compute alone (weights already in bank 0)
    ls.fill(0, 0)
    ls.acquire(0, comp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for l in range(n_layers):
        compute(l, 0)
    torch.cuda.synchronize()
    t_gemm = time.perf_counter() - t0
    ls.release(0, comp)
    progress(f"prefill: fills alone {t_fill * 1e3:.1f} ms, compute alone {t_gemm * 1e3:.1f} ms")
    # the grouped GEMM kernels alone, back to back on layer 0's routing
    L.route(b, logits[0])

    def gate_up(_):
        moe.moe_grouped_ffn_gate_up(b.wdt, banks[0], eb, slots, None, 0, xs[0], b.offsets, b.sorted_rows,
                                    T, k, E, H, I, b.out_rows, None, b.workspace)

    def down(_):
        moe.moe_grouped_ffn_down(b.wdt, banks[0], eb, slots, None, 0, xs[0], b.offsets, b.sorted_rows,
                                 T, k, E, H, I, b.out_rows, None, b.workspace)

    gu = time_back_to_back(gate_up, 1, 10)
    dn = time_back_to_back(down, 1, 10)
    gu_flop = 2.0 * T * k * 2 * I * H
    dn_flop = 2.0 * T * k * I * H
    layer_flop = gu_flop + dn_flop
    bp = host_to_device_gbs(lb, reps=3)
    ls.close()
    cpu = None if args.no_cpu_baseline else cpu_prefill_mxfp4(banks[0], logits[0], xs[0], c, T, args.cpu_seconds,
                                                              *cpu_threads(args), dtype=wdt)
    gu_tf = gu_flop / gu / 1e12
    peak = MFMA_FP8_PEAK_TFLOPS if native else MFMA_BF16_PEAK_TFLOPS
    line = out_line(
        T * n_layers / t_pipe, "layer-tokens/s", steps, warmup, t_pipe * 1e3,
        "fp4 x fp8 (MXFP4 weights, MXFP8 gate/up activations)" if native else "bf16 (MXFP4 weights)",
        f"synthetic (seeded N(0,0.02) weights quantized to MXFP4, {n_host} distinct pinned host layers streamed "
        "as layer l mod that; N(0,1) logits and activations)",
        {"workload": ("prefill layer MXFP4 weights with MXFP8 gate/up activations (native FP4 MFMA): "
                      if native else "prefill layer MXFP4: ") + "hidden 4096, 256 routed experts, top-6, intermediate 2048",
         "tokens_per_layer": T, "stacked_layers": n_layers, "host_layers_distinct": n_host,
         "layer_bytes": lb, "slots": "two HBM banks, one layer each"},
        {"kernel": ("mx8_quantize + grouped_gate_up<native fp4 x fp8>" if native else
                    "grouped_gate_up<mxfp4> (moe_grouped_ffn_gate_up)"), "bound": "mfma", "achieved": gu_tf,
         "peak": peak, "unit": "TFLOP/s", "frac": gu_tf / peak,
         "traffic": measured_traffic("prefill_mxfp4_a8" if native else "prefill_mxfp4"),
         "avg_launch_us": gu * 1e6, "algorithmic_flop_per_launch": gu_flop, "launches_timed": 10,
         "timing": "events around back-to-back gate_up launches on one layer's routing"},
        cpu,
        stack_tokens_per_s=T / t_pipe,
        pipeline={"t_overlapped_ms": t_pipe * 1e3, "t_fill_alone_ms": t_fill * 1e3, "t_gemm_alone_ms": t_gemm * 1e3,
                  "overlap_penalty": t_pipe / max(t_fill, t_gemm) - 1.0,
                  "fill_gbs": lb * n_layers / t_fill / 1e9, "host_to_device_gbs": bp},
        grouped_gemm={"gate_up_us": gu * 1e6, "down_us": dn * 1e6,
                      "tflops": layer_flop / (gu + dn) / 1e12,
                      "mfma_frac_bf16_peak": layer_flop / (gu + dn) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                      "layer_tflops": layer_flop / (t_gemm / n_layers) / 1e12})
    if not args.no_decode_leg and not native:
        del banks, host, b, xs, logits
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        line["decode_mxfp4"] = decode_leg(args)
    return line


def decode_leg(args):
    """The MXFP4 decode stack (43 layers, every expert resident; batch 64, then 1
    and 8), measured after the prefill line in the same run: its own value,
    roofline (gate_up against HBM) and CPU baseline."""
    import argparse as ap
    sub = ap.Namespace(**vars(args))
    sub.tokens, sub.layers, sub.extra_batches = 64, None, "1,8"
    sub.steps, sub.warmup = 10, 2
    d = workload_decode_mxfp4(sub)
    return {key: d[key] for key in ("value", "unit", "steps", "warmup", "ms_per_step", "dtype", "data", "config",
                                    "roofline", "layer_hbm_frac", "by_batch", "cpu_baseline") if key in d}


def cpu_prefill_mxfp4(bank, logits_d, x_d, c, T, seconds, threads, model, dtype=2):
    """The oracle on a bounded sample of one prefill layer, on one thread and on
    `threads` threads: routing of all T tokens, then whole experts (each with all
    of its tokens, ascending expert id) until the budget is spent; the layer time
    is extrapolated from the measured seconds per routed (token, expert) pair."""
    import synth
    import oracle
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    logits = logits_d.cpu().numpy()
    x = x_d.cpu().numpy().view(np.uint16)
    t0 = time.perf_counter()
    ids, _, _ = oracle.route_topk(logits, k)
    t_route = time.perf_counter() - t0
    jobs = expert_jobs(ids, E)[:max(4, 6 * threads)]
    weights = {e: bank[e].cpu().numpy() for e, _ in jobs}  # copied to the host before the timed calls

    def work(e, tok):
        return oracle.expert_rows(dtype, weights[e], H, I, x, tok)

    legs = {}
    for n in (1, threads):
        done, pairs, el = run_jobs(jobs, work, n, seconds)
        layer_s = t_route + el / pairs * T * k
        legs[n] = dict(value=T / layer_s,
                       sample=f"routing of {T} tokens + {len(done)} experts with {pairs} routed tokens of one MXFP4 "
                              f"prefill layer (H={H}, I={I}) on {n} thread(s), {t_route + el:.1f} s; layer time "
                              f"extrapolated to {T * k} routed tokens")
    return cpu_baseline_entry(legs[1], legs[threads], threads, model, "layer-tokens/s")


# ---------------------------------------------------------------------------
# cached_trace_bf16: 1000 single-token steps through a cold global-LRU cache.

def workload_cached_trace_bf16(args):
    import torch
    import synth
    from routed_expert_ffn_layer_amd import layer as L
    from routed_expert_ffn_layer_amd import moe
    c = synth.CONFIGS["cached_trace_bf16"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    n_layers = args.layers or c["layers"]
    tokens = args.steps or c["tokens"]
    warm_tokens = 20 if args.warmup is None else args.warmup
    n_host = args.host_layers or 8
    S = synth.cache_slots_for(c)
    dev = torch.device("cuda:0")
    eb = synth.expert_bytes(synth.BF16, H, I)
    stride = ((eb + 255) // 256) * 256
    host = []
    for j in range(n_host):
        h = torch.empty((E, eb), dtype=torch.uint8, pin_memory=True)
        h.copy_(synth.torch_bf16_expert_pool(E, H, I, seed=c["seed"] * 100 + j, device=dev).cpu())
        host.append(h)
    progress(f"cached trace: {n_host} pinned host layers ready")
    ptrs = (ctypes.c_void_p * (n_layers * E))(
        *[host[l % n_host].data_ptr() + e * eb for l in range(n_layers) for e in range(E)])
    slot_pool = torch.empty((S, stride), dtype=torch.uint8, device=dev)
    trace = synth.trace_logits(c["seed"], tokens, n_layers, E, c["zipf_s"], c["reuse_p"])
    trace_d = torch.from_numpy(trace).to(dev)
    xs = [torch.from_numpy(synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], 1, H, 7, l))
                           .view(np.int16)).to(dev) for l in range(n_layers)]
    b = L.LayerBuffers(1, E, k, H, I, moe.MOE_BF16)

    fill = None if args.fill_fraction is None else tuple(int(v) for v in args.fill_fraction.split("/"))
    if fill is not None:
        fwd = L.forward_cached_inplace
    else:
        fwd = L.forward_cached_split if args.split_waves else L.forward_cached

    def run(cache, n_tok):
        tot = dict(accesses=0, hits=0, misses=0, inplace=0, fill_bytes=0, waves=0)
        if fill is not None:
            cache.set_fill_fraction(*fill)
        for t in range(n_tok):
            for l in range(n_layers):
                _, waves = fwd(b, cache, l, trace_d[t, l:l + 1], xs[l], slot_pool, stride)
                for key in ("accesses", "hits", "misses", "inplace"):  # per step, repeated by every wave's call
                    tot[key] += waves[0][key]
                tot["fill_bytes"] += sum(w["fill_bytes"] for w in waves)
                tot["waves"] += len(waves)
        torch.cuda.synchronize()
        return tot

    fill_stream = torch.cuda.Stream()
    warm = moe.MoeCache(n_layers, E, S, expert_bytes=eb, slot_stride=stride, slot_pool=slot_pool,
                        host_expert_ptrs=ptrs, fill_stream=fill_stream)
    run(warm, warm_tokens)
    warm.close()
    progress("cached trace: warm-up done; timing the cold cache")
    cache = moe.MoeCache(n_layers, E, S, expert_bytes=eb, slot_stride=stride, slot_pool=slot_pool,
                         host_expert_ptrs=ptrs, fill_stream=fill_stream)
    t0 = time.perf_counter()
    tot = run(cache, tokens)
    el = time.perf_counter() - t0
    # elastic resize of the warm cache to half its slots (kept experts move device to device)
    half = S // 2
    new_pool = torch.empty((half, stride), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    moved = cache.resize(half, new_pool, stride)
    torch.cuda.synchronize()
    t_resize = time.perf_counter() - t1
    kept = int((moved >= 0).sum())
    resize = {"from_slots": S, "to_slots": half, "kept": kept, "ms": t_resize * 1e3,
              "moved_gbs": kept * eb / t_resize / 1e9,
              "hbm_frac": 2 * kept * eb / t_resize / 1e9 / HBM_PEAK_GBS}
    progress(f"cached trace: resize {S} -> {half} slots in {t_resize * 1e3:.1f} ms")
    cache.close()
    del new_pool
    progress(f"cached trace: {tokens} tokens in {el:.1f} s, miss rate {tot['misses'] / max(tot['accesses'], 1):.3f}")
    bp = host_to_device_gbs(eb)
    fill_gbs = tot["fill_bytes"] / el / 1e9
    link_gbs = (tot["fill_bytes"] + tot["inplace"] * eb) / el / 1e9
    cpu = None if args.no_cpu_baseline else cpu_cached_trace(trace, host, c, n_layers, n_host, S, args.cpu_seconds,
                                                             *cpu_threads(args))
    return out_line(
        tokens / el, "tokens/s", tokens, warm_tokens, el * 1e3 / tokens, "bf16",
        f"synthetic (seeded N(0,0.02) weights, {n_host} distinct pinned host layers serving layer l mod that; "
        "temporally correlated Zipf(1.0) Gumbel-top-k routing trace, reuse p=0.7)",
        {"workload": "cached decode trace bf16: 1000 tokens x 48 layers, hidden 2048, 256 experts, top-8, "
                     "intermediate 512, global LRU over 37% of the experts", "tokens": tokens,
         "stacked_layers": n_layers, "slots": S, "slot_pool_gb": round(S * stride / 1e9, 2),
         "host_layers_distinct": n_host,
         "waves": ("miss split: hits, then in-place misses while the others fill" if fill is not None else
                   "split (hits computed while misses fill)" if args.split_waves else "whole (FFN after all fills)"),
         "fill_fraction": None if fill is None else f"{fill[0]}/{fill[1]}"},
        {"kernel": "expert fills (hipMemcpyAsync pinned host -> HBM slots)" + (
            " and in-place expert reads (FFN loads from pinned host memory)" if fill is not None else ""),
         "bound": "pcie", "achieved": link_gbs, "peak": bp, "unit": "GB/s", "frac": link_gbs / bp, "traffic": None,
         "timing": "wall clock of the whole trace; bytes over the host link (fills + in-place reads); peak = measured "
                   "pinned host -> HBM bandwidth at one expert"},
        cpu, layer_tokens_per_s=tokens * n_layers / el,
        cache={"accesses": tot["accesses"], "hits": tot["hits"], "misses": tot["misses"],
               "inplace": tot["inplace"], "inplace_bytes": tot["inplace"] * eb,
               "link_gbs": (tot["fill_bytes"] + tot["inplace"] * eb) / el / 1e9,
               "miss_rate": tot["misses"] / max(tot["accesses"], 1), "fill_bytes": tot["fill_bytes"],
               "fill_gbs": fill_gbs, "host_to_device_gbs_one_expert": bp, "waves": tot["waves"],
               "expert_read_gbs": tot["accesses"] * eb / el / 1e9},
        resize=resize)


def cpu_cached_trace(trace, host, c, n_layers, n_host, S, seconds, threads, model):
    """The oracle on the first tokens of the same trace: its global LRU plus the
    layer for every (token, layer), until the budget is spent; on one thread and
    with each layer's experts spread over `threads` threads."""
    import synth
    import oracle
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    layers_host = [h.numpy() for h in host]
    xs = [synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], 1, H, 7, l)) for l in range(n_layers)]
    legs = {}
    for nthr in (1, threads):
        lru = oracle.LRU(S, n_layers, E)
        n = 0
        t0 = time.perf_counter()
        while n < trace.shape[0]:
            for l in range(n_layers):
                lg = trace[n, l:l + 1]
                ids, _, _ = oracle.route_topk(lg, k)
                counts = np.bincount(ids.ravel(), minlength=E).astype(np.int32)
                lru.step(l, counts)
                if nthr == 1:
                    oracle.layer(synth.BF16, layers_host[l % n_host], xs[l], lg, k, H, I)
                else:
                    oracle_layer_threads(synth.BF16, layers_host[l % n_host], xs[l], lg, k, H, I, nthr)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
        legs[nthr] = dict(value=n / el, sample=f"first {n} tokens of the trace through {n_layers} layers (oracle LRU "
                                               f"+ layer) on {nthr} thread(s), {el:.1f} s")
    return cpu_baseline_entry(legs[1], legs[threads], threads, model, "tokens/s")


def main():
    args = parse()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer runs on a single MI355X)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    fn = {"decode_bf16": workload_decode_bf16, "decode_mxfp4": workload_decode_mxfp4,
          "prefill_mxfp4": workload_prefill_mxfp4,
          "prefill_mxfp4_a8": lambda a: workload_prefill_mxfp4(a, native=True),
          "cached_trace_bf16": workload_cached_trace_bf16,
          "hostbw": workload_hostbw}[args.workload]
    print(json.dumps(fn(args)), flush=True)


if __name__ == "__main__":
    main()

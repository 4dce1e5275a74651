#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X, with the roofline of the dominant kernel
and the CPU oracle timed beside it.

Default workload: the bf16 decode layer (hidden 2048, 256 routed experts plus one
always-on shared expert, top-8, expert intermediate 512) at 16 tokens per layer,
stacked as 16 layers with distinct weights (16 replicas of the 257 experts, 26 GB)
so that the 256 MB Infinity Cache cannot serve re-used weights.  A step is one
pass of the whole path (top-k, permutation, grouped FFN gate_up + down, combine)
through the 16 layers; every layer has its own seeded logits and activations,
all resident in HBM before the timed region.  All experts are resident (fixed
identity slot table, no cache misses), as the workload specifies.

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "gate_up_mfma_bf16_decode_T16_counters.txt")
FFN_SOURCES = [os.path.join(ROOT, "routed_expert_ffn_layer_amd", "csrc", f) for f in ("ffn.hip", "common.hpp")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=16, help="tokens per layer (decode batch)")
    ap.add_argument("--layers", type=int, default=16, help="stacked layers with distinct weights")
    ap.add_argument("--extra-batches", default="1,4", help="other decode batches to report (not timed as value)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def ffn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per gate_up launch from the committed counter summary (rocprofv3
    FETCH_SIZE + WRITE_SIZE, scaled by the same counters on a copy of known size),
    or None if the kernel source changed since the counters were taken."""
    if not os.path.exists(COUNTERS):
        return None
    d = json.loads("\n".join(l for l in open(COUNTERS).read().splitlines() if not l.startswith("#")))
    if d.get("ffn_source_sha256") != ffn_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


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


def gate_up_bytes(n_experts_active, has_shared, T, k, H, I):
    """Algorithmic HBM bytes of one gate_up launch: each active expert's W13 once
    (2*I*H bf16), the T token rows of x, the SwiGLU intermediate written."""
    experts = n_experts_active + (1 if has_shared else 0)
    rows = T * k + (T if has_shared else 0)
    return experts * 2 * I * H * 2 + T * H * 2 + rows * I * 2


def layer_bytes(n_experts_active, has_shared, T, k, H, I):
    """Algorithmic HBM bytes of the whole layer: every active expert's weights once,
    logits, x, the intermediate (write + read), expert output rows (write + read),
    gate weights and the bf16 layer output."""
    experts = n_experts_active + (1 if has_shared else 0)
    rows = T * k + (T if has_shared else 0)
    w = experts * 3 * I * H * 2
    act = T * 256 * 4 + T * H * 2 + 2 * rows * I * 2 + 2 * rows * H * 4 + T * H * 2
    return w + act


def run_decode(args, T, n_layers, steps, warmup, time_kernel=True):
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

    def step():
        for l in range(n_layers):
            b = bufs[l]
            L.route(b, logits[l])
            gate_up(l)
            moe.moe_grouped_ffn_down(b.wdt, pools[l][:E], stride, slots, pools[l][E], I, xs[l], b.offsets,
                                     b.sorted_rows, T, k, E, H, I, b.out_rows, b.shared_out, b.workspace)
            L.combine(b, True)

    def gate_up(l):
        b = bufs[l]
        moe.moe_grouped_ffn_gate_up(b.wdt, pools[l][:E], stride, slots, pools[l][E], I, xs[l], b.offsets,
                                    b.sorted_rows, T, k, E, H, I, b.out_rows, b.shared_out, b.workspace)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    active = [int((b.counts > 0).sum().item()) for b in bufs]
    res = dict(T=T, layers=n_layers, steps=steps, seconds=elapsed, ms_per_step=1e3 * elapsed / steps,
               layer_tokens_per_s=T * n_layers * steps / elapsed, active_experts_mean=float(np.mean(active)))
    step_bytes = sum(layer_bytes(a, True, T, k, H, I) for a in active)
    res["layer_hbm_gbs"] = step_bytes * steps / elapsed / 1e9
    if time_kernel:
        # The dominant kernel, timed live on its launch stream: the same layers'
        # gate_up launches back to back (same inputs, same routing as the timed
        # steps), one event pair around each pass of n_layers launches, so the
        # events add no gap between launches and their own cost spreads over the pass.
        passes = max(4, steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for l in range(n_layers):
            gate_up(l)
        e0.record()
        for _ in range(passes):
            for l in range(n_layers):
                gate_up(l)
        e1.record()
        torch.cuda.synchronize()
        per_launch = e0.elapsed_time(e1) * 1e-3 / (passes * n_layers)
        gb = float(np.mean([gate_up_bytes(a, True, T, k, H, I) for a in active]))
        res["gate_up_avg_us"] = per_launch * 1e6
        res["gate_up_bytes_avg"] = gb
        res["gate_up_gbs"] = gb / per_launch / 1e9
        res["gate_up_launches_timed"] = passes * n_layers
    del pools
    torch.cuda.empty_cache()
    return res


def cpu_baseline(seconds):
    """The oracle (plain fp64 C, one thread) on a bounded sample of the same
    workload: decode layers of 16 tokens with the same shapes, until the budget
    is spent."""
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
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.layer(synth.BF16, experts, x, logits, k, H, I, shared=shared, I_shared=I)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 50:
            break
    return dict(value=T * n / el, unit="layer-tokens/s", cores=1, kind="oracle",
                sample=f"{n} decode layers of {T} tokens (H={H}, I={I}, {E} experts + shared, top-{k}), "
                       f"fp64 C oracle, single thread, {el:.1f} s")


def main():
    args = parse()
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
    main_res = run_decode(args, args.tokens, args.layers, args.steps, args.warmup)
    by_batch = {str(args.tokens): {k: main_res[k] for k in ("layer_tokens_per_s", "ms_per_step", "layer_hbm_gbs",
                                                           "gate_up_gbs", "gate_up_avg_us", "active_experts_mean")}}
    for tb in [int(v) for v in args.extra_batches.split(",") if v.strip()]:
        if tb == args.tokens:
            continue
        r = run_decode(args, tb, args.layers, max(10, args.steps // 2), 2)
        by_batch[str(tb)] = {k: r[k] for k in ("layer_tokens_per_s", "ms_per_step", "layer_hbm_gbs", "gate_up_gbs",
                                               "gate_up_avg_us", "active_experts_mean")}
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)
    achieved = main_res["gate_up_gbs"]
    out = {
        "metric": "MoE-layer tokens/s at 1 MI355X; % HBM BW (decode), % MFMA peak (prefill)",
        "value": main_res["layer_tokens_per_s"],
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) logits and activations)",
        "config": {"workload": "decode layer bf16: hidden 2048, 256 routed experts + 1 shared, top-8, "
                               "intermediate 512", "tokens_per_layer": args.tokens,
                   "stacked_layers": args.layers, "weights_in_hbm_gb": round(
                       args.layers * 257 * 6291456 / 1e9, 2), "slots": "all resident"},
        "roofline": {"kernel": "gate_up_mfma<bf16> (moe_grouped_ffn_gate_up)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(), "avg_launch_us": main_res["gate_up_avg_us"],
                     "algorithmic_bytes_per_launch": main_res["gate_up_bytes_avg"],
                     "launches_timed": main_res["gate_up_launches_timed"],
                     "timing": "events around back-to-back passes of the timed layers' gate_up launches"},
        "layer_hbm_frac": main_res["layer_hbm_gbs"] / HBM_PEAK_GBS,
        "by_batch": by_batch,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

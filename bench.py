"""Benchmark: one decode-layer step (o-proj + residual, router/top-k, routed experts || shared
expert, combine) per timed step, on one MI355X, through the C ABI.

Prints ONE JSON line on stdout (everything else goes to stderr).  Default workload: the
full-size layer (hidden 7168, 384 experts top-8, SwiGLU intermediate 2048, bf16 weights,
~34 GB of routed experts resident in HBM) at batch 1.

Timing protocol: weights and inputs are resident in HBM before timing starts.  Each timed
step is {flush the last-level cache by streaming a 1 GiB buffer; event A; the step's
launches; event B} on one stream, so every weight byte is fetched from HBM; value = median(B - A).
Steps are submitted as eager launches on one stream by default (on this GPU a replayed HIP
graph costs more per kernel node than an eager launch); the graph-replay time is reported
beside it.  The whole bracket (synchronize on both sides, flushes included) is reported as
wall_ms_per_iter_incl_flush.  A "warm" figure (back-to-back steps, no flush) is reported separately and
never used for the roofline fraction.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 1 << 30
COPY_BYTES = 256 << 20
# rocprofv3 HBM byte counters per dominant kernel and workload: committed summaries, valid only
# while the kernel's sources hash to what they were when the counters were taken
TRAFFIC_RECORDS = {("gemv", "full_b1", 1): "profiles/topk_gateup_gemv_full_b1.json",
                   ("gemv", "tp_rank", 1): "profiles/gemv_tp_rank_b1.json",
                   ("splitk_mfma", "tp_rank", 8): "profiles/mfma_tp_rank_b8.json",
                   ("splitk_mfma", "tp_rank", 64): "profiles/mfma_tp_rank_b64.json",
                   ("splitk_mfma", "full_b8", 8): "profiles/grouped_mfma_full_b8.json",
                   ("splitk_mfma", "verify_b8", 8): "profiles/grouped_mfma_verify_b8.json",
                   ("splitk_mfma", "full_b64", 64): "profiles/grouped_mfma_full_b64.json",
                   ("gemv", "full_b8", 2): "profiles/topk_shared_gateup_gemv_full_b8_batch2.json",
                   ("gemv", "tp_rank", 2): "profiles/topk_shared_gateup_gemv_tp_rank_b2.json",
                   ("gemv", "full_norm", 1): "profiles/topk_gateup_gemv_full_norm_b1.json",
                   ("splitk_mfma", "full_norm", 8): "profiles/grouped_mfma_full_norm_b8.json"}


def measured_traffic(path_name: str, workload: str, B: int):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of the dominant kernel, or None when no
    record exists or the kernel's sources changed since it was taken."""
    import hashlib
    rel = TRAFFIC_RECORDS.get((path_name, workload, B))
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    rec = json.load(open(os.path.join(ROOT, rel)))
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def unique_bytes(cfg, n_act: int) -> dict:
    wb = cfg.wbytes
    H, Ko, E, I, Is = cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.inter, cfg.shared_inter
    parts = {
        "oproj": wb * H * Ko,
        "router": wb * E * H + 4 * E,
        "shared_gateup": wb * 2 * Is * H,
        "routed_gateup": wb * n_act * 2 * I * H,
        "shared_down": wb * H * Is,
        "routed_down": wb * n_act * H * I,
    }
    if cfg.norm:
        parts["norm"] = wb * H
    parts["total"] = sum(parts.values())
    return parts


def cpu_baseline(cfg, B: int, reps: int) -> dict:
    """The fp64 oracle on the host cores, on one step of the same workload (bounded sample)."""
    import numpy as np

    import oracle as O
    import synth

    x, r = synth.host_tokens(cfg, B)
    dense = {n: synth.host_weight(cfg, n) for n in ("w_o", "w_r", "ws13", "ws2")}
    bias = synth.host_bias(cfg)
    # routing first (untimed) to pre-generate exactly the experts the step touches
    gamma = synth.host_norm_weight(cfg)
    probe = O.layer_step(x, r, O.LayerWeights(dense["w_o"], dense["w_r"], bias,
                                              lambda e: (np.zeros((2 * cfg.inter, cfg.hidden)),
                                                         np.zeros((cfg.hidden, cfg.inter))),
                                              dense["ws13"], dense["ws2"], norm_weight=gamma),
                         cfg.top_k, norm_eps=synth.NORM_EPS)
    experts = {int(e): synth.host_expert(cfg, int(e)) for e in probe["act"]}
    W = O.LayerWeights(dense["w_o"], dense["w_r"], bias, lambda e: experts[int(e)], dense["ws13"],
                       dense["ws2"], norm_weight=gamma)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.layer_step(x, r, W, cfg.top_k, norm_eps=synth.NORM_EPS)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    cores = len(os.sched_getaffinity(0))
    return {"value": t * 1e6, "unit": "us/step", "tokens_per_s": B / t, "cores": cores,
            "kind": "oracle", "reps": reps,
            "sample": f"one whole step of {cfg.name} at batch {B} ({len(experts)} routed experts "
                      f"touched); fp64 numpy incl. bf16->fp64 upcasts; weights pre-generated"}


def time_steps(layer, B, x, r, out, idx, gate, ws, s, flush, steps, warmup):
    """Median us of `steps` flushed eager steps (same protocol as the headline)."""
    import torch
    with torch.cuda.stream(s):
        for _ in range(warmup):
            flush.add_(1.0)
            layer.layer_decode(B, x, r, out, ws, idx, gate, stream=s)
    s.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with torch.cuda.stream(s):
        for a, b in evs:
            flush.add_(1.0)
            a.record(s)
            layer.layer_decode(B, x, r, out, ws, idx, gate, stream=s)
            b.record(s)
    s.synchronize()
    return statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)


def kernel_times(layer, B, x, r, out, idx, gate, ws, s, flush, steps) -> dict:
    """Mean us per kernel record over `steps` flushed eager steps, from the library's HIP events
    recorded around each launch on the stream it is launched on."""
    import torch
    layer.set_kernel_timing(True)
    layer.read_kernel_timing()
    with torch.cuda.stream(s):
        for _ in range(steps):
            flush.add_(1.0)
            layer.layer_decode(B, x, r, out, ws, idx, gate, stream=s)
    s.synchronize()
    recs = layer.read_kernel_timing()
    layer.set_kernel_timing(False)
    kernels = {}
    for name, ms in recs:
        kernels.setdefault(name, []).append(ms * 1e3)
    return {k: statistics.mean(v) for k, v in kernels.items()}


def roofline_for(path_name, by, kernels, workload, B):
    """The dominant kernel's achieved HBM rate: its algorithmic bytes per launch over its
    event-timed average duration.  GEMV path: the routed gate/up launch, which also runs the
    top-k and streams the shared expert's gate/up rows (layers with a norm: its down rows);
    split-K path: the gate/up record (routed
    and shared rows, and on small intermediates the SwiGLU launch that sums its K chunks)."""
    if path_name == "gemv" and "topk_shared_gateup_gemv" in kernels:
        # the routed gate/up launch whose prologue streams the shared expert's gate/up rows
        name, nbytes = "topk_shared_gateup_gemv", by["routed_gateup"] + by["shared_gateup"]
    elif path_name == "gemv":
        name, nbytes = "topk_gateup_gemv_routed", by["routed_gateup"] + by["shared_down"]
    else:
        name, nbytes = "gateup_mfma", by["routed_gateup"] + by["shared_gateup"]
    if name not in kernels:
        return None
    ach = nbytes / (kernels[name] * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(path_name, workload, B),
            "traffic_unit": "HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)",
            "bytes_per_launch": nbytes, "avg_launch_us": round(kernels[name], 3)}


def sweep(main_cfg, main_w, args, s, flush) -> dict:
    """The other workloads: batch 2 / 8 / 64 of the full-size layer, an 8-token speculative-verify
    batch (correlated tokens of one sequence) and the layer with an RMSNorm before the router
    and experts at batch 1 / 8, on the same resident weights (only the router bias and the
    norm weight differ), and one TP rank's share at batch 1, 2, 8, 64."""
    import torch

    import synth
    import synth.device as sd
    from moe_layer_skinny_amd import kk

    out = {}
    cases = ([("full_b8", 2), ("full_b8", 8), ("full_b64", 64), ("verify_b8", 8), ("full_norm", 1),
              ("full_norm", 8)] + [("tp_rank", b) for b in (1, 2, 8, 64)])
    weights = {}
    for name, B in cases:
        cfg = synth.CONFIGS[name]
        same = (cfg.hidden, cfg.oproj_in, cfg.inter) == (main_cfg.hidden, main_cfg.oproj_in,
                                                         main_cfg.inter)
        if name not in weights:
            share = main_w if same else next((v for k, v in weights.items()
                                              if synth.CONFIGS[k].oproj_in == cfg.oproj_in), None)
            log(f"[bench] sweep {name}: weights {'shared' if share is not None else 'filled'}")
            weights[name] = sd.device_weights(cfg, share_from=share)
        w = weights[name]
        layer = kk.Layer(kk.make_config(cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.top_k,
                                        cfg.inter, cfg.shared_inter, cfg.dtype,
                                        norm_eps=synth.NORM_EPS), w, B)
        x, r, _, _ = sd.device_tokens(cfg, B)
        o = torch.empty(B, cfg.hidden, dtype=torch.bfloat16, device="cuda")
        idx = torch.empty(B, cfg.top_k, dtype=torch.int32, device="cuda")
        gate = torch.empty(B, cfg.top_k, dtype=torch.float32, device="cuda")
        ws = layer.new_workspace()
        us = time_steps(layer, B, x, r, o, idx, gate, ws, s, flush, args.steps, max(2, args.warmup))
        n_act = int(torch.unique(idx).numel())
        parts = unique_bytes(cfg, n_act)
        by = parts["total"]
        gbs = by / (us * 1e-6) / 1e9
        lp = layer.query_plan(B)
        kern = {} if args.no_timing_pass else kernel_times(layer, B, x, r, o, idx, gate, ws, s,
                                                            flush, max(5, args.steps // 2))
        out[f"{name}@{B}"] = {"us_per_step": round(us, 3), "tokens_per_s": round(B / (us * 1e-6), 1),
                              "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                              "n_act": n_act, "unique_bytes": by,
                              "path": lp["path_name"],
                              "kernels_per_step": lp["kernels_per_step"],
                              "kernel_us_eager": {k: round(v, 3) for k, v in kern.items()},
                              "roofline": roofline_for(lp["path_name"], parts, kern, name, B)}
        log(f"[bench] {name}@{B}: {out[f'{name}@{B}']}")
        layer.close()
    return out


def chain_sweep(main_cfg, main_w, args, s, flush) -> dict:
    """Consecutive layers with distinct weights (kk_chain_decode), eager, with and without the
    next layer's weight prefetch on the auxiliary stream: us per chained step and per layer."""
    import torch

    import synth
    import synth.device as sd
    from moe_layer_skinny_amd import kk

    out = {}
    for name, B in (("chain_full", 1), ("chain_tp", 1), ("chain_tp", 8)):
        cfg = synth.CONFIGS[name]
        layers, keep = [], []
        for l in range(cfg.layers):
            lc = synth.layer_of(cfg, l)
            same = (lc.hidden, lc.oproj_in, lc.inter, lc.layer_seed) == (
                main_cfg.hidden, main_cfg.oproj_in, main_cfg.inter, main_cfg.layer_seed)
            w = sd.device_weights(lc, share_from=main_w if same else None)
            keep.append(w)
            layers.append(kk.Layer(kk.make_config(lc.hidden, lc.oproj_in, lc.n_experts, lc.top_k,
                                                  lc.inter, lc.shared_inter, lc.dtype,
                                                  norm_eps=synth.NORM_EPS), w, B))
        xs, r0, _, _ = sd.device_chain_tokens(cfg, B)
        outs = [torch.empty(B, cfg.hidden, dtype=torch.bfloat16, device="cuda") for _ in layers]
        ws = layers[0].new_workspace()
        for prefetch in (False, True):
            with torch.cuda.stream(s):
                for _ in range(max(2, args.warmup)):
                    flush.add_(1.0)
                    kk.chain_decode(layers, B, xs, r0, outs, ws, stream=s, prefetch=prefetch)
            s.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            with torch.cuda.stream(s):
                for a, b in evs:
                    flush.add_(1.0)
                    a.record(s)
                    kk.chain_decode(layers, B, xs, r0, outs, ws, stream=s, prefetch=prefetch)
                    b.record(s)
            s.synchronize()
            us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)
            key = f"{name}@{B}" + ("+prefetch" if prefetch else "")
            out[key] = {"layers": cfg.layers, "us_per_step": round(us, 3),
                        "us_per_layer": round(us / cfg.layers, 3)}
            log(f"[bench] {key}: {out[key]}")
        for layer in layers:
            layer.close()
        del keep
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="full_b1")
    ap.add_argument("--batch", type=int, default=0, help="default: the workload's first batch")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-timing-pass", action="store_true")
    ap.add_argument("--mode", choices=["eager", "graph"], default="eager",
                    help="how each timed step is submitted (eager: one launch per kernel on one stream)")
    ap.add_argument("--two-stream", action="store_true",
                    help="shared expert's gate/up on the auxiliary stream")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the batch 8/64 and TP-rank-share measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with two device copies of 256 MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import synth.device as sd
    from moe_layer_skinny_amd import kk

    cfg = synth.CONFIGS[args.config]
    B = args.batch or cfg.batches[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] {cfg.name} B={B}: filling weights on device")
    w = sd.device_weights(cfg, device=dev)
    layer = kk.Layer(kk.make_config(cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.top_k, cfg.inter,
                                    cfg.shared_inter, cfg.dtype, norm_eps=synth.NORM_EPS), w, B)
    plan = layer.query_plan(B)
    x, r, _, _ = sd.device_tokens(cfg, B, device=dev)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty(B, cfg.hidden, dtype=dt, device=dev)
    idx = torch.empty(B, cfg.top_k, dtype=torch.int32, device=dev)
    gate = torch.empty(B, cfg.top_k, dtype=torch.float32, device=dev)
    ws = layer.new_workspace(dev)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    s = torch.cuda.Stream(dev)

    def step(mode=args.mode):
        layer.layer_decode(B, x, r, out, ws, idx, gate, stream=s, graph=(mode == "graph"),
                           two_stream=args.two_stream)

    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            flush.add_(1.0)
            step()
    s.synchronize()
    n_act = int(torch.unique(idx).numel())
    by = unique_bytes(cfg, n_act)

    # ---- timed region: K steps, each preceded by an (untimed) cache flush
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        for a, b in evs:
            flush.add_(1.0)
            a.record(s)
            step()
            b.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    med = statistics.median(us)
    p10, p90 = us[int(0.1 * (len(us) - 1))], us[int(0.9 * (len(us) - 1))]

    # ---- the other submission mode, same protocol (reported, not the headline)
    other = "graph" if args.mode == "eager" else "eager"
    with torch.cuda.stream(s):
        step(other)
    s.synchronize()
    oevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    with torch.cuda.stream(s):
        for a, b in oevs:
            flush.add_(1.0)
            a.record(s)
            step(other)
            b.record(s)
    s.synchronize()
    other_us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in oevs)

    # ---- warm figure: back-to-back steps, no flush (cache-assisted; not the headline)
    wa, wb_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        wa.record(s)
        for _ in range(args.steps):
            step()
        wb_.record(s)
    s.synchronize()
    warm_us = wa.elapsed_time(wb_) * 1e3 / args.steps

    # ---- per-kernel durations (eager launches, library HIP events on each kernel's stream)
    kernels = {}
    if not args.no_timing_pass:
        if args.two_stream:
            layer.set_kernel_timing(True)
            layer.read_kernel_timing()
            with torch.cuda.stream(s):
                for _ in range(args.steps):
                    flush.add_(1.0)
                    layer.layer_decode(B, x, r, out, ws, idx, gate, stream=s, two_stream=True)
            s.synchronize()
            for name, ms in layer.read_kernel_timing():
                kernels.setdefault(name, []).append(ms * 1e3)
            layer.set_kernel_timing(False)
            kernels = {k: statistics.mean(v) for k, v in kernels.items()}
        else:
            kernels = kernel_times(layer, B, x, r, out, idx, gate, ws, s, flush, args.steps)
    roofline = roofline_for(plan["path_name"], by, kernels, cfg.name, B)

    gbs = by["total"] / (med * 1e-6) / 1e9
    res = {
        "metric": "µs per decode-layer step + achieved HBM GB/s (% of peak) at batch 1/8/64",
        "value": round(med, 3), "unit": "us/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(med / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "accum_dtype": "f32",
        "data": "synthetic (seeded Philox + Box-Muller: weights N(0,0.02), tokens N(0,1); random init)",
        "config": {"workload": cfg.name, "description": cfg.description, "batch": B,
                   "hidden": cfg.hidden, "oproj_in": cfg.oproj_in, "n_experts": cfg.n_experts,
                   "top_k": cfg.top_k, "inter": cfg.inter, "shared_inter": cfg.shared_inter,
                   "router_bias": cfg.bias, "path": plan["path_name"],
                   "kernels_per_step": plan["kernels_per_step"], "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(B / (med * 1e-6), 1),
        "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "unique_bytes": by["total"], "n_act": n_act,
        "p10_us": round(p10, 3), "p90_us": round(p90, 3),
        "wall_ms_per_iter_incl_flush": round(wall * 1e3 / args.steps, 4),
        "warm_us_per_step_no_flush": round(warm_us, 3),
        "submission": args.mode + ("+two_stream" if args.two_stream else ""),
        f"{other}_us_per_step": round(other_us, 3),
        "kernel_us_eager": {k: round(v, 3) for k, v in kernels.items()},
        "roofline": roofline,
    }
    layer.close()
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_sweep:
        res["batch_sweep"] = sweep(cfg, w, args, s, flush)
        res["chain_sweep"] = chain_sweep(cfg, w, args, s, flush)
    if not args.no_cpu:
        log("[bench] timing the oracle on the host cores")
        res["cpu_baseline"] = cpu_baseline(cfg, B, args.cpu_reps)
        if not args.no_sweep:
            # the batch-8 metric point: one step (about 37 experts) per repetition
            c8 = synth.CONFIGS["full_b8"]
            res["cpu_baseline_sweep"] = {"full_b8@8": cpu_baseline(c8, 8, 1)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark: MoE-layer tokens/s on one MI355X, with the roofline of each
workload's dominant kernel and the CPU oracle beside it.

The line's headline (`value`, `config`, `roofline`, `cpu_baseline`) is the
largest workload: one GLM-class MoE layer (hidden 6144, 256 routed SwiGLU
experts of intermediate 2048 in packed int4 with per-row f32 scales, top-8
sigmoid+bias routing with 8 groups / 4 kept, routed scaling 2.5, a 2048-wide
int4 shared expert), T = 2048 tokens, bf16 in and out.  One step = one
HIP-graph replay of moe_layer_forward.  Its dominant kernel, the routed
gate/up grouped GEMM, is HBM-bound (its weight stream), so its roofline is
against the 8 TB/s HBM peak, with its matrix-core fraction beside it.

The other workloads ride along under their own keys, each with its own
roofline and CPU baseline:
  c1  a decode step through 23 stacked Nano-shape layers, T = 32 (HIP graph of
      23 chained moe_layer_forward_chain calls); expert kernel against HBM;
  c2  a Nano-shape prefill layer, T = 4096 (8 hot experts); gate/up GEMM
      against the bf16 matrix-core peak;
  c4  a Nano-shape layer, T = 16384 (Zipf experts, int8 shared expert); same;
  c0  one Nano-shape layer, T = 16: cold (24 copies of the layer's weights
      rotated so that no weight is in the 256 MB last-level cache when it is
      read) and warm (one copy, repeated).
The CPU oracle is timed on each on a bounded sample, on all host threads, and
on one thread for c0-c2.

--config cN prints only that workload's line (its fields at the top level).
--copy-calibration MIB runs only a plain device-to-device copy of that size
(the reference kernel for scaling hardware byte counters) and exits.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 matrix-core peak


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_traffic(name, sources):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    summary (profiles/<name>.json), or None when any of its kernel sources
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        rec = json.load(open(path))
        for src in sources:
            digest = hashlib.sha256(open(os.path.join(ROOT, "int4_routed_expert_02_amd", "csrc", src),
                                         "rb").read()).hexdigest()
            if rec.get("sources", {}).get(src) != digest:
                return None
    except (OSError, ValueError, AttributeError):
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None,
                    help="only this workload's line (c0..c4); default: c3 headline with c1, c2, c4, c0 beside it")
    ap.add_argument("--no-extras", action="store_true", help="the c3 headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="adaptive expert top-p of the workload's router (0 = off, the workloads' own setting)")
    ap.add_argument("--act-q8", action="store_true",
                    help="Q8_0-style int8 activations for the expert matmuls (tiled configurations)")
    ap.add_argument("--int2-frac", type=float, default=0.0,
                    help="fraction of routed experts stored as packed int2 (cold-tail experts; the tiled configurations and the c1 decode step)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the headline's CPU-oracle sample")
    ap.add_argument("--cpu-seconds-extra", type=float, default=4.0,
                    help="budget of each other CPU-oracle sample (the extras and the one-thread runs)")
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--cold-copies", type=int, default=24, help="rotated weight copies of the cold c0 layer")
    ap.add_argument("--quantize", action="store_true",
                    help="time the per-row int4 quantiser on the GLM-class routed gate/up weights instead")
    ap.add_argument("--bias-update", action="store_true",
                    help="time the aux-loss-free bias update (E = 256) instead")
    ap.add_argument("--regime-sweep", action="store_true",
                    help="time the small-batch and the tiled regime at the Nano layer shape over T (cold weights) "
                         "instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB, 5 times (counter calibration), and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "launches": 5}), flush=True)
        return

    import int4_routed_expert_02_amd as moe
    import synth

    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    moe.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.quantize:
        return bench_quantize(args, moe, torch, np)
    if args.bias_update:
        return bench_bias_update(args, moe, torch, np)
    if args.regime_sweep:
        return bench_regime_sweep(args, moe, synth, torch, np, dev)

    def variant(cfg):
        if args.top_p:
            cfg = cfg.with_(top_p=args.top_p)
        if args.act_q8:
            if cfg.T <= 32:
                sys.exit("--act-q8 is a mode of the tiled configurations (c2, c3, c4)")
            cfg = cfg.with_(act_q8=True)
        if args.int2_frac:
            if cfg.T <= 32 and cfg.layers == 1:
                sys.exit("--int2-frac is a mode of the tiled configurations (c2, c3, c4) and of the c1 decode step")
            cfg = cfg.with_(int2_frac=args.int2_frac)
        return cfg

    def run(name, cpu_s, one_thread):
        cfg = variant(synth.CONFIGS[name])
        progress(f"{name}: {cfg.name}")
        if name == "c0":
            return bench_c0(args, cfg, moe, synth, torch, np, dev, cpu_s, one_thread)
        if cfg.T > 32:
            return bench_prefill(args, cfg, moe, synth, torch, np, dev, cpu_s, one_thread)
        return bench_decode(args, cfg, moe, synth, torch, np, dev, cpu_s, one_thread)

    if args.config:
        line = run(args.config, args.cpu_seconds, args.config in ("c0", "c1", "c2"))
        print(json.dumps(line), flush=True)
        return
    line = run("c3", args.cpu_seconds, False)
    torch.cuda.empty_cache()
    if not args.no_extras:
        extras = {}
        for name in ("c1", "c2", "c4", "c0"):
            r = run(name, args.cpu_seconds_extra, name in ("c0", "c1", "c2"))
            for key in ("n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "data"):
                r.pop(key, None)
            extras[name] = r
            torch.cuda.empty_cache()
        line["other_workloads"] = extras
    print(json.dumps(line), flush=True)


def cpu_baseline(oracle, work, cpu_s, unit_name, sample_fmt, threads=None):
    """Time work(n) -> units done (growing n) until cpu_s seconds are spent;
    returns the cpu_baseline object (units per second)."""
    prev = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    try:
        used = oracle.num_threads()
        done, spent, n = 0, 0.0, 1
        while spent < cpu_s:
            t0 = time.perf_counter()
            got = work(n)
            spent += time.perf_counter() - t0
            if got is None:
                break
            done += got
            # grow the sample so that the next call fits in what is left of the budget
            rate = done / spent
            n = max(1, min(2 * n, int((cpu_s - spent) * rate / max(got / n, 1e-9)) or 1))
    finally:
        oracle.set_num_threads(prev)
    return {"value": round(done / spent, 3), "unit": unit_name, "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(), "sample": sample_fmt(done, spent)}


def bench_decode(args, cfg, moe, synth, torch, np, dev, cpu_s, one_thread):
    """The decode step: 23 stacked Nano-shape layers, T = 32, each layer's
    combine taking the next layer's router logits (HIP graph per step)."""
    L, T, H = cfg.layers, cfg.T, cfg.H
    flags = moe.MOE_ADD_RESIDUAL  # bf16 out, residual added: the layer output is the next layer's input

    layers, arrays = [], []
    for l in range(L):
        d = synth.layer(cfg, l, with_hidden=False)
        layers.append(moe.MoeLayer(cfg, d, dev))
        arrays.append(d)
    x0_np = synth.hidden(cfg, 0)
    xs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L + 1)]
    xs[0].copy_(torch.from_numpy(x0_np.view(np.int16)).view(torch.bfloat16))
    wss = [layers[l].workspace(T, flags) for l in range(L)]
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    def lflags(l):
        return flags | (moe.MOE_LOGITS_GIVEN if l else 0)

    def step(s):
        for l in range(L):
            nxt = layers[l + 1] if l + 1 < L else None
            layers[l].forward_chain(xs[l], xs[l + 1], wss[l], lflags(l), nxt, wss[l + 1] if nxt is not None else None,
                                    stream=s)

    with torch.cuda.stream(stream):
        step(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(stream)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tok_s = T / (ms_per_step / 1e3)

    # the dominant kernel: the fused expert kernel, timed by HIP events on its
    # own stream around a graph of the 23 layers' expert stages alone
    # (MOE_STAGE_EXPERTS_ONLY: the same launches, reading the routing the step
    # left in each workspace), replayed back to back
    P = T * cfg.k

    def eflags(l):
        return lflags(l) | moe.MOE_STAGE_EXPERTS_ONLY

    with torch.cuda.stream(stream):
        step(stream)
        for l in range(L):
            layers[l].forward(xs[l], xs[l + 1], wss[l], eflags(l), stream=stream)
    torch.cuda.synchronize()
    egraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(egraph, stream=stream):
        for l in range(L):
            layers[l].forward(xs[l], xs[l + 1], wss[l], eflags(l), stream=stream)
    torch.cuda.synchronize()
    for _ in range(2):
        egraph.replay()
    torch.cuda.synchronize()
    ea = torch.cuda.Event(enable_timing=True)
    eb = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ea.record(stream)
        for _ in range(args.roofline_reps):
            egraph.replay()
        eb.record(stream)
    torch.cuda.synchronize()
    avg_ms = ea.elapsed_time(eb) / (args.roofline_reps * L)

    n_act, p_kept, act_w = [], [], []
    for l in range(L):
        pid, _, _, _ = moe.moe_layer_routing(moe.shape_of(cfg, T, flags), wss[l])
        base = wss[l].data_ptr()
        ids = wss[l][pid - base:pid - base + 4 * P].view(torch.int32).cpu().numpy()
        act = np.unique(ids[ids >= 0])  # (-1: a pair dropped by adaptive top-p)
        n_act.append(int(act.size))
        p_kept.append(int((ids >= 0).sum()))
        # the chosen experts' rows in their own formats (int2 cold-tail experts: half the bytes) and f32 scales
        eb = arrays[l].get("expert_bits")
        bits = eb[act].astype(np.int64) if eb is not None else np.full(act.size, 4, dtype=np.int64)
        act_w.append(int(np.sum(3 * cfg.I * H * bits // 8)) + int(act.size) * 4 * (2 * cfg.I + H))
    # algorithmic bytes of one expert-kernel launch: the weights (int4 rows and
    # f32 row scales) of every chosen routed expert and of the shared expert,
    # the activations and router logits read once, the layer output written
    # once (bf16)
    sh_w = (3 * cfg.I_sh * H * cfg.shared_bits // 8 + 4 * (2 * cfg.I_sh + H)) if cfg.shared_bits else 0
    ex_bytes = [aw + sh_w + 2 * T * H + 4 * T * cfg.E + 2 * T * H for aw in act_w]
    alg_per_launch = float(np.mean(ex_bytes))
    achieved = alg_per_launch / (avg_ms / 1e3) / 1e9  # GB/s
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": (measured_traffic("k_dec_expert_c1_traffic", ["decode.hip"])
                            if not cfg.int2_frac and not cfg.top_p else None),
                "kernel": "k_dec_expert (fused gate/up/SwiGLU/down of the chosen and shared experts)",
                "avg_launch_us": round(avg_ms * 1e3, 2), "alg_bytes_per_launch": int(alg_per_launch),
                "launches_timed": args.roofline_reps * L, "active_experts_mean": round(float(np.mean(n_act)), 2)}

    # step-level HBM fraction: algorithmic bytes of the whole step / step time
    step_bytes = 0
    for l in range(L):
        step_bytes += act_w[l]
        if cfg.shared_bits:
            step_bytes += 3 * cfg.I_sh * H * cfg.shared_bits // 8 + 4 * (2 * cfg.I_sh + H)
        step_bytes += 4 * cfg.E * H + 4 * cfg.E + 2 * T * H * 2 + 8 * T * cfg.k

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        import oracle
        lws = [oracle.LayerWeights(cfg, arrays[l]) for l in range(L)]
        state = {"x": x0_np, "l": 0}

        def work(n):
            for _ in range(n):
                l = state["l"] % L
                out = oracle.layer_forward(cfg, lws[l], state["x"], residual=True)[0]
                state["x"] = torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                state["l"] += 1
            return n * T / L  # decode-step tokens: T per 23 layer passes

        fmt = (lambda done, spent: f"{done * L / T:.0f} layer passes ({done / T:.2f} decode steps of {L} layers, "
                                   f"T={T}) in {spent:.1f} s, f64-accumulating C oracle, OpenMP over tokens/rows")
        cpu = cpu_baseline(oracle, work, cpu_s, "tokens/s", fmt)
        if one_thread:
            state.update(x=x0_np, l=0)
            cpu1 = cpu_baseline(oracle, work, cpu_s, "tokens/s", fmt, threads=1)

    line = {
        "metric": "MoE-layer tokens/s (decode step, 23 stacked int4 MoE layers)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 MFMA gate/up, f16 MFMA down, int4 weights, f32 accumulate",
        "data": "synthetic (seeded, random-init weights of the Colibri-Nano MoE layer shape)",
        "config": {"workload": cfg.name, "T": T, "layers": L, "H": H, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
                   "I_shared": cfg.I_sh, "global_batch": T, "parallelism": "single GPU",
                   "chained": "each layer's combine takes the next layer's router logits", "top_p": cfg.top_p,
                   "int2_frac": cfg.int2_frac},
        "step_hbm_GBs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_alg_bytes": int(step_bytes),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if cpu1 is not None:
        line["cpu_baseline_1thread"] = cpu1
    return line


def bench_c0(args, cfg, moe, synth, torch, np, dev, cpu_s, one_thread):
    """One Nano-shape layer, T = 16 (the small-batch regime): cold, with the
    weights of `cold_copies` identical layer copies rotated so that each call
    reads weights no recent call has touched (24 x 54 MB > the 256 MB
    last-level cache), and warm, one copy repeated.  Each is a HIP graph of
    `cold_copies` moe_layer_forward calls; the time per layer is the graph's
    time divided by the calls."""
    T, H, n = cfg.T, cfg.H, args.cold_copies
    d = synth.layer(cfg)
    copies = [moe.MoeLayer(cfg, d, dev) for _ in range(n)]
    x = torch.from_numpy(d["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
    flags = 0
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    wss = [c.workspace(T, flags) for c in copies]
    stream = torch.cuda.Stream(device=dev)

    def timed(order):
        with torch.cuda.stream(stream):
            for i, c in enumerate(order):
                copies[c].forward(x, outs[i], wss[i], flags, stream=stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i, c in enumerate(order):
                copies[c].forward(x, outs[i], wss[i], flags, stream=stream)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(args.steps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (args.steps * n)

    ms_cold = timed(list(range(n)))
    ms_warm = timed([0] * n)
    # algorithmic bytes of the layer: chosen routed experts, shared expert,
    # router, x in, out, ids and weights
    sh = moe.shape_of(cfg, T, flags)
    pid, _, _, _ = moe.moe_layer_routing(sh, wss[0])
    ids = wss[0][pid - wss[0].data_ptr():pid - wss[0].data_ptr() + 4 * T * cfg.k].view(torch.int32).cpu().numpy()
    n_act = int(np.unique(ids).size)
    alg = (n_act * (3 * cfg.I * H // 2 + 4 * (2 * cfg.I + H)) + 3 * cfg.I_sh * H // 2 + 4 * (2 * cfg.I_sh + H)
           + 4 * cfg.E * H + 4 * cfg.E + 2 * T * H * 2 + 8 * T * cfg.k)
    gbs_cold = alg / (ms_cold / 1e3) / 1e9
    gbs_warm = alg / (ms_warm / 1e3) / 1e9
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        import oracle
        lw = oracle.LayerWeights(cfg, d)

        def work(k):
            for _ in range(k):
                oracle.layer_forward(cfg, lw, d["hidden"])
            return k * T

        fmt = lambda done, spent: f"{done // T} passes of the T={T} layer in {spent:.1f} s, C oracle"
        cpu = cpu_baseline(oracle, work, cpu_s, "tokens/s", fmt)
        if one_thread:
            cpu1 = cpu_baseline(oracle, work, cpu_s, "tokens/s", fmt, threads=1)
    line = {
        "metric": "MoE-layer tokens/s (one Nano-shape layer, T=16, weights cold in HBM)",
        "value": round(T / (ms_cold / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms_cold, 5),
        "config": {"workload": cfg.name, "T": T, "H": H, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
                   "I_shared": cfg.I_sh, "rotated_weight_copies": n},
        "warm": {"value": round(T / (ms_warm / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms_warm, 5),
                 "hbm_GBs": round(gbs_warm, 1),
                 "note": "one weight copy repeated: the weights stay in the last-level cache"},
        "layer_alg_bytes": int(alg), "active_experts": n_act,
        "roofline": {"bound": "hbm", "achieved": round(gbs_cold, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs_cold / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "the whole layer (logits, fused expert kernel, combine), cold weights",
                     "avg_launch_us": round(ms_cold * 1e3, 2), "alg_bytes_per_launch": int(alg)},
        "cpu_baseline": cpu,
    }
    if cpu1 is not None:
        line["cpu_baseline_1thread"] = cpu1
    return line


def bench_regime_sweep(args, moe, synth, torch, np, dev):
    """Where the small-batch regime stops paying: one Nano-shape layer
    (moe_layer_forward, bf16 out) over T, with the weights of `cold_copies`
    identical layer copies rotated (no weight in the last-level cache when it
    is read), in the small-batch regime (MOE_REGIME_SMALL: chunks of 32
    tokens) and in the tiled regime (MOE_REGIME_TILED), whatever the default
    for that T.  Each point is a HIP graph of one call per copy; time per
    layer = graph time / copies."""
    base = synth.CONFIGS["c0"]
    n = args.cold_copies
    Tmax = 256
    d = synth.layer(base.with_(T=Tmax))
    copies = [moe.MoeLayer(base, d, dev) for _ in range(n)]
    xall = torch.from_numpy(d["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
    stream = torch.cuda.Stream(device=dev)
    rows = []
    for T in (1, 2, 4, 8, 16, 24, 32, 40, 48, 64, 80, 96, 128, 192, 256):
        x = xall[:T].contiguous()
        point = {"T": T}
        default_small = moe.moe_layer_routing(moe.shape_of(base, T, 0), copies[0].workspace(T, 0))[2] is None
        point["default"] = "small_batch" if default_small else "tiled"
        for name, fl in (("small_batch", moe.MOE_REGIME_SMALL), ("tiled", moe.MOE_REGIME_TILED)):
            outs = [torch.empty((T, base.H), dtype=torch.bfloat16, device=dev) for _ in range(n)]
            wss = [c.workspace(T, fl) for c in copies]
            with torch.cuda.stream(stream):
                for i, c in enumerate(copies):
                    c.forward(x, outs[i], wss[i], fl, stream=stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i, c in enumerate(copies):
                    c.forward(x, outs[i], wss[i], fl, stream=stream)
            torch.cuda.synchronize()
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for _ in range(args.steps):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (args.steps * n)
            point[name + "_us"] = round(us, 2)
            point[name + "_tok_s"] = round(T / (us * 1e-6), 1)
            del g, outs, wss
        rows.append(point)
        progress(f"regime sweep {point}")
    line = {"metric": "MoE-layer time per call by regime (Nano shape, cold weights)", "unit": "us",
            "config": {"workload": "one Nano-shape layer (H=1024, E=64 top-2, I=512, int4 shared I=2048) over T",
                       "rotated_weight_copies": n},
            "points": rows}
    print(json.dumps(line), flush=True)


def bench_quantize(args, moe, torch, np):
    """The step before the path: per-row symmetric int4 quantisation of the
    GLM-class layer's routed gate and up weights (256 experts x 2 x 2048 rows
    of 6144) from bf16, N(0, s^2) rows with s ~ U(0.005, 0.05), seeded on the
    device.  One step = the whole family."""
    rows, cols = 256 * 2 * 2048, 6144
    g = torch.Generator(device="cuda")
    g.manual_seed(1300)
    src = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 65536):
        sd = torch.empty(65536, 1, device="cuda").uniform_(0.005, 0.05, generator=g)
        src[r0:r0 + 65536] = (torch.randn(65536, cols, device="cuda", generator=g) * sd).to(torch.bfloat16)
    q = torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda")
    qs = torch.empty(rows, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    for _ in range(args.warmup):
        moe.moe_quantize_rows(src, 4, q, qs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        moe.moe_quantize_rows(src, 4, q, qs)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    alg = rows * cols * 2 + rows * cols // 2 + rows * 4
    gbs = alg / (ms * 1e-3) / 1e9
    line = {"metric": "per-row int4 quantiser throughput (bf16 source -> packed int4 + f32 scales)",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32 arithmetic on bf16 input", "data": "synthetic (seeded on the device)",
            "config": {"workload": "GLM-class routed gate+up family: 1048576 rows x 6144, bf16", "rows": rows,
                       "cols": cols, "bits": 4},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "k_quantize_rows<bf16,4>", "avg_launch_us": round(ms * 1e3, 2),
                         "alg_bytes_per_launch": alg}}
    if not args.no_cpu_baseline:
        import oracle
        n = 2048
        sample = src[:n].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.quantize_rows(sample, 4)
            done += n
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(done * (cols * 2 + cols // 2 + 4) / dt / 1e9, 3), "unit": "GB/s",
                                "cores": oracle.num_threads(), "kind": "oracle",
                                "sample": f"the first {n} rows, {done // n} passes in {dt:.1f} s, C oracle, OpenMP over rows"}
    print(json.dumps(line), flush=True)


def bench_bias_update(args, moe, torch, np):
    """The training-side step after the histogram: one aux-loss-free bias
    update for E = 256 experts (the GLM-class layer), counts of a 16384-pair
    step.  Latency-bound: 12 bytes per expert."""
    E = 256
    rng = np.random.default_rng(1300)
    counts = torch.from_numpy(rng.multinomial(16384, np.full(E, 1.0 / E)).astype(np.int32)).cuda()
    bias = torch.from_numpy((rng.standard_normal(E) * 0.01).astype(np.float32)).cuda()
    st = torch.cuda.current_stream()
    for _ in range(args.warmup):
        moe.moe_bias_update(counts, bias, 1e-3)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        moe.moe_bias_update(counts, bias, 1e-3)
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    alg = 12 * E
    line = {"metric": "aux-loss-free bias updates per second (E = 256)", "value": round(1e6 / us, 1),
            "unit": "updates/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic (seeded multinomial counts)",
            "config": {"workload": "one bias update, E = 256, counts of 16384 pairs", "E": E},
            "roofline": {"bound": "hbm", "achieved": round(alg / (us * 1e-6) / 1e9, 3), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 7), "traffic": None,
                         "kernel": "k_bias_update", "avg_launch_us": round(us, 2), "alg_bytes_per_launch": alg}}
    if not args.no_cpu_baseline:
        import oracle
        c, b = counts.cpu().numpy(), bias.cpu().numpy()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 2.0):
            b = oracle.bias_update(c, b, 1e-3)
            n += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(n / dt, 1), "unit": "updates/s", "cores": 1, "kind": "oracle",
                                "sample": f"{n} updates in {dt:.1f} s, C oracle through ctypes"}
    print(json.dumps(line), flush=True)


def bench_prefill(args, cfg, moe, synth, torch, np, dev, cpu_s, one_thread):
    """One large-batch layer (the tiled grouped-GEMM regime): tokens/s of one
    moe_layer_forward (bf16 out), the layer against both roofs, and the
    routed gate/up grouped GEMM (the dominant kernel) against its binding
    roof: HBM when its algorithmic bytes take longer at 8 TB/s than its flops
    at the matrix-core peak (the GLM-class layer), else the matrix cores."""
    T, H = cfg.T, cfg.H
    t0 = time.time()
    d = synth.layer(cfg)
    layer = moe.MoeLayer(cfg, d, dev)
    progress(f"{cfg.name.split(':')[0]}: inputs generated and uploaded in {time.time() - t0:.1f} s")
    x = torch.from_numpy(d["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    flags = 0
    ws = layer.workspace(T, flags)
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        layer.forward(x, out, ws, flags, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        layer.forward(x, out, ws, flags, stream=stream)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # the routed gate/up grouped GEMM (+ SwiGLU), bracketed by HIP events inside
    # real layer passes on the kernel's stream, each pass queued behind a
    # GPU-side delay so host enqueue time never lands between the events
    sh = moe.shape_of(cfg, T, flags)
    kms = []
    with torch.cuda.stream(stream):
        for _ in range(args.roofline_reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            stream.synchronize()
            torch.cuda._sleep(2_000_000)
            moe.moe_layer_forward_profiled(sh, layer.weights, x, out, ws, a, b, stream=stream)
            stream.synchronize()
            kms.append(a.elapsed_time(b))
    avg_ms = float(np.mean(kms))
    # the routed rows the pass computed (fewer than T*k when adaptive top-p drops pairs)
    _, _, poff, _ = moe.moe_layer_routing(sh, ws)
    off = ws[poff - ws.data_ptr():poff - ws.data_ptr() + 4 * (cfg.E + 1)].view(torch.int32).cpu().numpy()
    P = int(off[-1])
    counts = np.diff(off)
    touched = int(np.count_nonzero(counts))
    q8 = bool(cfg.act_q8)
    ebits = d.get("expert_bits")
    wb = (lambda e: int(ebits[e])) if ebits is not None else (lambda e: 4)
    # gate/up kernel: the touched experts' gate and up rows (int4 or int2) and
    # their f32 scales, x read once (bf16), h written once (f16; f32 + int8
    # codes in the Q8 mode are intermediates past this)
    gu_w = sum(2 * cfg.I * H * wb(e) // 8 + 8 * cfg.I for e in range(cfg.E) if counts[e])
    gu_bytes = gu_w + 2 * T * H + 2 * P * cfg.I
    gu_flops = 4.0 * P * cfg.I * H
    peak = INT8_PEAK_TOPS if q8 else BF16_PEAK_TFLOPS  # a contraction takes the peak of its own type
    t_hbm, t_mma = gu_bytes / (HBM_PEAK_GBS * 1e9), gu_flops / (peak * 1e12)
    gu_gbs = gu_bytes / (avg_ms / 1e3) / 1e9
    gu_tf = gu_flops / (avg_ms / 1e3) / 1e12
    kname = ("k_ffn_q8 gate/up (routed grouped GEMM + SwiGLU, int8 activations x int4 weights on i8 MFMA)" if q8 else
             "routed gate/up grouped GEMM + SwiGLU (int4 weights on bf16 MFMA)")
    traffic = None
    if cfg.name.startswith("c3") and not q8 and not cfg.int2_frac and not cfg.top_p:
        traffic = measured_traffic("k_ffn_gateup_c3_traffic", ["ffn.hip", "ffn_common.h"])
    if t_hbm >= t_mma:
        roofline = {"bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": round(gu_tf, 1), "peak": peak, "unit": "TOP/s" if q8 else "TFLOP/s",
                    "frac": round(gu_tf / peak, 4), "traffic": traffic}
    roofline.update({"kernel": kname, "avg_launch_us": round(avg_ms * 1e3, 2),
                     "alg_bytes_per_launch": int(gu_bytes), "alg_flops_per_launch": gu_flops,
                     "hbm_frac": round(gu_gbs / HBM_PEAK_GBS, 4), "mfma_frac": round(gu_tf / peak, 4),
                     "launches_timed": len(kms)})
    # the layer: algorithmic bytes (touched experts' three matrices and scales,
    # the shared expert, the router, x in, out, ids and weights) and flops
    sh_bytes = (3 * cfg.I_sh * H * cfg.shared_bits // 8 + 4 * (2 * cfg.I_sh + H)) if cfg.shared_bits else 0
    layer_bytes = (sum(3 * cfg.I * H * wb(e) // 8 + 4 * (2 * cfg.I + H) for e in range(cfg.E) if counts[e])
                   + sh_bytes + 4 * cfg.E * H + 4 * cfg.E + 2 * T * H * 2 + 8 * T * cfg.k)
    layer_flops = 6.0 * P * H * cfg.I + (6.0 * T * H * cfg.I_sh if cfg.shared_bits else 0.0)
    t_s = ms_per_step / 1e3
    lt_hbm, lt_mma = layer_bytes / (HBM_PEAK_GBS * 1e9), layer_flops / (peak * 1e12)

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        import oracle
        lw = oracle.LayerWeights(cfg, d)
        state = {"off": 0}

        def work(n):
            o = state["off"] % T
            take = min(n, T - o)
            oracle.layer_forward(cfg.with_(T=take), lw, d["hidden"][o:o + take])
            state["off"] += take
            return take

        fmt = (lambda done, spent: f"{done} tokens of the batch as sub-batches (router, permutation, routed and "
                                   f"shared FFN, combine) in {spent:.1f} s, f64-accumulating C oracle")
        cpu = cpu_baseline(oracle, work, cpu_s, "tokens/s", fmt)
        if one_thread:
            state["off"] = 0
            cpu1 = cpu_baseline(oracle, work, cpu_s, "tokens/s", fmt, threads=1)
    line = {
        "metric": f"MoE-layer tokens/s (prefill layer, {cfg.name.split(':')[0]})",
        "value": round(T / t_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("i8 MFMA (Q8_0-style activations x int4/int8 weights), i32 block sums, f32 accumulate" if q8 else
                  "bf16 MFMA gate/up, f16 MFMA down, int4 weights, f32 accumulate"),
        "data": "synthetic (seeded)",
        "config": {"workload": cfg.name, "T": T, "H": H, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
                   "I_shared": cfg.I_sh, "shared_bits": cfg.shared_bits, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "rsf": cfg.rsf, "global_batch": T,
                   "parallelism": "single GPU", "top_p": cfg.top_p, "routed_pairs": P, "act_q8": q8,
                   "int2_frac": cfg.int2_frac},
        "layer": {"alg_bytes": int(layer_bytes), "alg_flops": layer_flops, "experts_touched": touched,
                  "hbm_GBs": round(layer_bytes / t_s / 1e9, 1), "hbm_frac": round(layer_bytes / t_s / 1e9 / HBM_PEAK_GBS, 4),
                  "TFLOPs": round(layer_flops / t_s / 1e12, 1),
                  "mfma_frac": round(layer_flops / t_s / 1e12 / peak, 4),
                  "bound": "hbm" if lt_hbm >= lt_mma else "mfma",
                  "roofline_frac": round(max(lt_hbm, lt_mma) / t_s, 4),
                  "ideal_us": round(max(lt_hbm, lt_mma) * 1e6, 1),
                  "rows_per_expert_max": int(counts.max()), "rows_per_expert_min": int(counts.min())},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if cpu1 is not None:
        line["cpu_baseline_1thread"] = cpu1
    return line


if __name__ == "__main__":
    main()

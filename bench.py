#!/usr/bin/env python3
"""Benchmark: MoE-layer decode step on one MI355X.

Workload: a decode step through 23 stacked Nano-shape MoE layers (hidden 1024,
64 routed SwiGLU experts of intermediate 512 in packed int4 with per-row f32
scales, top-2 sigmoid+bias routing, a 2048-wide int4 shared expert), T = 32
tokens, bf16 hidden state, the residual added in each layer's combine.  Every
layer has its own seeded weights (828 MB of layer weights per step in total,
more than the 256 MB last-level cache, so each step streams them from HBM).
One step = one HIP-graph replay of the 23 moe_layer_forward calls.

Prints one JSON line: tokens/s for the step, plus
  roofline:     the fused expert kernel (the step's weight stream: every chosen
                routed expert and the shared expert) against HBM peak; its
                average duration comes from HIP events on its stream around
                back-to-back replays of the 23 layers' expert stages;
  cpu_baseline: the CPU oracle on a bounded sample of the same workload.

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


def sh_of(moe, cfg, T, flags):
    return moe.shape_of(cfg, T, flags)


def measured_traffic(root):
    """HBM bytes per expert-kernel launch from the committed rocprofv3 counter
    summary, or None when the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(root, "profiles", "k_dec_expert_c1_traffic.json")
    src = os.path.join(root, "int4_routed_expert_02_amd", "csrc", "decode.hip")
    try:
        rec = json.load(open(path))
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("decode_hip_sha256") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c1", help="workload key (c1 = the decode step this line reports)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="adaptive expert top-p of the workload's router (0 = off, the workloads' own setting)")
    ap.add_argument("--act-q8", action="store_true",
                    help="Q8_0-style int8 activations for the expert matmuls (tiled configurations)")
    ap.add_argument("--int2-frac", type=float, default=0.0,
                    help="fraction of routed experts stored as packed int2 (cold-tail experts; tiled configurations)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--quantize", action="store_true",
                    help="time the per-row int4 quantiser on the GLM-class routed gate/up weights instead")
    ap.add_argument("--bias-update", action="store_true",
                    help="time the aux-loss-free bias update (E = 256) instead")
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
    cfg = synth.CONFIGS[args.config]
    if args.top_p:
        cfg = cfg.with_(top_p=args.top_p)
    if args.act_q8:
        if cfg.T <= 32:
            sys.exit("--act-q8 is a mode of the tiled configurations (c2, c3, c4)")
        cfg = cfg.with_(act_q8=True)
    if args.int2_frac:
        if cfg.T <= 32:
            sys.exit("--int2-frac is a mode of the tiled configurations (c2, c3, c4)")
        cfg = cfg.with_(int2_frac=args.int2_frac)
    if cfg.T > 32:
        return bench_prefill(args, cfg, moe, synth, torch, np, dev)
    L, T, H = cfg.layers, cfg.T, cfg.H
    flags = moe.MOE_ADD_RESIDUAL  # bf16 out, residual added: the layer output is the next layer's input

    # ---- inputs resident in HBM before timing
    t0 = time.time()
    layers, arrays = [], []
    for l in range(L):
        d = synth.layer(cfg, l, with_hidden=False)
        layers.append(moe.MoeLayer(cfg, d, dev))
        arrays.append(d)
    x0_np = synth.hidden(cfg, 0)
    gen_s = time.time() - t0
    xs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L + 1)]
    xs[0].copy_(torch.from_numpy(x0_np.view(np.int16)).view(torch.bfloat16))
    wss = [layers[l].workspace(T, flags) for l in range(L)]
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    # the chained step: each layer's combine also takes the next layer's router
    # logits of the output row just written, so layers 2..L run no logits
    # kernel (MOE_LOGITS_GIVEN)
    def lflags(l):
        return flags | (moe.MOE_LOGITS_GIVEN if l else 0)

    def step(s):
        for l in range(L):
            nxt = layers[l + 1] if l + 1 < L else None
            layers[l].forward_chain(xs[l], xs[l + 1], wss[l], lflags(l), nxt, wss[l + 1] if nxt is not None else None,
                                    stream=s)

    # eager once (validates arguments), then capture the step in a HIP graph
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
    ms_total = ev0.elapsed_time(ev1)
    t_wall0 = time.time()
    ms_per_step = ms_total / args.steps
    tok_s = T / (ms_per_step / 1e3)

    # ---- roofline of the dominant kernel: the fused expert kernel (gate/up +
    # SwiGLU + down of every chosen routed expert and of the shared expert, one
    # launch per layer, each taking its routing decision from the router
    # logits in its workspace).  Its duration is measured with
    # HIP events on the kernel's own stream around a HIP graph of the 23
    # layers' expert stages alone (MOE_STAGE_EXPERTS_ONLY: the same launches as
    # in the step above, reading the routing the step left in each workspace),
    # replayed back to back: average = elapsed / launches.
    P = T * cfg.k

    def eflags(l):
        return lflags(l) | moe.MOE_STAGE_EXPERTS_ONLY

    with torch.cuda.stream(stream):
        step(stream)  # leave each layer's routing in its workspace
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

    n_act, p_kept = [], []
    for l in range(L):
        pid, _, _, _ = moe.moe_layer_routing(sh_of(moe, cfg, T, flags), wss[l])
        base = wss[l].data_ptr()
        ids = wss[l][pid - base:pid - base + 4 * P].view(torch.int32).cpu().numpy()
        n_act.append(int(np.unique(ids[ids >= 0]).size))  # (-1: a pair dropped by adaptive top-p)
        p_kept.append(int((ids >= 0).sum()))
    # algorithmic bytes of one expert-kernel launch: the weights (int4 rows and
    # f32 row scales) of every chosen routed expert and of the shared expert,
    # the activations and routing logits read once, one f32 output row per
    # (token, expert) pair and per token for the shared expert
    sh_w = (3 * cfg.I_sh * H * cfg.shared_bits // 8 + 4 * (2 * cfg.I_sh + H)) if cfg.shared_bits else 0
    ex_bytes = [na * (3 * cfg.I * H // 2 + 4 * (2 * cfg.I + H)) + sh_w + 2 * T * H + 4 * T * cfg.E
                + 4 * pk * H + (4 * T * H if cfg.shared_bits else 0) for na, pk in zip(n_act, p_kept)]
    alg_per_launch = float(np.mean(ex_bytes))
    achieved = alg_per_launch / (avg_ms / 1e3) / 1e9  # GB/s
    traffic = measured_traffic(ROOT)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_dec_expert<4,1> (routing + fused gate/up/SwiGLU/down of the chosen and shared experts)",
                "avg_launch_us": round(avg_ms * 1e3, 2), "alg_bytes_per_launch": int(alg_per_launch),
                "launches_timed": args.roofline_reps * L, "active_experts_mean": round(float(np.mean(n_act)), 2)}

    # step-level HBM fraction: algorithmic bytes of the whole step / step time
    step_bytes = 0
    for l in range(L):
        step_bytes += n_act[l] * (3 * cfg.I * H // 2 + 4 * (2 * cfg.I + H))
        if cfg.shared_bits:
            step_bytes += 3 * cfg.I_sh * H * cfg.shared_bits // 8 + 4 * (2 * cfg.I_sh + H)
        step_bytes += 4 * cfg.E * H + 4 * cfg.E + 2 * T * H * 2 + 8 * T * cfg.k

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        lws = [oracle.LayerWeights(cfg, arrays[l]) for l in range(L)]
        x = x0_np
        n_layers_done, t_cpu0 = 0, time.time()
        while time.time() - t_cpu0 < args.cpu_seconds or n_layers_done < L:
            l = n_layers_done % L
            out = oracle.layer_forward(cfg, lws[l], x, residual=True)[0]
            x = torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            n_layers_done += 1
        cpu_s = time.time() - t_cpu0
        steps_done = n_layers_done / L
        cpu = {"value": round(T * steps_done / cpu_s, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{n_layers_done} layer passes ({steps_done:.2f} decode steps of 23 layers, T={T}) "
                         f"in {cpu_s:.1f} s, f64-accumulating C oracle, OpenMP over tokens/rows"}

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
                   "chained": "each layer's combine takes the next layer's router logits", "top_p": cfg.top_p},
        "step_hbm_GBs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_alg_bytes": int(step_bytes),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
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


def bench_prefill(args, cfg, moe, synth, torch, np, dev):
    """One large-batch layer (the tiled grouped-GEMM regime): tokens/s of one
    moe_layer_forward (bf16 out), and the routed gate/up grouped GEMM against
    the bf16 matrix-core peak."""
    T, H, P = cfg.T, cfg.H, cfg.T * cfg.k
    d = synth.layer(cfg)
    layer = moe.MoeLayer(cfg, d, dev)
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
    P = int(ws[poff - ws.data_ptr() + 4 * cfg.E:poff - ws.data_ptr() + 4 * cfg.E + 4].view(torch.int32).item())
    gu_flops = 4.0 * P * cfg.I * H
    achieved = gu_flops / (avg_ms / 1e3) / 1e12
    layer_flops = 6.0 * P * H * cfg.I + (6.0 * T * H * cfg.I_sh if cfg.shared_bits else 0.0)
    q8 = bool(cfg.act_q8)
    peak = INT8_PEAK_TOPS if q8 else BF16_PEAK_TFLOPS  # a contraction takes the peak of its own type
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TOP/s" if q8 else "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                "kernel": ("k_ffn_q8 gate/up (routed grouped GEMM + SwiGLU, int8 activations x int4 weights on "
                           "i8 MFMA)" if q8 else
                           "k_ffn gate/up (routed grouped GEMM + SwiGLU, int4 weights on bf16 MFMA)"),
                "avg_launch_us": round(avg_ms * 1e3, 2), "alg_flops_per_launch": gu_flops,
                "launches_timed": len(kms)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        lw = oracle.LayerWeights(cfg, d)
        n, spent, done = 4, 0.0, 0
        while spent < args.cpu_seconds and done < T:
            take = min(n, T - done)
            t0 = time.time()
            oracle.layer_forward(cfg.with_(T=take), lw, d["hidden"][done:done + take])
            spent += time.time() - t0
            done += take
            n *= 2
        cpu = {"value": round(done / spent, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"the first {done} tokens of the batch as sub-batches (router, permutation, routed and "
                         f"shared FFN, combine) in {spent:.1f} s, f64-accumulating C oracle"}
    line = {
        "metric": f"MoE-layer tokens/s (prefill layer, {cfg.name})",
        "value": round(T / (ms_per_step / 1e3), 1),
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
                   "I_shared": cfg.I_sh, "shared_bits": cfg.shared_bits, "global_batch": T,
                   "parallelism": "single GPU", "top_p": cfg.top_p, "routed_pairs": P, "act_q8": q8,
                   "int2_frac": cfg.int2_frac},
        "layer_TFLOPs": round(layer_flops / (ms_per_step / 1e3) / 1e12, 1),
        "layer_mfma_frac": round(layer_flops / (ms_per_step / 1e3) / 1e12 / peak, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

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
  roofline:     the routed gate/up grouped-GEMM kernel (the largest weight
                stream of the step) against HBM peak, its duration measured with
                HIP events around each launch on its own stream;
  cpu_baseline: the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c1", help="workload key (c1 = the decode step this line reports)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--roofline-reps", type=int, default=10)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import int4_routed_expert_02_amd as moe
    import synth

    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    moe.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
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

    def step(s):
        for l in range(L):
            layers[l].forward(xs[l], xs[l + 1], wss[l], flags, stream=s)

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

    # ---- roofline of the dominant kernel: the expert gate/up weight stream
    # (routed experts the batch selected + the shared expert, one launch per
    # layer).  HIP events are recorded right before and after that kernel on
    # its own stream inside real layer passes (moe_layer_forward_profiled);
    # each pass is queued behind a short GPU-side delay so that host enqueue
    # time never lands between the events.
    P = T * cfg.k
    sh_f = moe.shape_of(cfg, T, flags)
    pairs = []
    with torch.cuda.stream(stream):
        for rep in range(args.roofline_reps):
            evl = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
            for a, b in evl:  # materialise the events before handing their handles to the library
                a.record(stream)
                b.record(stream)
            stream.synchronize()
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(2_000_000)
            for l in range(L):
                moe.moe_layer_forward_profiled(sh_f, layers[l].weights, xs[l], xs[l + 1], wss[l], evl[l][0],
                                               evl[l][1], stream=stream)
            pairs.append(evl)
    torch.cuda.synchronize()
    n_act = []
    for l in range(L):
        pid, _, _, _ = moe.moe_layer_routing(sh_f, wss[l])
        base = wss[l].data_ptr()
        ids = wss[l][pid - base:pid - base + 4 * P].view(torch.int32).cpu().numpy()
        n_act.append(int(np.unique(ids).size))
    sh_bytes = (cfg.I_sh * H * cfg.shared_bits // 8 + 8 * cfg.I_sh) if cfg.shared_bits else 0
    gu_bytes = [na * (cfg.I * H + 8 * cfg.I) + sh_bytes + 2 * T * H + 4 * P * cfg.I + 4 * T * cfg.I_sh + 4 * P
                for na in n_act]
    k_ms, k_b = [], []
    for evl in pairs:
        for l, (a, b) in enumerate(evl):
            k_ms.append(a.elapsed_time(b))
            k_b.append(gu_bytes[l])
    avg_ms = float(np.mean(k_ms))
    achieved = float(np.sum(k_b)) / (float(np.sum(k_ms)) / 1e3) / 1e9  # GB/s
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "k_dec_gateup<4> (expert gate/up + SwiGLU weight stream)",
                "avg_launch_us": round(avg_ms * 1e3, 2), "alg_bytes_per_launch": int(np.mean(gu_bytes)),
                "launches_timed": len(k_ms)}

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
        "dtype": "bf16 MFMA, int4 weights, f32 accumulate",
        "data": "synthetic (seeded, random-init weights of the Colibri-Nano MoE layer shape)",
        "config": {"workload": cfg.name, "T": T, "layers": L, "H": H, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
                   "I_shared": cfg.I_sh, "global_batch": T, "parallelism": "single GPU"},
        "step_hbm_GBs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_alg_bytes": int(step_bytes),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

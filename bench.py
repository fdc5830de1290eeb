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

    # ---- roofline of the dominant kernel: routed gate/up + SwiGLU (the largest weight stream)
    # Each launch reads the gate and up rows (int4) and scales of every expert its layer
    # routes to, the gathered hidden rows, and writes h (f32) for every pair.
    sh = moe.shape_of(cfg, T, 0)
    P = T * cfg.k
    routing = []
    for l in range(L):
        pid, pw, poff, psrt = moe.moe_layer_routing(moe.shape_of(cfg, T, flags), wss[l])
        off = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
        srt = torch.empty(P, dtype=torch.int32, device=dev)
        base = wss[l].data_ptr()
        off.copy_(wss[l][poff - base:poff - base + 4 * (cfg.E + 1)].view(torch.int32))
        srt.copy_(wss[l][psrt - base:psrt - base + 4 * P].view(torch.int32))
        routing.append((off, srt))
    torch.cuda.synchronize()
    alg_bytes = []
    for l in range(L):
        counts = np.diff(routing[l][0].cpu().numpy())
        n_act = int(np.count_nonzero(counts))
        alg_bytes.append(n_act * (2 * cfg.I * H // 2 + 2 * cfg.I * 4) + P * H * 2 + P * cfg.I * 4)
    y_dummy = torch.empty((P, H), dtype=torch.float32, device=dev)
    wsf = torch.empty(moe.moe_workspace_bytes(sh, moe.MOE_WS_EXPERT_FFN), dtype=torch.uint8, device=dev)
    evs = []
    with torch.cuda.stream(stream):
        for rep in range(args.roofline_reps):
            for l in range(L):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                moe.moe_expert_ffn(moe.shape_of(cfg, T, moe.MOE_STAGE_GATEUP_ONLY), xs[l], layers[l].weights,
                                   routing[l][0], routing[l][1], None, y_dummy, wsf, stream=stream)
                b.record(stream)
                evs.append((a, b, alg_bytes[l]))
    torch.cuda.synchronize()
    k_ms = [a.elapsed_time(b) for a, b, _ in evs]
    k_bytes = [nb for _, _, nb in evs]
    avg_ms = float(np.mean(k_ms))
    achieved = float(np.sum(k_bytes)) / (float(np.sum(k_ms)) / 1e3) / 1e9  # GB/s
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "k_ffn gate/up+SwiGLU (routed, 16-row tiles)",
                "avg_launch_us": round(avg_ms * 1e3, 2), "alg_bytes_per_launch": int(np.mean(alg_bytes))}

    # step-level HBM fraction: algorithmic bytes of the whole step / step time
    step_bytes = 0
    for l in range(L):
        counts = np.diff(routing[l][0].cpu().numpy())
        n_act = int(np.count_nonzero(counts))
        step_bytes += n_act * (3 * cfg.I * H // 2 + 4 * (2 * cfg.I + H))
        step_bytes += 3 * cfg.I_sh * H // 2 + 4 * (2 * cfg.I_sh + H)
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

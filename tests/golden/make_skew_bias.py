"""Calibrate the per-rank router-bias offsets of the skewed workloads.

The prefill workload wants its 8 hottest experts at ~3x the mean load, and the
large-batch workload wants expert popularity to follow Zipf(s = 1.2).  Neither
target says how to get there; the reading taken here mirrors the aux-loss-free
balancing of the model card ("Architecture": sigmoid+bias router with
DeepSeek-V3-style aux-loss-free balancing) run toward a skewed target: a fixed
number of additive bias updates, each moving an expert's bias by a step
proportional to log(target load / observed load), measured with the oracle's
router on a separate calibration batch (the workload seed + 50000).  The frozen
offsets are stored by popularity rank in synth/skew_bias.json; the generator
adds them to the N(0, 0.01) bias of the experts that a seeded permutation
ranks.  Re-run with:  python tests/golden/make_skew_bias.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

ITERS = 80
STEP = 0.03


def calibrate(key: str) -> dict:
    cfg = synth.CONFIGS[key]
    target = synth.skew_targets(cfg)
    P = cfg.T * cfg.k
    rank_of = synth.skew_ranking(cfg)  # rank r -> expert id
    W, base_bias = synth.router(cfg, with_skew=False)
    x = synth.hidden(cfg, seed=cfg.seed + 50000)
    off = np.zeros(cfg.E, np.float64)
    best = None
    for it in range(ITERS):
        bias = base_bias.copy()
        bias[rank_of] = (bias[rank_of].astype(np.float64) + off).astype(np.float32)
        ids, _, _, _ = oracle.router(cfg, x, W, bias)
        load = np.bincount(ids.ravel(), minlength=cfg.E)[rank_of] / P
        err = float(np.max(np.abs(np.log(np.maximum(load, 0.5 / P)) - np.log(target))))
        if best is None or err < best[0]:
            best = (err, off.copy(), load.copy())
        off += STEP * (np.log(target) - np.log(np.maximum(load, 0.5 / P)))
    err, off, load = best
    return {
        "offset_by_rank": [float(np.float32(v)) for v in off],
        "target_share_by_rank": [float(v) for v in target],
        "calibration_share_by_rank": [float(v) for v in load],
        "max_abs_log_error": err,
        "calibration": f"oracle router on {cfg.T} tokens, seed {cfg.seed + 50000}, {ITERS} updates of step {STEP}",
    }


def main():
    out = {name: calibrate(key) for key, name in (("c2", "hot8x3"), ("c4", "zipf1.2"))}
    path = os.path.join(ROOT, "synth", "skew_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    for k, v in out.items():
        print(k, "max |log(load/target)| =", round(v["max_abs_log_error"], 4))


if __name__ == "__main__":
    main()

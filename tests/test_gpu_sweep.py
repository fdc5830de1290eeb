"""GPU parity over a seeded sweep of layer shapes (both regimes, both tile
paths, with and without precomputed row sums; small-batch shapes with int2
experts, top-p and group limits): the HIP path through the C
ABI against the CPU oracle, at the bars of test_gpu_parity.py.  The shapes
are drawn once from a fixed seed and kept where moe_validate_shape accepts
them and the oracle finishes quickly."""
import numpy as np
import pytest

import int4_routed_expert_02_amd as moe
import synth
from gpu_util import check_output, check_routing, check_routing_top_p, run_layer, say

pytestmark = pytest.mark.gpu


def _sweep(n=14, seed=20261203):
    rng = np.random.default_rng(seed)
    out = {}
    tries = 0
    while len(out) < n and tries < 2000:
        tries += 1
        E = int(rng.choice([4, 8, 16, 32, 64, 128, 256]))
        k = int(rng.integers(1, min(8, E) + 1))
        H = int(rng.choice([256, 512, 1024, 2048, 3072]))
        I = int(rng.choice([64, 128, 192, 256, 512, 1024, 2048]))
        shared = int(rng.choice([0, 4, 4, 8]))
        I_sh = int(rng.choice([128, 512, 2048])) if shared else 128
        T = int(rng.choice([1, 7, 16, 33, 64, 65, 130, 257, 400]))
        n_group, topk_group = 1, 1
        if E >= 16 and rng.random() < 0.4:
            n_group = int(rng.choice([g for g in (2, 4, 8) if E % g == 0]))
            topk_group = int(rng.integers(1, n_group + 1))
            if k > topk_group * (E // n_group):
                continue
        rsf = float(rng.choice([1.0, 2.5]))
        cost = T * (k * 3 * H * I + (3 * H * I_sh if shared else 0))
        if cost > 6e8:
            continue
        cfg = synth.LayerConfig(f"sweep{len(out)}", T=T, H=H, E=E, k=k, I=I, I_sh=I_sh, n_group=n_group,
                                topk_group=topk_group, rsf=rsf, shared_bits=shared, seed=7000 + len(out))
        out[cfg.name] = cfg
    return out


def _sweep_tiled(n=10, seed=20261204):
    """Few experts and enough rows per expert for the pipelined tiles, with
    contractions of 2048 and more (precomputed row sums) mixed in."""
    rng = np.random.default_rng(seed)
    out = {}
    tries = 0
    while len(out) < n and tries < 2000:
        tries += 1
        E = int(rng.choice([4, 8]))
        k = int(rng.integers(1, 3))
        H = int(rng.choice([1024, 2048, 3072]))
        I = int(rng.choice([256, 512, 2048]))
        shared = int(rng.choice([0, 4, 8]))
        I_sh = int(rng.choice([512, 2048])) if shared else 128
        T = int(rng.choice([100, 130, 257]))
        rsf = float(rng.choice([1.0, 2.5]))
        cost = T * (k * 3 * H * I + (3 * H * I_sh if shared else 0))
        if cost > 2e9:
            continue
        cfg = synth.LayerConfig(f"tiled{len(out)}", T=T, H=H, E=E, k=k, I=I, I_sh=I_sh, rsf=rsf,
                                shared_bits=shared, seed=7100 + len(out))
        out[cfg.name] = cfg
    return out


def _sweep_small(n=12, seed=20261205):
    """Shapes the small-batch kernel takes (H % 1024, I % 512, top-k <= 16,
    T <= 64: one or two chunks of 32 tokens), with int2 cold-tail experts,
    adaptive top-p and group limits mixed in."""
    rng = np.random.default_rng(seed)
    out = {}
    tries = 0
    while len(out) < n and tries < 2000:
        tries += 1
        E = int(rng.choice([8, 16, 64, 128, 256]))
        k = int(rng.integers(1, min(16, E) + 1))
        H = int(rng.choice([1024, 2048]))
        I = int(rng.choice([512, 1024]))
        shared = int(rng.choice([0, 4, 8]))
        I_sh = int(rng.choice([512, 2048])) if shared else 512
        T = int(rng.choice([1, 5, 17, 32, 33, 64]))
        n_group, topk_group = 1, 1
        if E >= 16 and rng.random() < 0.4:
            n_group = int(rng.choice([g for g in (2, 4, 8) if E % g == 0]))
            topk_group = int(rng.integers(1, n_group + 1))
            if k > topk_group * (E // n_group):
                continue
        int2_frac = float(rng.choice([0.0, 0.3, 1.0]))
        top_p = float(rng.choice([0.0, 0.0, 0.5]))
        top_p = top_p if k >= 2 else 0.0  # (top-1 never drops a pair)
        cost = T * (k * 3 * H * I + (3 * H * I_sh if shared else 0))
        if cost > 1.5e9:
            continue
        cfg = synth.LayerConfig(f"small{len(out)}", T=T, H=H, E=E, k=k, I=I, I_sh=I_sh, n_group=n_group,
                                topk_group=topk_group, rsf=float(rng.choice([1.0, 2.5])), shared_bits=shared,
                                int2_frac=int2_frac, top_p=top_p, seed=7200 + len(out))
        out[cfg.name] = cfg
    return out


SWEEP = {**_sweep(), **_sweep_tiled(), **_sweep_small()}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()


@pytest.mark.parametrize("name", sorted(SWEEP))
def test_sweep_layer_parity(name):
    cfg = SWEEP[name]
    if moe.moe_validate_shape(moe.shape_of(cfg)) != moe.MOE_OK:
        pytest.skip("shape outside what the kernels cover")
    say(f"[sweep] {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} I_sh={cfg.I_sh} "
        f"shared={cfg.shared_bits} groups={cfg.n_group}/{cfg.topk_group} rsf={cfg.rsf}")
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d)
    if name.startswith("small"):
        assert offsets is None, f"{name}: the small-batch regime was not taken"
    chk = check_routing_top_p if cfg.top_p else check_routing
    ex = chk(cfg, d, d["hidden"], ids, w, offsets, srt, tag=name)
    check_output(cfg, d, d["hidden"], got, ex, tag=f"{name} (exempt {int(ex.sum())})")

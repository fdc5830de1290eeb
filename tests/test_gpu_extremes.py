"""GPU parity at the edges of the shapes the library accepts: the largest
top_k of each regime (16 in the small-batch kernel, 64 in the tiled one),
every expert chosen (k = E), one and two routed experts, group limits that
keep one group or all of them, the smallest accepted H and I, and the
small-batch shapes run through both regimes.  The HIP path through the C
ABI against the CPU oracle, at the bars of test_gpu_parity.py: ids
bit-exact outside near ties, weights, the permutation, outputs within
1e-2 of the oracle's RMS."""
import pytest

import int4_routed_expert_02_amd as moe
import synth
from gpu_util import check_output, check_routing, is_decode, run_layer, say, small_cfg

pytestmark = pytest.mark.gpu

_C1 = synth.CONFIGS["c1"]

EXT = {
    # the small-batch kernel's largest top_k, plain and group-limited
    "k16_small_batch_E64": _C1.with_(T=32, k=16, layers=1, seed=61),
    "k16_small_batch_E256_grouped": _C1.with_(T=20, E=256, k=16, n_group=8, topk_group=4, rsf=2.5, layers=1,
                                              seed=63),
    # top_k 16 past the small-batch cut (tiled)
    "k16_tiled_E64": _C1.with_(T=150, k=16, layers=1, seed=62),
    # the tiled kernels' largest top_k: 64 of 256 experts in 64 groups of 4, 32 groups kept
    "k64_E256_tiled": small_cfg(E=256, k=64, T=40, H=256, I=64, I_sh=64, n_group=64, topk_group=32, rsf=2.5,
                                seed=64),
    # every expert chosen: the weights are the normalised scores of all experts
    "k_eq_E": small_cfg(E=8, k=8, T=50, seed=65),
    # a single routed expert (weight 1 for every token), and two with top-1
    "E1": small_cfg(E=1, k=1, T=100, seed=66),
    "E2_k1": small_cfg(E=2, k=1, T=33, seed=67),
    # group limits at their extremes: one group kept, every group kept
    "groups_keep_one": small_cfg(E=64, k=4, n_group=8, topk_group=1, T=80, seed=68),
    "groups_keep_all": small_cfg(E=64, k=6, n_group=8, topk_group=8, T=80, seed=69),
    # the smallest H and I the kernels take (H % 128, I % 64)
    "smallest_H_I": small_cfg(H=128, I=64, I_sh=64, E=16, k=2, T=70, seed=70),
}

# each shape in the regime the layer picks, and the shapes the small-batch
# kernel covers in the other regime too
CASES = [(n, "auto") for n in EXT] + [(n, "tiled") for n, c in EXT.items() if is_decode(c)] + \
        [(n, "small") for n, c in EXT.items() if not is_decode(c) and is_decode(c, T=32)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()


@pytest.mark.parametrize("name,regime", CASES)
def test_extreme_shape(name, regime):
    cfg = EXT[name]
    flags = moe.MOE_OUT_F32 | {"auto": 0, "tiled": moe.MOE_REGIME_TILED, "small": moe.MOE_REGIME_SMALL}[regime]
    say(f"[extreme] {name} ({regime}): T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} "
        f"groups {cfg.n_group}/{cfg.topk_group} shared={cfg.shared_bits}")
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d, flags=flags)
    # the small-batch regime materialises no permutation
    small = regime == "small" or (regime == "auto" and is_decode(cfg))
    assert (offsets is None) == small, f"{name}: regime {regime} not taken"
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag=f"{name} {regime}")
    check_output(cfg, d, d["hidden"], got, ex, tag=f"{name} {regime} (exempt {int(ex.sum())})")

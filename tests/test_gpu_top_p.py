"""Adaptive expert top-p on the GPU against the oracle's top-p mode (both
regimes, both selection paths): ids bit-exact and weights within 1e-5 outside
near ties of the selection and near the top-p cut; dropped pairs read -1 and
weight 0 and get no rows in the permutation; outputs within the layer bar."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_output, check_routing_top_p, is_decode, run_layer, say, small_cfg

pytestmark = pytest.mark.gpu


CASES = {
    # small-batch regime, lane selection path (E <= 64, k <= 3, no groups)
    "dec_lanes_c0_T32": synth.CONFIGS["c0"].with_(T=32, seed=71, top_p=0.51),
    # small-batch regime, wave selection path (group-limited, k = 8)
    "dec_grouped_T20": synth.CONFIGS["c3"].with_(T=20, H=1024, I=512, I_sh=1024, seed=72, top_p=0.7),
    # tiled regime
    "tiled_c2_T700": synth.CONFIGS["c2"].with_(T=700, seed=73, top_p=0.51),
    "tiled_grouped": small_cfg(T=300, E=16, k=4, n_group=4, topk_group=2, rsf=2.5, seed=74, top_p=0.6,
                               w_std=0.1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_top_p_layer(name):
    cfg = CASES[name]
    say(f"top-p case {name}: T={cfg.T} E={cfg.E} k={cfg.k} p={cfg.top_p} decode={is_decode(cfg)}")
    d = synth.layer(cfg)
    out, ids, w, offsets, srt = run_layer(cfg, d)
    exempt = check_routing_top_p(cfg, d, d["hidden"], ids, w, offsets, srt, name)
    check_output(cfg, d, d["hidden"], out, exempt, tag=name)


def test_top_p_off_matches_plain():
    """top_p = 1 (off) gives the same bits as the plain router."""
    cfg = synth.CONFIGS["c0"].with_(T=24, seed=75)
    d = synth.layer(cfg)
    a = run_layer(cfg, d)
    b = run_layer(cfg.with_(top_p=1.0), d)
    for x, y in zip(a, b):
        assert (x is None and y is None) or np.array_equal(x, y)


def test_top_p_chain_matches_unchained():
    """Stacked decode with top-p: each chained combine (which also skips the
    dropped pairs' planes) takes the next layer's logits; every layer equals the
    unchained call on the same input (routing outside near ties, outputs)."""
    import torch
    import int4_routed_expert_02_amd as moe
    from gpu_util import dev_bf16, ws_view
    cfg = synth.CONFIGS["c1"].with_(layers=4, top_p=0.51, seed=1177)
    T, k, H = cfg.T, cfg.k, cfg.H
    flags = moe.MOE_ADD_RESIDUAL
    layers = [moe.MoeLayer(cfg, synth.layer(cfg, l, with_hidden=False)) for l in range(cfg.layers)]
    wss = [ly.workspace(T, flags) for ly in layers]
    ws_ref = layers[0].workspace(T, flags)
    sh = moe.shape_of(cfg, T, flags)
    x = dev_bf16(synth.hidden(cfg, 0))
    dropped = 0
    for l, ly in enumerate(layers):
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        nxt = layers[l + 1] if l + 1 < len(layers) else None
        ly.forward_chain(x, out, wss[l], flags | (moe.MOE_LOGITS_GIVEN if l else 0), nxt,
                         wss[l + 1] if nxt is not None else None)
        ref = torch.empty_like(out)
        ly.forward(x, ref, ws_ref, flags)
        torch.cuda.synchronize()
        pid, pw, _, _ = moe.moe_layer_routing(sh, wss[l])
        rid, rw, _, _ = moe.moe_layer_routing(sh, ws_ref)
        ids = ws_view(wss[l], pid, T * k, torch.int32).cpu().numpy().reshape(T, k)
        w = ws_view(wss[l], pw, T * k, torch.float32).cpu().numpy().reshape(T, k)
        r_ids = ws_view(ws_ref, rid, T * k, torch.int32).cpu().numpy().reshape(T, k)
        r_w = ws_view(ws_ref, rw, T * k, torch.float32).cpu().numpy().reshape(T, k)
        dropped += int((ids == -1).sum())
        same = np.all(ids == r_ids, axis=1)
        assert (~same).sum() <= 1, f"layer {l}: {int((~same).sum())} tokens routed differently"
        werr = float(np.max(np.abs(w[same] - r_w[same]))) if same.any() else 0.0
        assert werr <= 1e-5
        a, b = out.float().cpu().numpy()[same], ref.float().cpu().numpy()[same]
        rms = float(np.sqrt(np.mean(b.astype(np.float64) ** 2)))
        err = float(np.max(np.abs(a - b))) / rms
        say(f"top-p chain layer {l}: {int((ids == -1).sum())} dropped pairs, max|chained-unchained|/rms = {err:.3e}")
        assert err <= 1e-2
        x = out
    assert dropped > 0

"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: expert ids bit-exact except near-tie tokens (k-th/(k+1)-th biased score
gap < 1e-5, or the group boundary gap for group-limited routing); combine
weights within 1e-5; the permutation bit-exact (compared as the oracle's
permutation of the GPU's ids); outputs max|gpu - oracle| <= 1e-2 * RMS(oracle)
against the oracle's f32 math on the dequantised weights.
"""
import numpy as np
import pytest

import int4_routed_expert_02_amd as moe
import oracle
import synth
from gpu_util import (GAP_EXEMPT, W_TOL, check_output, check_routing, dev_bf16, reference_permutation, run_layer,
                      say, small_cfg, ws_view)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()


SMALL = {
    "c0": synth.CONFIGS["c0"],
    "c0_T100_ragged": synth.CONFIGS["c0"].with_(T=100, seed=11),
    "T1": synth.CONFIGS["c0"].with_(T=1, seed=12),
    "E8_small": small_cfg(E=8, T=50),
    "grouped_E32_k4": small_cfg(E=32, k=4, n_group=4, topk_group=2, rsf=2.5, T=64),
    "grouped_E64_k8_g8": small_cfg(E=64, k=8, n_group=8, topk_group=4, rsf=2.5, T=40, I=64, I_sh=128),
    "E256_k8_g8": small_cfg(E=256, k=8, n_group=8, topk_group=4, rsf=2.5, T=24, H=256, I=64, I_sh=64),
    "no_shared": small_cfg(shared_bits=0, T=70),
    "int8_shared": small_cfg(shared_bits=8, T=70),
    "c2_shape_T700": synth.CONFIGS["c2"].with_(T=700, seed=21),
    "c2_shape_T2000": synth.CONFIGS["c2"].with_(T=2000, seed=22),
    "c4_shape_T1500": synth.CONFIGS["c4"].with_(T=1500, seed=23),
    "c3_shape_T6": synth.CONFIGS["c3"].with_(T=6, seed=24),
    # H = 6144 in the tiled regime with enough rows per expert for the
    # 64-row down tiles of 256 columns (ragged groups, 300 tokens)
    "c3_H6144_E32_T300": synth.CONFIGS["c3"].with_(T=300, E=32, k=4, n_group=4, topk_group=2, seed=30),
    # small-batch regime (T <= 32, H % 1024 == 0)
    "dec_c2_skew_T32": synth.CONFIGS["c2"].with_(T=32, seed=25),
    "dec_c4_int8_T24": synth.CONFIGS["c4"].with_(T=24, seed=26),
    "dec_H2048_T9": synth.CONFIGS["c0"].with_(T=9, H=2048, I=1024, I_sh=1536, seed=27),
    "dec_no_shared_T32": synth.CONFIGS["c0"].with_(T=32, shared_bits=0, seed=28),
    "dec_grouped_T20": synth.CONFIGS["c3"].with_(T=20, H=1024, I=512, I_sh=1024, seed=29),
    # the small-batch regime in two chunks of up to 32 tokens (33 <= T <= 64)
    "dec_chunked_T33": synth.CONFIGS["c0"].with_(T=33, seed=34),
    "dec_chunked_T64": synth.CONFIGS["c0"].with_(T=64, seed=35),
    "dec_chunked_grouped_T50": synth.CONFIGS["c3"].with_(T=50, H=1024, I=512, I_sh=1024, seed=36),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_parity_small(name):
    cfg = SMALL[name]
    say(f"[layer parity] {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} shared={cfg.shared_bits}")
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d)
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag=name)
    check_output(cfg, d, d["hidden"], got, ex, tag=f"{name} (exempt {int(ex.sum())})")


def test_small_regime_in_chunks():
    """MOE_REGIME_SMALL at T = 100 (four chunks, the last of 4 tokens): the
    oracle's routing and outputs on every token, and each chunk's rows
    bit-equal to a call on that chunk's tokens alone."""
    import torch
    cfg = synth.CONFIGS["c0"].with_(T=100, seed=37)
    d = synth.layer(cfg)
    flags = moe.MOE_OUT_F32 | moe.MOE_REGIME_SMALL
    got, ids, w, offsets, srt = run_layer(cfg, d, flags=flags)
    assert offsets is None and srt is None
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag="small regime T=100")
    check_output(cfg, d, d["hidden"], got, ex, tag="small regime T=100")
    for t0, t1 in ((32, 64), (96, 100)):
        part, pids, pw, _, _ = run_layer(cfg.with_(T=t1 - t0), d, flags=moe.MOE_OUT_F32,
                                         hidden=np.ascontiguousarray(d["hidden"][t0:t1]))
        assert np.array_equal(part, got[t0:t1]), f"chunk {t0}:{t1} differs from its own call"
        assert np.array_equal(pids, ids[t0:t1]) and np.array_equal(pw, w[t0:t1])


@pytest.mark.parametrize("T", [1, 16, 32])
def test_regime_tiled_flag_at_small_T(T):
    """MOE_REGIME_TILED runs the tiled kernels where the small-batch regime
    would serve the shape: the same bar against the oracle, and the
    permutation is materialised."""
    cfg = synth.CONFIGS["c0"].with_(T=T, seed=90 + T)
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d, flags=moe.MOE_OUT_F32 | moe.MOE_REGIME_TILED)
    assert offsets is not None and srt is not None
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag=f"tiled T={T}")
    check_output(cfg, d, d["hidden"], got, ex, tag=f"tiled T={T}")


@pytest.mark.parametrize("cfg", [small_cfg(T=300, E=16), synth.CONFIGS["c0"].with_(T=32, E=16, seed=33)],
                         ids=["generic_T300", "decode_T32"])
def test_many_rows_per_expert_and_empty_experts(cfg):
    """Bias forces every token onto experts 3 and 9: multi-tile experts, 14 empty experts."""
    d = synth.layer(cfg)
    d["router_bias"][3] += 10.0
    d["router_bias"][9] += 9.0
    got, ids, w, offsets, srt = run_layer(cfg, d)
    assert set(np.unique(ids)) == {3, 9}
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag="two experts")
    check_output(cfg, d, d["hidden"], got, ex, tag="two experts")


def test_bf16_output_with_residual():
    cfg = synth.CONFIGS["c0"].with_(T=48, seed=31)
    d = synth.layer(cfg)
    flags = moe.MOE_ADD_RESIDUAL
    got, ids, w, offsets, srt = run_layer(cfg, d, flags=flags)
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag="bf16+res")
    check_output(cfg, d, d["hidden"], got, ex, residual=True, bf16_out=True, tag="bf16+res")


@pytest.mark.parametrize("T", [1000, 32])
def test_deterministic_bits(T):
    cfg = synth.CONFIGS["c2"].with_(T=T, seed=41)
    d = synth.layer(cfg)
    layer = moe.MoeLayer(cfg, d)
    a = run_layer(cfg, d, layer=layer)
    b = run_layer(cfg, d, layer=layer)
    for x, y in zip(a, b):
        assert (x is None and y is None) or np.array_equal(x, y)


@pytest.mark.parametrize("T", [8, 40, 400, 1500])
def test_integer_exact_gateup_sums(T):
    """Integer-valued x (|x| <= 8) and int4 weights: every product and partial sum
    is an integer below 2^24, so the raw gate/up sums are exact and must equal the
    oracle's bit for bit (this pins the unpack, the k-slot order and the 136*rowsum
    correction)."""
    import torch
    cfg = small_cfg(T=T, E=8, k=2, H=256, I=64, seed=50 + T)
    d = synth.layer(cfg)
    x = synth.small_int_hidden(cfg, 8)
    lw = oracle.LayerWeights(cfg, d)
    o_ids, _, _, _ = oracle.router(cfg, x, d["router_w"], d["router_bias"])
    _, offsets, srt, _ = oracle.permute(cfg, o_ids)
    g_ref, u_ref = oracle.gateup_int_sums(cfg, x, lw, offsets, srt)
    layer = moe.MoeLayer(cfg, d)
    sh = moe.shape_of(cfg, T, moe.MOE_TEST_GATEUP_SUMS)
    y = torch.zeros((T * cfg.k, cfg.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(sh, moe.MOE_WS_EXPERT_FFN), dtype=torch.uint8, device="cuda")
    moe.moe_expert_ffn(sh, dev_bf16(x), layer.weights, torch.from_numpy(offsets).cuda(),
                       torch.from_numpy(srt).cuda(), None, y, ws)
    torch.cuda.synchronize()
    yc = y.cpu().numpy().astype(np.float64)
    assert np.array_equal(yc[:, :cfg.I], g_ref)
    assert np.array_equal(yc[:, cfg.I:2 * cfg.I], u_ref)


SPLIT_CFGS = {
    "c0_T64": synth.CONFIGS["c0"].with_(T=64, seed=61, rsf=1.5),
    # contractions of 2048 and more: the gate/up and down GEMMs take precomputed row sums
    "H2048_T64": synth.CONFIGS["c0"].with_(T=64, H=2048, I=2048, I_sh=2048, seed=62, rsf=1.5),
}


@pytest.mark.parametrize("cname", sorted(SPLIT_CFGS))
def test_split_api_matches_oracle(cname):
    """router -> permute -> expert_ffn (routed, pre-scaled) -> expert_ffn (shared) -> combine."""
    import torch
    cfg = SPLIT_CFGS[cname]
    d = synth.layer(cfg)
    layer = moe.MoeLayer(cfg, d)
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    sh = moe.shape_of(cfg)
    x = dev_bf16(d["hidden"])
    dv = dict(device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, **dv)
    w = torch.empty((T, k), dtype=torch.float32, **dv)
    gap = torch.empty((T,), dtype=torch.float32, **dv)
    wsp = torch.empty(moe.moe_workspace_bytes(sh, moe.MOE_WS_PERMUTE), dtype=torch.uint8, **dv)
    moe.moe_router(sh, x, layer.router_w, layer.router_bias, ids, w, gap, wsp)
    counts = torch.empty((E,), dtype=torch.int32, **dv)
    offsets = torch.empty((E + 1,), dtype=torch.int32, **dv)
    srt = torch.empty((T * k,), dtype=torch.int32, **dv)
    inv = torch.empty((T * k,), dtype=torch.int32, **dv)
    moe.moe_permute(sh, ids, counts, offsets, srt, inv, wsp)
    torch.cuda.synchronize()
    ids_c, w_c = ids.cpu().numpy(), w.cpu().numpy()
    ex = check_routing(cfg, d, d["hidden"], ids_c, w_c, offsets.cpu().numpy(), srt.cpu().numpy(), tag="split")
    o_ids = oracle.router(cfg, d["hidden"], d["router_w"], d["router_bias"])[0]
    o_counts, _, _, o_inv = reference_permutation(cfg, ids_c, o_ids)
    assert np.array_equal(counts.cpu().numpy(), o_counts) and np.array_equal(inv.cpu().numpy(), o_inv)
    # routed experts, pre-scaled by rsf * w
    y = torch.empty((T * k, H), dtype=torch.float32, **dv)
    wsf = torch.empty(moe.moe_workspace_bytes(sh, moe.MOE_WS_EXPERT_FFN), dtype=torch.uint8, **dv)
    pscale = (w * cfg.rsf).reshape(-1).contiguous()
    moe.moe_expert_ffn(sh, x, layer.weights, offsets, srt, pscale, y, wsf)
    # shared expert through the same call: E = 1, k = 1, identity permutation
    sh1 = moe.shape(T, H, 1, 1, cfg.I_sh, 0, 0, 1, 1, 1.0, 0)
    w1 = moe.MoeWeights()
    w1.gate, w1.up, w1.down = layer.weights.sh_gate, layer.weights.sh_up, layer.weights.sh_down
    off1 = torch.tensor([0, T], dtype=torch.int32, **dv)
    ident = torch.arange(T, dtype=torch.int32, **dv)
    ysh = torch.empty((T, H), dtype=torch.float32, **dv)
    ws1 = torch.empty(moe.moe_workspace_bytes(sh1, moe.MOE_WS_EXPERT_FFN), dtype=torch.uint8, **dv)
    moe.moe_expert_ffn(sh1, x, w1, off1, ident, None, ysh, ws1)
    out = torch.empty((T, H), dtype=torch.float32, **dv)
    moe.moe_combine(moe.shape_of(cfg, flags=moe.MOE_OUT_F32), y, inv, None, ysh, None, out)
    # and the unscaled form: combine applies rsf * w itself
    y2 = torch.empty_like(y)
    moe.moe_expert_ffn(sh, x, layer.weights, offsets, srt, None, y2, wsf)
    out2 = torch.empty_like(out)
    moe.moe_combine(moe.shape_of(cfg, flags=moe.MOE_OUT_F32), y2, inv, w, ysh, None, out2)
    torch.cuda.synchronize()
    lw = oracle.LayerWeights(cfg, d)
    ref_sh = oracle.shared_ffn(cfg, d["hidden"], lw)
    err_sh = np.abs(ysh.cpu().numpy() - ref_sh).max() / np.sqrt(np.mean(ref_sh.astype(np.float64) ** 2))
    say(f"split: shared expert max err/rms {err_sh:.3e}")
    assert err_sh <= 1e-2
    check_output(cfg, d, d["hidden"], out.cpu().numpy(), ex, tag="split pre-scaled")
    check_output(cfg, d, d["hidden"], out2.cpu().numpy(), ex, tag="split combine-scaled")


FULL = ["c0", "c2", "c4", "c3"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """The full workload in the benchmark's launch configuration (moe_layer_forward,
    f32 output); routing and permutation checked on every token, outputs on
    every token (c0, c2, c4) or, for the GLM-class layer, whose oracle runs
    about 40 tokens/s, on 514 tokens: the first, the last and a seeded sample
    of 512."""
    cfg = synth.CONFIGS[name]
    say(f"[full] {name}: generating T={cfg.T} E={cfg.E} H={cfg.H}")
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d)
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag=name)
    toks = None
    if cfg.H > 2048:
        rng = np.random.default_rng(7)
        toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(np.arange(1, cfg.T - 1), 512, replace=False)]))
    check_output(cfg, d, d["hidden"], got, ex, tokens=toks, tag=f"{name} (skipped {int(ex.sum())})")
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    say(f"{name}: rows per expert max {counts.max()} min {counts.min()} active {np.count_nonzero(counts)}")


_ORACLE_STACK = {}


def oracle_stack(cfg):
    """The oracle's own 23-layer decode step from the seeded input: per layer
    its input, output (residual added), ids, w and tie gaps; the next input is
    the output rounded to bf16 (nearest even, torch on the CPU)."""
    import torch
    if cfg.name in _ORACLE_STACK:
        return _ORACLE_STACK[cfg.name]
    x = synth.hidden(cfg, 0)
    layers = []
    for l in range(cfg.layers):
        d = synth.layer(cfg, l, with_hidden=False)
        out, ids, w, gap, ggap = oracle.layer_forward(cfg, oracle.LayerWeights(cfg, d), x, residual=True)
        layers.append((x, out, ids, w, (gap < GAP_EXEMPT) | (ggap < GAP_EXEMPT)))
        x = torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _ORACLE_STACK[cfg.name] = layers
    return layers


def test_decode_stack_on_oracle_trajectory():
    """The benchmark's decode step: 23 stacked layers, T=32, bf16 out with the
    residual added.  The oracle runs its own stack from the seeded input; each
    GPU layer (moe_layer_forward, the benchmark's launch) runs on the oracle's
    input to that layer and is checked against the oracle's layer: routing of
    every token, all outputs.  (Values flow from the oracle to the GPU only.)"""
    cfg = synth.CONFIGS["c1"]
    for l, (x, _, _, _, _) in enumerate(oracle_stack(cfg)):
        d = synth.layer(cfg, l, with_hidden=False)
        got, ids, w, offsets, srt = run_layer(cfg, d, flags=moe.MOE_ADD_RESIDUAL, hidden=x)
        ex = check_routing(cfg, d, x, ids, w, offsets, srt, tag=f"c1 layer {l}")
        check_output(cfg, d, x, got, ex, residual=True, bf16_out=True, tag=f"c1 layer {l}")


def _identity_layer(cfg):
    """The c1 shape with every expert weight scale zero: routed and shared
    experts add exactly 0, so with the residual the layer's bf16 output is its
    input, bit for bit."""
    d = synth.layer(cfg, 0, with_hidden=False)
    d["experts_qs"][:] = 0.0
    d["shared_qs"][:] = 0.0
    return moe.MoeLayer(cfg, d)


def test_decode_chain_against_oracle():
    """The benchmark's chained decode step, layer by layer, against the oracle
    on the oracle's own 23-layer trajectory.  Layer 0 runs as in the step
    (chained, computing its own logits).  Every later layer runs as in the
    step too (MOE_LOGITS_GIVEN, chained to the next layer), on the oracle's
    input to it, with its router logits written by the chained combine of the
    identity layer (zero weight scales) run on that same input -- the kernel
    that writes them in the step.  Checked: routing of every token, all
    outputs; layer 0 gives the unchained call's bits exactly, the later
    layers' outputs lie within 1e-4 of the RMS of the unchained call's (their
    logits are the same sums in another order)."""
    import torch
    cfg = synth.CONFIGS["c1"]
    T, k, H, L = cfg.T, cfg.k, cfg.H, cfg.layers
    flags = moe.MOE_ADD_RESIDUAL
    stack = oracle_stack(cfg)
    layers = [moe.MoeLayer(cfg, synth.layer(cfg, l, with_hidden=False)) for l in range(L)]
    wss = [ly.workspace(T, flags) for ly in layers]
    ident = _identity_layer(cfg)
    ws_id = ident.workspace(T, flags)
    ws_ref = layers[0].workspace(T, flags)
    sh = moe.shape_of(cfg, T, flags)
    for l in range(L):
        x_np = stack[l][0]
        x = dev_bf16(x_np)
        if l:
            back = torch.empty_like(x)
            ident.forward_chain(x, back, ws_id, flags, layers[l], wss[l])
            torch.cuda.synchronize()
            assert torch.equal(back, x), f"layer {l}: the identity layer changed its input"
        out = torch.empty_like(x)
        nxt = layers[l + 1] if l + 1 < L else None
        layers[l].forward_chain(x, out, wss[l], flags | (moe.MOE_LOGITS_GIVEN if l else 0), nxt,
                                wss[l + 1] if nxt is not None else None)
        ref = torch.empty_like(x)
        layers[l].forward(x, ref, ws_ref, flags)
        torch.cuda.synchronize()
        d = synth.layer(cfg, l, with_hidden=False)
        pid, pw, _, _ = moe.moe_layer_routing(sh, wss[l])
        ids = ws_view(wss[l], pid, T * k, torch.int32).cpu().numpy().reshape(T, k)
        w = ws_view(wss[l], pw, T * k, torch.float32).cpu().numpy().reshape(T, k)
        ex = check_routing(cfg, d, x_np, ids, w, None, None, tag=f"chained layer {l}")
        got = out.float().cpu().numpy()
        check_output(cfg, d, x_np, got, ex, residual=True, bf16_out=True, tag=f"chained layer {l}")
        rid, _, _, _ = moe.moe_layer_routing(sh, ws_ref)
        r_ids = ws_view(ws_ref, rid, T * k, torch.int32).cpu().numpy().reshape(T, k)
        if l == 0:
            assert torch.equal(out, ref), "layer 0: chained and unchained outputs differ"
        else:
            same = np.all(ids == r_ids, axis=1)
            a, b = got[same].astype(np.float64), ref.float().cpu().numpy()[same].astype(np.float64)
            rms = float(np.sqrt(np.mean(b * b)))
            diff = float(np.max(np.abs(a - b))) / rms if same.any() else 0.0
            # (a weight that moved by f32 rounding can flip one bf16 rounding: an ulp of the value)
            ulp = np.abs(b) * 2.0 ** -7
            assert np.all(np.abs(a - b) <= np.maximum(ulp, 1e-4 * rms)), f"layer {l}: {diff}"


CHAIN_STACKS = {
    "c1": synth.CONFIGS["c1"],
    # an int8 shared expert: its units share the expert launch with the int4 routed ones
    "c4_int8_shared_T32": synth.CONFIGS["c4"].with_(T=32, layers=4, seed=37),
    # a quarter of the routed experts in int2 (widened to int4 in the expert kernel)
    "c1_int2_quarter": synth.CONFIGS["c1"].with_(layers=4, seed=38, int2_frac=0.25),
}


@pytest.mark.parametrize("cname", sorted(CHAIN_STACKS))
def test_decode_chain_matches_unchained(cname):
    """The chained decode step (moe_layer_forward_chain: each combine takes the
    next layer's router logits) over a layer stack (the 23-layer c1 step, and
    four c4-shape layers with an int8 shared expert), on its own trajectory.
    At every layer the chained call is compared with the unchained
    moe_layer_forward on the same input -- the path
    test_decode_stack_on_oracle_trajectory checks against the oracle: the
    routing (ids bit-exact outside near ties, w within 1e-5) and the output."""
    import torch
    cfg = CHAIN_STACKS[cname]
    T, k, H = cfg.T, cfg.k, cfg.H
    flags = moe.MOE_ADD_RESIDUAL
    layers = [moe.MoeLayer(cfg, synth.layer(cfg, l, with_hidden=False)) for l in range(cfg.layers)]
    wss = [ly.workspace(T, flags) for ly in layers]
    ws_ref = layers[0].workspace(T, flags)
    sh = moe.shape_of(cfg, T, flags)
    x = dev_bf16(synth.hidden(cfg, 0))
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
        same = np.all(ids == r_ids, axis=1)
        # (two f32 summation orders of the same logits can only part at a near tie)
        assert (~same).sum() <= 1, f"layer {l}: {int((~same).sum())} tokens routed differently"
        werr = float(np.max(np.abs(w[same] - r_w[same]))) if same.any() else 0.0
        assert werr <= 1e-5, f"layer {l}: chained weights differ by {werr}"
        a, b = out.float().cpu().numpy()[same], ref.float().cpu().numpy()[same]
        rms = float(np.sqrt(np.mean(b.astype(np.float64) ** 2)))
        err = float(np.max(np.abs(a - b))) / rms
        say(f"chain layer {l}: max|chained-unchained|/rms = {err:.3e}, weights {werr:.1e}, "
            f"{int((~same).sum())} tokens routed differently")
        if l == 0:
            # the same logits kernel: the same bits
            assert torch.equal(out, ref), "layer 0: chained and unchained outputs differ"
        else:
            # weights that moved by f32 rounding can flip a bf16 rounding (an ulp of the value)
            ulp = np.abs(b.astype(np.float64)) * 2.0 ** -7
            assert np.all(np.abs(a - b) <= np.maximum(ulp, 1e-4 * rms)), f"layer {l}: {err}"
        x = out


GRAPH_TILED = {
    "c2_T700": synth.CONFIGS["c2"].with_(T=700, seed=51),
    # H = 6144: the x row sums on the second stream, waited for by an event
    "c3_H6144_T300": synth.CONFIGS["c3"].with_(T=300, E=32, k=4, n_group=4, topk_group=2, seed=52),
}


@pytest.mark.parametrize("cname", sorted(GRAPH_TILED))
def test_tiled_graph_replays_match_eager(cname):
    """The tiled path (the shared expert forked onto the library's second
    stream and joined back) captured in a HIP graph and replayed several
    times with eager work between the replays: every replay gives the eager
    call's bits."""
    import torch
    cfg = GRAPH_TILED[cname]
    d = synth.layer(cfg)
    ly = moe.MoeLayer(cfg, d)
    x = dev_bf16(d["hidden"])
    flags = moe.MOE_OUT_F32
    ws = ly.workspace(cfg.T, flags)
    ref = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    out = torch.empty_like(ref)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        ly.forward(x, ref, ws, flags, stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        ly.forward(x, out, ws, flags, stream=stream)
    torch.cuda.synchronize()
    for r in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs"
        _ = (x.float() * 2).sum().item()


def test_decode_graph_replays_match_eager():
    """The benchmark's way of running the small-batch path: a chained stack
    (four layers, T = 32, MOE_LOGITS_GIVEN after the first) and a two-chunk
    layer (T = 64) captured in one HIP graph and replayed several times with
    eager work between the replays: every replay gives the eager bits."""
    import torch
    cfg = synth.CONFIGS["c1"]
    T, L = cfg.T, 4
    flags = moe.MOE_ADD_RESIDUAL
    layers = [moe.MoeLayer(cfg, synth.layer(cfg, l, with_hidden=False)) for l in range(L)]
    wss = [ly.workspace(T, flags) for ly in layers]
    xs = [torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda") for _ in range(L + 1)]
    xs[0].copy_(dev_bf16(synth.hidden(cfg, 0)))
    c2 = synth.CONFIGS["c0"].with_(T=64, seed=52)
    d2 = synth.layer(c2)
    ly2 = moe.MoeLayer(c2, d2)
    x2 = dev_bf16(d2["hidden"])
    ws2 = ly2.workspace(64, moe.MOE_OUT_F32)
    out2 = torch.empty((64, c2.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        for l in range(L):
            nxt = layers[l + 1] if l + 1 < L else None
            layers[l].forward_chain(xs[l], xs[l + 1], wss[l], flags | (moe.MOE_LOGITS_GIVEN if l else 0), nxt,
                                    wss[l + 1] if nxt is not None else None, stream=stream)
        ly2.forward(x2, out2, ws2, moe.MOE_OUT_F32, stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in xs[1:]] + [out2.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for x in xs[1:]:
            x.zero_()
        out2.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = xs[1:] + [out2]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs"
        _ = (x2.float() * 2).sum().item()

"""GPU: routed experts in int4 or int2 each (MOE_EXPERT_MIXED, the cold-tail
experts) against the oracle.

Bars as in test_gpu_parity.py: routing bit-exact outside near ties (the
router does not see the formats), outputs within 1e-2 * RMS of the oracle's
layer with each expert dequantised in its own format.
"""
import numpy as np
import pytest

import int4_routed_expert_02_amd as moe
import synth
from gpu_util import check_output, check_routing, check_routing_top_p, is_decode, run_layer, say, small_cfg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()


CASES = {
    "T1_all_int2": synth.CONFIGS["c0"].with_(T=1, seed=12, int2_frac=1.0),
    "c0_T16_quarter": synth.CONFIGS["c0"].with_(T=16, int2_frac=0.25),
    "c0_T100_ragged_half": synth.CONFIGS["c0"].with_(T=100, seed=11, int2_frac=0.5),
    "c2_shape_T700_quarter": synth.CONFIGS["c2"].with_(T=700, seed=21, int2_frac=0.25),
    "c4_int8_shared_T300": synth.CONFIGS["c4"].with_(T=300, seed=23, int2_frac=0.3),
    "grouped_E64_k8_all_int2": small_cfg(E=64, k=8, n_group=8, topk_group=4, rsf=2.5, T=40, I=64, I_sh=128,
                                         int2_frac=1.0),
    "no_shared_E8": small_cfg(E=8, T=50, shared_bits=0, int2_frac=0.5),
    "c3_shape_T256": synth.CONFIGS["c3"].with_(T=256, seed=24, int2_frac=0.25),
    "grouped_top_p": synth.CONFIGS["c3"].with_(T=64, H=1024, I=512, I_sh=1024, seed=26, top_p=0.6, int2_frac=0.5),
}


# every case in the regime the layer picks; the shapes the small-batch kernel
# takes (T <= 64) also forced through the tiled kernels
REGIMES = [(n, "auto") for n in CASES] + [(n, "tiled") for n, c in CASES.items() if is_decode(c)]


@pytest.mark.parametrize("name,regime", REGIMES)
def test_mixed_int2_layer_parity(name, regime):
    cfg = CASES[name]
    d = synth.layer(cfg)
    flags = moe.MOE_OUT_F32 | (moe.MOE_REGIME_TILED if regime == "tiled" else 0)
    got, ids, w, offsets, srt = run_layer(cfg, d, flags=flags)
    assert (offsets is None) == (regime == "auto" and is_decode(cfg)), f"{name}: regime {regime} not taken"
    chk = check_routing_top_p if cfg.top_p else check_routing
    ex = chk(cfg, d, d["hidden"], ids, w, offsets, srt, tag=f"int2 {name} {regime}")
    cold = np.isin(ids, np.nonzero(d["expert_bits"] == 2)[0])
    say(f"int2 {name}: {int(cold.sum())} of {ids.size} pairs on int2 experts")
    assert cold.any()
    toks = None
    if cfg.T * cfg.H > 200 * 1024:
        rng = np.random.default_rng(9)
        toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 48, replace=False)]))
    check_output(cfg, d, d["hidden"], got, ex, tokens=toks, tag=f"int2 {name}")


def _int4_reencoding(cfg, d):
    """The same layer with every int2 expert's codes stored as packed int4
    (element 2c + i in nibble i of byte c, two's complement) and no format
    array: the same weight values, all in the int4 format."""
    H, I = cfg.H, cfg.I
    mat = I * H // 2

    def widen(b2, rows, cols):
        b = b2.reshape(rows, cols // 4)
        f = np.stack([(b >> (2 * j)) & 3 for j in range(4)], -1).reshape(rows, cols).astype(np.int8)
        f[f >= 2] -= 4
        n = (f.astype(np.uint8) & 0xF).reshape(rows, cols // 2, 2)
        return (n[..., 0] | (n[..., 1] << 4)).astype(np.uint8).ravel()

    q = d["experts_q"].copy()
    for e in np.nonzero(d["expert_bits"] == 2)[0]:
        src = d["experts_q"][e]
        q[e, 0:mat] = widen(src[0:mat // 2], I, H)
        q[e, mat:2 * mat] = widen(src[mat:mat + mat // 2], I, H)
        q[e, 2 * mat:3 * mat] = widen(src[2 * mat:2 * mat + mat // 2], H, I)
    d4 = {k: v for k, v in d.items() if k != "expert_bits"}
    d4["experts_q"] = q
    return cfg.with_(int2_frac=0.0), d4


@pytest.mark.parametrize("T,frac", [(1, 1.0), (16, 0.25), (32, 1.0), (50, 0.5)])
def test_small_batch_int2_equals_int4_reencoding(T, frac):
    """The small-batch kernel widens an int2 expert's codes to int4 in
    registers and runs the int4 body on them: the layer must give the same
    bits as the same weights stored as int4 (T = 50: two chunks)."""
    import torch
    cfg = synth.CONFIGS["c0"].with_(T=T, seed=90 + T, int2_frac=frac)
    assert is_decode(cfg)
    d = synth.layer(cfg)
    got, ids, _, offsets, _ = run_layer(cfg, d)
    assert offsets is None, "the small-batch regime was not taken"
    cfg4, d4 = _int4_reencoding(cfg, d)
    ref, ids4, _, _, _ = run_layer(cfg4, d4)
    assert np.array_equal(ids, ids4)
    cold = np.isin(ids, np.nonzero(d["expert_bits"] == 2)[0])
    say(f"int2 = int4 re-encoding, T={T}: {int(cold.sum())} of {ids.size} pairs on int2 experts")
    assert cold.any()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
        f"max diff {float(np.max(np.abs(got - ref)))}"


def test_mixed_residual_bf16():
    cfg = synth.CONFIGS["c0"].with_(T=64, seed=41, int2_frac=0.5)
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d, flags=moe.MOE_ADD_RESIDUAL)
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag="int2 residual")
    check_output(cfg, d, d["hidden"], got, ex, residual=True, bf16_out=True, tag="int2 residual bf16")


def test_mixed_needs_the_bits_array():
    import torch
    cfg = synth.CONFIGS["c0"].with_(T=8, int2_frac=0.5)
    d = synth.layer(cfg)
    ly = moe.MoeLayer(cfg, d)
    ly.weights.expert_bits = None
    x = torch.zeros((8, cfg.H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((8, cfg.H), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError):
        ly.forward(x, out, ly.workspace(8, moe.MOE_OUT_F32), moe.MOE_OUT_F32)


@pytest.mark.parametrize("T", [40, 1000])
def test_split_expert_ffn_mixed(T):
    """moe_expert_ffn with MOE_EXPERT_MIXED (16-row and pipelined tiles) on
    the oracle's own routing and permutation, against oracle_expert_ffn: every
    sorted row of every expert, int4 and int2 alike."""
    import torch
    import oracle
    cfg = synth.CONFIGS["c0"].with_(T=T, seed=81 + T, int2_frac=0.5)
    d = synth.layer(cfg)
    ly = moe.MoeLayer(cfg, d)
    o_ids, o_w, _, _ = oracle.router(cfg, d["hidden"], d["router_w"], d["router_bias"])
    _, offsets, srt, _ = oracle.permute(cfg, o_ids)
    pscale = (o_w.reshape(-1) * np.float32(cfg.rsf)).astype(np.float32)
    ref = oracle.expert_ffn(cfg, d["hidden"], oracle.LayerWeights(cfg, d), offsets, srt, pscale)
    sh = moe.shape_of(cfg)
    dv = dict(device="cuda")
    x = torch.from_numpy(d["hidden"].view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.empty((T * cfg.k, cfg.H), dtype=torch.float32, **dv)
    ws = torch.empty(moe.moe_workspace_bytes(sh, moe.MOE_WS_EXPERT_FFN), dtype=torch.uint8, **dv)
    moe.moe_expert_ffn(sh, x, ly.weights, torch.from_numpy(offsets).cuda(), torch.from_numpy(srt).cuda(),
                       torch.from_numpy(pscale).cuda(), y, ws)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    rows = int(offsets[-1])
    rms = float(np.sqrt(np.mean(ref[:rows].astype(np.float64) ** 2)))
    err = float(np.abs(got[:rows] - ref[:rows]).max()) / rms
    say(f"split mixed T={T}: max|gpu-oracle|/rms = {err:.3e} over {rows} rows")
    assert err <= 1e-2


def test_int2_full_size_c3_sampled():
    """The GLM-class 2048-token layer with a quarter of its experts in int2,
    in the launch configuration bench.py --int2-frac times: routing on every
    token, outputs on a seeded sample the oracle computes one by one."""
    cfg = synth.CONFIGS["c3"].with_(int2_frac=0.25)
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d)
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag="int2 c3")
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 24, replace=False)]))
    check_output(cfg, d, d["hidden"], got, ex, tokens=toks, tag="int2 c3 full size")

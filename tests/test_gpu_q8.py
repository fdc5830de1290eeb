"""GPU: the Q8_0-style int8-activation mode (MOE_ACT_Q8) against the oracle's
matching mode.

Bars: the activation codes and block scales of moe_quantize_act_q8 bit-exact
(integer decisions taken in f32 on both sides); the layer's routing as in
the plain mode (the router does not see the mode); outputs within
1e-2 * RMS of the oracle's Q8 layer (x codes are exact; h is quantised from
the GPU's own f32 h, whose last bits can move a code by one near a rounding
boundary).
"""
import numpy as np
import pytest

import int4_routed_expert_02_amd as moe
import oracle
import synth
from gpu_util import check_output, check_routing, check_routing_top_p, run_layer, say, small_cfg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()


def _quant_inputs():
    rng = np.random.default_rng(31)
    x_bf16 = synth.hidden(synth.CONFIGS["c0"].with_(T=37, seed=31), 0)  # bf16 bits [37][1024]
    f = (rng.standard_normal((53, 384)) * rng.choice([1e-20, 1e-3, 1.0, 1e4], size=(53, 1))).astype(np.float32)
    f[3] = 0.0                      # an all-zero row
    f[5, 32:64] = 0.0               # an all-zero block
    f[7, :32] = np.float32(63.5)    # d exactly 0.5
    f[7, 1:8] = [0.25, 0.75, -0.75, 1.25, 0.26, -63.5, 10.0]  # ties to even
    return {"bf16_T37": x_bf16, "f32_mixed": f}


@pytest.mark.parametrize("name", ["bf16_T37", "f32_mixed"])
def test_quantize_act_q8_bit_exact(name):
    import torch
    src = _quant_inputs()[name]
    oq, od = oracle.quantize_act_q8(src)
    if src.dtype == np.uint16:
        dev = torch.from_numpy(src.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        dev = torch.from_numpy(src).cuda()
    q, d = moe.moe_quantize_act_q8(dev)
    torch.cuda.synchronize()
    q, d = q.cpu().numpy(), d.cpu().numpy()
    nq = int((q != oq).sum())
    nd = int((d.view(np.uint32) != od.view(np.uint32)).sum())
    say(f"q8 quantiser {name}: {nq} codes and {nd} scales differ of {q.size} / {d.size}")
    assert nq == 0 and nd == 0


CASES = {
    "T1": synth.CONFIGS["c0"].with_(T=1, seed=12, act_q8=True),
    "c0_T16": synth.CONFIGS["c0"].with_(T=16, act_q8=True),
    "c0_T100_ragged": synth.CONFIGS["c0"].with_(T=100, seed=11, act_q8=True),
    "c2_shape_T700": synth.CONFIGS["c2"].with_(T=700, seed=21, act_q8=True),
    "c4_int8_shared_T300": synth.CONFIGS["c4"].with_(T=300, seed=23, act_q8=True),
    "grouped_E64_k8": small_cfg(E=64, k=8, n_group=8, topk_group=4, rsf=2.5, T=40, I=64, I_sh=128, act_q8=True),
    "no_shared_E8": small_cfg(E=8, T=50, shared_bits=0, act_q8=True),
    "c3_shape_T64": synth.CONFIGS["c3"].with_(T=64, seed=24, act_q8=True),
    "grouped_top_p": synth.CONFIGS["c3"].with_(T=64, H=1024, I=512, I_sh=1024, seed=25, top_p=0.6, act_q8=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_q8_layer_parity(name):
    cfg = CASES[name]
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d)
    chk = check_routing_top_p if cfg.top_p else check_routing
    ex = chk(cfg, d, d["hidden"], ids, w, offsets, srt, tag=f"q8 {name}")
    toks = None
    if cfg.T * cfg.H > 200 * 1024:
        rng = np.random.default_rng(9)
        toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 48, replace=False)]))
    check_output(cfg, d, d["hidden"], got, ex, tokens=toks, tag=f"q8 {name}")


def test_q8_residual_bf16_and_plain_mode_differ():
    """bf16 output with the residual through the Q8 mode matches the oracle's
    Q8 layer; and the mode changes the result (it is not the plain path)."""
    cfg = synth.CONFIGS["c0"].with_(T=64, seed=41, act_q8=True)
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d, flags=moe.MOE_ADD_RESIDUAL)
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag="q8 residual")
    check_output(cfg, d, d["hidden"], got, ex, residual=True, bf16_out=True, tag="q8 residual bf16")
    plain, *_ = run_layer(cfg.with_(act_q8=False), d, flags=moe.MOE_ADD_RESIDUAL)
    assert not np.array_equal(plain, got)


def test_q8_full_size_c3_sampled():
    """The GLM-class 2048-token layer in the Q8 mode: routing on every token,
    outputs on a seeded sample the oracle computes one by one."""
    cfg = synth.CONFIGS["c3"].with_(act_q8=True)
    d = synth.layer(cfg)
    got, ids, w, offsets, srt = run_layer(cfg, d)
    ex = check_routing(cfg, d, d["hidden"], ids, w, offsets, srt, tag="q8 c3")
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 24, replace=False)]))
    check_output(cfg, d, d["hidden"], got, ex, tokens=toks, tag="q8 c3 full size")


def test_q8_empty_batch_is_a_no_op():
    """T = 0 in the Q8 mode: the call succeeds and writes nothing."""
    import torch
    cfg = synth.CONFIGS["c0"].with_(T=4, act_q8=True)
    d = synth.layer(cfg)
    ly = moe.MoeLayer(cfg, d)
    x = torch.zeros((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, cfg.H), 7.0, dtype=torch.float32, device="cuda")
    ws = ly.workspace(4, moe.MOE_OUT_F32)
    moe.moe_layer_forward(moe.shape_of(cfg, 0, moe.MOE_OUT_F32), ly.weights, x, out, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)

"""moe_layer_forward_noalloc (the entry point for callers that cannot
allocate) against moe_layer_forward through the C ABI: two calls in a row on
the library's static scratch, the second with a smaller input, each equal bit
for bit to moe_layer_forward on a caller workspace, in both regimes."""
import numpy as np
import pytest

import int4_routed_expert_02_amd as moe
import synth
from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()


CASES = {
    # tiled regime (the shared expert runs on the caller's stream here, on a second stream there)
    "tiled_c2_shape": (synth.CONFIGS["c2"].with_(T=700, seed=81), 250),
    "tiled_grouped_E64": (synth.CONFIGS["c0"].with_(T=300, E=64, k=8, n_group=8, topk_group=4, rsf=2.5, seed=82), 77),
    # small-batch regime
    "decode_c0_shape": (synth.CONFIGS["c0"].with_(T=32, seed=83), 5),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("flags", [moe.MOE_OUT_F32, moe.MOE_ADD_RESIDUAL], ids=["f32", "bf16_residual"])
def test_noalloc_matches_layer_forward(name, flags):
    import torch
    cfg, t_small = CASES[name]
    d = synth.layer(cfg)
    ly = moe.MoeLayer(cfg, d)
    odt = torch.float32 if flags & moe.MOE_OUT_F32 else torch.bfloat16
    for T in (cfg.T, t_small):
        x = dev_bf16(d["hidden"][:T])
        sh = moe.shape_of(cfg, T, flags)
        assert moe.moe_workspace_bytes(sh, moe.MOE_WS_LAYER) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        got = torch.full((T, cfg.H), float("nan"), dtype=odt, device="cuda")
        moe.moe_layer_forward_noalloc(sh, ly.weights, x, got)
        ref = torch.empty_like(got)
        ws = ly.workspace(T, flags)
        ly.forward(x, ref, ws, flags)
        torch.cuda.synchronize()
        same = torch.equal(got, ref)
        say(f"noalloc {name} T={T} flags={flags}: bit-equal {same}, "
            f"max|diff| {float((got.float() - ref.float()).abs().max()):.3e}")
        assert same


def test_noalloc_rejects_oversized_shape():
    """The 16384-token Nano-shape layer needs more workspace than the scratch holds."""
    cfg = synth.CONFIGS["c4"]
    sh = moe.shape_of(cfg, cfg.T, moe.MOE_OUT_F32)
    assert moe.moe_workspace_bytes(sh, moe.MOE_WS_LAYER) > moe.MOE_NOALLOC_SCRATCH_BYTES
    lib = moe.load()
    import ctypes
    rc = lib.moe_layer_forward_noalloc(ctypes.byref(sh), ctypes.byref(moe.MoeWeights()), None, None, None)
    assert rc == moe.MOE_ERR_WORKSPACE

"""The C ABI library loads and exports every symbol include/moe.h declares, and
its host-side validation answers without any device work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def moe():
    import int4_routed_expert_02_amd as m
    if not os.path.exists(m.LIB_PATH):
        from int4_routed_expert_02_amd import _build
        _build.build()
    m.load()
    return m


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(moe):
    names = declared_functions()
    assert len(names) >= 9
    lib = moe.load()
    for n in names:
        assert hasattr(lib, n), n
    assert set(moe.EXPORTS) == set(names)


def test_status_strings(moe):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert moe.status_string(code).startswith("MOE_")
    assert moe.status_string(42) == "unknown status"


def good(moe, **kw):
    base = dict(T=16, H=1024, E=64, top_k=2, I=512, I_shared=2048, shared_bits=4, n_group=1, topk_group=1, rsf=1.0)
    base.update(kw)
    return moe.shape(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(top_k=65, E=64), -2),
    (dict(T=-1), -2),
    (dict(H=1023), -2),
    (dict(shared_bits=3), -2),
    (dict(E=64, n_group=3), -2),
    (dict(E=64, n_group=8, topk_group=9), -2),
    (dict(E=64, n_group=8, topk_group=1, top_k=9), -2),
    (dict(E=8, n_group=8, topk_group=4), -2),
    (dict(H=1000), -3),
    (dict(I=500), -3),
    (dict(I_shared=2000), -3),
    (dict(E=512, top_k=2), -3),
    (dict(shared_bits=0, I_shared=0), 0),
    (dict(T=100, flags=0x8000), 0),                     # MOE_REGIME_SMALL on a shape it serves
    (dict(H=1152, flags=0x8000), -3),                   # ... on one it does not (H % 1024)
    (dict(flags=0x8000 | 0x4000), -3),                  # with MOE_REGIME_TILED
    (dict(flags=0x8000 | 0x1000), -3),                  # with MOE_ACT_Q8
    (dict(flags=0x8000 | 0x2000), 0),                   # with MOE_EXPERT_MIXED (int2 experts widened in registers)
    (dict(E=256, top_k=8, n_group=8, topk_group=4, H=6144, I=2048, rsf=2.5), 0),
    (dict(flags=0x1000), 0),            # MOE_ACT_Q8
    (dict(flags=0x2000), 0),            # MOE_EXPERT_MIXED
    (dict(flags=0x3000), -3),           # both: the Q8 kernels have no int2 form
    (dict(flags=0x2000 | 4), -3),       # mixed with MOE_EXPERT_INT8
])
def test_validation(moe, kw, code):
    assert moe.moe_validate_shape(good(moe, **kw)) == code


def test_workspace_sizes(moe):
    s = good(moe)
    # the int8-activation mode takes the tiled layout (with its code and
    # scale buffers); the mixed-format mode takes the regime's own layout
    dec = moe.moe_workspace_bytes(s, moe.MOE_WS_LAYER)
    q8 = moe.moe_workspace_bytes(good(moe, flags=moe.MOE_ACT_Q8), moe.MOE_WS_LAYER)
    mixed = moe.moe_workspace_bytes(good(moe, flags=moe.MOE_EXPERT_MIXED), moe.MOE_WS_LAYER)
    tiled = moe.moe_workspace_bytes(good(moe, flags=moe.MOE_REGIME_TILED), moe.MOE_WS_LAYER)
    mixed_tiled = moe.moe_workspace_bytes(good(moe, flags=moe.MOE_EXPERT_MIXED | moe.MOE_REGIME_TILED),
                                          moe.MOE_WS_LAYER)
    assert q8 > tiled > 0 and dec > 0 and mixed == dec and mixed_tiled == tiled != dec
    assert moe.moe_workspace_bytes(s, moe.MOE_WS_LAYER) > 16 * 2 * 1024 * 4
    assert moe.moe_workspace_bytes(s, moe.MOE_WS_PERMUTE) > 0
    assert moe.moe_workspace_bytes(s, moe.MOE_WS_EXPERT_FFN) >= 32 * 512 * 2
    assert moe.moe_workspace_bytes(good(moe, H=1000), moe.MOE_WS_LAYER) == 0
    assert moe.moe_workspace_bytes(s, 99) == 0


FAKE = 1 << 20  # an aligned address that is never dereferenced: every call below fails validation first


def test_errors_before_any_enqueue(moe):
    lib = moe.load()
    vp = ctypes.c_void_p
    w = moe.MoeWeights()
    for f in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        setattr(w, f, moe.MoeQMat(FAKE, FAKE, 0, 0))
    w.router_w = FAKE
    w.router_bias = FAKE
    s = good(moe)
    # bad shape
    assert lib.moe_layer_forward(ctypes.byref(good(moe, H=1023)), ctypes.byref(w), vp(FAKE), vp(FAKE), vp(FAKE),
                                 1 << 30, None) == moe.MOE_ERR_SHAPE
    # null hidden
    assert lib.moe_layer_forward(ctypes.byref(s), ctypes.byref(w), None, vp(FAKE), vp(FAKE), 1 << 30,
                                 None) == moe.MOE_ERR_NULL
    # misaligned hidden
    assert lib.moe_layer_forward(ctypes.byref(s), ctypes.byref(w), vp(FAKE + 2), vp(FAKE), vp(FAKE), 1 << 30,
                                 None) == moe.MOE_ERR_ALIGN
    # misaligned weight stride
    w2 = moe.MoeWeights.from_buffer_copy(w)
    w2.gate = moe.MoeQMat(FAKE, FAKE, 24, 0)
    assert lib.moe_layer_forward(ctypes.byref(s), ctypes.byref(w2), vp(FAKE), vp(FAKE), vp(FAKE), 1 << 30,
                                 None) == moe.MOE_ERR_ALIGN
    # workspace too small
    need = moe.moe_workspace_bytes(s, moe.MOE_WS_LAYER)
    assert lib.moe_layer_forward(ctypes.byref(s), ctypes.byref(w), vp(FAKE), vp(FAKE), vp(FAKE), need - 1,
                                 None) == moe.MOE_ERR_WORKSPACE
    # misaligned workspace
    assert lib.moe_layer_forward(ctypes.byref(s), ctypes.byref(w), vp(FAKE), vp(FAKE), vp(FAKE + 16), need,
                                 None) == moe.MOE_ERR_ALIGN
    # gate/up with different expert strides are not covered
    w3 = moe.MoeWeights.from_buffer_copy(w)
    w3.up = moe.MoeQMat(FAKE, FAKE, 16, 0)
    assert lib.moe_layer_forward(ctypes.byref(s), ctypes.byref(w3), vp(FAKE), vp(FAKE), vp(FAKE), need,
                                 None) == moe.MOE_ERR_UNSUPPORTED
    # the layer's routed experts are int4: the int8 row format is moe_expert_ffn's (shared expert)
    s8 = good(moe, flags=moe.MOE_EXPERT_INT8)
    assert lib.moe_layer_forward(ctypes.byref(s8), ctypes.byref(w), vp(FAKE), vp(FAKE), vp(FAKE),
                                 moe.moe_workspace_bytes(s8, moe.MOE_WS_LAYER), None) == moe.MOE_ERR_UNSUPPORTED
    # moe_expert_ffn with gate/up of different expert strides: rejected before any enqueue
    assert lib.moe_expert_ffn(ctypes.byref(s), vp(FAKE), ctypes.byref(w3), vp(FAKE), vp(FAKE), None, vp(FAKE),
                              vp(FAKE), 1 << 30, None) == moe.MOE_ERR_UNSUPPORTED
    # the no-allocation entry point: a shape whose layer workspace exceeds its scratch is refused
    huge = good(moe, T=16384)
    assert moe.moe_workspace_bytes(huge, moe.MOE_WS_LAYER) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_layer_forward_noalloc(ctypes.byref(huge), ctypes.byref(w), vp(FAKE), vp(FAKE),
                                         None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_layer_forward_noalloc(ctypes.byref(good(moe, H=1023)), ctypes.byref(w), vp(FAKE), vp(FAKE),
                                         None) == moe.MOE_ERR_SHAPE
    # the experts-only profiling stage exists only in the small-batch regime, for one chunk (T <= 32)
    big = good(moe, T=64, flags=moe.MOE_STAGE_EXPERTS_ONLY)
    need_big = moe.moe_workspace_bytes(big, moe.MOE_WS_LAYER)
    assert lib.moe_layer_forward(ctypes.byref(big), ctypes.byref(w), vp(FAKE), vp(FAKE), vp(FAKE), need_big,
                                 None) == moe.MOE_ERR_UNSUPPORTED
    # T == 0 is a no-op
    assert lib.moe_layer_forward(ctypes.byref(good(moe, T=0)), ctypes.byref(w), None, None, None, 0, None) == 0
    assert lib.moe_router(ctypes.byref(good(moe, T=0)), None, None, None, None, None, None, None, 0, None) == 0
    assert lib.moe_permute(ctypes.byref(good(moe, T=0)), None, None, None, None, None, None, 0, None) == 0
    # split calls validate too
    assert lib.moe_router(ctypes.byref(s), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE), 0,
                          None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_combine(ctypes.byref(s), None, vp(FAKE), None, None, None, vp(FAKE), None) == moe.MOE_ERR_NULL
    assert lib.moe_expert_ffn(ctypes.byref(good(moe, I=1024, flags=moe.MOE_TEST_GATEUP_SUMS)), vp(FAKE), ctypes.byref(w),
                              vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), 1 << 30, None) == moe.MOE_ERR_UNSUPPORTED


def test_regime_rule(moe):
    """The small-batch regime (no sorted pair list) serves T <= 64 by default
    (two chunks of 32), the tiled one from 65 on; MOE_REGIME_SMALL and
    MOE_REGIME_TILED decide at any T (host-side pointer arithmetic only)."""
    lib = moe.load()
    ws = ctypes.c_void_p(FAKE)

    def decode(sh):
        need = moe.moe_workspace_bytes(sh, moe.MOE_WS_LAYER)
        off = ctypes.POINTER(ctypes.c_int32)()
        assert lib.moe_layer_routing(ctypes.byref(sh), ws, need, None, None, ctypes.byref(off), None) == 0
        return not bool(off)

    assert decode(good(moe, T=1)) and decode(good(moe, T=32)) and decode(good(moe, T=33)) and decode(good(moe, T=64))
    assert not decode(good(moe, T=65)) and not decode(good(moe, T=4096))
    assert decode(good(moe, T=1000, flags=moe.MOE_REGIME_SMALL))
    assert not decode(good(moe, T=8, flags=moe.MOE_REGIME_TILED))
    assert not decode(good(moe, T=8, flags=moe.MOE_ACT_Q8))
    # the small-batch workspace holds the routing of the whole batch and one chunk's buffers
    w64 = moe.moe_workspace_bytes(good(moe, T=64), moe.MOE_WS_LAYER)
    w32 = moe.moe_workspace_bytes(good(moe, T=32), moe.MOE_WS_LAYER)
    assert w32 < w64 < 2 * w32


def test_product_path_has_no_fallback(moe, tmp_path, monkeypatch):
    """Without the built library the binding raises instead of computing anything."""
    import importlib
    import sys as _sys
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        moe.load()
    # the package never imports the oracle
    src = open(os.path.join(ROOT, "int4_routed_expert_02_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("oracle_", "")
    assert "import oracle" not in src


@pytest.mark.parametrize("args,code", [
    (dict(rows=-1), -2),
    (dict(cols=0), -2),
    (dict(bits=5), -2),
    (dict(bits=4, cols=7), -2),
    (dict(fmt=2), -2),
    (dict(rows=0), 0),
    (dict(src=None), -1),
    (dict(qs=None), -1),
    (dict(src=FAKE + 2, fmt=0), -5),
    (dict(src=FAKE + 1, fmt=1), -5),
    (dict(qs=FAKE + 2), -5),
])
def test_quantize_rows_validation(moe, args, code):
    a = dict(src=FAKE, fmt=0, rows=4, cols=16, bits=4, q=FAKE, qs=FAKE)
    a.update(args)
    assert moe.load().moe_quantize_rows(a["src"], a["fmt"], a["rows"], a["cols"], a["bits"], a["q"], a["qs"],
                                        None) == code


@pytest.mark.parametrize("args,code", [
    (dict(E=0), -2),
    (dict(counts=None), -1),
    (dict(bias=None), -1),
    (dict(counts=FAKE + 2), -5),
    (dict(bias=FAKE + 1), -5),
])
def test_bias_update_validation(moe, args, code):
    a = dict(E=64, counts=FAKE, bias=FAKE)
    a.update(args)
    assert moe.load().moe_bias_update(a["E"], a["counts"], a["bias"], 0.001, None) == code


def _fake_weights(moe):
    w = moe.MoeWeights()
    w.router_w, w.router_bias = FAKE, FAKE
    for m in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        setattr(w, m, moe.MoeQMat(FAKE, FAKE, 0, 0))
    return w


@pytest.mark.parametrize("case,code", [
    ("next ws missing", -1),
    ("T differs", -2),
    ("f32 out", -3),
    ("tiled regime", -3),
    ("logits given, tiled", -3),
    ("two chunks", -3),      # the small-batch regime at T = 64 runs in two chunks: not chainable
])
def test_chain_validation(moe, case, code):
    T = 100 if "tiled" in case else 64 if case == "two chunks" else 32
    flags = moe.MOE_OUT_F32 if case == "f32 out" else 0
    if case == "logits given, tiled":
        flags |= moe.MOE_LOGITS_GIVEN
    s = good(moe, T=T, flags=flags)
    ns = good(moe, T=16 if case == "T differs" else T)
    w = _fake_weights(moe)
    nbytes = moe.moe_workspace_bytes(s, moe.MOE_WS_LAYER)
    nnbytes = moe.moe_workspace_bytes(ns, moe.MOE_WS_LAYER)
    nxt = None if case == "logits given, tiled" else w
    nws = None if case == "next ws missing" else FAKE
    st = moe.load().moe_layer_forward_chain(ctypes.byref(s), ctypes.byref(w), FAKE, FAKE, FAKE, nbytes,
                                            ctypes.byref(ns), ctypes.byref(nxt) if nxt is not None else None, nws,
                                            nnbytes, None)
    assert st == code


@pytest.mark.parametrize("args,code", [
    (dict(rows=-1), -2),
    (dict(cols=0), -2),
    (dict(cols=48), -2),          # not whole 32-blocks
    (dict(fmt=2), -2),
    (dict(rows=0), 0),
    (dict(src=None), -1),
    (dict(q=None), -1),
    (dict(d=None), -1),
    (dict(src=FAKE + 4), -5),     # the block loads are 16-byte vectors
    (dict(q=FAKE + 8), -5),
    (dict(d=FAKE + 2), -5),
])
def test_quantize_act_q8_validation(moe, args, code):
    a = dict(src=FAKE, fmt=1, rows=4, cols=64, q=FAKE, d=FAKE)
    a.update(args)
    assert moe.load().moe_quantize_act_q8(a["src"], a["fmt"], a["rows"], a["cols"], a["q"], a["d"], None) == code

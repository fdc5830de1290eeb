"""The seeded generator: its streams follow the published generators, and its
arrays have the workload's distributions and layout."""
import numpy as np
import pytest

import moe_testutil as U

M64 = (1 << 64) - 1


def _splitmix64(state):
    state = (state + 0x9E3779B97F4A7C15) & M64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return state, z ^ (z >> 31)


def _rotl(v, k):
    return ((v << k) | (v >> (64 - k))) & M64


def _xoshiro_stream(seed, layer, tensor, row, n):
    """Pure-Python SplitMix64 key folding + xoshiro256** (Blackman & Vigna)."""
    x, k = _splitmix64(seed)
    x, k = _splitmix64(k ^ ((layer * 0xD1B54A32D192ED03) & M64))
    x, k = _splitmix64(k ^ ((tensor * 0x8CB92BA72F3D8DD7) & M64))
    x = k ^ ((row * 0xABC98388FB8FAC03 + 0x632BE59BD9B4E019) & M64)
    s = []
    for _ in range(4):
        x, z = _splitmix64(x)
        s.append(z)
    out = []
    for _ in range(n):
        out.append((_rotl((s[1] * 5) & M64, 7) * 9) & M64)
        t = (s[1] << 17) & M64
        s[2] ^= s[0]
        s[3] ^= s[1]
        s[1] ^= s[2]
        s[0] ^= s[3]
        s[2] ^= t
        s[3] = _rotl(s[3], 45)
    return out


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 0 gives 0xE220A8397B1DCDAF first (the reference C code's output)
    _, z = _splitmix64(0)
    assert z == 0xE220A8397B1DCDAF


@pytest.mark.parametrize("key", [(1000, 0, 3, 0), (1100, 22, 5, 4095), (7, 1, 0, 123456)])
def test_stream_matches_published_algorithm(synth_mod, key):
    got = synth_mod.raw_u64(*key, 16)
    ref = np.array(_xoshiro_stream(*key, 16), np.uint64)
    assert np.array_equal(got, ref)


def test_int4_range_and_uniformity(synth_mod):
    cfg = synth_mod.CONFIGS["c0"]
    q, qs = synth_mod.experts(cfg)
    vals = U.unpack_int4(q[:8], 2 * q.shape[1])
    assert vals.min() >= -7 and vals.max() <= 7
    counts = np.bincount(vals.ravel().astype(np.int64) + 7, minlength=15)
    expect = vals.size / 15
    assert np.all(np.abs(counts - expect) < 6 * np.sqrt(expect))
    assert qs.min() >= cfg.scale_lo and qs.max() <= cfg.scale_hi


def test_hidden_and_router_distributions(synth_mod):
    cfg = synth_mod.CONFIGS["c2"]
    x = U.bf16_to_f32(synth_mod.hidden(cfg))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    W, _ = synth_mod.router(cfg, with_skew=False)
    assert abs(W.std() - 0.02) < 0.0005
    cfg0 = synth_mod.CONFIGS["c0"]
    _, b = synth_mod.router(cfg0)
    assert abs(b.std() - 0.01) < 0.005


def test_layout_is_independent_of_placement(synth_mod):
    """A tensor's rows are the same whether written adjacent (gate|up|down per
    expert) or as a separate tensor."""
    import ctypes
    cfg = synth_mod.CONFIGS["c0"].with_(E=4)
    q, _ = synth_mod.experts(cfg)
    H, I = cfg.H, cfg.I
    sep = np.empty((cfg.E, I, H // 2), np.uint8)
    synth_mod.lib().synth_int4_packed(cfg.seed, 0, synth_mod.T_UP_Q, cfg.E * I, H, cfg.qmax4,
                                      ctypes.c_void_p(sep.ctypes.data), H // 2, I, I * H // 2)
    mat = I * H // 2
    assert np.array_equal(q[:, mat:2 * mat].reshape(cfg.E, I, H // 2), sep)


def test_int8_shared_range(synth_mod):
    cfg = synth_mod.CONFIGS["c4"].with_(I_sh=256, H=128)
    q, qs = synth_mod.shared(cfg)
    v = q.view(np.int8)
    assert v.min() >= -127 and v.max() <= 127 and v.min() < -120 and v.max() > 120
    lo, hi = cfg.scale_lo * 7 / 127, cfg.scale_hi * 7 / 127
    assert qs.min() >= lo and qs.max() <= hi


def test_deterministic(synth_mod):
    cfg = synth_mod.CONFIGS["c0"]
    a = synth_mod.layer(cfg)
    b = synth_mod.layer(cfg)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k

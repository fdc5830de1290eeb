"""Seeded synthetic MoE-layer inputs in the container layout.

The workloads are single MoE FFN layers of Colibri-Nano's shape (hidden 1024,
64 routed experts of intermediate 512, top-2, a 2048-wide shared expert; the
NanoColibri README's model table and the Colibri-Nano model card's
"Architecture" line) and one GLM-class layer (hidden 6144, 256 experts of
intermediate 2048, top-8 with group-limited selection and a routed scaling
factor; the colibri README's "What's implemented" list names the
DeepSeek-V3-style router with noaux_tc and routed_scaling_factor, and ~19 MB
int4 experts).

Nothing here computes any part of the layer: the module draws numbers
(``synth.c``) and places them in arrays.  The one input that depends on the
router -- the skewed selection bias of the prefill workloads -- is a fixed
table of per-rank offsets in ``skew_bias.json``; a committed script next to
the tests calibrates it with the oracle on a separate batch.

Layout of one synthetic layer (all host numpy arrays):
  hidden       [T, H]           uint16, raw bf16 bits
  router_w     [E, H]           float32, one row per expert
  router_bias  [E]              float32
  experts_q    [E, 3*I*H/2]     uint8: gate [I][H/2] | up [I][H/2] | down [H][I/2]
  experts_qs   [E, 2*I + H]     float32: gate [I] | up [I] | down [H]
  shared_q     [3*I_sh*H/2] (int4) or [3*I_sh*H] (int8), same gate|up|down order
  shared_qs    [2*I_sh + H]     float32
Each expert's three matrices are adjacent, as the colibri README's "Never wait
for the disk twice" section describes for its on-disk experts.
"""
from __future__ import annotations

import ctypes
import json
import os
import subprocess
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# tensor ids of the per-row streams
T_HIDDEN, T_ROUTER_W, T_ROUTER_B = 0, 1, 2
T_GATE_Q, T_UP_Q, T_DOWN_Q = 3, 4, 5
T_GATE_S, T_UP_S, T_DOWN_S = 6, 7, 8
T_SH_GATE_Q, T_SH_UP_Q, T_SH_DOWN_Q = 9, 10, 11
T_SH_GATE_S, T_SH_UP_S, T_SH_DOWN_S = 12, 13, 14
T_SKEW_PERM = 15
T_SMALL_X = 16


def build() -> str:
    """Compile synth.c into libsynth.so (plain gcc, OpenMP across rows)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i32, i64, f32 = ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        vp = ctypes.c_void_p
        L.synth_normal_f32.argtypes = [u64, i32, i32, i64, i64, f32, f32, vp]
        L.synth_normal_bf16.argtypes = [u64, i32, i32, i64, i64, f32, vp]
        L.synth_uniform_f32.argtypes = [u64, i32, i32, i64, f32, f32, vp]
        L.synth_int4_packed.argtypes = [u64, i32, i32, i64, i64, i32, vp, i64, i64, i64]
        L.synth_int8.argtypes = [u64, i32, i32, i64, i64, i32, vp, i64, i64, i64]
        L.synth_scales.argtypes = [u64, i32, i32, i64, f32, f32, vp, i64, i64]
        L.synth_permutation.argtypes = [u64, i32, i32, i32, vp]
        L.synth_small_int_bf16.argtypes = [u64, i32, i32, i64, i64, i32, vp]
        L.synth_raw_u64.argtypes = [u64, i32, i32, i64, i64, vp]
        for f in (L.synth_normal_f32, L.synth_normal_bf16, L.synth_uniform_f32, L.synth_int4_packed,
                  L.synth_int8, L.synth_scales, L.synth_permutation, L.synth_small_int_bf16,
                  L.synth_raw_u64):
            f.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


@dataclass(frozen=True)
class LayerConfig:
    """Shape and input recipe of one synthetic MoE layer workload."""
    name: str
    T: int
    H: int = 1024
    E: int = 64
    k: int = 2
    I: int = 512
    I_sh: int = 2048
    n_group: int = 1
    topk_group: int = 1
    rsf: float = 1.0
    shared_bits: int = 4          # 0 = no shared expert
    layers: int = 1
    seed: int = 1000
    skew: Optional[str] = None    # None | "hot8x3" | "zipf1.2"
    top_p: float = 0.0            # adaptive expert top-p (0 = keep all top_k)
    act_q8: bool = False          # Q8_0-style int8 activations for the expert matmuls
    int2_frac: float = 0.0        # fraction of routed experts stored as packed int2 (cold-tail experts)
    # value distributions
    x_std: float = 1.0
    w_std: float = 0.02
    b_std: float = 0.01
    qmax4: int = 7
    qmax8: int = 127
    scale_lo: float = 0.002
    scale_hi: float = 0.006

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The five workloads (sizes of the pages' models; see the module docstring).
CONFIGS = {
    "c0": LayerConfig("c0: one Nano-shape MoE layer, T=16", T=16, seed=1000),
    "c1": LayerConfig("c1: decode step through 23 stacked Nano-shape MoE layers, T=32", T=32,
                      layers=23, seed=1100),
    "c2": LayerConfig("c2: Nano-shape prefill layer, T=4096, 8 hot experts at ~3x load", T=4096,
                      seed=1200, skew="hot8x3"),
    "c3": LayerConfig("c3: GLM-class layer H=6144, 256x I=2048 top-8, groups 8/4, rsf 2.5, T=2048",
                      T=2048, H=6144, E=256, k=8, I=2048, I_sh=2048, n_group=8, topk_group=4,
                      rsf=2.5, seed=1300),
    "c4": LayerConfig("c4: Nano-shape layer T=16384, Zipf(1.2) expert popularity, int8 shared expert",
                      T=16384, shared_bits=8, seed=1400, skew="zipf1.2"),
}


def skew_table() -> dict:
    path = os.path.join(_HERE, "skew_bias.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f)


def skew_ranking(cfg: LayerConfig, layer: int = 0) -> np.ndarray:
    """Seeded order of experts by intended popularity (rank 0 = hottest)."""
    perm = np.empty(cfg.E, np.int32)
    lib().synth_permutation(cfg.seed, layer, T_SKEW_PERM, cfg.E, _p(perm))
    return perm


def skew_targets(cfg: LayerConfig) -> Optional[np.ndarray]:
    """Target share of the T*k routed pairs per popularity rank, or None."""
    if cfg.skew is None:
        return None
    if cfg.skew == "hot8x3":
        # 8 experts at 3x the mean load, the rest share what is left equally
        hot = 3.0 / cfg.E
        rest = (1.0 - 8 * hot) / (cfg.E - 8)
        return np.array([hot] * 8 + [rest] * (cfg.E - 8))
    if cfg.skew == "zipf1.2":
        r = np.arange(1, cfg.E + 1, dtype=np.float64)
        w = r ** -1.2
        return w / w.sum()
    raise ValueError(cfg.skew)


def bias_offsets(cfg: LayerConfig, layer: int = 0, table: Optional[dict] = None) -> np.ndarray:
    """Per-expert additive bias offsets that realise the config's skew (zeros if none)."""
    off = np.zeros(cfg.E, np.float32)
    if cfg.skew is None:
        return off
    table = skew_table() if table is None else table
    if cfg.skew not in table:
        raise RuntimeError(f"skew table has no entry for {cfg.skew}; run tests/golden/make_skew_bias.py")
    by_rank = np.asarray(table[cfg.skew]["offset_by_rank"], np.float32)
    off[skew_ranking(cfg, layer)] = by_rank
    return off


def hidden(cfg: LayerConfig, layer: int = 0, seed: Optional[int] = None, T: Optional[int] = None) -> np.ndarray:
    T = cfg.T if T is None else T
    x = np.empty((T, cfg.H), np.uint16)
    lib().synth_normal_bf16(cfg.seed if seed is None else seed, layer, T_HIDDEN, T, cfg.H, cfg.x_std, _p(x))
    return x


def small_int_hidden(cfg: LayerConfig, vmax: int, layer: int = 0) -> np.ndarray:
    x = np.empty((cfg.T, cfg.H), np.uint16)
    lib().synth_small_int_bf16(cfg.seed, layer, T_SMALL_X, cfg.T, cfg.H, vmax, _p(x))
    return x


def router(cfg: LayerConfig, layer: int = 0, with_skew: bool = True, table: Optional[dict] = None):
    W = np.empty((cfg.E, cfg.H), np.float32)
    b = np.empty((cfg.E,), np.float32)
    lib().synth_normal_f32(cfg.seed, layer, T_ROUTER_W, cfg.E, cfg.H, 0.0, cfg.w_std, _p(W))
    lib().synth_normal_f32(cfg.seed, layer, T_ROUTER_B, 1, cfg.E, 0.0, cfg.b_std, _p(b))
    if with_skew and cfg.skew is not None:
        b = (b + bias_offsets(cfg, layer, table)).astype(np.float32)
    return W, b


def experts(cfg: LayerConfig, layer: int = 0):
    """Routed experts: gate|up|down adjacent per expert, with their scales."""
    E, H, I = cfg.E, cfg.H, cfg.I
    mat = I * H // 2
    blk = 3 * mat
    q = np.empty((E, blk), np.uint8)
    L = lib()
    # gate and up: rows = output channel i (E*I rows of H/2 bytes), down: E*H rows of I/2 bytes
    L.synth_int4_packed(cfg.seed, layer, T_GATE_Q, E * I, H, cfg.qmax4, _p(q), H // 2, I, blk)
    L.synth_int4_packed(cfg.seed, layer, T_UP_Q, E * I, H, cfg.qmax4,
                        ctypes.c_void_p(q.ctypes.data + mat), H // 2, I, blk)
    L.synth_int4_packed(cfg.seed, layer, T_DOWN_Q, E * H, I, cfg.qmax4,
                        ctypes.c_void_p(q.ctypes.data + 2 * mat), I // 2, H, blk)
    sblk = 2 * I + H
    qs = np.empty((E, sblk), np.float32)
    L.synth_scales(cfg.seed, layer, T_GATE_S, E * I, cfg.scale_lo, cfg.scale_hi, _p(qs), I, sblk)
    L.synth_scales(cfg.seed, layer, T_UP_S, E * I, cfg.scale_lo, cfg.scale_hi,
                   ctypes.c_void_p(qs.ctypes.data + 4 * I), I, sblk)
    L.synth_scales(cfg.seed, layer, T_DOWN_S, E * H, cfg.scale_lo, cfg.scale_hi,
                   ctypes.c_void_p(qs.ctypes.data + 8 * I), H, sblk)
    return q, qs


def shared(cfg: LayerConfig, layer: int = 0):
    """Shared expert: gate|up|down adjacent; int4 packed or int8 per cfg.shared_bits."""
    H, I = cfg.H, cfg.I_sh
    L = lib()
    if cfg.shared_bits == 0:
        return None, None
    if cfg.shared_bits == 4:
        mat = I * H // 2
        q = np.empty((3 * mat,), np.uint8)
        L.synth_int4_packed(cfg.seed, layer, T_SH_GATE_Q, I, H, cfg.qmax4, _p(q), H // 2, I, 0)
        L.synth_int4_packed(cfg.seed, layer, T_SH_UP_Q, I, H, cfg.qmax4,
                            ctypes.c_void_p(q.ctypes.data + mat), H // 2, I, 0)
        L.synth_int4_packed(cfg.seed, layer, T_SH_DOWN_Q, H, I, cfg.qmax4,
                            ctypes.c_void_p(q.ctypes.data + 2 * mat), I // 2, H, 0)
        lo, hi = cfg.scale_lo, cfg.scale_hi
    elif cfg.shared_bits == 8:
        mat = I * H
        q = np.empty((3 * mat,), np.int8)
        L.synth_int8(cfg.seed, layer, T_SH_GATE_Q, I, H, cfg.qmax8, _p(q), H, I, 0)
        L.synth_int8(cfg.seed, layer, T_SH_UP_Q, I, H, cfg.qmax8,
                     ctypes.c_void_p(q.ctypes.data + mat), H, I, 0)
        L.synth_int8(cfg.seed, layer, T_SH_DOWN_Q, H, I, cfg.qmax8,
                     ctypes.c_void_p(q.ctypes.data + 2 * mat), I, H, 0)
        # int8 rows carry the same effective weight range as the int4 experts
        lo = cfg.scale_lo * cfg.qmax4 / cfg.qmax8
        hi = cfg.scale_hi * cfg.qmax4 / cfg.qmax8
    else:
        raise ValueError(cfg.shared_bits)
    qs = np.empty((2 * I + H,), np.float32)
    L.synth_scales(cfg.seed, layer, T_SH_GATE_S, I, lo, hi, _p(qs), I, 0)
    L.synth_scales(cfg.seed, layer, T_SH_UP_S, I, lo, hi, ctypes.c_void_p(qs.ctypes.data + 4 * I), I, 0)
    L.synth_scales(cfg.seed, layer, T_SH_DOWN_S, H, lo, hi, ctypes.c_void_p(qs.ctypes.data + 8 * I), H, 0)
    return q, qs


def expert_bits(cfg: LayerConfig, layer: int = 0) -> np.ndarray:
    """uint8 [E]: 2 for the cold-tail experts (a seeded choice of round(int2_frac * E)), 4 for the rest."""
    bits = np.full(cfg.E, 4, np.uint8)
    n2 = int(round(cfg.int2_frac * cfg.E))
    if n2:
        rng = np.random.default_rng([cfg.seed, layer, 0x1D2])
        bits[rng.choice(cfg.E, n2, replace=False)] = 2
    return bits


def _int2_rows(rng, rows: int, cols: int) -> np.ndarray:
    """rows x cols codes uniform over {-1, 0, 1}, packed four per byte (element
    4c + j in bits 2j..2j+1 of byte c, two's complement)."""
    c = (rng.integers(-1, 2, size=(rows, cols)).astype(np.int32) & 3).astype(np.uint8).reshape(rows, cols // 4, 4)
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def make_int2_experts(cfg: LayerConfig, layer: int, q: np.ndarray, qs: np.ndarray, bits: np.ndarray):
    """Re-draw the cold-tail experts in place as packed int2: each matrix in
    the first half of its int4-sized region (the rest zero), its scales times
    qmax4 so the weights keep their magnitude."""
    E, H, I = cfg.E, cfg.H, cfg.I
    mat = I * H // 2
    for e in np.nonzero(bits == 2)[0]:
        rng = np.random.default_rng([cfg.seed, layer, 0x1D2, int(e)])
        q[e] = 0
        q[e, 0:mat // 2] = _int2_rows(rng, I, H).ravel()
        q[e, mat:mat + mat // 2] = _int2_rows(rng, I, H).ravel()
        q[e, 2 * mat:2 * mat + mat // 2] = _int2_rows(rng, H, I).ravel()
        qs[e] *= np.float32(cfg.qmax4)


def layer(cfg: LayerConfig, layer_idx: int = 0, with_hidden: bool = True, table: Optional[dict] = None) -> dict:
    """All inputs of one layer as a dict of host arrays (see module docstring)."""
    W, b = router(cfg, layer_idx, table=table)
    q, qs = experts(cfg, layer_idx)
    eb = None
    if cfg.int2_frac > 0:
        eb = expert_bits(cfg, layer_idx)
        make_int2_experts(cfg, layer_idx, q, qs, eb)
    sq, sqs = shared(cfg, layer_idx)
    d = dict(router_w=W, router_bias=b, experts_q=q, experts_qs=qs, shared_q=sq, shared_qs=sqs)
    if eb is not None:
        d["expert_bits"] = eb
    if with_hidden:
        d["hidden"] = hidden(cfg, layer_idx)
    return d


def raw_u64(seed: int, layer: int, tensor: int, row: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().synth_raw_u64(seed, layer, tensor, row, n, _p(out))
    return out

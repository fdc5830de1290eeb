"""ctypes wrapper of the CPU oracle (oracle_moe.c).

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this module.  The HIP product path never
does, and it shares no code with it.

All arrays are host numpy arrays in the container layout documented in
``synth``; bf16 values are passed as their raw uint16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_moe.c")
_LIB = os.path.join(_HERE, "liboracle_moe.so")

ADD_RESIDUAL = 2
ACT_Q8 = 4         # Q8_0-style int8 activations (ORACLE_ACT_Q8)


def build() -> str:
    """Compile the oracle: -O2, OpenMP over independent outputs, no -ffast-math, no intrinsics."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wno-unknown-pragmas",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("shared_bits", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("top_p", ctypes.c_float)]


class QMat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("qs", ctypes.c_void_p),
                ("q_stride_bytes", ctypes.c_int64), ("qs_stride_floats", ctypes.c_int64)]


class Weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", QMat), ("up", QMat), ("down", QMat),
                ("sh_gate", QMat), ("sh_up", QMat), ("sh_down", QMat), ("expert_bits", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB_OVERRIDE")  # mutation tests load a planted-mistake build
        if path is None:
            path = _LIB
            if not os.path.exists(_LIB):
                build()
        L = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        S, W = ctypes.POINTER(Shape), ctypes.POINTER(Weights)
        sig = {
            "oracle_bf16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
            "oracle_f32_to_bf16": ([ctypes.c_float], ctypes.c_uint16),
            "oracle_unpack_int4_row": ([vp, i32, vp], None),
            "oracle_unpack_int2_row": ([vp, i32, vp], None),
            "oracle_pack_int4_row": ([vp, i32, vp], None),
            "oracle_dequant_row": ([vp, i32, vp, i32, vp], None),
            "oracle_router_scores": ([S, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "oracle_router": ([S, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "oracle_permute": ([S, vp, vp, vp, vp, vp], ctypes.c_int),
            "oracle_expert_ffn": ([S, vp, W, vp, vp, vp, vp], ctypes.c_int),
            "oracle_shared_ffn": ([S, vp, W, vp], ctypes.c_int),
            "oracle_combine": ([S, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "oracle_layer_forward": ([S, W, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "oracle_layer_tokens": ([S, W, vp, vp, i32, vp, vp, vp], ctypes.c_int),
            "oracle_layer_forward_dense": ([S, W, vp, vp], ctypes.c_int),
            "oracle_gateup_int_sums": ([S, vp, W, vp, vp, vp, vp], ctypes.c_int),
            "oracle_num_threads": ([], ctypes.c_int),
            "oracle_set_num_threads": ([ctypes.c_int], None),
            "oracle_quantize_rows": ([vp, i32, ctypes.c_int64, i32, i32, vp, vp], ctypes.c_int),
            "oracle_quantize_act_q8": ([vp, i32, ctypes.c_int64, i32, vp, vp], ctypes.c_int),
            "oracle_bias_update": ([i32, vp, vp, ctypes.c_float, vp], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _chk(st: int, what: str):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def shape_of(cfg, T: Optional[int] = None, residual: bool = False) -> Shape:
    flags = (ADD_RESIDUAL if residual else 0) | (ACT_Q8 if getattr(cfg, "act_q8", False) else 0)
    return Shape(cfg.T if T is None else T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_sh, cfg.shared_bits,
                 cfg.n_group, cfg.topk_group, cfg.rsf, flags, float(getattr(cfg, "top_p", 0.0)))


class LayerWeights:
    """Keeps the numpy arrays alive and exposes the ctypes weights struct."""

    def __init__(self, cfg, d: dict):
        self.cfg = cfg
        self.arrays = d
        H, I, Ish = cfg.H, cfg.I, cfg.I_sh
        q, qs = d["experts_q"], d["experts_qs"]
        mat = I * H // 2
        blk, sblk = q.shape[1] if q.ndim == 2 else 3 * mat, 2 * I + H
        base, sbase = q.ctypes.data, qs.ctypes.data
        w = Weights()
        w.router_w = d["router_w"].ctypes.data
        w.router_bias = d["router_bias"].ctypes.data
        w.gate = QMat(base, sbase, blk, sblk)
        w.up = QMat(base + mat, sbase + 4 * I, blk, sblk)
        w.down = QMat(base + 2 * mat, sbase + 8 * I, blk, sblk)
        if cfg.shared_bits:
            sq, sqs = d["shared_q"], d["shared_qs"]
            smat = Ish * H // 2 if cfg.shared_bits == 4 else Ish * H
            w.sh_gate = QMat(sq.ctypes.data, sqs.ctypes.data, 0, 0)
            w.sh_up = QMat(sq.ctypes.data + smat, sqs.ctypes.data + 4 * Ish, 0, 0)
            w.sh_down = QMat(sq.ctypes.data + 2 * smat, sqs.ctypes.data + 8 * Ish, 0, 0)
        eb = d.get("expert_bits")
        w.expert_bits = eb.ctypes.data if eb is not None else None
        self.w = w

    def ref(self):
        return ctypes.byref(self.w)


def router_scores(cfg, hidden, W, bias):
    T = hidden.shape[0]
    sh = shape_of(cfg, T)
    z = np.empty((T, cfg.E), np.float32)
    s = np.empty_like(z)
    b = np.empty_like(z)
    _chk(lib().oracle_router_scores(ctypes.byref(sh), _p(hidden), _p(W), _p(bias), _p(z), _p(s), _p(b)),
         "oracle_router_scores")
    return z, s, b


def router(cfg, hidden, W, bias):
    T = hidden.shape[0]
    sh = shape_of(cfg, T)
    ids = np.empty((T, cfg.k), np.int32)
    w = np.empty((T, cfg.k), np.float32)
    gap = np.empty((T,), np.float32)
    ggap = np.empty((T,), np.float32)
    _chk(lib().oracle_router(ctypes.byref(sh), _p(hidden), _p(W), _p(bias), _p(ids), _p(w), _p(gap), _p(ggap)),
         "oracle_router")
    return ids, w, gap, ggap


def permute(cfg, ids):
    T = ids.shape[0]
    sh = shape_of(cfg, T)
    P = T * cfg.k
    counts = np.empty((cfg.E,), np.int32)
    offsets = np.empty((cfg.E + 1,), np.int32)
    sorted_ = np.empty((P,), np.int32)
    inv = np.empty((P,), np.int32)
    ids = np.ascontiguousarray(ids, np.int32)
    _chk(lib().oracle_permute(ctypes.byref(sh), _p(ids), _p(counts), _p(offsets), _p(sorted_), _p(inv)),
         "oracle_permute")
    return counts, offsets, sorted_, inv


def expert_ffn(cfg, hidden, lw: LayerWeights, offsets, sorted_, pair_scale=None):
    T = hidden.shape[0]
    sh = shape_of(cfg, T)
    y = np.empty((T * cfg.k, cfg.H), np.float32)
    _chk(lib().oracle_expert_ffn(ctypes.byref(sh), _p(hidden), lw.ref(), _p(offsets), _p(sorted_),
                                 _p(pair_scale), _p(y)), "oracle_expert_ffn")
    return y


def shared_ffn(cfg, hidden, lw: LayerWeights):
    T = hidden.shape[0]
    sh = shape_of(cfg, T)
    out = np.empty((T, cfg.H), np.float32)
    _chk(lib().oracle_shared_ffn(ctypes.byref(sh), _p(hidden), lw.ref(), _p(out)), "oracle_shared_ffn")
    return out


def combine(cfg, y_pairs, inv, topk_w=None, shared_out=None, residual=None, T=None):
    T = inv.shape[0] // cfg.k if T is None else T
    sh = shape_of(cfg, T)
    out = np.empty((T, cfg.H), np.float32)
    _chk(lib().oracle_combine(ctypes.byref(sh), _p(y_pairs), _p(inv), _p(topk_w), _p(shared_out),
                              _p(residual), _p(out)), "oracle_combine")
    return out


def layer_forward(cfg, lw: LayerWeights, hidden, residual: bool = False):
    T = hidden.shape[0]
    sh = shape_of(cfg, T, residual)
    out = np.empty((T, cfg.H), np.float32)
    ids = np.empty((T, cfg.k), np.int32)
    w = np.empty((T, cfg.k), np.float32)
    gap = np.empty((T,), np.float32)
    ggap = np.empty((T,), np.float32)
    _chk(lib().oracle_layer_forward(ctypes.byref(sh), lw.ref(), _p(hidden), _p(out), _p(ids), _p(w), _p(gap),
                                    _p(ggap)), "oracle_layer_forward")
    return out, ids, w, gap, ggap


def layer_tokens(cfg, lw: LayerWeights, hidden, tokens, ids=None, w=None, residual: bool = False):
    T = hidden.shape[0]
    sh = shape_of(cfg, T, residual)
    tokens = np.ascontiguousarray(tokens, np.int32)
    out = np.empty((len(tokens), cfg.H), np.float32)
    if ids is not None:
        ids = np.ascontiguousarray(ids, np.int32)
        w = np.ascontiguousarray(w, np.float32)
    _chk(lib().oracle_layer_tokens(ctypes.byref(sh), lw.ref(), _p(hidden), _p(tokens), len(tokens), _p(ids),
                                   _p(w), _p(out)), "oracle_layer_tokens")
    return out


def layer_forward_dense(cfg, lw: LayerWeights, hidden, residual: bool = False):
    T = hidden.shape[0]
    sh = shape_of(cfg, T, residual)
    out = np.empty((T, cfg.H), np.float32)
    _chk(lib().oracle_layer_forward_dense(ctypes.byref(sh), lw.ref(), _p(hidden), _p(out)),
         "oracle_layer_forward_dense")
    return out


def gateup_int_sums(cfg, hidden, lw: LayerWeights, offsets, sorted_):
    T = hidden.shape[0]
    sh = shape_of(cfg, T)
    g = np.empty((T * cfg.k, cfg.I), np.float64)
    u = np.empty_like(g)
    _chk(lib().oracle_gateup_int_sums(ctypes.byref(sh), _p(hidden), lw.ref(), _p(offsets), _p(sorted_),
                                      _p(g), _p(u)), "oracle_gateup_int_sums")
    return g, u


def unpack_int4_row(row: np.ndarray, cols: int) -> np.ndarray:
    out = np.empty((cols,), np.int32)
    lib().oracle_unpack_int4_row(_p(np.ascontiguousarray(row, np.uint8)), cols, _p(out))
    return out


def pack_int4_row(vals: np.ndarray) -> np.ndarray:
    vals = np.ascontiguousarray(vals, np.int32)
    out = np.empty(((len(vals) + 1) // 2,), np.uint8)
    lib().oracle_pack_int4_row(_p(vals), len(vals), _p(out))
    return out


def dequant_row(q: np.ndarray, bits: int, scale: float, cols: int) -> np.ndarray:
    out = np.empty((cols,), np.float32)
    s = np.array([scale], np.float32)
    lib().oracle_dequant_row(_p(np.ascontiguousarray(q)), bits, _p(s), cols, _p(out))
    return out


def bf16_to_f32(bits: int) -> float:
    return float(lib().oracle_bf16_to_f32(bits))


def f32_to_bf16(f: float) -> int:
    return int(lib().oracle_f32_to_bf16(f))


def quantize_rows(src: np.ndarray, bits: int):
    """Per-row symmetric quantiser: src [rows][cols] f32, or uint16 holding bf16
    bits.  Returns (codes, scales): codes uint8 [rows][cols/2] packed int4 or
    int8 [rows][cols]; scales f32 [rows]."""
    src = np.ascontiguousarray(src)
    if src.ndim != 2 or src.dtype not in (np.float32, np.uint16):
        raise ValueError("src must be a 2-D float32 or uint16 (bf16 bits) array")
    rows, cols = src.shape
    q = np.zeros((rows, cols // 2) if bits == 4 else (rows, cols), dtype=np.uint8 if bits == 4 else np.int8)
    qs = np.zeros(rows, dtype=np.float32)
    _chk(lib().oracle_quantize_rows(_p(src), 1 if src.dtype == np.uint16 else 0, rows, cols, bits, _p(q), _p(qs)),
         "oracle_quantize_rows")
    return q, qs


def quantize_act_q8(src: np.ndarray):
    """Q8_0-style activation codes: src [rows][cols] f32, or uint16 holding bf16
    bits (cols % 32 == 0).  Returns (codes int8 [rows][cols], d f32 [rows][cols/32])."""
    src = np.ascontiguousarray(src)
    if src.ndim != 2 or src.dtype not in (np.float32, np.uint16):
        raise ValueError("src must be a 2-D float32 or uint16 (bf16 bits) array")
    rows, cols = src.shape
    q = np.zeros((rows, cols), dtype=np.int8)
    d = np.zeros((rows, max(cols // 32, 1)), dtype=np.float32)
    _chk(lib().oracle_quantize_act_q8(_p(src), 1 if src.dtype == np.uint16 else 0, rows, cols, _p(q), _p(d)),
         "oracle_quantize_act_q8")
    return q, d


def bias_update(counts: np.ndarray, bias: np.ndarray, gamma: float) -> np.ndarray:
    """One aux-loss-free balancing step: the updated f32 bias for these expert counts."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty_like(bias)
    _chk(lib().oracle_bias_update(len(bias), _p(counts), _p(bias), gamma, _p(out)), "oracle_bias_update")
    return out


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the oracle's later calls from this thread (results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))

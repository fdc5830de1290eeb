"""Independent numpy helpers for the tests.

These decode the container format and evaluate textbook pieces (a dense SwiGLU
MLP, a stable sort) with numpy, written separately from the C oracle so that a
test can compare the oracle against something other than itself.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(f: np.ndarray) -> np.ndarray:
    u = np.asarray(f, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def unpack_int4(packed: np.ndarray, cols: int) -> np.ndarray:
    """[..., cols/2] uint8 -> [..., cols] int8; low nibble first, two's complement."""
    b = np.asarray(packed, np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (cols,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def unpack_int2(packed: np.ndarray, cols: int) -> np.ndarray:
    """[..., cols/4] uint8 -> [..., cols] int8; field j of byte c is element 4c + j, two's complement."""
    b = np.asarray(packed, np.uint8)
    out = np.empty(b.shape[:-1] + (cols,), np.int8)
    for j in range(4):
        f = ((b >> (2 * j)) & 3).astype(np.int16)
        out[..., j::4] = np.where(f >= 2, f - 4, f)
    return out


def pack_int4(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, np.int16)
    lo = (q[..., 0::2] & 0xF).astype(np.uint8)
    hi = (q[..., 1::2] & 0xF).astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


def expert_mats(cfg, d: dict, e: int):
    """Dequantised f64 (gate [I,H], up [I,H], down [H,I]) of routed expert e (numpy decode)."""
    H, I = cfg.H, cfg.I
    mat = I * H // 2
    q = d["experts_q"][e]
    qs = d["experts_qs"][e]
    if "expert_bits" in d and d["expert_bits"][e] == 2:
        q2 = mat // 2
        g = unpack_int2(q[:q2].reshape(I, H // 4), H).astype(np.float64) * qs[:I, None].astype(np.float64)
        u = unpack_int2(q[mat:mat + q2].reshape(I, H // 4), H).astype(np.float64) * qs[I:2 * I, None].astype(np.float64)
        dn = unpack_int2(q[2 * mat:2 * mat + q2].reshape(H, I // 4), I).astype(np.float64) * qs[2 * I:, None].astype(np.float64)
        return g, u, dn
    g = unpack_int4(q[:mat].reshape(I, H // 2), H).astype(np.float64) * qs[:I, None].astype(np.float64)
    u = unpack_int4(q[mat:2 * mat].reshape(I, H // 2), H).astype(np.float64) * qs[I:2 * I, None].astype(np.float64)
    dn = unpack_int4(q[2 * mat:].reshape(H, I // 2), I).astype(np.float64) * qs[2 * I:, None].astype(np.float64)
    return g, u, dn


def shared_mats(cfg, d: dict):
    H, I = cfg.H, cfg.I_sh
    q, qs = d["shared_q"], d["shared_qs"]
    if cfg.shared_bits == 4:
        mat = I * H // 2
        g = unpack_int4(q[:mat].reshape(I, H // 2), H)
        u = unpack_int4(q[mat:2 * mat].reshape(I, H // 2), H)
        dn = unpack_int4(q[2 * mat:].reshape(H, I // 2), I)
    else:
        mat = I * H
        g = q[:mat].view(np.int8).reshape(I, H)
        u = q[mat:2 * mat].view(np.int8).reshape(I, H)
        dn = q[2 * mat:].view(np.int8).reshape(H, I)
    f = np.float64
    return (g.astype(f) * qs[:I, None].astype(f), u.astype(f) * qs[I:2 * I, None].astype(f),
            dn.astype(f) * qs[2 * I:, None].astype(f))


def swiglu_mlp(x: np.ndarray, g: np.ndarray, u: np.ndarray, dn: np.ndarray) -> np.ndarray:
    """Dense SwiGLU MLP in float64: down(silu(x gate^T) * (x up^T))."""
    a = x @ g.T
    b = x @ u.T
    h = a / (1.0 + np.exp(-a)) * b
    return h @ dn.T


def rel_max_err(a: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if rms == 0.0:
        return float(np.max(np.abs(np.asarray(a, np.float64) - ref))) if ref.size else 0.0
    return float(np.max(np.abs(np.asarray(a, np.float64) - ref)) / rms)

"""Python binding of the MI355X MoE-layer library (libmoe_hip.so, include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch provides device memory and the current stream.  If the HIP
library is missing, every call raises -- there is no CPU fallback.

The functions mirror the C ABI names:
  moe_router, moe_permute, moe_expert_ffn, moe_combine, moe_layer_forward,
  moe_workspace_bytes, moe_validate_shape, moe_status_string, moe_layer_routing,
  moe_quantize_rows, moe_bias_update, moe_layer_forward_chain, moe_quantize_act_q8
and ``MoeLayer`` keeps one layer's device weights and workspace.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_hip.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_UNSUPPORTED = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_ALIGN = -5
MOE_ERR_HIP = -6

MOE_OUT_F32 = 1
MOE_ADD_RESIDUAL = 2
MOE_EXPERT_INT8 = 4
MOE_TEST_GATEUP_SUMS = 0x100
MOE_STAGE_GATEUP_ONLY = 0x200
MOE_STAGE_EXPERTS_ONLY = 0x400
MOE_LOGITS_GIVEN = 0x800
MOE_ACT_Q8 = 0x1000
MOE_EXPERT_MIXED = 0x2000
MOE_REGIME_TILED = 0x4000
MOE_REGIME_SMALL = 0x8000

MOE_SRC_F32 = 0
MOE_SRC_BF16 = 1

MOE_WS_PERMUTE = 1
MOE_WS_EXPERT_FFN = 2
MOE_WS_LAYER = 3

EXPORTS = ["moe_router", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_profiled", "moe_workspace_bytes", "moe_validate_shape", "moe_status_string",
           "moe_layer_routing", "moe_quantize_rows", "moe_bias_update", "moe_layer_forward_chain",
           "moe_quantize_act_q8", "moe_layer_forward_noalloc"]

MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("shared_bits", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("top_p", ctypes.c_float)]


class MoeQMat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("qs", ctypes.c_void_p),
                ("q_stride_bytes", ctypes.c_int64), ("qs_stride_floats", ctypes.c_int64)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", MoeQMat), ("up", MoeQMat), ("down", MoeQMat),
                ("sh_gate", MoeQMat), ("sh_up", MoeQMat), ("sh_down", MoeQMat), ("expert_bits", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe_hip.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, S, W = ctypes.c_void_p, ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights)
        sz = ctypes.c_size_t
        sig = {
            "moe_router": [S, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_permute": [S, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_expert_ffn": [S, vp, W, vp, vp, vp, vp, vp, sz, vp],
            "moe_combine": [S, vp, vp, vp, vp, vp, vp, vp],
            "moe_layer_forward": [S, W, vp, vp, vp, sz, vp],
            "moe_layer_forward_profiled": [S, W, vp, vp, vp, sz, vp, vp, vp],
            "moe_layer_forward_noalloc": [S, W, vp, vp, vp],
            "moe_layer_forward_chain": [S, W, vp, vp, vp, sz, S, W, vp, sz, vp],
            "moe_validate_shape": [S],
            "moe_layer_routing": [S, vp, sz, vp, vp, vp, vp],
            "moe_quantize_rows": [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, vp],
            "moe_quantize_act_q8": [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp, vp, vp],
            "moe_bias_update": [ctypes.c_int32, vp, vp, ctypes.c_float, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [S, ctypes.c_int]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


moe_status_string = status_string


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def shape(T, H, E, top_k, I, I_shared=0, shared_bits=0, n_group=1, topk_group=1, rsf=1.0, flags=0,
          top_p=0.0) -> MoeShape:
    return MoeShape(T, H, E, top_k, I, I_shared, shared_bits, n_group, topk_group, rsf, flags, top_p)


def shape_of(cfg, T: Optional[int] = None, flags: int = 0) -> MoeShape:
    """MoeShape of a synth.LayerConfig-like object (fields T,H,E,k,I,I_sh,...)."""
    if getattr(cfg, "act_q8", False):
        flags |= MOE_ACT_Q8
    if getattr(cfg, "int2_frac", 0.0) > 0:
        flags |= MOE_EXPERT_MIXED
    return shape(cfg.T if T is None else T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_sh, cfg.shared_bits, cfg.n_group,
                 cfg.topk_group, cfg.rsf, flags, float(getattr(cfg, "top_p", 0.0)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def moe_validate_shape(sh: MoeShape) -> int:
    return load().moe_validate_shape(ctypes.byref(sh))


def moe_workspace_bytes(sh: MoeShape, which: int = MOE_WS_LAYER) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(sh), which))


def moe_router(sh: MoeShape, hidden, router_w, router_bias, topk_ids, topk_w, sel_gap, ws, stream=None):
    _check(load().moe_router(ctypes.byref(sh), _ptr(hidden), _ptr(router_w), _ptr(router_bias), _ptr(topk_ids),
                             _ptr(topk_w), _ptr(sel_gap), _ptr(ws), ws.numel() if ws is not None else 0,
                             _stream(stream)), "moe_router")


def moe_permute(sh: MoeShape, topk_ids, counts, offsets, sorted_pairs, inv_pos, ws, stream=None):
    _check(load().moe_permute(ctypes.byref(sh), _ptr(topk_ids), _ptr(counts), _ptr(offsets), _ptr(sorted_pairs),
                              _ptr(inv_pos), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_permute")


def moe_expert_ffn(sh: MoeShape, hidden, weights: MoeWeights, offsets, sorted_pairs, pair_scale, y_pairs, ws,
                   stream=None):
    _check(load().moe_expert_ffn(ctypes.byref(sh), _ptr(hidden), ctypes.byref(weights), _ptr(offsets),
                                 _ptr(sorted_pairs), _ptr(pair_scale), _ptr(y_pairs), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream)), "moe_expert_ffn")


def moe_combine(sh: MoeShape, y_pairs, inv_pos, topk_w, shared_out, residual, out, stream=None):
    _check(load().moe_combine(ctypes.byref(sh), _ptr(y_pairs), _ptr(inv_pos), _ptr(topk_w), _ptr(shared_out),
                              _ptr(residual), _ptr(out), _stream(stream)), "moe_combine")


def moe_layer_forward(sh: MoeShape, weights: MoeWeights, hidden, out, ws, stream=None):
    _check(load().moe_layer_forward(ctypes.byref(sh), ctypes.byref(weights), _ptr(hidden), _ptr(out), _ptr(ws),
                                    ws.numel() if ws is not None else 0, _stream(stream)), "moe_layer_forward")


def moe_layer_forward_profiled(sh: MoeShape, weights: MoeWeights, hidden, out, ws, ev_start, ev_stop, stream=None):
    """moe_layer_forward with torch.cuda.Event objects recorded around the expert gate/up kernel."""
    _check(load().moe_layer_forward_profiled(ctypes.byref(sh), ctypes.byref(weights), _ptr(hidden), _ptr(out),
                                             _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream),
                                             ev_start.cuda_event, ev_stop.cuda_event), "moe_layer_forward_profiled")


def moe_layer_forward_noalloc(sh: MoeShape, weights: MoeWeights, hidden, out, stream=None):
    """moe_layer_forward on the library's static scratch: no workspace, no allocation (include/moe.h)."""
    _check(load().moe_layer_forward_noalloc(ctypes.byref(sh), ctypes.byref(weights), _ptr(hidden), _ptr(out),
                                            _stream(stream)), "moe_layer_forward_noalloc")


def moe_layer_forward_chain(sh: MoeShape, weights: MoeWeights, hidden, out, ws, next_sh: Optional[MoeShape] = None,
                            next_weights: Optional[MoeWeights] = None, next_ws=None, stream=None):
    """One layer of a chained small-batch decode step (include/moe.h)."""
    _check(load().moe_layer_forward_chain(ctypes.byref(sh), ctypes.byref(weights), _ptr(hidden), _ptr(out), _ptr(ws),
                                          ws.numel(), ctypes.byref(next_sh) if next_sh is not None else None,
                                          ctypes.byref(next_weights) if next_weights is not None else None,
                                          _ptr(next_ws), next_ws.numel() if next_ws is not None else 0,
                                          _stream(stream)), "moe_layer_forward_chain")


def moe_layer_routing(sh: MoeShape, ws):
    """Device pointers (ints) of ids, w, offsets, sorted inside a layer workspace."""
    p = [ctypes.c_void_p() for _ in range(4)]
    _check(load().moe_layer_routing(ctypes.byref(sh), _ptr(ws), ws.numel(), *[ctypes.byref(x) for x in p]),
           "moe_layer_routing")
    return [x.value for x in p]


def moe_quantize_rows(src, bits: int, q=None, qs=None, stream=None):
    """Per-row symmetric quantiser (include/moe.h): src a 2-D float32 or
    bfloat16 GPU tensor.  Allocates the outputs when not given and returns
    (q, qs): q uint8 [rows][cols/2] (packed int4) or int8 [rows][cols], qs
    float32 [rows]."""
    import torch
    if src.dim() != 2 or src.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("src must be a 2-D float32 or bfloat16 tensor")
    rows, cols = src.shape
    if q is None:
        q = torch.empty((rows, cols // 2) if bits == 4 else (rows, cols),
                        dtype=torch.uint8 if bits == 4 else torch.int8, device=src.device)
    if qs is None:
        qs = torch.empty(rows, dtype=torch.float32, device=src.device)
    fmt = MOE_SRC_BF16 if src.dtype == torch.bfloat16 else MOE_SRC_F32
    _check(load().moe_quantize_rows(_ptr(src), fmt, rows, cols, bits, _ptr(q), _ptr(qs), _stream(stream)),
           "moe_quantize_rows")
    return q, qs


def moe_quantize_act_q8(src, q=None, d=None, stream=None):
    """Q8_0-style activation codes (include/moe.h): src a 2-D float32 or
    bfloat16 GPU tensor with cols % 32 == 0.  Returns (q int8 [rows][cols],
    d float32 [rows][cols/32]), allocated when not given."""
    import torch
    if src.dim() != 2 or src.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("src must be a 2-D float32 or bfloat16 tensor")
    rows, cols = src.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=src.device)
    if d is None:
        d = torch.empty((rows, max(cols // 32, 1)), dtype=torch.float32, device=src.device)
    fmt = MOE_SRC_BF16 if src.dtype == torch.bfloat16 else MOE_SRC_F32
    _check(load().moe_quantize_act_q8(_ptr(src), fmt, rows, cols, _ptr(q), _ptr(d), _stream(stream)),
           "moe_quantize_act_q8")
    return q, d


def moe_bias_update(counts, router_bias, gamma: float, stream=None):
    """Aux-loss-free balancing step (include/moe.h): router_bias (f32 [E], GPU)
    is updated in place from counts (int32 [E], GPU)."""
    if counts.numel() != router_bias.numel():
        raise ValueError("counts and router_bias must both have E elements")
    _check(load().moe_bias_update(router_bias.numel(), _ptr(counts), _ptr(router_bias), gamma, _stream(stream)),
           "moe_bias_update")


def qmat(q, qs, q_stride_bytes: int = 0, qs_stride_floats: int = 0, q_offset: int = 0, qs_offset: int = 0) -> MoeQMat:
    """A matrix family inside device tensors q (bytes) and qs (f32), at byte / float offsets."""
    return MoeQMat(_ptr(q) + q_offset, _ptr(qs) + 4 * qs_offset, q_stride_bytes, qs_stride_floats)


class MoeLayer:
    """One layer's weights on the device, in the container layout:
    experts_q [E, 3*I*H/2] u8 (gate|up|down per expert), experts_qs [E, 2I+H] f32,
    shared_q / shared_qs likewise for the shared expert, router_w [E,H], router_bias [E]."""

    def __init__(self, cfg, arrays: dict, device="cuda"):
        import torch
        self.cfg = cfg
        dev = torch.device(device)

        def up(a):
            return None if a is None else torch.from_numpy(a).to(dev)

        self.router_w = up(arrays["router_w"])
        self.router_bias = up(arrays["router_bias"])
        self.experts_q = up(arrays["experts_q"])
        self.experts_qs = up(arrays["experts_qs"])
        self.shared_q = up(arrays.get("shared_q"))
        self.shared_qs = up(arrays.get("shared_qs"))
        self.expert_bits = up(arrays.get("expert_bits"))
        H, I, Ish = cfg.H, cfg.I, cfg.I_sh
        mat = I * H // 2
        blk, sblk = 3 * mat, 2 * I + H
        w = MoeWeights()
        w.router_w = _ptr(self.router_w)
        w.router_bias = _ptr(self.router_bias)
        w.gate = qmat(self.experts_q, self.experts_qs, blk, sblk, 0, 0)
        w.up = qmat(self.experts_q, self.experts_qs, blk, sblk, mat, I)
        w.down = qmat(self.experts_q, self.experts_qs, blk, sblk, 2 * mat, 2 * I)
        if cfg.shared_bits:
            smat = Ish * H // 2 if cfg.shared_bits == 4 else Ish * H
            w.sh_gate = qmat(self.shared_q, self.shared_qs, 0, 0, 0, 0)
            w.sh_up = qmat(self.shared_q, self.shared_qs, 0, 0, smat, Ish)
            w.sh_down = qmat(self.shared_q, self.shared_qs, 0, 0, 2 * smat, 2 * Ish)
        if self.expert_bits is not None:
            w.expert_bits = _ptr(self.expert_bits)
        self.weights = w

    def workspace(self, T: int, flags: int = 0):
        import torch
        n = moe_workspace_bytes(shape_of(self.cfg, T, flags), MOE_WS_LAYER)
        return torch.empty(n, dtype=torch.uint8, device=self.router_w.device)

    def forward(self, hidden, out, ws, flags: int = 0, stream=None):
        moe_layer_forward(shape_of(self.cfg, hidden.shape[0], flags), self.weights, hidden, out, ws, stream)
        return out

    def forward_chain(self, hidden, out, ws, flags: int = 0, nxt: Optional["MoeLayer"] = None, next_ws=None,
                      stream=None):
        """moe_layer_forward_chain: this layer, and the router logits of `nxt`
        (if given) from `out` into next_ws.  Pass MOE_LOGITS_GIVEN in flags
        when the previous layer's chained call wrote this one's logits."""
        T = hidden.shape[0]
        moe_layer_forward_chain(shape_of(self.cfg, T, flags), self.weights, hidden, out, ws,
                                shape_of(nxt.cfg, T) if nxt is not None else None,
                                nxt.weights if nxt is not None else None, next_ws, stream)
        return out

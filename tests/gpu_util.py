"""Shared helpers of the GPU parity tests (device upload, workspace views, checks)."""
from __future__ import annotations

import sys

import numpy as np

import int4_routed_expert_02_amd as moe
import oracle
import synth

GAP_EXEMPT = 1e-5    # near-tie exemption of the routing comparison
W_TOL = 1e-5         # combine-weight tolerance
OUT_TOL = 1e-2       # max |gpu - oracle| <= OUT_TOL * RMS(oracle)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(a_u16: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).cuda().view(torch.bfloat16)


def ws_view(ws, ptr: int, n: int, dtype):
    import torch
    itemsize = torch.tensor([], dtype=dtype).element_size()
    off = ptr - ws.data_ptr()
    return ws[off:off + n * itemsize].view(dtype)


def run_layer(cfg, d, flags=moe.MOE_OUT_F32, hidden=None, layer=None):
    """One moe_layer_forward call; returns output and the routing the GPU computed."""
    import torch
    layer = layer or moe.MoeLayer(cfg, d)
    xh = d["hidden"] if hidden is None else hidden
    x = dev_bf16(xh)
    T = x.shape[0]
    odt = torch.float32 if flags & moe.MOE_OUT_F32 else torch.bfloat16
    out = torch.empty((T, cfg.H), dtype=odt, device="cuda")
    ws = layer.workspace(T, flags)
    layer.forward(x, out, ws, flags)
    torch.cuda.synchronize()
    sh = moe.shape_of(cfg, T, flags)
    pid, pw, poff, psrt = moe.moe_layer_routing(sh, ws)
    P = T * cfg.k
    ids = ws_view(ws, pid, P, torch.int32).cpu().numpy().reshape(T, cfg.k)
    w = ws_view(ws, pw, P, torch.float32).cpu().numpy().reshape(T, cfg.k)
    # the small-batch regime does not materialise the permutation (NULL pointers)
    offsets = ws_view(ws, poff, cfg.E + 1, torch.int32).cpu().numpy() if poff else None
    srt = ws_view(ws, psrt, P, torch.int32).cpu().numpy() if psrt else None
    return out.float().cpu().numpy(), ids, w, offsets, srt


def reference_permutation(cfg, gpu_ids, oracle_ids):
    """The permutation the GPU must produce for its own ids: the oracle's (of
    its own ids) when every id agrees; otherwise (a near-tie token chose
    differently) the stable counting sort of the GPU ids by numpy's stable
    argsort, a library routine.  Returns counts, offsets, sorted, inv."""
    if np.array_equal(gpu_ids, oracle_ids):
        return oracle.permute(cfg, oracle_ids)
    flat = np.asarray(gpu_ids, np.int64).reshape(-1)
    srt = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=cfg.E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    inv = np.empty_like(srt)
    inv[srt] = np.arange(len(srt), dtype=np.int32)
    return counts, offsets, srt, inv


def check_routing(cfg, d, hidden, ids, w, offsets, srt, tag=""):
    """ids bit-exact and w within W_TOL outside near ties; permutation exact.
    A near-tie (exempt) token that chose the oracle's ids is held to the same
    bars as the others.  Returns the mask of the tokens left out of output
    comparisons: exempt tokens whose ids differ from the oracle's."""
    o_ids, o_w, gap, ggap = oracle.router(cfg, hidden, d["router_w"], d["router_bias"])
    exempt = (gap < GAP_EXEMPT) | (ggap < GAP_EXEMPT)
    differs = np.any(ids != o_ids, axis=1)
    skip = exempt & differs
    bad = np.nonzero(differs & ~exempt)[0]
    assert bad.size == 0, f"{tag}: ids differ on {bad.size} non-exempt tokens, first {bad[:5]}"
    keep = ~skip
    if keep.any():
        werr = float(np.max(np.abs(w[keep] - o_w[keep])))
        assert werr <= W_TOL, f"{tag}: weight error {werr}"
    if exempt.any():
        say(f"{tag}: {int(exempt.sum())} near-tie tokens, {int(skip.sum())} of them routed differently")
    # exempt tokens: still a valid selection (k distinct ids in range)
    assert np.all((ids >= 0) & (ids < cfg.E))
    assert all(len(set(r)) == cfg.k for r in ids.tolist())
    if offsets is not None:
        _, o_off, o_srt, _ = reference_permutation(cfg, ids, o_ids)
        assert np.array_equal(offsets, o_off), f"{tag}: offsets differ"
        assert np.array_equal(srt, o_srt), f"{tag}: sorted pairs differ"
    return skip


def check_output(cfg, d, hidden, got, exempt, tokens=None, residual=False, bf16_out=False, tag=""):
    """Output rows against the oracle's own layer (its own routing), on the
    tokens not in `exempt` (check_routing's mask: near-tie tokens that
    legitimately chose other experts; their routing is checked for
    validity)."""
    lw = oracle.LayerWeights(cfg, d)
    T = hidden.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    toks = toks[~np.asarray(exempt)[toks]]
    ref = oracle.layer_tokens(cfg, lw, hidden, toks, residual=residual).astype(np.float64)
    g = got[toks].astype(np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    diff = np.abs(g - ref)
    if bf16_out:
        # the bf16 store adds up to half an ulp of the value itself
        diff = np.maximum(diff - np.abs(ref) * 2.0 ** -8, 0.0)
    err = float(diff.max()) / rms
    say(f"{tag}: max|gpu-oracle|/rms = {err:.3e} (rms {rms:.4f}, {len(toks)} tokens)")
    assert err <= OUT_TOL, f"{tag}: {err}"
    return err


def is_decode(cfg, T=None) -> bool:
    """Whether moe_layer_forward takes the small-batch path for this shape."""
    T = cfg.T if T is None else T
    return (T <= 64 and cfg.E <= 256 and cfg.k <= 16 and cfg.H % 1024 == 0 and cfg.I % 512 == 0
            and (cfg.shared_bits == 0 or cfg.I_sh % 512 == 0))


def small_cfg(**kw):
    base = dict(name="small", T=64, H=256, E=16, k=2, I=128, I_sh=256, seed=4242)
    base.update(kw)
    return synth.LayerConfig(**base)


def _cut_margin(w0, ids0, p):
    """Per token: the distance of p to the nearest f32 running mass of the
    weight ranking (where the kept set would change under a tiny perturbation)."""
    out = np.empty(w0.shape[0])
    for t in range(w0.shape[0]):
        rank = sorted(range(w0.shape[1]), key=lambda j: (-w0[t][j], ids0[t][j]))
        mass, best = np.float32(0), np.inf
        for j in rank:
            mass = np.float32(mass + w0[t][j])
            best = min(best, abs(float(mass) - p))
        out[t] = best
    return out


def check_routing_top_p(cfg, d, hidden, ids, w, offsets, srt, tag=""):
    """check_routing for adaptive expert top-p: the oracle's truncated routing
    outside near ties and near cut points, dropped slots -1 / weight 0, kept
    weights summing to 1, the permutation over the kept pairs only."""
    o_ids0, o_w0, gap, ggap = oracle.router(cfg.with_(top_p=0.0), hidden, d["router_w"], d["router_bias"])
    o_ids, o_w, _, _ = oracle.router(cfg, hidden, d["router_w"], d["router_bias"])
    exempt = (gap < GAP_EXEMPT) | (ggap < GAP_EXEMPT) | (_cut_margin(o_w0, o_ids0, cfg.top_p) < GAP_EXEMPT)
    keep = ~exempt
    say(f"{tag}: {int((o_ids == -1).sum())} of {o_ids.size} pairs dropped by the oracle, {int(exempt.sum())} exempt tokens")
    assert (o_ids == -1).any(), "the case drops no pair"
    bad = np.nonzero(np.any(ids[keep] != o_ids[keep], axis=1))[0]
    assert bad.size == 0, f"{tag}: ids differ on {bad.size} non-exempt tokens"
    werr = float(np.max(np.abs(w[keep] - o_w[keep]))) if keep.any() else 0.0
    assert werr <= W_TOL, f"{tag}: weight error {werr}"
    # every token: kept ids distinct and in range, dropped slots -1 / weight 0, kept weights sum to 1
    for t in range(ids.shape[0]):
        live = ids[t] >= 0
        assert live.any() and np.all(ids[t][live] < cfg.E) and len(set(ids[t][live])) == live.sum()
        assert np.all(ids[t][~live] == -1) and np.all(w[t][~live] == 0.0)
        assert abs(float(w[t][live].sum()) - 1.0) < 1e-5
    if offsets is not None:
        flat = ids.reshape(-1).astype(np.int64)
        live = np.nonzero(flat >= 0)[0]
        order = live[np.argsort(flat[live], kind="stable")]
        counts = np.bincount(flat[live], minlength=cfg.E)
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)])), f"{tag}: offsets"
        assert np.array_equal(srt[:len(live)], order), f"{tag}: sorted pairs"
    return exempt

"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test compares the oracle with something other than itself: printed
figures, closed forms, library routines (numpy / scipy), brute force on tiny
inputs, invariants, or special cases that reduce to a dense SwiGLU MLP.
"""
import itertools
import json
import os
import subprocess
import sys

import numpy as np
import pytest
from scipy.special import expit

import moe_testutil as U

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def tiny_cfg(synth_mod, **kw):
    base = dict(name="tiny", T=12, H=64, E=8, k=2, I=32, I_sh=48, seed=77)
    base.update(kw)
    return synth_mod.LayerConfig(**base)


def make(synth_mod, oracle_mod, cfg):
    d = synth_mod.layer(cfg)
    return d, oracle_mod.LayerWeights(cfg, d)


# ------------------------------------------------------------------ formats

def test_int4_nibble_order_golden(oracle_mod):
    g = _gold("int4_nibble_order.json")
    for case in g["cases"]:
        vals = oracle_mod.unpack_int4_row(np.array([case["byte"]], np.uint8), 2)
        assert list(vals) == case["elements"], case
        assert oracle_mod.pack_int4_row(np.array(case["elements"]))[0] == case["byte"]


def test_int4_pack_unpack_exhaustive(oracle_mod):
    allb = np.arange(256, dtype=np.uint8)
    vals = oracle_mod.unpack_int4_row(allb, 512)
    assert np.array_equal(oracle_mod.pack_int4_row(vals), allb)
    pairs = np.array([(a, b) for a in range(-8, 8) for b in range(-8, 8)], np.int32).ravel()
    assert np.array_equal(oracle_mod.unpack_int4_row(oracle_mod.pack_int4_row(pairs), pairs.size), pairs)
    # the numpy decoder of the tests agrees with the oracle's on every byte
    assert np.array_equal(U.unpack_int4(allb, 512).astype(np.int32), vals)


def test_int8_dequant_all_values(oracle_mod):
    q = np.arange(-128, 128, dtype=np.int8)
    out = oracle_mod.dequant_row(q, 8, 0.25, 256)
    assert np.array_equal(out, q.astype(np.float32) * np.float32(0.25))


def test_int4_dequant_is_product(oracle_mod):
    q = np.arange(256, dtype=np.uint8)
    s = np.float32(0.0037)
    out = oracle_mod.dequant_row(q, 4, float(s), 512)
    assert np.array_equal(out, U.unpack_int4(q, 512).astype(np.float32) * s)


def test_bf16_rne_golden(oracle_mod):
    for case in _gold("bf16_rne.json")["cases"]:
        f = np.array([int(case["f32_bits"], 16)], np.uint32).view(np.float32)[0]
        assert oracle_mod.f32_to_bf16(float(f)) == int(case["bf16_bits"], 16), case
    for bits in (0x3F80, 0xC0A0, 0x0001, 0x7F7F):
        assert np.float32(oracle_mod.bf16_to_f32(bits)) == U.bf16_to_f32(np.array([bits]))[0]


def test_page_byte_figures(synth_mod):
    """Byte accounting of the packed format against the pages' printed sizes."""
    g = _gold("page_figures.json")
    ge = g["glm_expert"]
    cfg = synth_mod.CONFIGS["c3"]
    q_bytes = 3 * cfg.H * cfg.I // 2
    assert (cfg.H, cfg.I) == (ge["H"], ge["I"])
    assert abs(q_bytes / 1e6 - ge["approx_MB"]) / ge["approx_MB"] < ge["rel_tol"]
    per_expert = q_bytes + 4 * (2 * cfg.I + cfg.H)
    cr = g["glm_cold_read"]
    tok = cr["layers"] * cr["experts_per_layer"] * per_expert
    assert abs(tok / 1e9 - cr["approx_GB"]) / cr["approx_GB"] < cr["rel_tol"]
    rc = g["glm_routed_expert_count"]
    assert rc["layers"] * rc["experts_per_layer"] + rc["mtp_head_experts"] == rc["count"]
    # Nano: the int4 routed experts plus the int8 shared experts fit inside the
    # ~1.4 GB container and the rest is the ~0.3 GB resident dense part.
    nc = g["nano_container"]
    c0 = synth_mod.CONFIGS["c0"]
    assert (c0.H, c0.E, c0.I, c0.I_sh) == (nc["H"], nc["E"], nc["I"], nc["I_shared"])
    routed = nc["moe_layers"] * c0.E * (3 * c0.H * c0.I // 2 + 4 * (2 * c0.I + c0.H))
    shared8 = nc["moe_layers"] * (3 * c0.H * c0.I_sh + 4 * (2 * c0.I_sh + c0.H))
    assert routed + shared8 < nc["container_GB"] * 1e9
    assert routed > (nc["container_GB"] - nc["resident_GB"]) * 1e9 * 0.95
    # the synthetic layer has exactly that many bytes
    d = synth_mod.experts(c0.with_(E=2))
    assert d[0].nbytes + d[1].nbytes == 2 * (3 * c0.H * c0.I // 2 + 4 * (2 * c0.I + c0.H))


# ------------------------------------------------------------------- router

def test_router_scores_against_library(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, T=40, H=256, E=16)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    z, s, b = oracle_mod.router_scores(cfg, x, W, bias)
    zf = U.bf16_to_f32(x).astype(np.float64) @ W.astype(np.float64).T
    # z is the double dot rounded once to f32: within one f32 ulp of numpy's double matmul
    assert np.all(np.abs(z - zf) <= np.spacing(np.abs(zf).astype(np.float32)))
    assert np.array_equal(s, expit(z.astype(np.float64)).astype(np.float32))
    assert np.array_equal(b, s + bias[None, :])


def test_router_zero_weights_closed_form(synth_mod, oracle_mod):
    """W = 0: every score is sigmoid(0) = 1/2, so selection is the top-k of the
    bias alone (ties -> lower id) and every weight is exactly 1/k."""
    for k in (1, 2, 4):
        cfg = tiny_cfg(synth_mod, T=5, E=16, k=k, rsf=2.5)
        x = synth_mod.hidden(cfg)
        W = np.zeros((cfg.E, cfg.H), np.float32)
        bias = np.array([0.1, 0.3, 0.3, -0.2, 0.05, 0.3, 0.0, 0.2, 0.1, -0.1, 0.25, 0.25, 0.0, 0.01, -0.5, 0.2],
                        np.float32)
        z, s, b = oracle_mod.router_scores(cfg, x, W, bias)
        assert np.all(s == 0.5)
        ids, w, gap, _ = oracle_mod.router(cfg, x, W, bias)
        order = sorted(range(cfg.E), key=lambda e: (-(np.float32(0.5) + bias[e]), e))[:k]
        assert all(list(ids[t]) == order for t in range(cfg.T))
        assert np.all(w == np.float32(1.0 / k))


def _brute_select(b_row, s_row, k, n_group, topk_group):
    E = len(b_row)
    Eg = E // n_group
    allowed = list(range(E))
    if n_group > 1 and topk_group < n_group:
        # group score: the largest f32 sum over all pairs of distinct experts of the group
        G = []
        for g in range(n_group):
            mem = range(g * Eg, (g + 1) * Eg)
            G.append(max(np.float32(b_row[a]) + np.float32(b_row[c]) for a, c in itertools.combinations(mem, 2)))
        best = None
        for sub in itertools.combinations(range(n_group), topk_group):
            key = (sum(float(G[g]) for g in sub), [-g for g in sub])
            if best is None or key > best[0]:
                best = (key, sub)
        kept = set(best[1])
        allowed = [e for e in range(E) if e // Eg in kept]
    order = sorted(allowed, key=lambda e: (-float(b_row[e]), e))
    ids = order[:k]
    ssum = sum(float(s_row[e]) for e in ids)
    return ids, [float(s_row[e]) / ssum for e in ids]


@pytest.mark.parametrize("E,k,ng,kg", [(8, 2, 1, 1), (16, 3, 1, 1), (16, 4, 4, 2), (12, 2, 3, 1), (16, 8, 8, 4)])
def test_router_brute_force(synth_mod, oracle_mod, E, k, ng, kg):
    cfg = tiny_cfg(synth_mod, T=64, H=64, E=E, k=k, n_group=ng, topk_group=kg, seed=500 + E + k)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    W *= 8  # widen the score spread so selections differ across tokens
    _, s, b = oracle_mod.router_scores(cfg, x, W, bias)
    ids, w, gap, ggap = oracle_mod.router(cfg, x, W, bias)
    for t in range(cfg.T):
        bi, bw = _brute_select(b[t], s[t], k, ng, kg)
        assert list(ids[t]) == bi, t
        assert np.allclose(w[t], bw, rtol=1e-6, atol=0)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6
        assert gap[t] >= 0


def test_router_group_no_op_special_case(synth_mod, oracle_mod):
    """n_group = 1, or keeping every group, is plain top-k."""
    cfg1 = tiny_cfg(synth_mod, T=64, E=16, k=3)
    x = synth_mod.hidden(cfg1)
    W, bias = synth_mod.router(cfg1)
    ref = oracle_mod.router(cfg1, x, W, bias)
    for ng in (2, 4, 8):
        got = oracle_mod.router(cfg1.with_(n_group=ng, topk_group=ng), x, W, bias)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_router_gap_definition(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, T=32, E=16, k=2)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    _, s, b = oracle_mod.router_scores(cfg, x, W, bias)
    ids, _, gap, ggap = oracle_mod.router(cfg, x, W, bias)
    for t in range(cfg.T):
        srt = sorted(b[t].tolist(), reverse=True)
        assert gap[t] == np.float32(np.float32(srt[1]) - np.float32(srt[2]))
    assert np.all(np.isinf(ggap))


def _brute_gaps(b_row, k, n_group, topk_group):
    """Tie gaps of group-limited selection by enumeration: ggap = the f32
    difference between the kept group of lowest score and the best dropped
    group, where the kept set is the best-scoring subset of topk_group groups
    (group score: the largest f32 sum of two distinct members); gap = the f32
    difference between the k-th and (k+1)-th largest b among the experts of
    the kept groups (inf when no allowed expert is left over)."""
    E = len(b_row)
    Eg = E // n_group
    G = [max(np.float32(b_row[a]) + np.float32(b_row[c])
             for a, c in itertools.combinations(range(g * Eg, (g + 1) * Eg), 2)) for g in range(n_group)]
    best = None
    for sub in itertools.combinations(range(n_group), topk_group):
        key = (sum(float(G[g]) for g in sub), [-g for g in sub])
        if best is None or key > best[0]:
            best = (key, sub)
    kept = set(best[1])
    worst_kept = min(G[g] for g in kept)
    best_dropped = max(G[g] for g in range(n_group) if g not in kept)
    ggap = np.float32(worst_kept - best_dropped)
    allowed = sorted((float(b_row[e]) for e in range(E) if e // Eg in kept), reverse=True)
    gap = np.float32(np.float32(allowed[k - 1]) - np.float32(allowed[k])) if len(allowed) > k else np.float32(np.inf)
    return gap, ggap


@pytest.mark.parametrize("E,k,ng,kg", [(16, 4, 4, 2), (12, 2, 3, 1), (16, 8, 8, 4), (32, 8, 8, 4), (16, 4, 4, 1)])
def test_router_group_gaps_brute_force(synth_mod, oracle_mod, E, k, ng, kg):
    """Group-limited routing: both tie gaps (the quantities the GPU tests use to
    exempt near-tie tokens) against enumeration of the group subsets.  The
    (16, 4, 4, 1) case keeps one group of four experts for k = 4, so nothing
    is left over and gap is infinite."""
    cfg = tiny_cfg(synth_mod, T=64, H=64, E=E, k=k, n_group=ng, topk_group=kg, seed=900 + E + k + kg)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    W *= 8
    _, s, b = oracle_mod.router_scores(cfg, x, W, bias)
    _, _, gap, ggap = oracle_mod.router(cfg, x, W, bias)
    for t in range(cfg.T):
        bg, bgg = _brute_gaps(b[t], k, ng, kg)
        assert ggap[t] == bgg, (t, ggap[t], bgg)
        assert gap[t] == bg, (t, gap[t], bg)
        assert ggap[t] >= 0 and gap[t] >= 0
    if (E, k, ng, kg) == (16, 4, 4, 1):
        assert np.all(np.isinf(gap))


def test_router_group_gap_worked_example(synth_mod, oracle_mod):
    """A hand-computed token (W = 0, so s = 1/2 and b = 1/2 + bias): four
    groups of four; group scores (top-two sums of b) 1.9, 1.5, 1.2, 1.45 ->
    keep groups 0 and 1, ggap = 1.5 - 1.45; top-3 of the kept experts are
    1.0, 0.9, 0.8 with 0.7 next -> gap = 0.8 - 0.7."""
    cfg = tiny_cfg(synth_mod, T=1, E=16, k=3, n_group=4, topk_group=2)
    x = synth_mod.hidden(cfg)
    W = np.zeros((cfg.E, cfg.H), np.float32)
    b_target = np.array([1.0, 0.9, 0.1, 0.2,   0.8, 0.7, 0.3, 0.0,
                         0.6, 0.6, 0.5, 0.4,   0.75, 0.7, 0.2, 0.1], np.float32)
    bias = (b_target - np.float32(0.5)).astype(np.float32)
    _, _, b = oracle_mod.router_scores(cfg, x, W, bias)
    ids, _, gap, ggap = oracle_mod.router(cfg, x, W, bias)
    assert list(ids[0]) == [0, 1, 4]
    G = [np.float32(b[0][0] + b[0][1]), np.float32(b[0][4] + b[0][5]), np.float32(b[0][8] + b[0][9]),
         np.float32(b[0][12] + b[0][13])]
    assert ggap[0] == np.float32(G[1] - G[3])
    assert abs(float(ggap[0]) - 0.05) < 1e-6
    assert gap[0] == np.float32(b[0][4] - b[0][5])
    assert abs(float(gap[0]) - 0.1) < 1e-6


# -------------------------------------------------------------- permutation

def test_permute_is_stable_argsort_and_invariants(synth_mod, oracle_mod):
    cfg = synth_mod.CONFIGS["c0"].with_(T=300)
    d = synth_mod.layer(cfg)
    ids, w, _, _ = oracle_mod.router(cfg, d["hidden"], d["router_w"], d["router_bias"])
    counts, offsets, srt, inv = oracle_mod.permute(cfg, ids)
    flat = ids.ravel()
    assert np.array_equal(srt, np.argsort(flat, kind="stable"))
    assert counts.sum() == cfg.T * cfg.k
    assert np.array_equal(counts, np.bincount(flat, minlength=cfg.E))
    assert offsets[0] == 0 and offsets[-1] == cfg.T * cfg.k and np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(srt), np.arange(cfg.T * cfg.k))
    assert np.array_equal(inv[srt], np.arange(cfg.T * cfg.k))
    for e in range(cfg.E):
        seg = srt[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(flat[seg] == e)
    # k distinct experts per token
    assert all(len(set(r)) == cfg.k for r in ids.tolist())
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)


# ------------------------------------------------------------------ the FFN

def test_single_expert_is_dense_swiglu(synth_mod, oracle_mod):
    """E = 1, k = 1, no shared expert: the layer is rsf times a dense SwiGLU MLP."""
    cfg = tiny_cfg(synth_mod, T=10, E=1, k=1, shared_bits=0, rsf=1.75)
    d, lw = make(synth_mod, oracle_mod, cfg)
    out, ids, w, _, _ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    assert np.all(ids == 0) and np.all(w == 1.0)
    x = U.bf16_to_f32(d["hidden"]).astype(np.float64)
    ref = 1.75 * U.swiglu_mlp(x, *U.expert_mats(cfg, d, 0))
    assert U.rel_max_err(out, ref) < 2e-6


@pytest.mark.parametrize("bits", [4, 8])
def test_shared_expert_is_dense_swiglu(synth_mod, oracle_mod, bits):
    cfg = tiny_cfg(synth_mod, T=9, shared_bits=bits, I_sh=80)
    d, lw = make(synth_mod, oracle_mod, cfg)
    got = oracle_mod.shared_ffn(cfg, d["hidden"], lw)
    x = U.bf16_to_f32(d["hidden"]).astype(np.float64)
    ref = U.swiglu_mlp(x, *U.shared_mats(cfg, d))
    assert U.rel_max_err(got, ref) < 2e-6


def test_layer_against_numpy_sparse_sum(synth_mod, oracle_mod):
    """Whole layer against a numpy evaluation of sum_j rsf*w_j*FFN_{id_j}(x) + shared(x),
    using the oracle's routing (the router is pinned separately)."""
    cfg = tiny_cfg(synth_mod, T=16, E=8, k=3, rsf=1.5, n_group=4, topk_group=2)
    d, lw = make(synth_mod, oracle_mod, cfg)
    out, ids, w, _, _ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    x = U.bf16_to_f32(d["hidden"]).astype(np.float64)
    mats = [U.expert_mats(cfg, d, e) for e in range(cfg.E)]
    ref = U.swiglu_mlp(x, *U.shared_mats(cfg, d))
    for t in range(cfg.T):
        for j in range(cfg.k):
            ref[t] += 1.5 * float(w[t, j]) * U.swiglu_mlp(x[t:t + 1], *mats[ids[t, j]])[0]
    assert U.rel_max_err(out, ref) < 2e-6


def test_identical_experts_make_routing_irrelevant(synth_mod, oracle_mod):
    """All experts equal: the routed part is rsf*FFN(x) whatever the routing (sum w = 1)."""
    cfg = tiny_cfg(synth_mod, T=20, E=8, k=2, shared_bits=0, rsf=2.0)
    d = synth_mod.layer(cfg)
    d["experts_q"][:] = d["experts_q"][0]
    d["experts_qs"][:] = d["experts_qs"][0]
    lw = oracle_mod.LayerWeights(cfg, d)
    out, _, _, _, _ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    x = U.bf16_to_f32(d["hidden"]).astype(np.float64)
    ref = 2.0 * U.swiglu_mlp(x, *U.expert_mats(cfg, d, 0))
    assert U.rel_max_err(out, ref) < 2e-6


@pytest.mark.parametrize("kw", [dict(), dict(E=8, k=3, n_group=4, topk_group=2, rsf=2.5), dict(shared_bits=8)])
def test_sparse_equals_dense_mask(synth_mod, oracle_mod, kw):
    cfg = tiny_cfg(synth_mod, **kw)
    d, lw = make(synth_mod, oracle_mod, cfg)
    sparse, *_ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    dense = oracle_mod.layer_forward_dense(cfg, lw, d["hidden"])
    assert np.allclose(sparse, dense, rtol=2e-7, atol=1e-9)


def test_rsf_linearity(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, T=16)
    d, lw = make(synth_mod, oracle_mod, cfg)
    sh = oracle_mod.shared_ffn(cfg, d["hidden"], lw).astype(np.float64)
    o1, *_ = oracle_mod.layer_forward(cfg.with_(rsf=1.0), lw, d["hidden"])
    o3, *_ = oracle_mod.layer_forward(cfg.with_(rsf=3.0), lw, d["hidden"])
    assert np.allclose(o3 - sh, 3.0 * (o1 - sh), rtol=1e-5, atol=1e-6)


def test_residual_adds_input(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, T=8)
    d, lw = make(synth_mod, oracle_mod, cfg)
    o0, *_ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    o1, *_ = oracle_mod.layer_forward(cfg, lw, d["hidden"], residual=True)
    x = U.bf16_to_f32(d["hidden"])
    assert np.allclose(o1, o0.astype(np.float64) + x, rtol=0, atol=1e-6)


def test_token_subset_matches_full(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, T=24, E=8, k=2)
    d, lw = make(synth_mod, oracle_mod, cfg)
    out, ids, w, _, _ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    toks = np.array([0, 5, 23, 7])
    assert np.array_equal(oracle_mod.layer_tokens(cfg, lw, d["hidden"], toks), out[toks])
    assert np.array_equal(oracle_mod.layer_tokens(cfg, lw, d["hidden"], toks, ids, w), out[toks])


def test_split_calls_compose_to_layer(synth_mod, oracle_mod):
    """router -> permute -> expert_ffn (pre-scaled) -> shared -> combine equals the layer."""
    cfg = tiny_cfg(synth_mod, T=16, rsf=2.0)
    d, lw = make(synth_mod, oracle_mod, cfg)
    x = d["hidden"]
    out, *_ = oracle_mod.layer_forward(cfg, lw, x)
    ids, w, _, _ = oracle_mod.router(cfg, x, d["router_w"], d["router_bias"])
    counts, offsets, srt, inv = oracle_mod.permute(cfg, ids)
    y = oracle_mod.expert_ffn(cfg, x, lw, offsets, srt)
    sh = oracle_mod.shared_ffn(cfg, x, lw)
    assert np.array_equal(oracle_mod.combine(cfg, y, inv, w, sh), out)
    ys = oracle_mod.expert_ffn(cfg, x, lw, offsets, srt, pair_scale=(2.0 * w).astype(np.float32).ravel())
    assert np.allclose(oracle_mod.combine(cfg, ys, inv, None, sh), out, rtol=1e-6, atol=1e-7)


def test_integer_sums_exact(synth_mod, oracle_mod):
    """Integer-valued inputs: the gate/up sums are exact integers equal to numpy's int64 matmul."""
    cfg = tiny_cfg(synth_mod, T=16, H=128, E=4, k=2, I=64)
    d, lw = make(synth_mod, oracle_mod, cfg)
    x = synth_mod.small_int_hidden(cfg, 8)
    ids, _, _, _ = oracle_mod.router(cfg, x, d["router_w"], d["router_bias"])
    _, offsets, srt, _ = oracle_mod.permute(cfg, ids)
    g, u = oracle_mod.gateup_int_sums(cfg, x, lw, offsets, srt)
    xi = U.bf16_to_f32(x).astype(np.int64)
    mat = cfg.I * cfg.H // 2
    for r in range(cfg.T * cfg.k):
        e = int(np.searchsorted(offsets, r, side="right") - 1)
        t = srt[r] // cfg.k
        qg = U.unpack_int4(d["experts_q"][e][:mat].reshape(cfg.I, -1), cfg.H).astype(np.int64)
        qu = U.unpack_int4(d["experts_q"][e][mat:2 * mat].reshape(cfg.I, -1), cfg.H).astype(np.int64)
        assert np.array_equal(g[r], (qg @ xi[t]).astype(np.float64))
        assert np.array_equal(u[r], (qu @ xi[t]).astype(np.float64))


# ------------------------------------------------------------------ quantiser (NEXT-2)
# Per-row symmetric quantisation with one f32 scale per row (colibri-nano
# README, "Converting a checkpoint yourself"); the codes are the nearest
# integer multiples of the scale, ties to even (numpy's rounding, which the
# pages' converter uses), and the scale maps the row's largest magnitude to
# the largest code.

QMAX = {4: 7, 8: 127}


def _codes(oracle_mod, q, bits, cols):
    if bits == 4:
        return np.stack([oracle_mod.unpack_int4_row(r, cols) for r in q])
    return q.astype(np.int32)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_zero_rows(oracle_mod, bits):
    src = np.zeros((3, 10), np.float32)
    src[1, 3] = -0.0
    q, s = oracle_mod.quantize_rows(src, bits)
    assert np.all(s == 0) and np.all(_codes(oracle_mod, q, bits, 10) == 0)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_exact_round_trip(oracle_mod, bits):
    # codes with one +-qmax per row and scales m * 2^e (m odd, 5 bits): every
    # product q * s, and amax / qmax = s, is exact in f32, so quantising the
    # dequantised row must return the same codes and the same scale bits
    rng = np.random.default_rng(11)
    qm = QMAX[bits]
    rows, cols = 40, 34
    codes = rng.integers(-qm, qm + 1, size=(rows, cols))
    codes[np.arange(rows), rng.integers(0, cols, rows)] = qm * rng.choice([-1, 1], rows)
    scales = (rng.integers(0, 16, rows) * 2 + 1) * np.exp2(rng.integers(-14, 2, rows))
    src = (codes * scales[:, None]).astype(np.float32)
    assert np.array_equal(src.astype(np.float64), codes * scales[:, None])  # exact
    q, s = oracle_mod.quantize_rows(src, bits)
    assert np.array_equal(s, scales.astype(np.float32))
    assert np.array_equal(_codes(oracle_mod, q, bits, cols), codes)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_ties_go_to_even(oracle_mod, bits):
    qm = QMAX[bits]
    halves = np.arange(-qm, qm) + 0.5  # every half-way point inside the range
    want = np.where(np.floor(halves) % 2 == 0, np.floor(halves), np.ceil(halves))
    row = np.concatenate([[qm], halves]) * 0.125  # a power-of-two scale keeps them exact
    if len(row) % 2:
        row = np.concatenate([row, [0.0]])
        want = np.concatenate([want, [0.0]])
    q, s = oracle_mod.quantize_rows(row[None, :].astype(np.float32), bits)
    assert s[0] == np.float32(0.125)
    got = _codes(oracle_mod, q, bits, len(row))[0]
    assert got[0] == qm and np.array_equal(got[1:], want)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_nearest_code_brute_force(oracle_mod, bits):
    from fractions import Fraction
    rng = np.random.default_rng(5)
    qm = QMAX[bits]
    src = (rng.standard_normal((6, 64)) * rng.uniform(0.01, 3.0, (6, 1))).astype(np.float32)
    q, s = oracle_mod.quantize_rows(src, bits)
    codes = _codes(oracle_mod, q, bits, 64)
    for r in range(src.shape[0]):
        amax = np.max(np.abs(src[r]))
        assert s[r] == np.float32(amax) / np.float32(qm)  # the scale's definition, one f32 division
        S = Fraction(float(s[r]))
        for c in range(64):
            w = Fraction(float(src[r, c]))
            dist = sorted((abs(w - k * S), k) for k in range(-qm, qm + 1))
            if dist[1][0] - dist[0][0] < Fraction(1, 10**6) * S:
                continue  # (an exact tie or a near one; the tie rule has its own pin)
            assert codes[r, c] == dist[0][1], (r, c)
        assert np.max(np.abs(codes[r])) == qm


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_sign_and_power_of_two_scaling(oracle_mod, bits):
    rng = np.random.default_rng(9)
    src = rng.standard_normal((5, 48)).astype(np.float32)
    q, s = oracle_mod.quantize_rows(src, bits)
    qn, sn = oracle_mod.quantize_rows(-src, bits)
    q4, s4 = oracle_mod.quantize_rows(src * np.float32(4.0), bits)
    c, cn, c4 = (_codes(oracle_mod, a, bits, 48) for a in (q, qn, q4))
    assert np.array_equal(sn, s) and np.array_equal(cn, -c)
    assert np.array_equal(s4, s * 4) and np.array_equal(c4, c)


def test_quantizer_bf16_input_is_its_widened_value(oracle_mod):
    rng = np.random.default_rng(3)
    bits16 = (rng.standard_normal((4, 40)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    widened = (bits16.astype(np.uint32) << 16).view(np.float32)
    for b in (4, 8):
        qa, sa = oracle_mod.quantize_rows(bits16, b)
        qb, sb = oracle_mod.quantize_rows(widened, b)
        assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


# ------------------------------------------------------------------ bias update (NEXT-3)
# Aux-loss-free balancing (Colibri-Nano model card, "Architecture": sigmoid +
# bias router with DeepSeek-V3-style aux-loss-free balancing): after a step
# each expert's bias moves by gamma toward balance.

def test_bias_update_worked_example(oracle_mod):
    # loads 3, 1, 2, 2 against a mean of 2; power-of-two values keep the sums exact
    bias = np.array([0.5, -0.25, 0.125, 0.0], np.float32)
    out = oracle_mod.bias_update(np.array([3, 1, 2, 2]), bias, 0.0625)
    assert out.tolist() == [0.4375, -0.1875, 0.125, 0.0]


def test_bias_update_no_op_cases(oracle_mod):
    rng = np.random.default_rng(4)
    bias = (rng.standard_normal(16) * 0.01).astype(np.float32)
    assert np.array_equal(oracle_mod.bias_update(np.full(16, 5), bias, 0.01), bias)  # balanced
    assert np.array_equal(oracle_mod.bias_update(rng.integers(0, 9, 16), bias, 0.0), bias)  # gamma 0
    # a fractional mean (sum 7 over 4): nobody is exactly at it, everyone moves
    out = oracle_mod.bias_update(np.array([2, 2, 2, 1]), np.zeros(4, np.float32), 0.5)
    assert out.tolist() == [-0.5, -0.5, -0.5, 0.5]


def test_bias_update_drives_loads_toward_balance(synth_mod, oracle_mod):
    # the method's purpose: repeated router -> histogram -> update steps on a
    # batch skewed toward two experts bring the loads back toward the mean
    cfg = tiny_cfg(synth_mod, T=256, E=8, k=2, H=64, seed=91)
    d = synth_mod.layer(cfg)
    bias = d["router_bias"].copy()
    bias[:2] += np.float32(0.3)

    def loads(b):
        ids = oracle_mod.router(cfg, d["hidden"], d["router_w"], b)[0]
        return np.bincount(ids.reshape(-1), minlength=cfg.E)

    start = loads(bias)
    for _ in range(80):
        bias = oracle_mod.bias_update(loads(bias), bias, 0.005)
    end = loads(bias)
    mean = cfg.T * cfg.k / cfg.E
    assert start.max() / mean > 3.0
    assert end.max() / mean < 1.5 and end.min() / mean > 0.5


def test_thread_count_does_not_change_bits(synth_mod, oracle_mod, tmp_path):
    code = ("import sys, numpy as np; sys.path.insert(0, %r); import synth, oracle;"
            "cfg = synth.CONFIGS['c0'];"
            "d = synth.layer(cfg); lw = oracle.LayerWeights(cfg, d);"
            "o = oracle.layer_forward(cfg, lw, d['hidden'])[0]; np.save(sys.argv[1], o)"
            % os.path.dirname(GOLD.rstrip('/')).rsplit('/tests', 1)[0])
    outs = []
    for n in (1, 5):
        p = str(tmp_path / f"o{n}.npy")
        env = dict(os.environ, OMP_NUM_THREADS=str(n))
        subprocess.run([sys.executable, "-c", code, p], check=True, env=env)
        outs.append(np.load(p))
    assert np.array_equal(outs[0], outs[1])


# ------------------------------------------------------- adaptive expert top-p

def _controlled_router(cfg, z_row):
    """H = 2, hidden [1, 0] (exact in bf16), W[e] = [z_e, 0]: every token's
    logits are exactly the f32 values z_row."""
    x = np.zeros((cfg.T, 2), np.uint16)
    x[:, 0] = 0x3F80  # bf16 1.0
    W = np.zeros((cfg.E, 2), np.float32)
    W[:, 0] = np.asarray(z_row, np.float32)
    return x, W


def test_top_p_worked_example(synth_mod, oracle_mod):
    """Scores 1/2, 3/10, 1/5 (weights the same, their sum is 1); p = 0.7 keeps
    the two largest (running mass 0.5 < 0.7, then 0.8 >= 0.7), renormalised to
    0.5/0.8 = 0.625 and 0.3/0.8 = 0.375; the third is dropped (id -1, w 0)."""
    s_tgt = np.array([0.5, 0.3, 0.2])
    cfg = tiny_cfg(synth_mod, T=3, H=2, E=3, k=3, top_p=0.7)
    x, W = _controlled_router(cfg, np.log(s_tgt / (1 - s_tgt)))
    ids, w, _, _ = oracle_mod.router(cfg, x, W, np.zeros(3, np.float32))
    for t in range(cfg.T):
        assert list(ids[t]) == [0, 1, -1]
        assert np.allclose(w[t], [0.625, 0.375, 0.0], rtol=0, atol=1e-6) and w[t][2] == 0.0


def test_top_p_ties_keep_lower_id(synth_mod, oracle_mod):
    """Scores 1/2, 1/2, 1/4 -> weights 0.4, 0.4, 0.2; p = 0.3 is reached by the
    first ranked alone, and of the two equal weights the lower id ranks first
    (the selection order itself is b = s + bias, here the bias puts id 1 first)."""
    cfg = tiny_cfg(synth_mod, T=2, H=2, E=3, k=3, top_p=0.3)
    x, W = _controlled_router(cfg, [0.0, 0.0, np.log(1 / 3)])
    bias = np.array([0.0, 0.01, 0.0], np.float32)
    ids, w, _, _ = oracle_mod.router(cfg, x, W, bias)
    for t in range(cfg.T):
        # selection order [1, 0, 2]; the tie of ids 1 and 0 ranks id 0 first
        assert list(ids[t]) == [-1, 0, -1]
        assert list(w[t]) == [0.0, 1.0, 0.0]


def test_top_p_mass_reaching_p_exactly_stops(synth_mod, oracle_mod):
    """Two equal scores: weights exactly 1/2 each; p = 1/2 is reached by the
    first ranked (the lower id), so the second is dropped."""
    cfg = tiny_cfg(synth_mod, T=2, H=2, E=2, k=2, top_p=0.5)
    x, W = _controlled_router(cfg, [0.3, 0.3])
    ids, w, _, _ = oracle_mod.router(cfg, x, W, np.zeros(2, np.float32))
    for t in range(cfg.T):
        assert list(ids[t]) == [0, -1] and list(w[t]) == [1.0, 0.0]


def test_top_p_off_values_keep_everything(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, T=20, E=16, k=4, seed=91)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    ref = oracle_mod.router(cfg, x, W, bias)
    for p in (0.0, 1.0, 1.5, -0.2):
        got = oracle_mod.router(cfg.with_(top_p=p), x, W, bias)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_top_p_tiny_keeps_the_heaviest(synth_mod, oracle_mod):
    """p -> 0: one expert per token, the one of largest weight (= largest
    unbiased score among the selected), with weight exactly 1."""
    cfg = tiny_cfg(synth_mod, T=30, E=16, k=4, seed=92)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    W *= 8
    ids0, w0, _, _ = oracle_mod.router(cfg, x, W, bias)
    ids, w, _, _ = oracle_mod.router(cfg.with_(top_p=1e-6), x, W, bias)
    for t in range(cfg.T):
        kept = [j for j in range(cfg.k) if ids[t][j] >= 0]
        assert len(kept) == 1 and w[t][kept[0]] == 1.0
        best = max(range(cfg.k), key=lambda j: (w0[t][j], -ids0[t][j]))
        assert kept == [best] and ids[t][best] == ids0[t][best]


@pytest.mark.parametrize("p", [0.35, 0.7, 0.9])
def test_top_p_definition_invariants(synth_mod, oracle_mod, p):
    """The kept set is the shortest prefix of the weight ranking whose f32
    running mass reaches p; kept weights are the unbiased scores renormalised
    over the kept set; positions and ids of the kept selections are unchanged."""
    cfg = tiny_cfg(synth_mod, T=64, E=16, k=6, n_group=4, topk_group=3, seed=93)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    W *= 6
    _, s, _ = oracle_mod.router_scores(cfg, x, W, bias)
    ids0, w0, _, _ = oracle_mod.router(cfg, x, W, bias)
    ids, w, _, _ = oracle_mod.router(cfg.with_(top_p=p), x, W, bias)
    for t in range(cfg.T):
        rank = sorted(range(cfg.k), key=lambda j: (-w0[t][j], ids0[t][j]))
        mass, keep = np.float32(0), 0
        while keep < cfg.k and mass < np.float32(p):
            mass = np.float32(mass + w0[t][rank[keep]])
            keep += 1
        kept = set(rank[:keep])
        ssum = sum(float(s[t][ids0[t][j]]) for j in kept)
        for j in range(cfg.k):
            if j in kept:
                assert ids[t][j] == ids0[t][j]
                assert abs(w[t][j] - s[t][ids0[t][j]] / ssum) <= 1e-7
            else:
                assert ids[t][j] == -1 and w[t][j] == 0.0
        assert abs(float(w[t][list(kept)].sum()) - 1.0) < 1e-6


@pytest.mark.parametrize("kw", [dict(top_p=0.6, w_std=0.2), dict(E=8, k=3, n_group=4, topk_group=2, rsf=2.5, top_p=0.5, w_std=0.2)])
def test_top_p_sparse_equals_dense_mask(synth_mod, oracle_mod, kw):
    """With dropped pairs the sorted grouped path (permutation skips them, the
    combine skips them) equals the dense all-experts-times-mask path."""
    cfg = tiny_cfg(synth_mod, **kw)
    d, lw = make(synth_mod, oracle_mod, cfg)
    sparse, ids, *_ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    assert (ids == -1).any()
    dense = oracle_mod.layer_forward_dense(cfg, lw, d["hidden"])
    assert np.allclose(sparse, dense, rtol=2e-7, atol=1e-9)


def test_top_p_permutation_skips_dropped(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, T=40, E=8, k=3, top_p=0.6, seed=95)
    x = synth_mod.hidden(cfg)
    W, bias = synth_mod.router(cfg)
    ids, _, _, _ = oracle_mod.router(cfg, x, W, bias)
    counts, offsets, srt, inv = oracle_mod.permute(cfg, ids)
    flat = ids.reshape(-1)
    live = np.nonzero(flat >= 0)[0]
    assert counts.sum() == len(live) and offsets[-1] == len(live)
    assert np.all(inv[flat < 0] == -1)
    order = live[np.argsort(flat[live], kind="stable")]
    assert np.array_equal(srt[:len(live)], order)
    assert np.array_equal(inv[order], np.arange(len(live)))


# --------------------------------------------- Q8_0-style int8 activations

def test_q8_worked_example(oracle_mod):
    """One block with max |v| = 63.5, so d = 0.5 exactly: 0.25 / d = 0.5 and
    1.25 / d = 2.5 are ties (to even: 0 and 2), 0.75 / d = 1.5 goes to 2;
    then an all-zero block (d = 0, codes 0).  bf16 input gives the same."""
    blk = np.zeros(32, dtype=np.float32)
    blk[:8] = [63.5, 0.25, 0.75, -0.75, 1.25, 0.26, -63.5, 10.0]
    v = np.concatenate([blk, np.zeros(32, dtype=np.float32)])[None, :]
    q, d = oracle_mod.quantize_act_q8(v)
    assert d.tolist() == [[0.5, 0.0]]
    assert q[0, :8].tolist() == [127, 0, 2, -2, 2, 1, -127, 20]
    assert not q[0, 8:].any()
    qb, db = oracle_mod.quantize_act_q8(U.f32_to_bf16_rne(v))
    assert np.array_equal(qb, q) and np.array_equal(db, d)


def test_q8_nearest_code_and_bounds(oracle_mod):
    """Random blocks over many magnitudes: every code is the nearest integer to
    v / d (checked in f64 against all 255 codes, near-ties left out), |q| <=
    127 with 127 reached in every non-zero block, and d * 127 is max |v| to
    f32 rounding."""
    rng = np.random.default_rng(5)
    rows = []
    for e in (-30, -8, 0, 3, 30):
        rows.append((rng.standard_normal(256) * 10.0 ** e).astype(np.float32))
    rows.append(np.where(rng.random(256) < 0.7, 0.0, rng.standard_normal(256)).astype(np.float32))
    v = np.stack(rows)
    q, d = oracle_mod.quantize_act_q8(v)
    codes = np.arange(-127, 128, dtype=np.float64)
    checked = 0
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            vb = v[r, 32 * b:32 * b + 32].astype(np.float64)
            db = float(d[r, b])
            qb = q[r, 32 * b:32 * b + 32].astype(np.int64)
            amax = np.abs(vb).max()
            if amax == 0:
                assert db == 0 and not qb.any()
                continue
            assert abs(db * 127 - amax) <= 2e-7 * amax
            assert np.abs(qb).max() == 127
            t = vb / db
            near_tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4
            best = codes[np.argmin(np.abs(t[:, None] - codes[None, :]), axis=1)]
            assert np.array_equal(best[~near_tie].astype(np.int64), qb[~near_tie])
            checked += int((~near_tie).sum())
    assert checked > 1000


def test_q8_sign_power_of_two_and_block_independence(oracle_mod):
    rng = np.random.default_rng(6)
    v = rng.standard_normal((3, 128)).astype(np.float32)
    q, d = oracle_mod.quantize_act_q8(v)
    q2, d2 = oracle_mod.quantize_act_q8(-v * np.float32(2.0 ** -9))
    assert np.array_equal(q2, -q) and np.array_equal(d2, d * np.float32(2.0 ** -9))
    w = v.copy()
    w[:, 32:64] *= 1000.0  # another block's values leave the rest alone
    q3, d3 = oracle_mod.quantize_act_q8(w)
    keep = np.r_[0:32, 64:128]
    assert np.array_equal(q3[:, keep], q[:, keep])
    assert np.array_equal(d3[:, [0, 2, 3]], d[:, [0, 2, 3]])


def _q8_dequant(oracle_mod, v32):
    q, d = oracle_mod.quantize_act_q8(np.ascontiguousarray(v32, dtype=np.float32))
    return q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)


def _q8_mlp(oracle_mod, x, g, u, dn):
    """The Q8 expert through dequantised activations, in f64 matmuls (a route
    independent of the oracle's integer block sums): x' = d * q, g and u
    rounded to f32, h in f32, h' = d * q of h."""
    xq = _q8_dequant(oracle_mod, x)
    gg = (xq @ g.T).astype(np.float32).astype(np.float64)
    uu = (xq @ u.T).astype(np.float32).astype(np.float64)
    h = (gg * expit(gg) * uu).astype(np.float32)
    return _q8_dequant(oracle_mod, h) @ dn.T


@pytest.mark.parametrize("shared_bits", [4, 8])
def test_q8_layer_against_numpy_dequantised(synth_mod, oracle_mod, shared_bits):
    """The whole layer in Q8 mode against sum_j rsf*w_j*FFN'_{id_j}(x) +
    shared'(x) where FFN' runs the dequantised activations through f64
    matmuls of the dequantised weights (the routing is the plain one: the
    router does not see the mode)."""
    cfg = tiny_cfg(synth_mod, T=16, E=8, k=3, rsf=1.5, n_group=4, topk_group=2, shared_bits=shared_bits,
                   I_sh=64, act_q8=True)
    d, lw = make(synth_mod, oracle_mod, cfg)
    out, ids, w, _, _ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    plain = cfg.with_(act_q8=False)
    _, ids0, w0, _, _ = oracle_mod.layer_forward(plain, oracle_mod.LayerWeights(plain, d), d["hidden"])
    assert np.array_equal(ids, ids0) and np.array_equal(w, w0)
    x = U.bf16_to_f32(d["hidden"])
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        ref[t] = _q8_mlp(oracle_mod, x[t:t + 1], *U.shared_mats(cfg, d))[0]
        for j in range(cfg.k):
            ref[t] += 1.5 * float(w[t, j]) * _q8_mlp(oracle_mod, x[t:t + 1], *U.expert_mats(cfg, d, ids[t, j]))[0]
    assert U.rel_max_err(out, ref) < 2e-6


def test_q8_sparse_equals_dense_mask(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, I_sh=64, act_q8=True)
    d, lw = make(synth_mod, oracle_mod, cfg)
    sparse, *_ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    dense = oracle_mod.layer_forward_dense(cfg, lw, d["hidden"])
    assert np.allclose(sparse, dense, rtol=2e-7, atol=1e-9)


def test_q8_shape_rule(synth_mod, oracle_mod):
    """Q8 mode needs the contraction sizes in whole 32-blocks."""
    cfg = tiny_cfg(synth_mod, I=48, I_sh=64, act_q8=True)
    d, lw = make(synth_mod, oracle_mod, cfg)
    with pytest.raises(RuntimeError):
        oracle_mod.layer_forward(cfg, lw, d["hidden"])


# ------------------------------------------------ int2 cold-tail experts

def test_int2_byte_decode_golden_and_exhaustive(oracle_mod):
    """0xE4 = fields 00, 01, 10, 11 from the low bits: elements 0, 1, -2, -1;
    and every byte value against a direct reading of its four fields."""
    import ctypes
    def decode(row, cols):
        vals = np.zeros(cols, np.int32)
        oracle_mod.lib().oracle_unpack_int2_row(row.ctypes.data, cols, vals.ctypes.data)
        return vals
    assert decode(np.array([0xE4], np.uint8), 4).tolist() == [0, 1, -2, -1]
    allb = np.arange(256, dtype=np.uint8)
    got = decode(allb, 1024).reshape(256, 4)
    for b in range(256):
        want = [((b >> (2 * j)) & 3) - (4 if (b >> (2 * j)) & 2 else 0) for j in range(4)]
        assert got[b].tolist() == want
    s = np.array([0.75], np.float32)
    out = np.zeros(1024, np.float32)
    oracle_mod.lib().oracle_dequant_row(allb.ctypes.data, 2, s.ctypes.data, 1024, out.ctypes.data)
    assert np.array_equal(out, got.ravel().astype(np.float32) * np.float32(0.75))


def test_int2_layer_against_numpy_sparse_sum(synth_mod, oracle_mod):
    """A layer with half its routed experts in int2 against the numpy sum over
    the routing, each expert decoded by numpy in its own format."""
    cfg = tiny_cfg(synth_mod, T=16, E=8, k=3, rsf=1.5, int2_frac=0.5)
    d, lw = make(synth_mod, oracle_mod, cfg)
    assert (d["expert_bits"] == 2).sum() == 4
    out, ids, w, _, _ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    assert np.isin(ids, np.nonzero(d["expert_bits"] == 2)[0]).any()
    x = U.bf16_to_f32(d["hidden"]).astype(np.float64)
    ref = U.swiglu_mlp(x, *U.shared_mats(cfg, d))
    for t in range(cfg.T):
        for j in range(cfg.k):
            ref[t] += 1.5 * float(w[t, j]) * U.swiglu_mlp(x[t:t + 1], *U.expert_mats(cfg, d, ids[t, j]))[0]
    assert U.rel_max_err(out, ref) < 2e-6


@pytest.mark.parametrize("q8", [False, True])
def test_int2_expert_equals_its_int4_encoding(synth_mod, oracle_mod, q8):
    """Codes -1..1 fit int4: the same experts re-encoded as int4 (same scales)
    give the same bits, in the plain and in the Q8 mode."""
    cfg = tiny_cfg(synth_mod, T=16, E=8, k=2, I_sh=64, int2_frac=0.5, act_q8=q8)
    d, lw = make(synth_mod, oracle_mod, cfg)
    out2, *_ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    H, I = cfg.H, cfg.I
    mat = I * H // 2
    d4 = dict(d)
    q4 = d["experts_q"].copy()
    for e in np.nonzero(d["expert_bits"] == 2)[0]:
        q = d["experts_q"][e]
        for off, rows, cols in ((0, I, H), (mat, I, H), (2 * mat, H, I)):
            codes = U.unpack_int2(q[off:off + rows * cols // 4].reshape(rows, cols // 4), cols)
            q4[e, off:off + rows * cols // 2] = U.pack_int4(codes).ravel()
    d4["experts_q"] = q4
    d4["expert_bits"] = np.full(cfg.E, 4, np.uint8)
    out4, *_ = oracle_mod.layer_forward(cfg, oracle_mod.LayerWeights(cfg, d4), d["hidden"])
    assert np.array_equal(out2, out4)


def test_int2_sparse_equals_dense_mask(synth_mod, oracle_mod):
    cfg = tiny_cfg(synth_mod, int2_frac=0.4)
    d, lw = make(synth_mod, oracle_mod, cfg)
    sparse, *_ = oracle_mod.layer_forward(cfg, lw, d["hidden"])
    dense = oracle_mod.layer_forward_dense(cfg, lw, d["hidden"])
    assert np.allclose(sparse, dense, rtol=2e-7, atol=1e-9)

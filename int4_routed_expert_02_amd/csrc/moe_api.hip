// moe_api.hip -- the C ABI (include/moe.h): host-side validation, workspace
// layout and kernel launches.  Nothing here touches device memory from the host
// or synchronises; every error is detected before the first enqueue.
#include <string.h>

#include <mutex>

#include "moe.h"
#include "moe_launch.h"

namespace {

using moe::FfnArgs;

// A second stream per device (default priority, non-blocking) for work that
// does not depend on the routing: the tiled regime runs the shared expert on it
// while the router, the permutation and the routed GEMMs run on the caller's
// stream, forked and joined with events (a captured graph gets two branches);
// `xs` marks the layer input's row sums, which the side stream computes and
// the routed GEMMs wait for.  The mutex keeps one call's events from
// interleaving with another's.
struct SideStream {
    hipStream_t st = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, xs = nullptr;
};
constexpr int MAX_DEVICES = 64;
SideStream g_side[MAX_DEVICES];
std::mutex g_side_mu;

SideStream *side_stream(hipStream_t caller)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    SideStream &s = g_side[dev];
    if (!s.st) {
        // not created under graph capture: the caller's stream then runs everything
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
        // all four or none: a partial set is released and the next call tries again
        SideStream n;
        if (hipStreamCreateWithFlags(&n.st, hipStreamNonBlocking) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&n.join, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&n.xs, hipEventDisableTiming) != hipSuccess) {
            if (n.fork) (void)hipEventDestroy(n.fork);
            if (n.join) (void)hipEventDestroy(n.join);
            (void)hipStreamDestroy(n.st);
            return nullptr;
        }
        s = n;
    }
    return &s;
}

constexpr size_t WS_ALIGN = 256;

// The workspace of moe_layer_forward_noalloc: a file-scope device array, one
// copy per GPU, kept until the process ends.  Host code never passes its name
// to a kernel or a copy (on the host the name is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and is kept in g_scratch.
constexpr size_t NOALLOC_BYTES = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];
void *g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

// This device's copy of `scratch` (nullptr on failure).
void *scratch_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

size_t align_up(size_t v) { return (v + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int validate(const moe_shape *s)
{
    if (!s) return MOE_ERR_NULL;
    if (s->T < 0 || s->H <= 0 || s->E <= 0 || s->top_k <= 0 || s->I <= 0) return MOE_ERR_SHAPE;
    if (s->top_k > s->E) return MOE_ERR_SHAPE;
    if (s->H % 2 || s->I % 2) return MOE_ERR_SHAPE;
    if (s->shared_bits != 0 && s->shared_bits != 4 && s->shared_bits != 8) return MOE_ERR_SHAPE;
    if (s->shared_bits && (s->I_shared <= 0 || s->I_shared % 2)) return MOE_ERR_SHAPE;
    if (s->n_group <= 0 || s->E % s->n_group) return MOE_ERR_SHAPE;
    if (s->topk_group <= 0 || s->topk_group > s->n_group) return MOE_ERR_SHAPE;
    if (s->n_group > 1 && s->E / s->n_group < 2) return MOE_ERR_SHAPE;
    if (s->top_k > s->topk_group * (s->E / s->n_group)) return MOE_ERR_SHAPE;
    if ((int64_t)s->T * s->top_k > INT32_MAX / 2) return MOE_ERR_SHAPE;
    if (s->top_p != s->top_p) return MOE_ERR_SHAPE;  // NaN
    // what the gfx950 kernels cover
    if (s->H % 128 || s->I % 64) return MOE_ERR_UNSUPPORTED;
    if (s->shared_bits && s->I_shared % 64) return MOE_ERR_UNSUPPORTED;
    if (s->E > 256 || s->top_k > 64 || s->n_group > 64) return MOE_ERR_UNSUPPORTED;
    if ((s->flags & MOE_EXPERT_MIXED) && (s->flags & (MOE_ACT_Q8 | MOE_TEST_GATEUP_SUMS | MOE_EXPERT_INT8)))
        return MOE_ERR_UNSUPPORTED;
    if ((s->flags & MOE_REGIME_SMALL) &&
        ((s->flags & (MOE_REGIME_TILED | MOE_ACT_Q8)) ||
         !moe::decode_supported(s->H, s->E, s->top_k, s->I, s->I_shared, s->shared_bits)))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_qmat(const moe_qmat &m)
{
    if (!m.q || !m.qs) return MOE_ERR_NULL;
    if (!aligned(m.q, 16) || m.q_stride_bytes % 16 || !aligned(m.qs, 16) || m.qs_stride_floats % 4)
        return MOE_ERR_ALIGN;
    if (m.q_stride_bytes < 0 || m.qs_stride_floats < 0) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Workspace sections, in bytes, each 256-aligned.
struct Layout {
    size_t zpart, sbc, ids, w, gap, pscale, counts, offsets, sorted, inv, hbuf, shh, ypair, shy, total;
    // row sums: of the layer input (T), of the routed and shared h rows
    // (partials per 128-column tile of the gate/up GEMM)
    size_t xsum, hsum, shsum;
    // Q8_0-style activations: x codes and block scales, h (f32), its codes and scales (routed, shared)
    size_t xq, xd, hf, hq, hd, shf, shq, shd;
    bool decode;  // the small-batch path serves this shape (MOE_WS_LAYER)
};

// Largest batch the small-batch regime takes by default: two chunks of 32
// tokens.  Measured at the Nano shape (one layer, cold weights, bench.py
// --regime-sweep): the small-batch kernels are faster than the tiled ones up
// to 64 tokens and slower from 96 on.
constexpr int DEC_AUTO_MAX_T = 64;

bool use_decode(const moe_shape *s)
{
    if (s->flags & (MOE_ACT_Q8 | MOE_REGIME_TILED)) return false;  // the tiled kernels
    if (!moe::decode_supported(s->H, s->E, s->top_k, s->I, s->I_shared, s->shared_bits)) return false;
    return (s->flags & MOE_REGIME_SMALL) || s->T <= DEC_AUTO_MAX_T;
}

Layout layout(const moe_shape *s, int which)
{
    Layout L;
    memset(&L, 0, sizeof(L));
    const size_t T = (size_t)s->T, E = (size_t)s->E, k = (size_t)s->top_k, P = T * k;
    const int KS = moe::router_ks(s->T, s->H, s->E);
    const int sbt = moe::superblock_tokens(s->top_k);
    const size_t nsb = (T + sbt - 1) / sbt;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes ? bytes : 1);
        return o;
    };
    if (which == MOE_WS_PERMUTE) {
        // router partial logits or permutation histograms (never both at once)
        const size_t a = (size_t)KS * T * E * 4, b = nsb * E * 4;
        L.zpart = L.sbc = take(a > b ? a : b);
    } else if (which == MOE_WS_EXPERT_FFN) {
        L.hbuf = take(P * (size_t)s->I * 2);  // h, f16
        L.xsum = take(T * 4);
        L.hsum = take(P * (size_t)((s->I + 127) / 128) * 4);
    } else if (use_decode(s)) {
        // pair-indexed buffers, no permutation: the routing of the whole
        // batch; per chunk of tokens (reused by the chunks in turn) the
        // partial logits and the experts' partial outputs (one f16 plane per
        // 128-row intermediate unit)
        L.decode = true;
        const size_t Tc = T < (size_t)moe::DEC_CHUNK_TOKENS ? T : (size_t)moe::DEC_CHUNK_TOKENS, Pc = Tc * k;
        L.zpart = take(moe::DEC_LOGIT_PLANES * Tc * E * 4);
        L.ids = take(P * 4);
        L.w = take(P * 4);
        L.gap = take(T * 4);
        L.pscale = take(P * 4);
        L.ypair = take((size_t)(s->I / moe::DEC_CHUNK_ROWS) * Pc * (size_t)s->H * 2);
        if (s->shared_bits) L.shy = take((size_t)(s->I_shared / moe::DEC_CHUNK_ROWS) * Tc * (size_t)s->H * 2);
    } else {
        L.zpart = take((size_t)KS * T * E * 4);
        L.sbc = take(nsb * E * 4);
        L.ids = take(P * 4);
        L.w = take(P * 4);
        L.gap = take(T * 4);
        L.pscale = take(P * 4);
        L.counts = take(E * 4);
        L.offsets = take((E + 1) * 4);
        L.sorted = take(P * 4);
        L.inv = take(P * 4);
        L.hbuf = take(P * (size_t)s->I * 2);  // h, f16
        L.xsum = take(T * 4);
        L.hsum = take(P * (size_t)((s->I + 127) / 128) * 4);
        if (s->shared_bits) L.shsum = take(T * (size_t)((s->I_shared + 127) / 128) * 4);
        // the routed and shared output rows: f16, f32 in the Q8 mode
        const size_t yb = (s->flags & MOE_ACT_Q8) ? 4 : 2;
        L.ypair = take(P * (size_t)s->H * yb);
        if (s->shared_bits) {
            L.shh = take(T * (size_t)s->I_shared * 2);
            L.shy = take(T * (size_t)s->H * yb);
        }
        if (s->flags & MOE_ACT_Q8) {
            const size_t H = (size_t)s->H, I = (size_t)s->I, Is = (size_t)s->I_shared;
            L.xq = take(T * H);
            L.xd = take(T * (H / 32) * 4);
            L.hf = take(P * I * 4);
            L.hq = take(P * I);
            L.hd = take(P * (I / 32) * 4);
            if (s->shared_bits) {
                L.shf = take(T * Is * 4);
                L.shq = take(T * Is);
                L.shd = take(T * (Is / 32) * 4);
            }
        }
    }
    L.total = off;
    return L;
}

template <typename T>
T *at(void *ws, size_t off)
{
    return (T *)((char *)ws + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int check_ws(const moe_shape *s, int which, void *ws, size_t ws_bytes)
{
    const Layout L = layout(s, which);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (!ws) return MOE_ERR_NULL;
    if (!aligned(ws, WS_ALIGN)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

int run_ffn_down(const moe_shape *s, int wbits, const moe_qmat &down, int I, const int32_t *offsets,
                 const int32_t *sorted, int E, int rows, const float *pscale, const uint16_t *hbuf, void *y,
                 hipStream_t st, const uint8_t *ebits = nullptr, bool y_f16 = false, const float *hsum = nullptr);

// Precomputed row sums (of x for gate/up, of h for down) in place of the
// offset-correction MFMA of every k-step pay where the contraction is long:
// measured at K = 6144 (gate/up) and 2048 (down) of the GLM-class layer
// (layer 1.951 -> 1.909 ms on one box), and slower at the Nano shape's
// K = 1024 and 512 (c2 130 -> 137 us), whose short k loops gain little and
// pay the extra row-sum work.
constexpr int RS_MIN_K = 2048;

// The h-row sum partials a gate/up launch leaves in hsum (its pipelined
// tiles write them, where the down GEMM takes precomputed sums), or null.
const float *gateup_hsum(int wbits, int rows, int groups, int I, const uint8_t *ebits, const float *hsum)
{
    return hsum && !ebits && I >= RS_MIN_K && moe::ffn3_taken(0, wbits, rows, groups, I) ? hsum : nullptr;
}

// gate and up of a family with more than one expert share one expert stride
// (the kernels step both by it); a single expert's strides are never used.
bool strides_ok(const moe_qmat &gate, const moe_qmat &up, int E)
{
    return E == 1 || (gate.q_stride_bytes == up.q_stride_bytes && gate.qs_stride_floats == up.qs_stride_floats);
}

// The two grouped GEMMs of one expert family on sorted rows (the caller has
// checked strides_ok before its first enqueue).
int run_ffn(const moe_shape *s, int wbits, const uint16_t *hidden, const moe_qmat &gate, const moe_qmat &up,
            const moe_qmat &down, int I, const int32_t *offsets, const int32_t *sorted, int E, int kdiv, int rows,
            const float *pscale, uint16_t *hbuf, void *y, hipStream_t st, bool gateup_only = false,
            const uint8_t *ebits = nullptr, bool y_f16 = false, const float *xsum = nullptr, float *hsum = nullptr)
{
    FfnArgs g;
    memset(&g, 0, sizeof(g));
    g.A = hidden;
    g.lda = s->H;
    g.gather = sorted;
    g.kdiv = kdiv;
    g.offsets = offsets;
    g.E = E;
    g.M = rows;
    g.q0 = (const uint8_t *)gate.q;
    g.s0 = gate.qs;
    g.q1 = (const uint8_t *)up.q;
    g.s1 = up.qs;
    g.qstride = gate.q_stride_bytes;
    g.sstride = gate.qs_stride_floats;
    g.K = s->H;
    g.N = I;
    g.out = hbuf;
    g.ldo = I;
    g.ebits = ebits;
    // precomputed x row sums and the h row sums for the down GEMM (the
    // pipelined int4/int8 tiles; mixed families take the MFMA corrections)
    g.rsum = (ebits || s->H < RS_MIN_K) ? nullptr : xsum;
    g.rsum_parts = 1;
    const float *hs = gateup_hsum(wbits, rows, offsets ? E : 1, I, ebits, hsum);
    g.hsum = (float *)hs;
    hipError_t e = moe::launch_ffn(0, wbits, g, rows, offsets ? E : 1, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (gateup_only) return MOE_OK;
    return run_ffn_down(s, wbits, down, I, offsets, sorted, E, rows, pscale, hbuf, y, st, ebits, y_f16, hs);
}

// The down GEMM on h (f16) of sorted rows; y: f32 rows in sorted order (the
// split API), or (y_f16: the layer's own rows) f16 rows in pair order.
int run_ffn_down(const moe_shape *s, int wbits, const moe_qmat &down, int I, const int32_t *offsets,
                 const int32_t *sorted, int E, int rows, const float *pscale, const uint16_t *hbuf, void *y,
                 hipStream_t st, const uint8_t *ebits, bool y_f16, const float *hsum)
{
    FfnArgs d;
    memset(&d, 0, sizeof(d));
    d.A = hbuf;  // h in f16 [rows][I], k-slot order of the down weights
    d.lda = I;
    d.gather = nullptr;
    d.kdiv = 1;
    d.pair_of_row = sorted;
    d.offsets = offsets;
    d.E = E;
    d.M = rows;
    d.q0 = (const uint8_t *)down.q;
    d.s0 = down.qs;
    d.qstride = down.q_stride_bytes;
    d.sstride = down.qs_stride_floats;
    d.K = I;
    d.N = s->H;
    d.out = y;
    d.ldo = s->H;
    d.pscale = pscale;
    d.ebits = ebits;
    d.out_f16 = y_f16 ? 1 : 0;
    d.out_by_pair = y_f16 ? 1 : 0;
    d.rsum = hsum;  // the gate/up tiles' partials, one per 128 columns of h
    d.rsum_parts = I / 128;
    return hip_status(moe::launch_ffn(1, wbits, d, rows, offsets ? E : 1, st));
}

// Buffers of one expert family in the Q8_0-style activation mode.
struct Q8Bufs {
    const int8_t *xq;  // [T][H] codes of the layer input
    const float *xd;   // [T][H/32]
    float *hf;         // [rows][I] h
    int8_t *hq;        // [rows][I] its codes
    float *hd;         // [rows][I/32]
};

// The down GEMM of the Q8 mode: h quantised per 32-block, then int8 x int4/int8.
int run_ffn_q8_down(const moe_shape *s, int wbits, const moe_qmat &down, int I, const int32_t *offsets,
                    const int32_t *sorted, int E, int rows, const float *pscale, const Q8Bufs &b, float *y,
                    hipStream_t st)
{
    hipError_t e = moe::launch_quant_act_q8(b.hf, 0, rows, I, b.hq, b.hd, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    FfnArgs d;
    memset(&d, 0, sizeof(d));
    d.A = b.hq;
    d.ad = b.hd;
    d.lda = I;
    d.kdiv = 1;
    d.pair_of_row = sorted;
    d.offsets = offsets;
    d.E = E;
    d.M = rows;
    d.q0 = (const uint8_t *)down.q;
    d.s0 = down.qs;
    d.qstride = down.q_stride_bytes;
    d.sstride = down.qs_stride_floats;
    d.K = I;
    d.N = s->H;
    d.out = y;
    d.ldo = s->H;
    d.pscale = pscale;
    return hip_status(moe::launch_ffn_q8(1, wbits, d, rows, offsets ? E : 1, st));
}

// The two grouped GEMMs of one expert family on sorted rows, int8 activations
// (x codes gathered by token when `sorted` is given).
int run_ffn_q8(const moe_shape *s, int wbits, const moe_qmat &gate, const moe_qmat &up, const moe_qmat &down, int I,
               const int32_t *offsets, const int32_t *sorted, int E, int kdiv, int rows, const float *pscale,
               const Q8Bufs &b, float *y, hipStream_t st, bool gateup_only = false)
{
    FfnArgs g;
    memset(&g, 0, sizeof(g));
    g.A = b.xq;
    g.ad = b.xd;
    g.lda = s->H;
    g.gather = sorted;
    g.kdiv = kdiv;
    g.offsets = offsets;
    g.E = E;
    g.M = rows;
    g.q0 = (const uint8_t *)gate.q;
    g.s0 = gate.qs;
    g.q1 = (const uint8_t *)up.q;
    g.s1 = up.qs;
    g.qstride = gate.q_stride_bytes;
    g.sstride = gate.qs_stride_floats;
    g.K = s->H;
    g.N = I;
    g.out = b.hf;
    g.ldo = I;
    hipError_t e = moe::launch_ffn_q8(0, wbits, g, rows, offsets ? E : 1, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (gateup_only) return MOE_OK;
    return run_ffn_q8_down(s, wbits, down, I, offsets, sorted, E, rows, pscale, b, y, st);
}

}  // namespace

extern "C" {

int moe_validate_shape(const moe_shape *shape) { return validate(shape); }

const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: inconsistent shape";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside what the gfx950 kernels cover";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: misaligned pointer or stride";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown status";
    }
}

size_t moe_workspace_bytes(const moe_shape *shape, int which)
{
    if (validate(shape) != MOE_OK) return 0;
    if (which != MOE_WS_PERMUTE && which != MOE_WS_EXPERT_FFN && which != MOE_WS_LAYER) return 0;
    return layout(shape, which).total;
}

int moe_router(const moe_shape *s, const moe_bf16 *hidden, const float *router_w, const float *router_bias,
               int32_t *topk_ids, float *topk_w, float *sel_gap, void *ws, size_t ws_bytes, void *stream)
{
    int st = validate(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;
    if (!hidden || !router_w || !router_bias || !topk_ids || !topk_w) return MOE_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(router_w, 16)) return MOE_ERR_ALIGN;
    if ((st = check_ws(s, MOE_WS_PERMUTE, ws, ws_bytes))) return st;
    const Layout L = layout(s, MOE_WS_PERMUTE);
    const int KS = moe::router_ks(s->T, s->H, s->E);
    return hip_status(moe::launch_router(hidden, router_w, router_bias, s->T, s->H, s->E, s->top_k, s->n_group,
                                         s->topk_group, s->routed_scaling_factor, s->top_p, at<float>(ws, L.zpart), KS,
                                         topk_ids, topk_w, sel_gap, nullptr, nullptr, (hipStream_t)stream));
}

int moe_permute(const moe_shape *s, const int32_t *topk_ids, int32_t *counts, int32_t *offsets,
                int32_t *sorted_pairs, int32_t *inv_pos, void *ws, size_t ws_bytes, void *stream)
{
    int st = validate(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;
    if (!topk_ids || !counts || !offsets || !sorted_pairs || !inv_pos) return MOE_ERR_NULL;
    if ((st = check_ws(s, MOE_WS_PERMUTE, ws, ws_bytes))) return st;
    const Layout L = layout(s, MOE_WS_PERMUTE);
    const int P = s->T * s->top_k;
    const int sbt = moe::superblock_tokens(s->top_k);
    const int nsb = (s->T + sbt - 1) / sbt;
    hipStream_t hs = (hipStream_t)stream;
    int32_t *bc = at<int32_t>(ws, L.sbc);
    hipError_t e = moe::launch_pair_hist(topk_ids, P, s->E, sbt * s->top_k, nsb, bc, hs);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(moe::launch_scatter(topk_ids, bc, nsb, P, s->E, sbt * s->top_k, counts, offsets, sorted_pairs,
                                          inv_pos, hs));
}

int moe_expert_ffn(const moe_shape *s, const moe_bf16 *hidden, const moe_weights *w, const int32_t *offsets,
                   const int32_t *sorted_pairs, const float *pair_scale, float *y_pairs, void *ws, size_t ws_bytes,
                   void *stream)
{
    int st = validate(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;
    if (!hidden || !w || !offsets || !sorted_pairs || !y_pairs) return MOE_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(y_pairs, 16)) return MOE_ERR_ALIGN;
    if ((st = check_qmat(w->gate)) || (st = check_qmat(w->up)) || (st = check_qmat(w->down))) return st;
    if ((st = check_ws(s, MOE_WS_EXPERT_FFN, ws, ws_bytes))) return st;
    if (s->flags & MOE_ACT_Q8) return MOE_ERR_UNSUPPORTED;  // the int8-activation mode: moe_layer_forward
    if (!strides_ok(w->gate, w->up, s->E)) return MOE_ERR_UNSUPPORTED;
    const Layout L = layout(s, MOE_WS_EXPERT_FFN);
    const int wbits = (s->flags & MOE_EXPERT_INT8) ? 8 : 4;
    if ((s->flags & MOE_TEST_GATEUP_SUMS) && (wbits != 4 || 2 * s->I > s->H)) return MOE_ERR_UNSUPPORTED;
    if ((s->flags & MOE_EXPERT_MIXED) && !w->expert_bits) return MOE_ERR_NULL;
    float *xsum = at<float>(ws, L.xsum);
    // (the exactness test takes the precomputed sums at any K)
    if ((s->H >= RS_MIN_K || (s->flags & MOE_TEST_GATEUP_SUMS)) &&
        moe::launch_rowsum_bf16(hidden, s->H, s->T, s->H, xsum, (hipStream_t)stream) != hipSuccess)
        return MOE_ERR_HIP;
    if (s->flags & MOE_TEST_GATEUP_SUMS) {
        FfnArgs g;
        memset(&g, 0, sizeof(g));
        g.A = hidden;
        g.lda = s->H;
        g.gather = sorted_pairs;
        g.kdiv = s->top_k;
        g.offsets = offsets;
        g.E = s->E;
        g.q0 = (const uint8_t *)w->gate.q;
        g.s0 = w->gate.qs;
        g.q1 = (const uint8_t *)w->up.q;
        g.s1 = w->up.qs;
        g.qstride = w->gate.q_stride_bytes;
        g.sstride = w->gate.qs_stride_floats;
        g.K = s->H;
        g.N = s->I;
        g.out = y_pairs;
        g.ldo = s->H;
        g.rsum = xsum;
        g.rsum_parts = 1;
        return hip_status(moe::launch_ffn(2, 4, g, s->T * s->top_k, s->E, (hipStream_t)stream));
    }
    return run_ffn(s, wbits, hidden, w->gate, w->up, w->down, s->I, offsets, sorted_pairs, s->E, s->top_k,
                   s->T * s->top_k, pair_scale, at<uint16_t>(ws, L.hbuf), y_pairs, (hipStream_t)stream,
                   (s->flags & MOE_STAGE_GATEUP_ONLY) != 0,
                   (s->flags & MOE_EXPERT_MIXED) ? w->expert_bits : nullptr, false, xsum, at<float>(ws, L.hsum));
}

int moe_combine(const moe_shape *s, const float *y_pairs, const int32_t *inv_pos, const float *topk_w,
                const float *shared_out, const moe_bf16 *residual, void *out, void *stream)
{
    int st = validate(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;
    if (!y_pairs || !inv_pos || !out) return MOE_ERR_NULL;
    if (!aligned(y_pairs, 16) || !aligned(out, 16) || (shared_out && !aligned(shared_out, 16)) ||
        (residual && !aligned(residual, 8)))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_combine(y_pairs, inv_pos, topk_w, s->routed_scaling_factor, shared_out, residual,
                                          out, s->T, s->H, s->top_k, (s->flags & MOE_OUT_F32) ? 1 : 0, 0, 0,
                                          (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The layer forward behind moe_layer_forward(_profiled, _chain).  ns/nw/nws:
// the next layer of a chained small-batch step (nw null: not chained).
int forward_impl(const moe_shape *s, const moe_weights *w, const moe_bf16 *hidden, void *out, void *ws,
                 size_t ws_bytes, void *stream, void *ev_start, void *ev_stop, const moe_shape *ns,
                 const moe_weights *nw, void *nws, size_t nws_bytes, bool allow_side = true)
{
    int st = validate(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;
    if (!w || !hidden || !out || !w->router_w || !w->router_bias) return MOE_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(out, 16) || !aligned(w->router_w, 16)) return MOE_ERR_ALIGN;
    if ((st = check_qmat(w->gate)) || (st = check_qmat(w->up)) || (st = check_qmat(w->down))) return st;
    if (s->shared_bits &&
        ((st = check_qmat(w->sh_gate)) || (st = check_qmat(w->sh_up)) || (st = check_qmat(w->sh_down))))
        return st;
    if ((st = check_ws(s, MOE_WS_LAYER, ws, ws_bytes))) return st;
    // routed experts are packed int4 (int8 rows are a moe_expert_ffn format, for a shared expert)
    if (s->flags & MOE_EXPERT_INT8) return MOE_ERR_UNSUPPORTED;
    if (!strides_ok(w->gate, w->up, s->E)) return MOE_ERR_UNSUPPORTED;
    if ((s->flags & MOE_EXPERT_MIXED) && !w->expert_bits) return MOE_ERR_NULL;
    const uint8_t *ebits = (s->flags & MOE_EXPERT_MIXED) ? w->expert_bits : nullptr;
    const Layout L = layout(s, MOE_WS_LAYER);
    hipStream_t hs = (hipStream_t)stream;
    if ((s->flags & (MOE_STAGE_EXPERTS_ONLY | MOE_LOGITS_GIVEN)) && (!L.decode || s->T > moe::DEC_CHUNK_TOKENS))
        return MOE_ERR_UNSUPPORTED;
    Layout NL;
    if (nw) {
        // chained: the next layer's router logits from this layer's bf16 output
        if (!ns || !nws || !nw->router_w || !nw->router_bias) return MOE_ERR_NULL;
        if ((st = validate(ns))) return st;
        if (ns->T != s->T || ns->H != s->H) return MOE_ERR_SHAPE;
        NL = layout(ns, MOE_WS_LAYER);
        if (!L.decode || !NL.decode || (s->flags & (MOE_OUT_F32 | MOE_STAGE_EXPERTS_ONLY)) ||
            s->T > moe::DEC_CHUNK_TOKENS)
            return MOE_ERR_UNSUPPORTED;
        if (!aligned(nw->router_w, 16)) return MOE_ERR_ALIGN;
        if ((st = check_ws(ns, MOE_WS_LAYER, nws, nws_bytes))) return st;
    }
    if (L.decode) {
        moe::DecLaunch d;
        memset(&d, 0, sizeof(d));
        d.x = hidden;
        d.rw = w->router_w;
        d.rb = w->router_bias;
        d.T = s->T;
        d.H = s->H;
        d.E = s->E;
        d.k = s->top_k;
        d.n_group = s->n_group;
        d.topk_group = s->topk_group;
        d.rsf = s->routed_scaling_factor;
        d.top_p = s->top_p;
        d.ids = at<int32_t>(ws, L.ids);
        d.w = at<float>(ws, L.w);
        d.gap = at<float>(ws, L.gap);
        d.pscale = at<float>(ws, L.pscale);
        d.z = at<float>(ws, L.zpart);
        d.gq = (const uint8_t *)w->gate.q;
        d.uq = (const uint8_t *)w->up.q;
        d.dq = (const uint8_t *)w->down.q;
        d.gs = w->gate.qs;
        d.us = w->up.qs;
        d.ds = w->down.qs;
        d.qstride = w->gate.q_stride_bytes;
        d.dqstride = w->down.q_stride_bytes;
        d.sstride = w->gate.qs_stride_floats;
        d.dsstride = w->down.qs_stride_floats;
        d.I = s->I;
        d.ebits = ebits;
        if (s->shared_bits) {
            d.sgq = (const uint8_t *)w->sh_gate.q;
            d.suq = (const uint8_t *)w->sh_up.q;
            d.sdq = (const uint8_t *)w->sh_down.q;
            d.sgs = w->sh_gate.qs;
            d.sus = w->sh_up.qs;
            d.sds = w->sh_down.qs;
            d.shp = at<uint16_t>(ws, L.shy);
        }
        d.Ish = s->I_shared;
        d.sh_bits = s->shared_bits;
        d.y = at<uint16_t>(ws, L.ypair);
        d.res = (s->flags & MOE_ADD_RESIDUAL) ? hidden : nullptr;
        d.out = out;
        d.out_f32 = (s->flags & MOE_OUT_F32) ? 1 : 0;
        d.ev0 = (hipEvent_t)ev_start;
        d.ev1 = (hipEvent_t)ev_stop;
        d.experts_only = (s->flags & MOE_STAGE_EXPERTS_ONLY) ? 1 : 0;
        d.logits_given = (s->flags & MOE_LOGITS_GIVEN) ? 1 : 0;
        if (nw) {
            d.nrw = nw->router_w;
            d.nE = ns->E;
            d.nz = at<float>(nws, NL.zpart);
        }
        // chunks of up to DEC_CHUNK_TOKENS tokens, one after another on the
        // stream (each reuses the chunk-sized logit and partial-output
        // buffers); routing and output land at the chunk's rows.  The events
        // bracket the first chunk's expert kernel through the last's.
        const int CT = moe::DEC_CHUNK_TOKENS, nchunk = (s->T + CT - 1) / CT;
        const size_t osz = d.out_f32 ? 4 : 2;
        for (int c = 0; c < nchunk; ++c) {
            const int t0 = c * CT;
            moe::DecLaunch dc = d;
            dc.T = s->T - t0 < CT ? s->T - t0 : CT;
            dc.x = d.x + (size_t)t0 * s->H;
            dc.ids = d.ids + (size_t)t0 * s->top_k;
            dc.w = d.w + (size_t)t0 * s->top_k;
            dc.gap = d.gap + t0;
            dc.pscale = d.pscale + (size_t)t0 * s->top_k;
            if (d.res) dc.res = d.res + (size_t)t0 * s->H;
            dc.out = (char *)out + (size_t)t0 * s->H * osz;
            dc.ev0 = c == 0 ? d.ev0 : nullptr;
            dc.ev1 = c == nchunk - 1 ? d.ev1 : nullptr;
            const hipError_t e = moe::launch_decode(dc, hs);
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
        return MOE_OK;
    }
    const int P = s->T * s->top_k;
    const int KS = moe::router_ks(s->T, s->H, s->E);
    const int sbt = moe::superblock_tokens(s->top_k);
    const int nsb = (s->T + sbt - 1) / sbt;
    int32_t *ids = at<int32_t>(ws, L.ids), *sbc = at<int32_t>(ws, L.sbc);
    int32_t *counts = at<int32_t>(ws, L.counts), *offsets = at<int32_t>(ws, L.offsets);
    int32_t *sorted = at<int32_t>(ws, L.sorted), *inv = at<int32_t>(ws, L.inv);
    float *pscale = at<float>(ws, L.pscale);
    float *ypair = at<float>(ws, L.ypair);  // f32 in the Q8 mode, else f16 (uint16_t)

    if (s->flags & MOE_ACT_Q8) {
        // Q8_0-style int8 activations: x quantised once (routed and shared
        // experts read the same codes), each h before its down GEMM
        hipError_t e = moe::launch_router(hidden, w->router_w, w->router_bias, s->T, s->H, s->E, s->top_k,
                                          s->n_group, s->topk_group, s->routed_scaling_factor, s->top_p,
                                          at<float>(ws, L.zpart), KS, ids, at<float>(ws, L.w), at<float>(ws, L.gap),
                                          pscale, sbc, hs);
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = moe::launch_scatter(ids, sbc, nsb, P, s->E, sbt * s->top_k, counts, offsets, sorted, inv, hs);
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = moe::launch_quant_act_q8(hidden, 1, s->T, s->H, at<int8_t>(ws, L.xq), at<float>(ws, L.xd), hs);
        if (e != hipSuccess) return MOE_ERR_HIP;
        const Q8Bufs rb{at<int8_t>(ws, L.xq), at<float>(ws, L.xd), at<float>(ws, L.hf), at<int8_t>(ws, L.hq),
                        at<float>(ws, L.hd)};
        if (ev_start && hipEventRecord((hipEvent_t)ev_start, hs) != hipSuccess) return MOE_ERR_HIP;
        st = run_ffn_q8(s, 4, w->gate, w->up, w->down, s->I, offsets, sorted, s->E, s->top_k, P, pscale, rb, ypair,
                        hs, ev_stop != nullptr);
        if (st) return st;
        if (ev_stop) {
            if (hipEventRecord((hipEvent_t)ev_stop, hs) != hipSuccess) return MOE_ERR_HIP;
            st = run_ffn_q8_down(s, 4, w->down, s->I, offsets, sorted, s->E, P, pscale, rb, ypair, hs);
            if (st) return st;
        }
        if (s->shared_bits) {
            const Q8Bufs sb{at<int8_t>(ws, L.xq), at<float>(ws, L.xd), at<float>(ws, L.shf), at<int8_t>(ws, L.shq),
                            at<float>(ws, L.shd)};
            st = run_ffn_q8(s, s->shared_bits, w->sh_gate, w->sh_up, w->sh_down, s->I_shared, nullptr, nullptr, 1, 1,
                            s->T, nullptr, sb, at<float>(ws, L.shy), hs);
            if (st) return st;
        }
        return hip_status(moe::launch_combine(ypair, inv, nullptr, 1.f,
                                              s->shared_bits ? at<float>(ws, L.shy) : nullptr,
                                              (s->flags & MOE_ADD_RESIDUAL) ? hidden : nullptr, out, s->T, s->H,
                                              s->top_k, (s->flags & MOE_OUT_F32) ? 1 : 0, 0, 0, hs));
    }

    // row sums of the layer input (the gate/up GEMMs' offset correction),
    // read by the routed and the shared experts: computed first thing on the
    // side stream where there is one (the routed gate/up waits for its event,
    // long since recorded by then), else on the caller's stream
    float *xsum = at<float>(ws, L.xsum), *hsum = at<float>(ws, L.hsum);
    const bool xrs = s->H >= RS_MIN_K;  // the gate/up GEMMs take precomputed x row sums

    // the shared expert (no dependence on the routing) on the side stream,
    // except in the profiled call, whose events time the routed gate/up alone.
    // Once forked, the side stream is joined back on every path, errors too,
    // so a failing call leaves no open fork (nor a broken graph capture).
    SideStream *side = nullptr;
    std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
    if (s->shared_bits && !ev_start && !ev_stop && allow_side) {
        side_lock.lock();
        side = side_stream(hs);
        if (!side) side_lock.unlock();
    }
    // Launch order, set by measurement: where the shared expert holds at least
    // as much work as the routed experts (I_shared >= top_k * I) the router is
    // enqueued first, so its workgroups are not queued behind the shared
    // GEMM's and the shared tiles fill the machine around the small selection
    // and scatter grids (c2 layer 144 -> 130 us; c4 unchanged); where the
    // routed work dominates (c3) the shared expert goes first (router first
    // measured 1% slower there).
    const bool router_first = (long)s->I_shared >= (long)s->top_k * s->I;
    auto shared_side = [&]() -> int {
        if (!side) return MOE_OK;
        if (xrs && (moe::launch_rowsum_bf16(hidden, s->H, s->T, s->H, xsum, side->st) != hipSuccess ||
                    hipEventRecord(side->xs, side->st) != hipSuccess))
            return MOE_ERR_HIP;
        return run_ffn(s, s->shared_bits, hidden, w->sh_gate, w->sh_up, w->sh_down, s->I_shared, nullptr, nullptr, 1,
                       1, s->T, nullptr, at<uint16_t>(ws, L.shh), at<uint16_t>(ws, L.shy), side->st, false, nullptr,
                       true, xsum, at<float>(ws, L.shsum));
    };
    auto routed = [&]() -> int {
        if (!router_first) {
            const int r = shared_side();
            if (r) return r;
        }
        hipError_t e = moe::launch_router(hidden, w->router_w, w->router_bias, s->T, s->H, s->E, s->top_k,
                                          s->n_group, s->topk_group, s->routed_scaling_factor, s->top_p,
                                          at<float>(ws, L.zpart), KS, ids, at<float>(ws, L.w), at<float>(ws, L.gap),
                                          pscale, sbc, hs);
        if (e != hipSuccess) return MOE_ERR_HIP;
        if (router_first) {
            const int r = shared_side();
            if (r) return r;
        }
        e = moe::launch_scatter(ids, sbc, nsb, P, s->E, sbt * s->top_k, counts, offsets, sorted, inv, hs);
        if (e != hipSuccess) return MOE_ERR_HIP;
        if (xrs && side) {
            if (hipStreamWaitEvent(hs, side->xs, 0) != hipSuccess) return MOE_ERR_HIP;
        } else if (xrs && moe::launch_rowsum_bf16(hidden, s->H, s->T, s->H, xsum, hs) != hipSuccess) {
            return MOE_ERR_HIP;
        }
        if (ev_start && hipEventRecord((hipEvent_t)ev_start, hs) != hipSuccess) return MOE_ERR_HIP;
        int r = run_ffn(s, 4, hidden, w->gate, w->up, w->down, s->I, offsets, sorted, s->E, s->top_k, P, pscale,
                        at<uint16_t>(ws, L.hbuf), ypair, hs, ev_stop != nullptr, ebits, true, xsum, hsum);
        if (r) return r;
        if (ev_stop) {
            // profiled: the routed gate/up kernel ran alone between the events; now the down GEMM
            if (hipEventRecord((hipEvent_t)ev_stop, hs) != hipSuccess) return MOE_ERR_HIP;
            r = run_ffn_down(s, 4, w->down, s->I, offsets, sorted, s->E, P, pscale, at<uint16_t>(ws, L.hbuf),
                             ypair, hs, ebits, true, gateup_hsum(4, P, s->E, s->I, ebits, hsum));
            if (r) return r;
        }
        return MOE_OK;
    };
    if (side) {
        if (hipEventRecord(side->fork, hs) != hipSuccess || hipStreamWaitEvent(side->st, side->fork, 0) != hipSuccess)
            return MOE_ERR_HIP;  // nothing forked yet
        st = routed();
        const bool joined =
            hipEventRecord(side->join, side->st) == hipSuccess && hipStreamWaitEvent(hs, side->join, 0) == hipSuccess;
        side_lock.unlock();
        if (st) return st;
        if (!joined) return MOE_ERR_HIP;
    } else {
        st = routed();
        if (st) return st;
        if (s->shared_bits) {
            st = run_ffn(s, s->shared_bits, hidden, w->sh_gate, w->sh_up, w->sh_down, s->I_shared, nullptr, nullptr,
                         1, 1, s->T, nullptr, at<uint16_t>(ws, L.shh), at<uint16_t>(ws, L.shy), hs, false, nullptr,
                         true, xsum, at<float>(ws, L.shsum));
            if (st) return st;
        }
    }
    const uint16_t *shy = s->shared_bits ? at<uint16_t>(ws, L.shy) : nullptr;
    return hip_status(moe::launch_combine(ypair, inv, nullptr, 1.f, shy,
                                          (s->flags & MOE_ADD_RESIDUAL) ? hidden : nullptr, out, s->T, s->H,
                                          s->top_k, (s->flags & MOE_OUT_F32) ? 1 : 0, 1, 1, hs));
}

}  // namespace

extern "C" {

int moe_layer_forward(const moe_shape *s, const moe_weights *w, const moe_bf16 *hidden, void *out, void *ws,
                      size_t ws_bytes, void *stream)
{
    return forward_impl(s, w, hidden, out, ws, ws_bytes, stream, nullptr, nullptr, nullptr, nullptr, nullptr, 0);
}

int moe_layer_forward_profiled(const moe_shape *s, const moe_weights *w, const moe_bf16 *hidden, void *out,
                               void *ws, size_t ws_bytes, void *stream, void *ev_start, void *ev_stop)
{
    return forward_impl(s, w, hidden, out, ws, ws_bytes, stream, ev_start, ev_stop, nullptr, nullptr, nullptr, 0);
}

int moe_layer_forward_chain(const moe_shape *s, const moe_weights *w, const moe_bf16 *hidden, void *out, void *ws,
                            size_t ws_bytes, const moe_shape *next_shape, const moe_weights *next_weights,
                            void *next_ws, size_t next_ws_bytes, void *stream)
{
    return forward_impl(s, w, hidden, out, ws, ws_bytes, stream, nullptr, nullptr, next_shape, next_weights, next_ws,
                        next_ws_bytes);
}

int moe_layer_forward_noalloc(const moe_shape *s, const moe_weights *w, const moe_bf16 *hidden, void *out,
                              void *stream)
{
    int st = validate(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;
    const size_t need = layout(s, MOE_WS_LAYER).total;
    if (need > NOALLOC_BYTES) return MOE_ERR_WORKSPACE;
    if (s->flags & (MOE_STAGE_EXPERTS_ONLY | MOE_LOGITS_GIVEN)) return MOE_ERR_UNSUPPORTED;
    void *ws = scratch_ptr();
    if (!ws) return MOE_ERR_HIP;
    // the shared expert stays on `stream` (no second stream is created here)
    return forward_impl(s, w, hidden, out, ws, NOALLOC_BYTES, stream, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                        false);
}

int moe_bias_update(int32_t E, const int32_t *counts, float *router_bias, float gamma, void *stream)
{
    if (E < 1) return MOE_ERR_SHAPE;
    if (!counts || !router_bias) return MOE_ERR_NULL;
    if (!aligned(counts, 4) || !aligned(router_bias, 4)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_bias_update(E, counts, router_bias, gamma, (hipStream_t)stream));
}

int moe_quantize_rows(const void *src, int32_t src_format, int64_t rows, int32_t cols, int32_t bits, void *q,
                      float *qs, void *stream)
{
    if (rows < 0 || cols <= 0 || (bits != 4 && bits != 8) || (bits == 4 && cols % 2) ||
        (src_format != MOE_SRC_F32 && src_format != MOE_SRC_BF16))
        return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!src || !q || !qs) return MOE_ERR_NULL;
    if (!aligned(src, src_format == MOE_SRC_BF16 ? 2 : 4) || !aligned(qs, 4)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_quantize(src, src_format == MOE_SRC_BF16, (long)rows, cols, bits, q, qs,
                                           (hipStream_t)stream));
}

int moe_quantize_act_q8(const void *src, int32_t src_format, int64_t rows, int32_t cols, int8_t *q, float *d,
                        void *stream)
{
    if (rows < 0 || cols <= 0 || cols % 32 || (src_format != MOE_SRC_F32 && src_format != MOE_SRC_BF16))
        return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!src || !q || !d) return MOE_ERR_NULL;
    if (!aligned(src, 16) || !aligned(q, 16) || !aligned(d, 4)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_quant_act_q8(src, src_format == MOE_SRC_BF16, (long)rows, cols, q, d,
                                               (hipStream_t)stream));
}

int moe_layer_routing(const moe_shape *s, void *ws, size_t ws_bytes, int32_t **topk_ids, float **topk_w,
                      int32_t **offsets, int32_t **sorted_pairs)
{
    int st = validate(s);
    if (st) return st;
    if ((st = check_ws(s, MOE_WS_LAYER, ws, ws_bytes))) return st;
    const Layout L = layout(s, MOE_WS_LAYER);
    if (topk_ids) *topk_ids = at<int32_t>(ws, L.ids);
    if (topk_w) *topk_w = at<float>(ws, L.w);
    if (offsets) *offsets = L.decode ? nullptr : at<int32_t>(ws, L.offsets);
    if (sorted_pairs) *sorted_pairs = L.decode ? nullptr : at<int32_t>(ws, L.sorted);
    return MOE_OK;
}

}  // extern "C"

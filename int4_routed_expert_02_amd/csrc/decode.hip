// decode.hip -- the small-batch regime: a layer whose batch routes only a few
// rows to each expert is a weight stream, bound by HBM, not by the matrix cores.
//
// The engine chooses kernels per shape by measurement (colibri README, "What's
// implemented", integer-dot kernels: the single-row int4 case takes a
// different path from the batched one).  Here, for T <= 32 tokens:
//   k_dec_logits   router logits z = x W^T in f32 FMA, one workgroup per four
//                  experts (W is the largest read of the router);
//   k_dec_gateup   routed workgroups first select the top-k experts of every
//                  token from z (sigmoid + bias, moe_select.h; each workgroup
//                  takes the same decision, the first publishes ids, weights
//                  and rsf * w), then one workgroup per (active expert, 64
//                  intermediate rows): gathers
//                  the pairs routed to its expert (batch-union: the expert's
//                  rows are read once for all of them), streams its gate and up
//                  rows straight from HBM into registers, MFMA on 16-pair
//                  blocks, SwiGLU epilogue -> h [pair][I] f32;  the shared
//                  expert's rows form extra units over all T tokens;
//   k_dec_down     one workgroup per (expert, 128 output rows, 512-column chunk
//                  of the reduction): h as an exact hi + lo bf16 pair, down rows
//                  streamed to registers, epilogue scales by sd * rsf * w ->
//                  partial y [chunk][pair][H];  the shared expert's units are
//                  (128 output rows, 512-column chunk) over all T tokens;
//   k_dec_combine  out = sum_j sum_chunk y + sum_chunk shared partials (+ x),
//                  in a fixed order.
// Buffers are indexed by pair, so no permutation is materialised: each
// workgroup finds its expert's pairs by scanning the ids in ascending order.
//
// Weight loads: a wave owns 16 weight rows; lane (n = lane % 16, g = lane / 16)
// loads 16-byte chunks (4c + g) of row n, c = 0..CPL-1, so the four lane
// groups read 64 contiguous bytes of each row per instruction and the whole
// stage is in flight before the first MFMA.  The k-slots of chunk c, word w
// for lane group g are k = (4c + g) * 32 + 8w + [0, 8) (int4), and the A
// fragments are read from LDS at the same k.
#include "moe_device.h"
#include "moe_launch.h"
#include "moe_select.h"

namespace moe {

constexpr int DEC_MAXT = 32;  // tokens per layer call in this regime

// ------------------------------------------------------------------ router

constexpr int LG_KSPLIT = 16;  // K slices of the router logits, one per wave
constexpr int LG_NP = DEC_LOGIT_PLANES;  // partial logit planes (one per workgroup of 4 waves)
static_assert(LG_KSPLIT == 4 * LG_NP, "four K slices per plane");
constexpr int DEC_MAXK = 16;   // top-k limit of this regime (LDS lists of T * k pairs)

// Router logits on the matrix cores.  The f32 router row W_e is split exactly
// into three bf16 terms (hi + mid + lo carries all 24 mantissa bits), so three
// bf16 products against the bf16 hidden row give x . W_e to f32 accuracy.
// Workgroup = (16-expert tile, 16-token tile, group of 4 K slices); wave w
// takes slice 4 * group + w of H / 16 columns, the four wave tiles are added in
// wave order and written as one partial plane: zp[group][t][e].  The consumer
// adds the LG_NP planes in plane order.
__device__ __forceinline__ void split3_bf16(const f32x4 &a, const f32x4 &b, u32x4 &hi, u32x4 &mid, u32x4 &lo)
{
    float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    uint16_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = f32_to_bf16(v[i]);
        const float r1 = v[i] - bf16_to_f32(h[i]);
        m[i] = f32_to_bf16(r1);
        l[i] = f32_to_bf16(r1 - bf16_to_f32(m[i]));
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        hi[d] = (uint32_t)h[2 * d] | ((uint32_t)h[2 * d + 1] << 16);
        mid[d] = (uint32_t)m[2 * d] | ((uint32_t)m[2 * d + 1] << 16);
        lo[d] = (uint32_t)l[2 * d] | ((uint32_t)l[2 * d + 1] << 16);
    }
}

__global__ __launch_bounds__(256) void k_dec_logits(const uint16_t *__restrict__ x, const float *__restrict__ W,
                                                    int T, int H, int E, float *__restrict__ zp)
{
    __shared__ f32x4 red[3][WAVE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int net = (E + 15) / 16, ntt = (T + 15) / 16;
    const int et = blockIdx.x % net, tt = (blockIdx.x / net) % ntt, grp = blockIdx.x / (net * ntt);
    const int ksl = H / LG_KSPLIT;
    const int k0 = (grp * 4 + wave) * ksl;
    const int e = et * 16 + n, t = tt * 16 + n;
    const float *wrow = W + (size_t)(e < E ? e : 0) * H + k0 + g * 8;
    const uint16_t *xrow = x + (size_t)(t < T ? t : 0) * H + k0 + g * 8;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < ksl; kk += 64) {  // two 32-column steps per round, loads first
        f32x4 wa[2], wb[2];
        u32x4 xv[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            wa[s] = *(const f32x4 *)(wrow + kk + 32 * s);
            wb[s] = *(const f32x4 *)(wrow + kk + 32 * s + 4);
            xv[s] = *(const u32x4 *)(xrow + kk + 32 * s);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (e >= E) wa[s] = wb[s] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t >= T) xv[s] = u32x4{0u, 0u, 0u, 0u};
            u32x4 hi, mid, lo;
            split3_bf16(wa[s], wb[s], hi, mid, lo);
            acc = mfma_bf16(hi, xv[s], acc);
            acc = mfma_bf16(mid, xv[s], acc);
            acc = mfma_bf16(lo, xv[s], acc);
        }
    }
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            const f32x4 o = red[w][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += o[r];
        }
        // acc[r] = z[token tt*16 + n][expert et*16 + 4g + r]
        if (t < T) {
            float *dst = zp + ((size_t)grp * T + t) * E + et * 16 + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (et * 16 + 4 * g + r < E) dst[r] = acc[r];
        }
    }
}

__device__ __forceinline__ float dec_logit(const float *__restrict__ zp, int T, int E, int t, int e)
{
    float z = zp[(size_t)t * E + e];
#pragma unroll
    for (int p = 1; p < LG_NP; ++p) z += zp[((size_t)p * T + t) * E + e];
    return z;
}

// Selection for all T tokens of the batch, any E <= 256, k <= 16 and group
// limit (moe_select.h, one wave per token): wave w takes tokens w, w + 4, ...
// Results go to LDS (ids_l, w_l: [T][k]); with `pub` set the workgroup also
// writes ids, w, rsf * w and the tie gap to global memory.
template <int EPL>
__device__ __noinline__ void dec_select_waves(const float *__restrict__ zp, const float *__restrict__ bias, int T,
                                              int E, int k, int n_group, int topk_group, float rsf, int32_t *ids_l,
                                              float *w_l, bool pub, float *__restrict__ gap_g)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int t = wave; t < T; t += 4) {
        float s[EPL], b[EPL];
        bool ok[EPL];
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            const int e = lane * EPL + q;
            ok[q] = e < E;
            s[q] = ok[q] ? 1.0f / (1.0f + expf(-dec_logit(zp, T, E, t, e))) : 0.f;
            b[q] = ok[q] ? s[q] + bias[e] : -INFINITY;
        }
        select_token<EPL>(s, b, ok, lane, t, E, k, n_group, topk_group, rsf, ids_l, w_l, pub ? gap_g : nullptr,
                          nullptr, nullptr);
    }
}

// One selection candidate: selection score v (sigmoid + bias), unbiased score
// s, expert id i.  Order: larger v first, equal v -> lower id first (the
// order of moe_select.h); an empty slot (i = INT_MAX, v = -inf) loses to all.
struct Cand {
    float v, s;
    int i;
};
__device__ __forceinline__ bool cand_before(const Cand &a, const Cand &b)
{
    return a.v > b.v || (a.v == b.v && a.i < b.i);
}
__device__ __forceinline__ void cand_sort2(Cand &a, Cand &b)
{
    if (cand_before(b, a)) {
        const Cand t = a;
        a = b;
        b = t;
    }
}

// Fast selection when no group limit applies, E <= 64, E % 8 == 0 and k < KL:
// eight lanes per token (lane slice q scans experts 8q .. 8q + 7), each keeps
// its best KL candidates sorted, then three butterfly merges over the slices
// (bitonic: pair own entry j with the partner's entry KL - 1 - j, keep the
// better, re-sort) leave the batch-wide best KL in every lane of the token.
// The selected k are the first k, taken in that order; the weight of
// selection j is s_j over the sum of the selected s (summed in selection
// order); the tie gap is v_{k-1} - v_k.  Same results as moe_select.h.
template <int KL, typename Pre>
__device__ __forceinline__ void dec_select_lanes(const float *__restrict__ zp, const float *__restrict__ bias, int T,
                                                 int E, int k, int32_t *ids_l, float *w_l, bool pub,
                                                 float *__restrict__ gap_g, Pre &&pre)
{
    const int tid = threadIdx.x, t = tid >> 3, q = tid & 7;
    Cand c[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) c[j] = Cand{-INFINITY, 0.f, 0x7fffffff};
    const bool live = t < T && 8 * q < E;
    // the logits are requested first, then the caller's own requests (pre), so
    // that waiting for the logits never waits for those
    f32x4 pa[LG_NP][2], b0, b1;
    if (live) {
#pragma unroll
        for (int p = 0; p < LG_NP; ++p) {
            const f32x4 *pp = (const f32x4 *)(zp + ((size_t)p * T + t) * E + 8 * q);
            pa[p][0] = pp[0];
            pa[p][1] = pp[1];
        }
        b0 = *(const f32x4 *)(bias + 8 * q);
        b1 = *(const f32x4 *)(bias + 8 * q + 4);
    }
    pre();
    if (live) {
        float z[8];
        const f32x4 a0 = pa[0][0], a1 = pa[0][1];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            z[r] = a0[r];
            z[r + 4] = a1[r];
        }
#pragma unroll
        for (int p = 1; p < LG_NP; ++p)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                z[r] += pa[p][0][r];
                z[r + 4] += pa[p][1][r];
            }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float sc = __builtin_amdgcn_rcpf(1.0f + __expf(-z[r]));
            Cand x{sc + (r < 4 ? b0[r] : b1[r - 4]), sc, 8 * q + r};
            // insert into the sorted list (drop the last)
#pragma unroll
            for (int j = 0; j < KL; ++j)
                if (cand_before(x, c[j])) {
                    const Cand tmp = c[j];
                    c[j] = x;
                    x = tmp;
                }
        }
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        Cand o[KL];
#pragma unroll
        for (int j = 0; j < KL; ++j) {
            o[j].v = __shfl_xor(c[j].v, m, WAVE);
            o[j].s = __shfl_xor(c[j].s, m, WAVE);
            o[j].i = __shfl_xor(c[j].i, m, WAVE);
        }
#pragma unroll
        for (int j = 0; j < KL; ++j)
            if (cand_before(o[KL - 1 - j], c[j])) c[j] = o[KL - 1 - j];
        // c is now bitonic; sort it (KL <= 4)
        if (KL == 4) {
            cand_sort2(c[0], c[2]);
            cand_sort2(c[1], c[3]);
        }
        if (KL >= 3) {
            cand_sort2(c[0], c[1]);
            cand_sort2(c[KL - 2], c[KL - 1]);
            if (KL == 3) cand_sort2(c[0], c[1]);
        } else {
            cand_sort2(c[0], c[1]);
        }
    }
    if (t < T && q == 0) {
        float ssum = 0.f;
#pragma unroll
        for (int j = 0; j < KL - 1; ++j)
            if (j < k) ssum += c[j].s;
#pragma unroll
        for (int j = 0; j < KL - 1; ++j)
            if (j < k) {
                ids_l[t * k + j] = c[j].i;
                w_l[t * k + j] = c[j].s / ssum;
            }
        if (pub) {
            float nv = -INFINITY, kv = 0.f;
            bool has = false;
#pragma unroll
            for (int j = 0; j < KL; ++j) {
                if (j == k - 1) kv = c[j].v;
                if (j == k) {
                    nv = c[j].v;
                    has = c[j].i != 0x7fffffff;
                }
            }
            gap_g[t] = has ? kv - nv : INFINITY;
        }
    }
}

// ------------------------------------------------------------- pair lists

// Pairs routed to expert e in ascending order -> list (and their tokens ->
// tok); returns the count.
// Called by the whole workgroup; the result is in LDS after the barrier.
__device__ __forceinline__ int gather_pairs(const int32_t *__restrict__ ids, int P, int k, int e, int *list,
                                            int *tok, int *cnt)
{
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < WAVE) {
        int n = 0;
        for (int p0 = 0; p0 < P; p0 += WAVE) {
            const int p = p0 + lane;
            const bool hit = p < P && ids[p] == e;
            const uint64_t m = __ballot(hit);
            if (hit) {
                const int slot = n + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
                list[slot] = p;
                tok[slot] = p / k;
            }
            n += __popcll(m);
        }
        if (lane == 0) *cnt = n;
    }
    __syncthreads();
    return *cnt;
}

// The rank-th active expert (ascending id) of this batch, or -1 when fewer
// experts are active: units of inactive experts never get a workgroup slot
// ahead of active work.  `flags` is E <= 256 ints of LDS.  Whole workgroup.
__device__ __forceinline__ int active_expert(const int32_t *__restrict__ ids, int P, int E, int rank, int *flags,
                                             int *res)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < 256; e += 256) flags[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 256) {
        const int e = ids[p];
        if ((unsigned)e < (unsigned)E) flags[e] = 1;  // every writer stores 1
    }
    __syncthreads();
    if (wave == 0) {
        int before = 0, found = -1;
        for (int e0 = 0; e0 < E; e0 += WAVE) {
            const bool on = (e0 + lane < E) && flags[e0 + lane];
            const uint64_t m = __ballot(on);
            const int cnt = __popcll(m);
            if (found < 0 && rank < before + cnt) {
                const int want = rank - before;
                const bool me = on && __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)))) == want;
                const uint64_t hit = __ballot(me);
                found = e0 + (int)__builtin_ctzll(hit);
            }
            before += cnt;
        }
        if (lane == 0) *res = found;
    }
    __syncthreads();
    return *res;
}

struct DecArgs {
    const uint16_t *x;  // [T][H] bf16
    int T, H, k, E;
    int32_t *ids;        // [T*k] selected experts (written by the first routed gate/up workgroup)
    float *w, *gap;      // [T*k] combine weights, [T] tie gaps (same writer)
    const float *zp;     // [LG_NP][T][E] partial router logits
    const float *rb;     // [E] selection bias
    int n_group, topk_group;
    float rsf;
    int spec;  // routed units map to experts by index and fetch before routing
    // routed experts
    const uint8_t *gq, *uq, *dq;
    const float *gs, *us, *ds;
    int64_t qstride, dqstride, sstride, dsstride;
    int I;
    // shared expert
    const uint8_t *sgq, *suq, *sdq;
    const float *sgs, *sus, *sds;
    int Ish, sh_bits;
    // buffers
    float *h;      // [P][I]
    float *shh;    // [T][Ish]
    float *pscale;  // [P] rsf * w
    float *y;      // [P][H]
    float *shp;    // [Ish/512][T][H]
};

// The routing decision of the batch into LDS (every routed gate/up workgroup
// takes it, from the same logits, so all agree); the publishing workgroup
// also writes ids, w, rsf * w and the tie gaps to global memory.
// `pre` runs once, after the logits are requested and before they are used.
template <int EPL, typename Pre>
__device__ __forceinline__ void dec_route(const DecArgs &r, int T, int E, int k, int32_t *ids_l, float *w_l,
                                          bool pub, Pre &&pre)
{
    const bool grouped = r.n_group > 1 && r.topk_group < r.n_group;
    if (!grouped && E <= 64 && E % 8 == 0 && k <= 3) {
        if (k == 1)
            dec_select_lanes<2>(r.zp, r.rb, T, E, k, ids_l, w_l, pub, r.gap, pre);
        else if (k == 2)
            dec_select_lanes<3>(r.zp, r.rb, T, E, k, ids_l, w_l, pub, r.gap, pre);
        else
            dec_select_lanes<4>(r.zp, r.rb, T, E, k, ids_l, w_l, pub, r.gap, pre);
    } else {
        pre();
        dec_select_waves<EPL>(r.zp, r.rb, T, E, k, r.n_group, r.topk_group, r.rsf, ids_l, w_l, pub, r.gap);
    }
    __syncthreads();
    if (pub)
        for (int i = threadIdx.x; i < T * k; i += 256) {
            r.ids[i] = ids_l[i];
            r.w[i] = w_l[i];
            r.pscale[i] = r.rsf * w_l[i];
        }
}

// ------------------------------------------------------------------ gate/up

template <int CPL>
__device__ __forceinline__ void load_rows(u32x4 (&dst)[CPL], const uint8_t *row)
{
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[c] = *(const u32x4 *)(row + c * 64);
}

// The body of k_dec_gateup for a compile-time number of 16-row blocks (NMB).
// Per super-stage of KS columns: the activation rows are requested first, then
// the wave's whole weight slice, so the activations can be staged in LDS
// (interleaved, row sums taken) while the weights are still streaming in.
constexpr int GU_CPL = 8;  // 16-byte gate/up weight chunks per lane per row per super-stage

template <int WBITS, int NMB>
__device__ __forceinline__ void gateup_body(const DecArgs &a, bool shared, int n, const int *plist, const int *tok,
                                            uint16_t *sA, float *sPart, const uint8_t *grow, const uint8_t *urow,
                                            const u32x4 (&wg0)[GU_CPL], const u32x4 (&wu0)[GU_CPL], float sg,
                                            float su, float *dst, int I, int row)
{
    constexpr int CPL = GU_CPL;
    constexpr int SB = CPL * 64;           // weight bytes of a row per super-stage (512)
    constexpr int KS = SB * 8 / WBITS;     // columns per super-stage (1024 int4, 512 int8)
    constexpr int LDA = KS + 8;
    constexpr int CPR = KS / 8;            // 8-column activation chunks per row
    constexpr int XPT = CPR / 16;          // chunks per thread: a 16-thread group owns one row
    constexpr int NCH = 2;                 // independent accumulator chains per matrix
    static_assert(CPR == 128 || CPR == 64, "a row is 128 or 64 chunks");
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
    f32x4 acc[NMB][2][NCH];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) acc[mb][x][ch] = f32x4{0.f, 0.f, 0.f, 0.f};
    float rsum[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) rsum[mb] = 0.f;
    const int nss = a.H / KS;
    const uint16_t *ap = sA + (lane & 15) * LDA;
    const int rsub = tid >> 4, csub = tid & 15;  // row within a 16-row block, chunk phase
    const uint16_t *xrow[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        const int r = mb * 16 + rsub;
        xrow[mb] = (r < n) ? a.x + (size_t)(shared ? r : tok[r]) * a.H + csub * 8 : nullptr;
    }
    auto load_x = [&](u32x4 (&xr)[XPT], int mb, int ss) {
        if (xrow[mb]) {
#pragma unroll
            for (int j = 0; j < XPT; ++j) xr[j] = *(const u32x4 *)(xrow[mb] + (size_t)ss * KS + j * 128);
        } else {
#pragma unroll
            for (int j = 0; j < XPT; ++j) xr[j] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto stage_x = [&](u32x4 (&xr)[XPT], int mb) {
        uint16_t *dstrow = sA + (mb * 16 + rsub) * LDA + csub * 8;
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            u32x4 v = xr[j];
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d) s += bf16_lo(v[d]) + bf16_hi(v[d]);
            rsum[mb] += s;
            if (WBITS == 4) v = interleave_bf16x8(v);
            *(u32x4 *)(dstrow + j * 128) = v;
        }
    };
    for (int ss = 0; ss < nss; ++ss) {
        u32x4 xr[XPT];
        load_x(xr, 0, ss);
        u32x4 wg[CPL], wu[CPL];
        if (ss == 0) {  // the first super-stage's weights were requested by the caller
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                wg[c] = wg0[c];
                wu[c] = wu0[c];
            }
        } else {
            load_rows<CPL>(wg, grow + (size_t)ss * SB);
            load_rows<CPL>(wu, urow + (size_t)ss * SB);
        }
        if (ss > 0) __syncthreads();  // the previous super-stage's A reads are done
        stage_x(xr, 0);
#pragma unroll
        for (int mb = 1; mb < NMB; ++mb) {
            load_x(xr, mb, ss);
            stage_x(xr, mb);
        }
        if (ss == nss - 1) {
            // row sums: the 16 threads of a row are 16 consecutive lanes
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                float s = rsum[mb];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, WAVE);
                if (csub == 0) sPart[mb * 16 + rsub] = s;
            }
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if constexpr (WBITS == 4) {
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const u32x4 bg = unpack_int4x8(wg[c][wd]);
                    const u32x4 bu = unpack_int4x8(wu[c][wd]);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        const u32x4 af = *(const u32x4 *)(ap + mb * 16 * LDA + (4 * c + g) * 32 + 8 * wd);
                        acc[mb][0][wd % NCH] = mfma_bf16(af, bg, acc[mb][0][wd % NCH]);
                        acc[mb][1][wd % NCH] = mfma_bf16(af, bu, acc[mb][1][wd % NCH]);
                    }
                }
            } else {
#pragma unroll
                for (int wd = 0; wd < 2; ++wd) {
                    const u32x4 bg = unpack_int8x8(u32x2{wg[c][2 * wd], wg[c][2 * wd + 1]});
                    const u32x4 bu = unpack_int8x8(u32x2{wu[c][2 * wd], wu[c][2 * wd + 1]});
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        const u32x4 af = *(const u32x4 *)(ap + mb * 16 * LDA + (4 * c + g) * 16 + 8 * wd);
                        acc[mb][0][wd % NCH] = mfma_bf16(af, bg, acc[mb][0][wd % NCH]);
                        acc[mb][1][wd % NCH] = mfma_bf16(af, bu, acc[mb][1][wd % NCH]);
                    }
                }
            }
        }
    }
    const float bias = (WBITS == 4) ? INT4_BIAS : 0.f;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb * 16 + g * 4 + r;
            if (m >= n) continue;
            const float corr = bias * sPart[m];
            float ga = acc[mb][0][0][r], ua = acc[mb][1][0][r];
#pragma unroll
            for (int ch = 1; ch < NCH; ++ch) {
                ga += acc[mb][0][ch][r];
                ua += acc[mb][1][ch][r];
            }
            const float gv = (ga - corr) * sg;
            const float uv = (ua - corr) * su;
            const int orow = shared ? m : plist[m];
            dst[(size_t)orow * I + row] = fast_silu(gv) * uv;
        }
    }
}

// units: [0, nsh) shared (64 intermediate rows each), then E * (I/64) routed.
// Each wave owns 16 intermediate rows i and streams both their gate and up rows.
// Routed units first take the routing decision for the whole batch (every
// routed workgroup computes the same one from the logits).  With a.spec set
// (a batch expected to touch most experts) routed unit v belongs to expert
// v / (I/64) and requests its first weight stage before routing, so the
// selection overlaps the weight fetch; a unit whose expert nobody chose
// exits.  Otherwise unit v belongs to the (v / (I/64))-th chosen expert in
// ascending id order and fetches after routing (no wasted reads).
template <int WBITS, int EPL>
__global__ __launch_bounds__(256) void k_dec_gateup(DecArgs a)
{
    constexpr int KS = 512 * 8 / WBITS;
    constexpr int LDA = KS + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sA[DEC_MAXT * LDA];
    __shared__ float sPart[DEC_MAXT];
    __shared__ int plist[DEC_MAXT], tok[DEC_MAXT];
    __shared__ int flags[256];
    __shared__ int32_t sIds[DEC_MAXT * DEC_MAXK];
    __shared__ float sW[DEC_MAXT * DEC_MAXK];
    __shared__ int pcnt, ares;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;
    const int nsh = a.sh_bits ? a.Ish / 64 : 0;
    const int u = blockIdx.x;
    const bool shared = u < nsh;
    if ((shared ? a.sh_bits : 4) != WBITS) return;  // the launch instantiates one weight format
    const size_t rbytes = (size_t)a.H * WBITS / 8;
    u32x4 wg0[GU_CPL], wu0[GU_CPL];
    const uint8_t *grow, *urow;
    float sg, su;
    int row;
    auto fetch = [&](const uint8_t *gq, const uint8_t *uq, const float *gsc, const float *usc, int i0) {
        row = i0 + wave * 16 + (lane & 15);
        grow = gq + (size_t)row * rbytes + g * 16;
        urow = uq + (size_t)row * rbytes + g * 16;
        load_rows<GU_CPL>(wg0, grow);
        load_rows<GU_CPL>(wu0, urow);
        sg = gsc[row];
        su = usc[row];
    };
    int n, I;
    float *dst;
    if (shared) {
        fetch(a.sgq, a.suq, a.sgs, a.sus, u * 64);
        n = a.T;
        I = a.Ish;
        dst = a.shh;
    } else {
        const int v = u - nsh, per = a.I / 64;
        int e = v / per;
        dec_route<EPL>(a, a.T, a.E, a.k, sIds, sW, v == 0, [&]() {
            if (a.spec)
                fetch(a.gq + (size_t)e * a.qstride, a.uq + (size_t)e * a.qstride, a.gs + (size_t)e * a.sstride,
                      a.us + (size_t)e * a.sstride, (v % per) * 64);
        });
        if (!a.spec) {
            e = active_expert(sIds, a.T * a.k, a.E, v / per, flags, &ares);
            if (e < 0) return;
            fetch(a.gq + (size_t)e * a.qstride, a.uq + (size_t)e * a.qstride, a.gs + (size_t)e * a.sstride,
                  a.us + (size_t)e * a.sstride, (v % per) * 64);
        }
        n = gather_pairs(sIds, a.T * a.k, a.k, e, plist, tok, &pcnt);
        if (n == 0) return;  // (speculative units only) nobody chose this expert
        I = a.I;
        dst = a.h;
    }
    if (n <= 16)
        gateup_body<WBITS, 1>(a, shared, n, plist, tok, sA, sPart, grow, urow, wg0, wu0, sg, su, dst, I, row);
    else
        gateup_body<WBITS, 2>(a, shared, n, plist, tok, sA, sPart, grow, urow, wg0, wu0, sg, su, dst, I, row);
}

// ------------------------------------------------------------------- down

constexpr int DN_ROWS = 128;  // output rows per down unit (32 per wave)
// 16-byte weight chunks per lane per row of a 512-column unit (4 int4, 8 int8)
constexpr int dn_cpl(int wbits) { return 512 * wbits / 8 / 64; }

// The body of k_dec_down: h rows (f32) are requested first, then the wave's
// weight slice (2 blocks of 16 output rows); h is split into exact hi + lo
// bf16 planes in LDS while the weights stream in.  One 512-column chunk of the
// reduction per unit.
template <int WBITS, int NMB>
__device__ __forceinline__ void down_body(const DecArgs &a, bool shared, int n, const int *plist, uint16_t *sHi,
                                          uint16_t *sLo, float *sPart, const u32x4 (&w0)[dn_cpl(WBITS)],
                                          const u32x4 (&w1)[dn_cpl(WBITS)], const float *hsrc, int hld, int kbeg,
                                          float sd0, float sd1, int row0, int row1)
{
    constexpr int KC = 512;                   // reduction columns per unit
    constexpr int CPL = dn_cpl(WBITS);
    constexpr int LDA = KC + 8;
    constexpr int CPR = KC / 8;               // 64 chunks of 8 columns per row
    constexpr int XPT = NMB * 16 * CPR / 256;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
    f32x4 hv[XPT][2];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
        hv[i][0] = hv[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (r < n) {
            const float *hp = hsrc + (size_t)(shared ? r : plist[r]) * hld + kbeg + cc * 8;
            hv[i][0] = *(const f32x4 *)hp;
            hv[i][1] = *(const f32x4 *)(hp + 4);
        }
    }
    float rsum[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + 256 * i, r = c / CPR, cc = c % CPR;
        u32x4 hi, lo;
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t hb[2], lb[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const float v = hv[i][d / 2][(d % 2) * 2 + e2];
                hb[e2] = f32_to_bf16(v);
                const float hf = __uint_as_float(hb[e2] << 16);
                lb[e2] = f32_to_bf16(v - hf);
                s += hf + __uint_as_float(lb[e2] << 16);
            }
            hi[d] = hb[0] | (hb[1] << 16);
            lo[d] = lb[0] | (lb[1] << 16);
        }
        rsum[i] = s;
        if (WBITS == 4) {
            hi = interleave_bf16x8(hi);
            lo = interleave_bf16x8(lo);
        }
        *(u32x4 *)(sHi + r * LDA + cc * 8) = hi;
        *(u32x4 *)(sLo + r * LDA + cc * 8) = lo;
    }
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        float s = rsum[i];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o, WAVE);
        const int c = tid + 256 * i, r = c / CPR;
        if ((c % CPR) == 0) sPart[r] = s;
    }
    __syncthreads();
    // chains: [row block 0/1][hi/lo plane]
    f32x4 acc[NMB][2][2];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int x = 0; x < 2; ++x) acc[mb][x][0] = acc[mb][x][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *ah = sHi + (lane & 15) * LDA, *al = sLo + (lane & 15) * LDA;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if constexpr (WBITS == 4) {
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                const u32x4 b0 = unpack_int4x8(w0[c][wd]);
                const u32x4 b1 = unpack_int4x8(w1[c][wd]);
                const int ko = (4 * c + g) * 32 + 8 * wd;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const u32x4 fh = *(const u32x4 *)(ah + mb * 16 * LDA + ko);
                    const u32x4 fl = *(const u32x4 *)(al + mb * 16 * LDA + ko);
                    acc[mb][0][0] = mfma_bf16(fh, b0, acc[mb][0][0]);
                    acc[mb][1][0] = mfma_bf16(fh, b1, acc[mb][1][0]);
                    acc[mb][0][1] = mfma_bf16(fl, b0, acc[mb][0][1]);
                    acc[mb][1][1] = mfma_bf16(fl, b1, acc[mb][1][1]);
                }
            }
        } else {
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
                const u32x4 b0 = unpack_int8x8(u32x2{w0[c][2 * wd], w0[c][2 * wd + 1]});
                const u32x4 b1 = unpack_int8x8(u32x2{w1[c][2 * wd], w1[c][2 * wd + 1]});
                const int ko = (4 * c + g) * 16 + 8 * wd;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const u32x4 fh = *(const u32x4 *)(ah + mb * 16 * LDA + ko);
                    const u32x4 fl = *(const u32x4 *)(al + mb * 16 * LDA + ko);
                    acc[mb][0][0] = mfma_bf16(fh, b0, acc[mb][0][0]);
                    acc[mb][1][0] = mfma_bf16(fh, b1, acc[mb][1][0]);
                    acc[mb][0][1] = mfma_bf16(fl, b0, acc[mb][0][1]);
                    acc[mb][1][1] = mfma_bf16(fl, b1, acc[mb][1][1]);
                }
            }
        }
    }
    const float bias = (WBITS == 4) ? INT4_BIAS : 0.f;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb * 16 + g * 4 + r;
            if (m >= n) continue;
            const float corr = bias * sPart[m];
            const float v0 = (acc[mb][0][0][r] + acc[mb][0][1][r] - corr) * sd0;
            const float v1 = (acc[mb][1][0][r] + acc[mb][1][1][r] - corr) * sd1;
            if (shared) {
                float *o = a.shp + ((size_t)(kbeg / KC) * a.T + m) * a.H;
                o[row0] = v0;
                o[row1] = v1;
            } else {
                const int p = plist[m];
                const float ps = a.pscale[p];
                float *o = a.y + ((size_t)(kbeg / KC) * a.T * a.k + p) * a.H;
                o[row0] = v0 * ps;
                o[row1] = v1 * ps;
            }
        }
    }
}

// units: [0, nsh) shared (128 output rows x one 512-column chunk of Ish), then
// routed (expert, 128 output rows, one 512-column chunk of I).  The expert of
// a routed unit is its index / units-per-expert with a.spec set (weights are
// requested before the routing is read; units of unchosen experts exit),
// else the chosen expert of that rank in ascending id order.
template <int WBITS>
__global__ __launch_bounds__(256) void k_dec_down(DecArgs a)
{
    constexpr int LDA = 512 + 8;
    constexpr int CPL = dn_cpl(WBITS);
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][DEC_MAXT * LDA];  // hi, lo planes
    __shared__ float sPart[DEC_MAXT];
    __shared__ int plist[DEC_MAXT], tok[DEC_MAXT];
    __shared__ int flags[256];
    __shared__ int pcnt, ares;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;
    const int nkc = a.sh_bits ? a.Ish / 512 : 0;
    const int nsh = nkc * (a.H / DN_ROWS);
    const int u = blockIdx.x;
    const bool shared = u < nsh;
    if ((shared ? a.sh_bits : 4) != WBITS) return;
    u32x4 w0[CPL], w1[CPL];
    float sd0, sd1;
    int row0, row1;
    auto fetch = [&](const uint8_t *dq, const float *dsc, int K, int c0, int kbeg) {
        row0 = c0 + wave * 32 + (lane & 15);
        row1 = row0 + 16;
        const size_t rbytes = (size_t)K * WBITS / 8;
        const uint8_t *drow0 = dq + (size_t)row0 * rbytes + (size_t)kbeg * WBITS / 8 + g * 16;
        load_rows<CPL>(w0, drow0);
        load_rows<CPL>(w1, drow0 + 16 * rbytes);
        sd0 = dsc[row0];
        sd1 = dsc[row1];
    };
    int n, kbeg, hld;
    const float *hsrc;
    if (shared) {
        const int kc = u % nkc;
        kbeg = kc * 512;
        fetch(a.sdq, a.sds, a.Ish, (u / nkc) * DN_ROWS, kbeg);
        n = a.T;
        hsrc = a.shh;
        hld = a.Ish;
    } else {
        const int nkr = a.I / 512;
        const int v = u - nsh, per = (a.H / DN_ROWS) * nkr;
        const int c0 = ((v % per) / nkr) * DN_ROWS;
        kbeg = ((v % per) % nkr) * 512;
        int e = v / per;
        if (a.spec) {
            fetch(a.dq + (size_t)e * a.dqstride, a.ds + (size_t)e * a.dsstride, a.I, c0, kbeg);
        } else {
            e = active_expert(a.ids, a.T * a.k, a.E, v / per, flags, &ares);
            if (e < 0) return;
            fetch(a.dq + (size_t)e * a.dqstride, a.ds + (size_t)e * a.dsstride, a.I, c0, kbeg);
        }
        n = gather_pairs(a.ids, a.T * a.k, a.k, e, plist, tok, &pcnt);
        if (n == 0) return;  // (speculative units only) nobody chose this expert
        hsrc = a.h;
        hld = a.I;
    }
    if (n <= 16)
        down_body<WBITS, 1>(a, shared, n, plist, sA[0], sA[1], sPart, w0, w1, hsrc, hld, kbeg, sd0, sd1, row0, row1);
    else
        down_body<WBITS, 2>(a, shared, n, plist, sA[0], sA[1], sPart, w0, w1, hsrc, hld, kbeg, sd0, sd1, row0, row1);
}

// ---------------------------------------------------------------- combine

__global__ __launch_bounds__(256) void k_dec_combine(const float *__restrict__ y, int nkr, const float *__restrict__ shp,
                                                     int nkc, const uint16_t *__restrict__ res, void *__restrict__ out,
                                                     int T, int H, int k, int out_f32)
{
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int cpt = H / 4;
    if (idx >= (long)T * cpt) return;
    const int t = (int)(idx / cpt);
    const int c = (int)(idx % cpt) * 4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j)
        for (int kr = 0; kr < nkr; ++kr) {
            const f32x4 v = *(const f32x4 *)(y + (((size_t)kr * T + t) * k + j) * H + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += v[i];
        }
    for (int kc = 0; kc < nkc; ++kc) {
        const f32x4 v = *(const f32x4 *)(shp + ((size_t)kc * T + t) * H + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += v[i];
    }
    if (res) {
        const u32x2 v = *(const u32x2 *)(res + (size_t)t * H + c);
        acc[0] += bf16_lo(v[0]);
        acc[1] += bf16_hi(v[0]);
        acc[2] += bf16_lo(v[1]);
        acc[3] += bf16_hi(v[1]);
    }
    if (out_f32) {
        *(f32x4 *)((float *)out + (size_t)t * H + c) = acc;
    } else {
        *(u32x2 *)((uint16_t *)out + (size_t)t * H + c) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    }
}

// ---------------------------------------------------------------- launcher

bool decode_supported(int T, int H, int E, int k, int I, int Ish, int sh_bits)
{
    if (T > DEC_MAXT || E > 256 || k > DEC_MAXK) return false;
    if (H % 1024 || I % 512) return false;
    if (sh_bits && Ish % 512) return false;
    return true;
}

hipError_t launch_decode(const DecLaunch &d, hipStream_t st)
{
    DecArgs a;
    a.x = d.x;
    a.T = d.T;
    a.H = d.H;
    a.k = d.k;
    a.E = d.E;
    a.ids = d.ids;
    a.w = d.w;
    a.gap = d.gap;
    a.zp = d.z;
    a.rb = d.rb;
    a.n_group = d.n_group;
    a.topk_group = d.topk_group;
    a.rsf = d.rsf;
    a.spec = 0;
    a.gq = d.gq;
    a.uq = d.uq;
    a.dq = d.dq;
    a.gs = d.gs;
    a.us = d.us;
    a.ds = d.ds;
    a.qstride = d.qstride;
    a.dqstride = d.dqstride;
    a.sstride = d.sstride;
    a.dsstride = d.dsstride;
    a.I = d.I;
    a.sgq = d.sgq;
    a.suq = d.suq;
    a.sdq = d.sdq;
    a.sgs = d.sgs;
    a.sus = d.sus;
    a.sds = d.sds;
    a.Ish = d.Ish;
    a.sh_bits = d.sh_bits;
    a.h = d.h;
    a.shh = d.shh;
    a.pscale = d.pscale;
    a.y = d.y;
    a.shp = d.shp;

    {
        const int grid = ((d.E + 15) / 16) * ((d.T + 15) / 16) * LG_NP;
        hipLaunchKernelGGL(k_dec_logits, dim3(grid), dim3(256), 0, st, d.x, d.rw, d.T, d.H, d.E, d.z);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // gate/up: the int8 shared expert needs its own instantiation
    const int nsh_gu = d.sh_bits ? d.Ish / 64 : 0;
    const int ngu = nsh_gu + d.E * (d.I / 64);
    if (d.ev0) {
        e = hipEventRecord(d.ev0, st);
        if (e != hipSuccess) return e;
    }
    if (d.sh_bits == 8) hipLaunchKernelGGL((k_dec_gateup<8, 1>), dim3(nsh_gu), dim3(256), 0, st, a);
    if (d.E <= 64)
        hipLaunchKernelGGL((k_dec_gateup<4, 1>), dim3(ngu), dim3(256), 0, st, a);
    else if (d.E <= 128)
        hipLaunchKernelGGL((k_dec_gateup<4, 2>), dim3(ngu), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_dec_gateup<4, 4>), dim3(ngu), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e == hipSuccess && d.ev1) e = hipEventRecord(d.ev1, st);
    if (e != hipSuccess) return e;
    const int nkc = d.sh_bits ? d.Ish / 512 : 0;
    const int nkr = d.I / 512;
    const int nsh_d = nkc * (d.H / DN_ROWS);
    const int nd = nsh_d + d.E * (d.H / DN_ROWS) * nkr;
    if (d.sh_bits == 8) {
        hipLaunchKernelGGL(k_dec_down<8>, dim3(nsh_d), dim3(256), 0, st, a);
        hipLaunchKernelGGL(k_dec_down<4>, dim3(nd), dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL(k_dec_down<4>, dim3(nd), dim3(256), 0, st, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long nthreads = (long)d.T * (d.H / 4);
    hipLaunchKernelGGL(k_dec_combine, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, st, d.y, nkr, d.shp,
                       nkc, d.res, d.out, d.T, d.H, d.k, d.out_f32);
    return hipGetLastError();
}

}  // namespace moe

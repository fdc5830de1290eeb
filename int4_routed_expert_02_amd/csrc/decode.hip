// decode.hip -- the small-batch regime: a layer whose batch routes only a few
// rows to each expert is a weight stream, bound by HBM, not by the matrix cores.
//
// The engine chooses kernels per shape by measurement (colibri README, "What's
// implemented", integer-dot kernels: the single-row int4 case takes a
// different path from the batched one).  Here, for T <= 32 tokens:
//   k_dec_route    one workgroup per token: logits (f32 FMA), sigmoid + bias,
//                  top-k (moe_select.h), weights and rsf * w per pair;
//   k_dec_gateup   one workgroup per (expert, 64 intermediate rows): gathers
//                  the pairs routed to its expert (batch-union: the expert's
//                  rows are read once for all of them), streams its gate and up
//                  rows straight from HBM into registers, MFMA on 16-pair
//                  blocks, SwiGLU epilogue -> h [pair][I] f32;  the shared
//                  expert's rows form extra units over all T tokens;
//   k_dec_down     one workgroup per (expert, 64 output rows, 512-column chunk
//                  of the reduction): h as an exact hi + lo bf16 pair, down rows
//                  streamed to registers, epilogue scales by sd * rsf * w ->
//                  partial y [chunk][pair][H];  the shared expert's units are
//                  (64 output rows, 512-column chunk) over all T tokens;
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

template <int EPL>
__global__ __launch_bounds__(256) void k_dec_route(const uint16_t *__restrict__ x, const float *__restrict__ W,
                                                   const float *__restrict__ bias, int T, int H, int E, int k,
                                                   int n_group, int topk_group, float rsf, int32_t *__restrict__ ids,
                                                   float *__restrict__ w, float *__restrict__ gap,
                                                   float *__restrict__ pscale)
{
    extern __shared__ float xs[];  // H floats
    __shared__ float zs[256];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid * 8; i < H; i += 256 * 8) {
        const u32x4 v = *(const u32x4 *)(x + (size_t)t * H + i);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            xs[i + 2 * d] = bf16_lo(v[d]);
            xs[i + 2 * d + 1] = bf16_hi(v[d]);
        }
    }
    __syncthreads();
    // Q consecutive threads share one expert's dot product; thread q takes the
    // float4 columns q, q + Q, q + 2Q, ...  Eight loads are kept in flight and
    // four partial sums interleaved, then combined in a fixed order.
    int Q = 64;
    while (Q > 1 && Q * E > 256) Q >>= 1;
    const int q = tid % Q;
    const int nper = H / 4 / Q;  // float4 columns per thread
    const f32x4 *x4 = (const f32x4 *)xs;
    for (int e = tid / Q; e < E; e += 256 / Q) {
        const f32x4 *w4 = (const f32x4 *)(W + (size_t)e * H) + q;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        int i = 0;
        for (; i + 8 <= nper; i += 8) {
            f32x4 wv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) wv[u] = w4[(size_t)(i + u) * Q];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const f32x4 xv = x4[q + (i + u) * Q];
                float &ac = acc[u & 3];
                ac = fmaf(wv[u][0], xv[0], ac);
                ac = fmaf(wv[u][1], xv[1], ac);
                ac = fmaf(wv[u][2], xv[2], ac);
                ac = fmaf(wv[u][3], xv[3], ac);
            }
        }
        for (; i < nper; ++i) {
            const f32x4 wv = w4[(size_t)i * Q];
            const f32x4 xv = x4[q + i * Q];
            acc[0] = fmaf(wv[0], xv[0], acc[0]);
            acc[0] = fmaf(wv[1], xv[1], acc[0]);
            acc[0] = fmaf(wv[2], xv[2], acc[0]);
            acc[0] = fmaf(wv[3], xv[3], acc[0]);
        }
        float tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        for (int o = Q / 2; o > 0; o >>= 1) tot += __shfl_xor(tot, o, WAVE);
        if (q == 0) zs[e] = tot;
    }
    __syncthreads();
    if (wave == 0) {
        float s[EPL], b[EPL];
        bool ok[EPL];
#pragma unroll
        for (int qq = 0; qq < EPL; ++qq) {
            const int e = lane * EPL + qq;
            ok[qq] = e < E;
            s[qq] = 0.f;
            b[qq] = -INFINITY;
            if (ok[qq]) {
                s[qq] = 1.0f / (1.0f + expf(-zs[e]));
                b[qq] = s[qq] + bias[e];
            }
        }
        select_token<EPL>(s, b, ok, lane, t, E, k, n_group, topk_group, rsf, ids, w, gap, pscale, nullptr);
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
    for (int p = tid; p < P; p += 256) flags[ids[p]] = 1;  // every writer stores 1
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
    const int32_t *ids;  // [T*k]
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
    const float *pscale;  // [P]
    float *y;      // [P][H]
    float *shp;    // [Ish/512][T][H]
};

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
template <int WBITS, int NMB>
__device__ __forceinline__ void gateup_body(const DecArgs &a, bool shared, int n, const int *plist, const int *tok,
                                            uint16_t *sA,
                                            float *sPart, const uint8_t *grow, const uint8_t *urow, float sg,
                                            float su, float *dst, int I, int row)
{
    constexpr int CPL = 8;                 // 16-byte weight chunks per lane per row per super-stage
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
        load_rows<CPL>(wg, grow + (size_t)ss * SB);
        load_rows<CPL>(wu, urow + (size_t)ss * SB);
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
template <int WBITS>
__global__ __launch_bounds__(256) void k_dec_gateup(DecArgs a)
{
    constexpr int KS = 512 * 8 / WBITS;
    constexpr int LDA = KS + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sA[DEC_MAXT * LDA];
    __shared__ float sPart[DEC_MAXT];
    __shared__ int plist[DEC_MAXT], tok[DEC_MAXT];
    __shared__ int flags[256];
    __shared__ int pcnt, ares;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nsh = a.sh_bits ? a.Ish / 64 : 0;
    const int u = blockIdx.x;
    const bool shared = u < nsh;
    int i0, n, I, wb;
    const uint8_t *gq, *uq;
    const float *gsc, *usc;
    float *dst;
    if (shared) {
        i0 = u * 64;
        n = a.T;
        I = a.Ish;
        wb = a.sh_bits;
        gq = a.sgq;
        uq = a.suq;
        gsc = a.sgs;
        usc = a.sus;
        dst = a.shh;
    } else {
        const int v = u - nsh, per = a.I / 64;
        const int e = active_expert(a.ids, a.T * a.k, a.E, v / per, flags, &ares);
        if (e < 0) return;
        i0 = (v % per) * 64;
        I = a.I;
        wb = 4;
        n = gather_pairs(a.ids, a.T * a.k, a.k, e, plist, tok, &pcnt);
        gq = a.gq + (size_t)e * a.qstride;
        uq = a.uq + (size_t)e * a.qstride;
        gsc = a.gs + (size_t)e * a.sstride;
        usc = a.us + (size_t)e * a.sstride;
        dst = a.h;
    }
    if (wb != WBITS) return;  // the launch instantiates one weight format
    const int row = i0 + wave * 16 + (lane & 15);
    const int g = lane >> 4;
    const size_t rbytes = (size_t)a.H * WBITS / 8;
    const uint8_t *grow = gq + (size_t)row * rbytes + g * 16;
    const uint8_t *urow = uq + (size_t)row * rbytes + g * 16;
    const float sg = gsc[row], su = usc[row];
    if (n <= 16)
        gateup_body<WBITS, 1>(a, shared, n, plist, tok, sA, sPart, grow, urow, sg, su, dst, I, row);
    else
        gateup_body<WBITS, 2>(a, shared, n, plist, tok, sA, sPart, grow, urow, sg, su, dst, I, row);
}

// ------------------------------------------------------------------- down

constexpr int DN_ROWS = 128;  // output rows per down unit (32 per wave)

// The body of k_dec_down: h rows (f32) are requested first, then the wave's
// weight slice (2 blocks of 16 output rows); h is split into exact hi + lo
// bf16 planes in LDS while the weights stream in.  One 512-column chunk of the
// reduction per unit.
template <int WBITS, int NMB>
__device__ __forceinline__ void down_body(const DecArgs &a, bool shared, int n, const int *plist, uint16_t *sHi,
                                          uint16_t *sLo, float *sPart, const uint8_t *drow0,
                                          const uint8_t *drow1, const float *hsrc, int hld, int kbeg, float sd0,
                                          float sd1, int row0, int row1)
{
    constexpr int KC = 512;                   // reduction columns per unit
    constexpr int CPL = KC * WBITS / 8 / 64;  // weight chunks per lane per row (4 int4, 8 int8)
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
    u32x4 w0[CPL], w1[CPL];
    load_rows<CPL>(w0, drow0);
    load_rows<CPL>(w1, drow1);
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
// routed (active expert rank, 128 output rows, one 512-column chunk of I).
template <int WBITS>
__global__ __launch_bounds__(256) void k_dec_down(DecArgs a)
{
    constexpr int LDA = 512 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][DEC_MAXT * LDA];  // hi, lo planes
    __shared__ float sPart[DEC_MAXT];
    __shared__ int plist[DEC_MAXT], tok[DEC_MAXT];
    __shared__ int flags[256];
    __shared__ int pcnt, ares;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nkc = a.sh_bits ? a.Ish / 512 : 0;
    const int nsh = nkc * (a.H / DN_ROWS);
    const int u = blockIdx.x;
    const bool shared = u < nsh;
    int n, K, kbeg, wbits, c0;
    const uint8_t *dq;
    const float *dsc;
    const float *hsrc;
    int hld;
    if (shared) {
        const int kc = u % nkc;
        c0 = (u / nkc) * DN_ROWS;
        n = a.T;
        K = a.Ish;
        kbeg = kc * 512;
        wbits = a.sh_bits;
        dq = a.sdq;
        dsc = a.sds;
        hsrc = a.shh;
        hld = a.Ish;
    } else {
        const int nkr = a.I / 512;
        const int v = u - nsh, per = (a.H / DN_ROWS) * nkr;
        const int e = active_expert(a.ids, a.T * a.k, a.E, v / per, flags, &ares);
        if (e < 0) return;
        c0 = ((v % per) / nkr) * DN_ROWS;
        kbeg = ((v % per) % nkr) * 512;
        K = a.I;
        wbits = 4;
        n = gather_pairs(a.ids, a.T * a.k, a.k, e, plist, tok, &pcnt);
        dq = a.dq + (size_t)e * a.dqstride;
        dsc = a.ds + (size_t)e * a.dsstride;
        hsrc = a.h;
        hld = a.I;
    }
    if (wbits != WBITS) return;
    const int row0 = c0 + wave * 32 + (lane & 15), row1 = row0 + 16;
    const int g = lane >> 4;
    const size_t rbytes = (size_t)K * WBITS / 8;
    const uint8_t *drow0 = dq + (size_t)row0 * rbytes + (size_t)kbeg * WBITS / 8 + g * 16;
    const uint8_t *drow1 = drow0 + 16 * rbytes;
    const float sd0 = dsc[row0], sd1 = dsc[row1];
    if (n <= 16)
        down_body<WBITS, 1>(a, shared, n, plist, sA[0], sA[1], sPart, drow0, drow1, hsrc, hld, kbeg, sd0, sd1, row0,
                            row1);
    else
        down_body<WBITS, 2>(a, shared, n, plist, sA[0], sA[1], sPart, drow0, drow1, hsrc, hld, kbeg, sd0, sd1, row0,
                            row1);
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
    if (T > DEC_MAXT || E > 256) return false;
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

    const size_t lds_route = (size_t)d.H * sizeof(float);
    if (d.E <= 64)
        hipLaunchKernelGGL(k_dec_route<1>, dim3(d.T), dim3(256), lds_route, st, d.x, d.rw, d.rb, d.T, d.H, d.E, d.k,
                           d.n_group, d.topk_group, d.rsf, d.ids, d.w, d.gap, d.pscale);
    else if (d.E <= 128)
        hipLaunchKernelGGL(k_dec_route<2>, dim3(d.T), dim3(256), lds_route, st, d.x, d.rw, d.rb, d.T, d.H, d.E, d.k,
                           d.n_group, d.topk_group, d.rsf, d.ids, d.w, d.gap, d.pscale);
    else
        hipLaunchKernelGGL(k_dec_route<4>, dim3(d.T), dim3(256), lds_route, st, d.x, d.rw, d.rb, d.T, d.H, d.E, d.k,
                           d.n_group, d.topk_group, d.rsf, d.ids, d.w, d.gap, d.pscale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // gate/up: the int8 shared expert needs its own instantiation
    const int nsh_gu = d.sh_bits ? d.Ish / 64 : 0;
    const int ngu = nsh_gu + d.E * (d.I / 64);
    if (d.ev0) {
        e = hipEventRecord(d.ev0, st);
        if (e != hipSuccess) return e;
    }
    if (d.sh_bits == 8) {
        hipLaunchKernelGGL(k_dec_gateup<8>, dim3(nsh_gu), dim3(256), 0, st, a);
        hipLaunchKernelGGL(k_dec_gateup<4>, dim3(ngu), dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL(k_dec_gateup<4>, dim3(ngu), dim3(256), 0, st, a);
    }
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

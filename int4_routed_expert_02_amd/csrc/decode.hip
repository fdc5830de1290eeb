// decode.hip -- the small-batch regime: a layer whose batch routes only a few
// rows to each expert is a weight stream, bound by HBM, not by the matrix cores.
//
// The engine chooses kernels per shape by measurement (colibri README, "What's
// implemented", integer-dot kernels: the single-row int4 case takes a
// different path from the batched one).  Here, for T <= 32 tokens:
//   k_dec_logits          router logits z = x W^T (exact split-bf16 MFMA) as 4
//                         partial planes;
//   k_dec_expert          one workgroup per unit of 128 intermediate rows of a
//                         chosen expert (or of the shared expert): routed units
//                         first take the routing decision of the batch from
//                         the logits (every unit computes the same; the first
//                         publishes ids, weights and rsf * w), find their
//                         expert (the rank-th chosen one) and its pairs, then
//                         stream gate/up rows into registers a few chunks
//                         ahead of the MFMAs (16-pair blocks), SwiGLU -> h on
//                         chip in f16, and the down slice (all output rows x
//                         the unit's 128 columns) on f16 MFMA -> one f32
//                         partial output plane per unit, scaled by the down
//                         row scale and rsf * w;
//   k_dec_combine         out = the partial planes summed in a fixed order
//                         (+ x);
//   k_dec_combine_logits  the same, plus the next layer's router logits of
//                         the row it writes (stacked layers).
// Buffers are indexed by pair, so no permutation is materialised: each
// workgroup finds its expert's pairs by scanning the ids in ascending order.
//
// Weight loads: a wave owns 16 weight rows; lane (n = lane % 16, g = lane / 16)
// loads 16-byte chunks (4c + g) of row n, c = 0..CPL-1, so the four lane
// groups read 64 contiguous bytes of each row per instruction.  The k-slots
// of chunk c, word w for lane group g are k = (4c + g) * 32 + 8w + [0, 8)
// (int4), and the A fragments are read from LDS at the same k.
#include <type_traits>

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
                                              int E, int k, int n_group, int topk_group, float rsf, float top_p,
                                              int32_t *ids_l, float *w_l, bool pub, float *__restrict__ gap_g)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = blockDim.x / WAVE;
    for (int t = wave; t < T; t += nw) {
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
                          nullptr, nullptr, top_p);
    }
}

// Selection order as one 64-bit key: the score's bits made monotone in the
// float order (-0 taken as +0, NaN below everything), then the complement of
// the id, so a larger key is a larger score or, at equal scores, a lower id.
// Key 0 marks an empty or taken slot.
__device__ __forceinline__ uint64_t sel_key(float v, int id)
{
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0;
    uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    if (v != v) o = 0;
    return ((uint64_t)o << 32) | (0xFFFFFFFFu - (uint32_t)id);
}

// Data-parallel-primitive lane moves (no LDS round trip): DPP_X1 and DPP_X2
// swap lanes within each group of four (xor 1, xor 2), DPP_HM mirrors each
// half-row of eight (lane i <-> 7 - i), DPP_RM each row of sixteen.
constexpr int DPP_X1 = 0xB1, DPP_X2 = 0x4E, DPP_HM = 0x141, DPP_RM = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x)
{
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(x >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)x);
}

// maximum / bitwise or over each group of eight lanes, in every lane of it
__device__ __forceinline__ uint64_t max8_u64(uint64_t b)
{
    uint64_t x = dpp_u64<DPP_X1>(b);
    b = x > b ? x : b;
    x = dpp_u64<DPP_X2>(b);
    b = x > b ? x : b;
    x = dpp_u64<DPP_HM>(b);
    return x > b ? x : b;
}

__device__ __forceinline__ uint32_t or8_u32(uint32_t b)
{
    b |= dpp_u32<DPP_X1>(b);
    b |= dpp_u32<DPP_X2>(b);
    return b | dpp_u32<DPP_HM>(b);
}

// Fast selection when no group limit applies, E <= 64, E % 8 == 0 and
// k < KL: eight lanes per token (lane slice q holds experts 8q .. 8q + 7).
// KL rounds, each taking the best remaining key of the token: a lane's best
// of its eight, the maximum over the token's eight lanes, and the owner lane
// retires the winner.  Rounds 0 .. k-1 are the selection in order; round k
// gives the tie gap v_{k-1} - v_k.  The weight of selection j is s_j over the
// sum of the selected s (summed in selection order).  Same results as
// moe_select.h.  Waves holding no token skip the work.
template <int KL>
__device__ __forceinline__ void dec_select_lanes(const float *__restrict__ zp, const float *__restrict__ bias, int T,
                                                 int E, int k, float top_p, int32_t *ids_l, float *w_l, bool pub,
                                                 float *__restrict__ gap_g)
{
    const int tid = threadIdx.x, t = tid >> 3, q = tid & 7;
    if (__builtin_amdgcn_readfirstlane(tid >> 6) * 8 >= T) return;  // (wave-uniform)
    const bool live = t < T && 8 * q < E;
    uint64_t key[8];
    float sv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        key[r] = 0;
        sv[r] = 0.f;
    }
    if (live) {
        f32x4 pa[LG_NP][2];
#pragma unroll
        for (int p = 0; p < LG_NP; ++p) {
            const float *pz = zp + ((size_t)p * T + t) * E + 8 * q;
            pa[p][0] = *(const f32x4 *)pz;
            pa[p][1] = *(const f32x4 *)(pz + 4);
        }
        const f32x4 b0 = *(const f32x4 *)(bias + 8 * q), b1 = *(const f32x4 *)(bias + 8 * q + 4);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            float z = r < 4 ? pa[0][0][r] : pa[0][1][r - 4];
#pragma unroll
            for (int p = 1; p < LG_NP; ++p) z += r < 4 ? pa[p][0][r] : pa[p][1][r - 4];
            const float sc = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
            sv[r] = sc;
            key[r] = sel_key(sc + (r < 4 ? b0[r] : b1[r - 4]), 8 * q + r);
        }
    }
    int sid[KL];
    float ss[KL], vv[KL];
    bool has = true;
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        uint64_t b = key[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) b = key[r] > b ? key[r] : b;
        b = max8_u64(b);
        const int id = (int)(0xFFFFFFFFu - (uint32_t)b);
        uint32_t mine = 0;  // the winner's s from its owner lane (the others give 0 bits)
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (b != 0 && 8 * q + r == id) {
                mine = __float_as_uint(sv[r]);
                key[r] = 0;
            }
        ss[j] = __uint_as_float(or8_u32(mine));
        sid[j] = id;
        // the score of the key: invert the monotone map
        const uint32_t o = (uint32_t)(b >> 32);
        vv[j] = __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
        if (j == k) has = b != 0;
    }
    if (t < T && q == 0) {
        float ssum = 0.f;
#pragma unroll
        for (int j = 0; j < KL - 1; ++j)
            if (j < k) ssum += ss[j];
        float wj[KL - 1];
        bool keep[KL - 1];
#pragma unroll
        for (int j = 0; j < KL - 1; ++j) {
            wj[j] = j < k ? ss[j] / ssum : 0.f;
            keep[j] = j < k;
        }
        if (top_p > 0.f && top_p < 1.f) {
            // adaptive expert top-p, as in moe_select.h: rank by weight (equal
            // weights, lower id first), keep while the f32 running mass in rank
            // order is below p, renormalise over the kept scores
            int rank[KL - 1];
#pragma unroll
            for (int j = 0; j < KL - 1; ++j) {
                rank[j] = 0;
#pragma unroll
                for (int i = 0; i < KL - 1; ++i)
                    if (i < k && j < k && i != j && (wj[i] > wj[j] || (wj[i] == wj[j] && sid[i] < sid[j])))
                        ++rank[j];
            }
            float mass = 0.f, ks = 0.f;
#pragma unroll
            for (int r = 0; r < KL - 1; ++r)
#pragma unroll
                for (int j = 0; j < KL - 1; ++j)
                    if (j < k && rank[j] == r) {
                        keep[j] = mass < top_p;
                        mass += wj[j];
                        if (keep[j]) ks += ss[j];
                    }
#pragma unroll
            for (int j = 0; j < KL - 1; ++j) wj[j] = keep[j] ? ss[j] / ks : 0.f;
        }
#pragma unroll
        for (int j = 0; j < KL - 1; ++j)
            if (j < k) {
                ids_l[t * k + j] = keep[j] ? sid[j] : -1;
                w_l[t * k + j] = wj[j];
            }
        if (pub) {
            float nv = -INFINITY, kv = 0.f;
#pragma unroll
            for (int j = 0; j < KL; ++j) {
                if (j == k - 1) kv = vv[j];
                if (j == k) nv = vv[j];
            }
            gap_g[t] = has ? kv - nv : INFINITY;
        }
    }
}

// ------------------------------------------------------------- pair lists

// A unit's pair rows, one per lane: lane s < n holds pair row s (its pair
// index, token and output scale); other lanes hold pair 0, token 0, scale 0.
struct PairRows {
    int pair, tok;
    float psc;
};

// Every wave on its own (no LDS table, no barrier): the rank-th chosen
// expert of the batch (ascending id) from the ids in LDS, and the pairs
// routed to it in ascending order, compacted into lanes.  The chosen set is
// an or over the pairs of one-hot words (EW words of 64 experts), reduced
// within rows of sixteen lanes by lane moves and across the four rows in
// scalar registers.  Returns the expert (-1 when fewer experts are chosen)
// and the pair count, both wave-uniform.
template <int EW>
__device__ __forceinline__ int2 dec_locate_wave(const int32_t *ids, int P, int k, int E, int rank, PairRows &pr)
{
    constexpr int MAXC = DEC_MAXT * DEC_MAXK / WAVE;  // 64-pair chunks of the batch
    const int lane = threadIdx.x & 63;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes below this one
    // every chunk's ids read once, kept in registers
    int ev[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int p = c * WAVE + lane;
        ev[c] = c * WAVE < P && p < P ? ids[p] : -1;
    }
    uint32_t m[2 * EW];
#pragma unroll
    for (int w = 0; w < 2 * EW; ++w) m[w] = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int w = 0; w < 2 * EW; ++w)
            if ((unsigned)(ev[c] - 32 * w) < 32u && ev[c] < E) m[w] |= 1u << (ev[c] - 32 * w);
    int found = -1, before = 0;
#pragma unroll
    for (int w = 0; w < EW; ++w) {
        uint64_t mw = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t x = or8_u32(m[2 * w + h]);
            x |= dpp_u32<DPP_RM>(x);
            const uint32_t r = __builtin_amdgcn_readlane(x, 0) | __builtin_amdgcn_readlane(x, 16) |
                               __builtin_amdgcn_readlane(x, 32) | __builtin_amdgcn_readlane(x, 48);
            mw |= (uint64_t)r << (32 * h);
        }
        const int cnt = __popcll(mw);
        if (found < 0 && rank < before + cnt) {
            const bool me = ((mw >> lane) & 1ull) && __popcll(mw & lt) == rank - before;
            found = 64 * w + (int)__builtin_ctzll(__ballot(me));
        }
        before += cnt;
    }
    found = __builtin_amdgcn_readfirstlane(found);
    int n = 0;
    pr = PairRows{0, 0, 0.f};
    if (found >= 0) {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            if (c * WAVE >= P) break;
            const int p = c * WAVE + lane;
            const bool hit = ev[c] == found;
            const uint64_t bm = __ballot(hit);
            // forward permute: a hit lane sends its pair to lane n + (hits below it);
            // the others to lane 63, which no pair row reaches (n <= T <= 32)
            const int dst = hit ? n + __popcll(bm & lt) : 63;
            const int got = __builtin_amdgcn_ds_permute(dst * 4, p);
            const int cn = __popcll(bm);
            if (lane >= n && lane < n + cn) pr.pair = got;
            n += cn;
        }
        if (lane < n) pr.tok = pr.pair / k;
    }
    return int2{found, n};
}

struct DecArgs {
    const uint16_t *x;  // [T][H] bf16
    int T, H, k, E;
    int32_t *ids;        // [T*k] selected experts (written by the first routed workgroup)
    float *w, *gap;      // [T*k] combine weights, [T] tie gaps (same writer)
    float *pscale;       // [T*k] rsf * w (same writer)
    const float *zp;     // [LG_NP][T][E] partial router logits
    const float *rb;     // [E] selection bias
    int n_group, topk_group;
    float rsf, top_p;  // top_p: adaptive expert top-p (0 < top_p < 1), else all top_k kept
    // routed experts
    const uint8_t *gq, *uq, *dq;
    const float *gs, *us, *ds;
    int64_t qstride, dqstride, sstride, dsstride;
    int I;
    const uint8_t *ebits;  // [E] each routed expert's format, 4 or 2 (packed int2); null: all int4
    // shared expert
    const uint8_t *sgq, *suq, *sdq;
    const float *sgs, *sus, *sds;
    int Ish, sh_bits;
    // partial expert outputs, one plane per 128-row unit of the intermediate,
    // f16 (each partial rounded once to nearest even)
    uint16_t *yp;   // [I/128][T*k][H]   routed, scaled by rsf * w
    uint16_t *ysp;  // [Ish/128][T][H]   shared
};

// The routing decision of the batch into LDS (every routed workgroup takes
// it, from the same logits, so all agree); the publishing workgroup also
// writes ids, w, rsf * w and the tie gaps to global memory.
template <int EPL>
__device__ __forceinline__ void dec_route(const DecArgs &r, int T, int E, int k, int32_t *ids_l, float *w_l, bool pub)
{
    const bool grouped = r.n_group > 1 && r.topk_group < r.n_group;
    if (!grouped && E <= 64 && E % 8 == 0 && k <= 3) {
        if (k == 1)
            dec_select_lanes<2>(r.zp, r.rb, T, E, k, r.top_p, ids_l, w_l, pub, r.gap);
        else if (k == 2)
            dec_select_lanes<3>(r.zp, r.rb, T, E, k, r.top_p, ids_l, w_l, pub, r.gap);
        else
            dec_select_lanes<4>(r.zp, r.rb, T, E, k, r.top_p, ids_l, w_l, pub, r.gap);
    } else {
        dec_select_waves<EPL>(r.zp, r.rb, T, E, k, r.n_group, r.topk_group, r.rsf, r.top_p, ids_l, w_l, pub, r.gap);
    }
    __syncthreads();
    if (pub)
        for (int i = threadIdx.x; i < T * k; i += blockDim.x) {
            r.ids[i] = ids_l[i];
            r.w[i] = w_l[i];
            r.pscale[i] = r.rsf * w_l[i];
        }
}

// ------------------------------------------------------------- expert kernel

constexpr int DX_WAVES = 8;                         // waves per workgroup
constexpr int DX_THREADS = DX_WAVES * WAVE;         // 512
constexpr int DX_ROWS = DX_WAVES * 16;              // intermediate rows per unit (16 per wave)
static_assert(DX_ROWS == DEC_CHUNK_ROWS, "the workspace holds one output plane per unit chunk");
constexpr int DX_LDH = DX_ROWS + 8;                 // padded row of the on-chip h chunk (bf16)
constexpr int DX_TILES = 8;                         // down output tiles of 16 columns per wave per round
constexpr int DX_WCOLS = DX_TILES * 16;             // output columns per wave per round (128)
constexpr int DX_RCOLS = DX_WAVES * DX_WCOLS;       // output columns per round (1024)
constexpr int DX_LDY = DX_WCOLS + 4;                // padded row of a wave's staged down tile (floats)
constexpr int GU_CPL = 8;                           // 16-byte gate/up chunks per lane per row per super-stage
constexpr int GU_AHEAD = 4;                         // gate/up chunks in flight ahead of the MFMAs

// s_waitcnt for at most N outstanding vector-memory operations of the wave
// (gfx9 encoding; expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void dx_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Down weights of one round: lane (n, g) holds, for each of its wave's 8
// output tiles tt, the 32 values of intermediate [32g, 32g + 32) of the
// unit's chunk in output row 16 tt + n of the wave's 128: 16 bytes int4,
// 32 bytes int8.  Word s (int4) or words 2s, 2s + 1 (int8) feed k-step s.
template <int WBITS>
struct DownW {
    uint32_t d[DX_TILES][WBITS];
};

// Buffer resource over `bytes` bytes at `base` (raw, byte-addressed; loads
// beyond the range return zero).  `base` and `bytes` must be uniform over the
// wave; they are taken from the first lane so that the compiler keeps the
// descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t p = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void *ub = (void *)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// A lane's 8 rows are 16 * rstride bytes apart: one per-lane offset plus a
// uniform per-tile offset, so the loads share one address register.  Also
// the row scales of the wave's 128 columns, 4 per lane (lanes 32..63 repeat
// lanes 0..31: the write-out covers a row with 32 lanes).
template <int WBITS>
__device__ __forceinline__ void load_down(DownW<WBITS> &w, f32x4 &sd, const uint8_t *dq, const float *dsc,
                                          int64_t rstride, int H, int col0, int i0)
{
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    sd = *(const f32x4 *)(dsc + col0 + 4 * (lane & 31));
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(dq, (uint32_t)(H * rstride));
    const int voff = (int)((col0 + n) * rstride + (i0 + 32 * g) * WBITS / 8);
#pragma unroll
    for (int tt = 0; tt < DX_TILES; ++tt) {
        const int soff = (int)(tt * 16 * rstride);
#pragma unroll
        for (int h = 0; h < WBITS / 4; ++h) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * h, soff, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) w.d[tt][4 * h + q] = v[q];
        }
    }
}

// Int2 experts (element 4c + j of a row in bits 2j..2j+1 of byte c, two's
// complement) run the int4 body's arithmetic: each 16-byte chunk of an int4
// row (32 values) is 8 bytes of the int2 row, loaded at half the width, and
// eight codes (a 16-bit field) unpack straight to the bit patterns the int4
// unpacks give for the same values: 2^e + (code + 8), bf16 (HI = 0x4300) or
// f16 (0x6400), in their k-slot order (e0,e4),(e1,e5),(e2,e6),(e3,e7).
// t = w | w << 8 puts element j + 4 sixteen bits above element j; a field
// XOR 2 is code + 2 (0..3), plus 6 is code + 8 (6..9).  So the products and
// sums are those of the same weights stored as int4, bit for bit.
template <uint32_t HI>
__device__ __forceinline__ u32x4 unpack_int2x8_ks(uint32_t w)
{
    const uint32_t t = (w & 0xFFFFu) | ((w & 0xFFFFu) << 8);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = ((((t >> (2 * i)) & 0x00030003u) ^ 0x00020002u) + 0x00060006u) | (HI | (HI << 16));
    return r;
}

// codes 8 wd .. 8 wd + 7 of a lane's 32 in an int2 chunk (two 32-bit words)
__device__ __forceinline__ uint32_t int2_group(const u32x2 &c, int wd) { return c[wd >> 1] >> (16 * (wd & 1)); }

// The down slice of an int2 expert: as load_down<4>, each tile's 32 values
// in 8 bytes (rstride: bytes of an int2 row), unpacked where they are used.
struct DownW2 {
    u32x2 d[DX_TILES];
};

__device__ __forceinline__ void load_down2(DownW2 &w, f32x4 &sd, const uint8_t *dq, const float *dsc, int64_t rstride,
                                           int H, int col0, int i0)
{
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    sd = *(const f32x4 *)(dsc + col0 + 4 * (lane & 31));
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(dq, (uint32_t)(H * rstride));
    const int voff = (int)((col0 + n) * rstride + (i0 + 32 * g) / 4);
#pragma unroll
    for (int tt = 0; tt < DX_TILES; ++tt)
        w.d[tt] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, (int)(tt * 16 * rstride), 0));
}

// Position of intermediate j in a row of the on-chip h chunk: with int4
// weights each 8-group is stored in the unpack's k-slot order
// (j0, j4, j1, j5, j2, j6, j3, j7).
template <int WBITS>
__device__ __forceinline__ int h_pos(int j)
{
    return WBITS == 4 ? (j & ~7) | ((j & 3) << 1) | ((j >> 2) & 1) : j;
}

// LDS of the expert kernel.  The staged activations are dead once the gate/up
// MFMAs are done, so they share storage with the staged down tiles.
template <int WBITS>
struct alignas(16) DxSmem {
    static constexpr int KS = 512 * 8 / WBITS;  // columns per gate/up super-stage
    static constexpr int LDA = KS + 8;
    union {
        uint16_t a[DEC_MAXT * LDA];      // bf16 activation rows of the super-stage
        float y[DX_WAVES][16 * DX_LDY];  // each wave's 16 x 128 down tile (after the gate/up MFMAs)
    } u;
    int32_t ids[DEC_MAXT * DEC_MAXK];        // routing of the batch
    float w[DEC_MAXT * DEC_MAXK];
    uint16_t hh[DEC_MAXT * DX_LDH];          // h chunk, f16
    float xsum[DEC_MAXT];                    // activation row sums (by staged row = pair row)
};

// Activation staging: 16 threads per row, 32 rows; row r of the staging
// area holds token rtok(r).  Loads and stores are separate steps so that
// other requests can be issued in between; each thread keeps its row's
// running sum (over its chunks and all super-stages) in rsum.
template <int WBITS>
struct XStage {
    static constexpr int TPR = 16;
    static constexpr int XPT = DxSmem<WBITS>::KS / 8 / TPR;
    u32x4 v[XPT];
};

template <int WBITS>
__device__ __forceinline__ void xstage_load(XStage<WBITS> &xs, const DecArgs &a, int nr, int ss, const PairRows &pr)
{
    constexpr int TPR = XStage<WBITS>::TPR, KS = DxSmem<WBITS>::KS;
    const int srow = threadIdx.x / TPR, csub = threadIdx.x % TPR;
    const int tk = __shfl(pr.tok, srow, WAVE);  // staged row srow holds pair row srow (srow < 32)
    const uint16_t *src = srow < nr ? a.x + (size_t)tk * a.H + (size_t)ss * KS + csub * 8 : nullptr;
#pragma unroll
    for (int j = 0; j < XStage<WBITS>::XPT; ++j)
        xs.v[j] = src ? *(const u32x4 *)(src + j * 8 * TPR) : u32x4{0u, 0u, 0u, 0u};
}

template <int WBITS>
__device__ __forceinline__ void xstage_store(const XStage<WBITS> &xs, DxSmem<WBITS> &sm, int nr, float &rsum)
{
    constexpr int TPR = XStage<WBITS>::TPR, LDA = DxSmem<WBITS>::LDA;
    const int srow = threadIdx.x / TPR, csub = threadIdx.x % TPR;
    if (srow >= nr) return;
    uint16_t *dst = sm.u.a + srow * LDA + csub * 8;
#pragma unroll
    for (int j = 0; j < XStage<WBITS>::XPT; ++j) {
        u32x4 v = xs.v[j];
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) s += bf16_lo(v[d]) + bf16_hi(v[d]);
        rsum += s;
        if (WBITS == 4) v = interleave_bf16x8(v);
        *(u32x4 *)(dst + j * 8 * TPR) = v;
    }
}

// One unit: gate/up of 128 intermediate rows for the n pair rows of its batch
// (SwiGLU -> h chunk, on chip in f16), then
// y_part = h_chunk . D[:, chunk]^T for every output column, scaled by the
// down row scale and the row's output scale, stored to plane `chunk` of out.
// Each super-stage's activation rows (staged row r = pair row r, r < nr) are
// loaded here just before its weight rows, so they land first (vector loads
// complete in issue order) while the weights stream behind them.  Weight
// loads are issued gate/up first, then the down slice, a few chunks ahead of
// the MFMAs that consume them.
template <int WBITS, int NMB, bool I2 = false>
__device__ __forceinline__ void expert_body(const DecArgs &a, DxSmem<WBITS> &sm, int n, int nr, const PairRows &pr,
                                            float rsum, const uint8_t *grow, const uint8_t *urow, float sg,
                                            float su, const uint8_t *dq, const float *dsc, int64_t drstride,
                                            int i0, uint16_t *out, int nrows)
{
    static_assert(!I2 || WBITS == 4, "int2 experts run the int4 body");
    constexpr int CPL = GU_CPL;
    constexpr int SB = CPL * 64;           // weight bytes of a row per super-stage (512)
    constexpr int CB = I2 ? 32 : 64;       // bytes of a row per chunk step (an int2 row: half)
    constexpr int KS = DxSmem<WBITS>::KS;  // columns per super-stage (1024 int4, 512 int8)
    constexpr int LDA = DxSmem<WBITS>::LDA;
    constexpr int NCH = NMB == 1 ? 2 : 1;  // independent accumulator chains per matrix (register budget)
    constexpr int TPR = XStage<WBITS>::TPR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, ln = lane & 15;
    f32x4 acc[NMB][2][NCH];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) acc[mb][x][ch] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nss = a.H / KS;
    const uint16_t *ap[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) ap[mb] = sm.u.a + (mb * 16 + ln < n ? mb * 16 + ln : 0) * LDA;
    std::conditional_t<I2, DownW2, DownW<WBITS>> dw;
    f32x4 sdv;
    using WChunk = std::conditional_t<I2, u32x2, u32x4>;  // a lane's chunk as loaded
    WChunk wg[CPL], wu[CPL];
    auto down_load = [&](int col) {
        if constexpr (I2) load_down2(dw, sdv, dq, dsc, drstride, a.H, col, i0);
        else load_down<WBITS>(dw, sdv, dq, dsc, drstride, a.H, col, i0);
    };
    // One super-stage; the last one (a separate instance, LAST set) also
    // issues the down slice, so its loads stay where they are written
    // instead of moving to the loop's exit, behind the gate/up MFMAs.
    auto super_stage = [&](int ss, auto lastc) {
        constexpr bool LAST = decltype(lastc)::value;
        // gate and up chunk c in adjacent requests: the MFMAs on chunk c can
        // start once its pair has arrived
        auto issue_gu = [&](int c) {
            wg[c] = *(const WChunk *)(grow + (size_t)ss * (SB / 64 * CB) + c * CB);
            wu[c] = *(const WChunk *)(urow + (size_t)ss * (SB / 64 * CB) + c * CB);
        };
        XStage<WBITS> xs;
        xstage_load<WBITS>(xs, a, nr, ss, pr);
        // The first GU_AHEAD chunks now, each later one as an earlier chunk is
        // consumed (so a wave is not held at issue while the memory system is
        // saturated, and its MFMAs overlap the stream); the down slice after
        // the last gate/up chunk.
#pragma unroll
        for (int c = 0; c < GU_AHEAD; ++c) issue_gu(c);
        if (ss > 0) __syncthreads();  // the previous super-stage's A reads are done
        xstage_store<WBITS>(xs, sm, nr, rsum);
        // every load older than these gate/up chunks (the activation rows, the
        // row scales) has landed: waited for here by every wave, so the
        // epilogue does not wait on the counter for the down slice
        dx_wait_vm<2 * GU_AHEAD>();
        if (LAST) {
            // row sums: the TPR threads of a staged row are consecutive lanes
            float s = rsum;
#pragma unroll
            for (int o = 1; o < TPR; o <<= 1) s += __shfl_xor(s, o, WAVE);
            if (tid % TPR == 0 && tid / TPR < nr) sm.xsum[tid / TPR] = s;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (c + GU_AHEAD < CPL) issue_gu(c + GU_AHEAD);
            else if (LAST && c + GU_AHEAD == CPL) {
                down_load(wave * DX_WCOLS);
                asm volatile("" ::: "memory");  // keeps the compiler from sinking these loads to their use
            }
            if constexpr (WBITS == 4) {
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    u32x4 bg, bu;
                    if constexpr (I2) {
                        bg = unpack_int2x8_ks<0x4300u>(int2_group(wg[c], wd));
                        bu = unpack_int2x8_ks<0x4300u>(int2_group(wu[c], wd));
                    } else {
                        bg = unpack_int4x8(wg[c][wd]);
                        bu = unpack_int4x8(wu[c][wd]);
                    }
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        const u32x4 af = *(const u32x4 *)(ap[mb] + (4 * c + g) * 32 + 8 * wd);
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
                        const u32x4 af = *(const u32x4 *)(ap[mb] + (4 * c + g) * 16 + 8 * wd);
                        acc[mb][0][wd % NCH] = mfma_bf16(af, bg, acc[mb][0][wd % NCH]);
                        acc[mb][1][wd % NCH] = mfma_bf16(af, bu, acc[mb][1][wd % NCH]);
                    }
                }
            }
        }
    };
    for (int ss = 0; ss < nss - 1; ++ss) super_stage(ss, std::false_type{});
    super_stage(nss - 1, std::true_type{});
    // SwiGLU epilogue: h for (row m, intermediate wave * 16 + ln) -> on-chip
    // chunk in f16 (round to nearest even).
    const float bias = (WBITS == 4) ? INT4_BIAS : 0.f;
    const int hp = h_pos<WBITS>(wave * 16 + ln);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb * 16 + g * 4 + r;
            const float corr = bias * sm.xsum[m < n ? m : 0];
            float ga = acc[mb][0][0][r], ua = acc[mb][1][0][r];
#pragma unroll
            for (int ch = 1; ch < NCH; ++ch) {
                ga += acc[mb][0][ch][r];
                ua += acc[mb][1][ch][r];
            }
            const float h = m < n ? fast_silu((ga - corr) * sg) * ((ua - corr) * su) : 0.f;
            sm.hh[m * DX_LDH + hp] = __builtin_bit_cast(uint16_t, (_Float16)h);
        }
    }
    __syncthreads();
    // down on f16 matrix cores: A = h chunk (rows m, 128 k in four 32-steps),
    // one 16-row block at a time (the weights are unpacked again per block).
    // The B fragments hold q + 1032 (int4) or q + 1152 (int8): each tile
    // starts from minus that constant times the row sum of h, itself an MFMA
    // against a constant fragment, so the accumulation yields the sum over q.  Each wave stages
    // its 16 x 128 result in LDS and writes it out two rows at a time as
    // 16-byte stores scaled by the down row scale and the row's output scale.
    const int chunk = i0 / DX_ROWS;
    float *yl = sm.u.y[wave];
    for (int c0 = 0; c0 < a.H; c0 += DX_RCOLS) {
        const int col0 = c0 + wave * DX_WCOLS;
        if (c0 > 0) down_load(col0);
#pragma unroll 1
        for (int mb = 0; mb < NMB; ++mb) {
            if (mb * 16 >= n) break;
            u32x4 fh[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) fh[s] = *(const u32x4 *)(sm.hh + (mb * 16 + ln) * DX_LDH + 32 * g + 8 * s);
            // f16 1032 / 1152
            constexpr uint32_t CB16 = WBITS == 4 ? 0x64086408u : 0x64806480u;
            const u32x4 cb = u32x4{CB16, CB16, CB16, CB16};
            f32x4 cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) cs = mfma_f16(fh[s], cb, cs);
            const f32x4 d0 = -cs;
#pragma unroll
            for (int tt = 0; tt < DX_TILES; ++tt) {
                f32x4 d = d0;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 b;
                    if constexpr (I2) b = unpack_int2x8_ks<0x6400u>(int2_group(dw.d[tt], s));
                    else if constexpr (WBITS == 4) b = unpack_int4x8_f16(dw.d[tt][s]);
                    else b = unpack_int8x8_f16(u32x2{dw.d[tt][2 * s], dw.d[tt][2 * s + 1]});
                    d = mfma_f16(fh[s], b, d);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) yl[(4 * g + r) * DX_LDY + tt * 16 + ln] = d[r];
            }
            // read back two rows at a time (own wave's data: LDS order within the wave suffices)
            const int nrw = n - mb * 16;
            const int half = lane >> 5, q4 = 4 * (lane & 31);
#pragma unroll
            for (int rr = 0; rr < 16; rr += 2) {
                const int row = rr + half;
                const int m = mb * 16 + row;
                const float osc = __shfl(pr.psc, m, WAVE);  // pair row m's scale and pair (m < 32)
                const int prow = __shfl(pr.pair, m, WAVE);
                if (row < nrw) {
                    const f32x4 v = *(const f32x4 *)(yl + row * DX_LDY + q4);
                    f32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o[q] = v[q] * sdv[q] * osc;
                    *(u32x2 *)(out + ((size_t)chunk * nrows + prow) * a.H + col0 + q4) =
                        u32x2{pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3])};
                }
            }
        }
    }
}

// Units (logical index L): [0, nsh) shared-expert units (128 intermediate
// rows x up to 16 tokens: the two token halves of a chunk are adjacent
// units), then routed units (rank of the chosen expert in ascending id
// order, chunk).  Routed units first take the routing decision of the whole
// batch (every one computes the same from the logits), then gather the pairs
// routed to their expert; units beyond the chosen experts exit.  A unit's
// loads are its activation rows, its gate/up rows and its down slice (all
// output rows, the chunk's 128 columns), issued a few chunks ahead of the MFMAs.
//
// XCD-aware placement: workgroup b runs on XCD b % 8; logical units 4q ..
// 4q + 3 (chunks whose down slices share 128-byte lines, or the token
// halves of one chunk) are given workgroups on the same XCD, so shared data
// is fetched into one L2.
__device__ __forceinline__ int dx_logical_unit(int b)
{
    const int x = b & 7, s = b >> 3;
    return 4 * (x + 8 * (s >> 2)) + (s & 3);
}

__host__ __device__ __forceinline__ int dx_token_halves(int T) { return (T + 15) / 16; }

// Logical unit L in the weight format of its expert (WBITS: the shared
// expert's format for its units, int4 for the routed ones).
// MIX: a family of int4 and int2 experts (a.ebits), a separate instance so
// that int4-only layers run without the int2 body.
template <int WBITS, int EPL, bool MIX>
__device__ __forceinline__ void dec_unit(const DecArgs &a, DxSmem<WBITS> &sm, int L)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
    const int nth = dx_token_halves(a.T);
    const int nsh = a.sh_bits ? (a.Ish / DX_ROWS) * nth : 0;
    const bool shared = L < nsh;
    const size_t rbytes = (size_t)a.H * WBITS / 8;
    const uint8_t *grow, *urow, *dq;
    const float *dsc;
    float sg, su;
    int64_t drs;
    int i0;
    // (wb: the bits of the expert's rows, WBITS or 2 for an int2 routed
    // expert, whose 32-value chunks are 8 bytes instead of 16)
    auto locate = [&](const uint8_t *gq, const uint8_t *uq, const uint8_t *dqq, const float *gsc, const float *usc,
                      const float *dscc, int K, int chunk0, int wb) {
        i0 = chunk0;
        const int row = i0 + wave * 16 + (lane & 15);
        const size_t rb = wb == WBITS ? rbytes : (size_t)a.H * wb / 8;
        const int cb = wb == 2 ? 8 : 16;
        grow = gq + (size_t)row * rb + g * cb;
        urow = uq + (size_t)row * rb + g * cb;
        sg = gsc[row];
        su = usc[row];
        dq = dqq;
        dsc = dscc;
        drs = (int64_t)K * wb / 8;
    };
    int n, nrows, nr;
    uint16_t *out;
    const float rsum = 0.f;
    if (shared) {
        // 16 tokens of one half: staged rows r = pair rows r = token 16 th + r
        const int th = L % nth;
        n = a.T - 16 * th < 16 ? a.T - 16 * th : 16;
        nr = n;
        const PairRows pr{16 * th + lane, 16 * th + lane, 1.0f};
        locate(a.sgq, a.suq, a.sdq, a.sgs, a.sus, a.sds, a.Ish, (L / nth) * DX_ROWS, WBITS);
        nrows = a.T;
        out = a.ysp;
        expert_body<WBITS, 1>(a, sm, n, nr, pr, rsum, grow, urow, sg, su, dq, dsc, drs, i0, out, nrows);
        return;
    }
    // routed: the routing decision, then the unit's expert and pairs; only
    // the rows of those pairs are staged (row r = token of pair r)
    const int v = L - nsh, per = a.I / DX_ROWS;
    // the experts' formats (a mixed int4/int2 family): four per lane, loaded
    // now so that the routing hides the load
    uint32_t fmt4 = 0x04040404u;
    if (MIX) {
        fmt4 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) fmt4 |= (uint32_t)(4 * lane + j < a.E ? a.ebits[4 * lane + j] : 4) << (8 * j);
    }
    dec_route<EPL>(a, a.T, a.E, a.k, sm.ids, sm.w, v == 0);
    PairRows pr;
    const int2 un = dec_locate_wave<EPL>(sm.ids, a.T * a.k, a.k, a.E, v / per, pr);
    const int e = __builtin_amdgcn_readfirstlane(un.x);
    if (e < 0) return;
    n = __builtin_amdgcn_readfirstlane(un.y);
    nr = n;
    pr.psc = lane < n ? a.rsf * sm.w[pr.pair] : 0.f;
    const bool i2 = MIX && WBITS == 4 && ((__shfl(fmt4, e / 4, WAVE) >> (8 * (e % 4))) & 0xFFu) == 2u;  // wave-uniform
    locate(a.gq + (size_t)e * a.qstride, a.uq + (size_t)e * a.qstride, a.dq + (size_t)e * a.dqstride,
           a.gs + (size_t)e * a.sstride, a.us + (size_t)e * a.sstride, a.ds + (size_t)e * a.dsstride, a.I,
           (v % per) * DX_ROWS, i2 ? 2 : WBITS);
    nrows = a.T * a.k;
    out = a.yp;
    if constexpr (MIX && WBITS == 4) {
        if (i2) {
            if (n <= 16)
                expert_body<4, 1, true>(a, sm, n, nr, pr, rsum, grow, urow, sg, su, dq, dsc, drs, i0, out, nrows);
            else
                expert_body<4, 2, true>(a, sm, n, nr, pr, rsum, grow, urow, sg, su, dq, dsc, drs, i0, out, nrows);
            return;
        }
    }
    if (n <= 16)
        expert_body<WBITS, 1>(a, sm, n, nr, pr, rsum, grow, urow, sg, su, dq, dsc, drs, i0, out, nrows);
    else
        expert_body<WBITS, 2>(a, sm, n, nr, pr, rsum, grow, urow, sg, su, dq, dsc, drs, i0, out, nrows);
}

// One launch for every unit.  SH8 (an int8 shared expert): its units take
// the int8 body, the routed ones the int4 body, in one LDS area sized for
// either, so the routed units do not wait for a separate shared-expert
// launch to drain; otherwise every unit takes the int4 body.
template <bool SH8, int EPL, bool MIX>
__global__ __launch_bounds__(DX_THREADS, 1) void k_dec_expert(DecArgs a, int nunits)
{
    const int L = dx_logical_unit(blockIdx.x);
    if (L >= nunits) return;
    if constexpr (SH8) {
        __shared__ union {
            DxSmem<4> s4;
            DxSmem<8> s8;
        } sm;
        const int nsh = (a.Ish / DX_ROWS) * dx_token_halves(a.T);
        if (L < nsh)
            dec_unit<8, EPL, false>(a, sm.s8, L);
        else
            dec_unit<4, EPL, MIX>(a, sm.s4, L);
    } else {
        __shared__ DxSmem<4> sm;
        dec_unit<4, EPL, MIX>(a, sm, L);
    }
}

// ---------------------------------------------------------------- combine

constexpr int CB_SPLIT = 4;  // threads per output quad, each summing every 4th plane

// Bit j set: token t's selection slot j was dropped by adaptive top-p (id -1;
// its partial planes were never written).  ids is null when top-p is off.
__device__ __forceinline__ uint32_t dec_dropped_slots(const int32_t *ids, int t, int k)
{
    uint32_t m = 0;
    if (ids)
        for (int j = 0; j < k; ++j)
            if (ids[(size_t)t * k + j] < 0) m |= 1u << j;
    return m;
}

// The four f16 columns at c of this lane's planes p0, p0 + CB_SPLIT, ...
// (MAXL of them): every load is issued, unconditionally, before any result
// is used (a plane that is absent, past the last or dropped by top-p reads
// a valid address and is marked unused), so the MAXL requests are in flight
// together instead of one after another.
template <int MAXL>
__device__ __forceinline__ void dec_plane_loads(u32x2 (&hv)[MAXL], bool (&use)[MAXL], const uint16_t *yp,
                                                const uint16_t *ysp, bool live, int p0, int np, int nrp, int nkr,
                                                uint32_t dropped, size_t P, int T, int t, int k, int H, int c)
{
    // routed plane p is chunk p % nkr of the pair in slot p / nkr; the lane's
    // planes step by CB_SPLIT <= nkr, so chunk and slot advance without a
    // division.  Offsets are in elements (32 bits: the planes of this regime
    // hold well under 2^31 of them).
    int ch = p0 % nkr, j = p0 / nkr;
    const uint32_t rbase = (uint32_t)((size_t)t * k * H + c), sbase = (uint32_t)((size_t)t * H + c);
    const uint32_t rstep = (uint32_t)(P * H), sstep = (uint32_t)T * H;
#pragma unroll
    for (int i = 0; i < MAXL; ++i) {
        const int p = p0 + CB_SPLIT * i;
        use[i] = live && p < np && !(p < nrp && ((dropped >> j) & 1u));
        const uint16_t *src = !use[i] ? yp
                              : p < nrp ? yp + (rbase + (uint32_t)ch * rstep + (uint32_t)j * H)
                                        : ysp + (sbase + (uint32_t)(p - nrp) * sstep);
        hv[i] = *(const u32x2 *)src;
        ch += CB_SPLIT;
        if (ch >= nkr) {
            ch -= nkr;
            ++j;
        }
    }
}

// out[t] = sum over partial planes (routed pairs of t in order j, their
// chunks in order; then the shared expert's chunks) (+ x[t]).  Four
// consecutive lanes own one 4-column quad: lane q sums planes q, q + 4, ...
// with all its loads in flight together, then the four sums are added in
// lane order.  Fixed order throughout.
__global__ __launch_bounds__(256) void k_dec_combine(const uint16_t *__restrict__ yp, int nkr,
                                                     const uint16_t *__restrict__ ysp, int nks,
                                                     const uint16_t *__restrict__ res, void *__restrict__ out, int T,
                                                     int H, int k, int out_f32, const int32_t *__restrict__ ids)
{
    constexpr int MAXL = 16;  // planes per lane per batch
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int cpt = H / 4;
    const bool live = idx < (long)T * cpt * CB_SPLIT;
    const long quad = idx / CB_SPLIT;
    const int q = (int)(idx % CB_SPLIT);
    const int t = live ? (int)(quad / cpt) : 0;
    const int c = live ? (int)(quad % cpt) * 4 : 0;
    const size_t P = (size_t)T * k;
    const int nrp = k * nkr, np = nrp + nks;
    const uint32_t dropped = dec_dropped_slots(ids, live ? t : 0, k);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    auto add_planes = [&](const u32x2 (&hv)[MAXL], const bool (&use)[MAXL]) {
#pragma unroll
        for (int i = 0; i < MAXL; ++i) {
            const f32x4 v = use[i] ? f32x4{f16_lo(hv[i][0]), f16_hi(hv[i][0]), f16_lo(hv[i][1]), f16_hi(hv[i][1])}
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += v[e];
        }
    };
    u32x2 rv = u32x2{0u, 0u};
    if (np <= CB_SPLIT * MAXL) {
        // one batch (up to 64 planes): straight-line, the residual in flight
        // with the planes
        u32x2 hv[MAXL];
        bool use[MAXL];
        dec_plane_loads<MAXL>(hv, use, yp, ysp, live, q, np, nrp, nkr, dropped, P, T, t, k, H, c);
        rv = *(const u32x2 *)(res ? res + (size_t)t * H + c : yp);  // (used only with res)
        add_planes(hv, use);
    } else {
        for (int p0 = q; p0 < np; p0 += CB_SPLIT * MAXL) {
            u32x2 hv[MAXL];
            bool use[MAXL];
            dec_plane_loads<MAXL>(hv, use, yp, ysp, live, p0, np, nrp, nkr, dropped, P, T, t, k, H, c);
            add_planes(hv, use);
        }
        if (res) rv = *(const u32x2 *)(res + (size_t)t * H + c);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float s1 = __shfl_down(acc[e], 1, WAVE);
        const float s2 = __shfl_down(acc[e], 2, WAVE);
        const float s3 = __shfl_down(acc[e], 3, WAVE);
        acc[e] = ((acc[e] + s1) + s2) + s3;
    }
    if (!live || q != 0) return;
    if (res) {
        const u32x2 v = rv;
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

// Chained decode: k_dec_combine (same lanes and plane order per output
// quad, so the bf16 output is the same bits) that also takes the next
// layer's router logits of the row it writes, in the 4-plane form
// k_dec_expert reads.  Workgroup (token t, quarter g) covers columns
// [g H/4, (g+1) H/4): once that quarter of the output row is in LDS (as the
// next layer reads it, bf16), sixteen consecutive threads take an expert,
// thread j the 4-column groups j, j + 16, ... of the quarter (16-byte W
// loads, sixteen threads on 256 contiguous bytes), four experts per thread
// per round of 64; fused multiply-adds in that order, then the sixteen
// partial sums in a fixed butterfly; the sum goes to plane g.  The next
// layer adds the 4 planes as it does its own logits kernel's.  For H = 1024
// the first round's W values are loaded with the planes, before the combine.
constexpr int CL_SUBS = 16;  // threads per expert in the logits
constexpr int CL_EPT = 4;    // experts per thread per round (64 per round)
constexpr int CL_GPT = 4;    // 4-column groups per thread per expert (H = 1024: a quarter is 64 groups)

__global__ __launch_bounds__(256) void k_dec_combine_logits(const uint16_t *__restrict__ yp, int nkr,
                                                            const uint16_t *__restrict__ ysp, int nks,
                                                            const uint16_t *res,  // (not restrict: its load
                                                                                  // stays before the W loads)
                                                            uint16_t *__restrict__ out, int T, int H, int k,
                                                            const float *__restrict__ nrw, int nE,
                                                            float *__restrict__ nzp, const int32_t *__restrict__ ids)
{
    static_assert(DEC_LOGIT_PLANES == 4, "one plane per quarter of the row");
    extern __shared__ float xq[];  // [H / 4] this quarter of the output row
    constexpr int MAXL = 16, MAXF = 8;  // planes per lane per batch (generic path, straight-line path)
    const int tid = threadIdx.x;
    const int t = blockIdx.x / 4, g = blockIdx.x % 4;
    const int H4 = H / 4, c0 = g * H4;
    const int sub = tid % CL_SUBS, ex = tid / CL_SUBS;  // logits: experts ex + 16 i of the round, thread sub
    bool pre = false;                                   // wv holds the first round's W values
    f32x4 wv[CL_EPT][CL_GPT];
    const size_t P = (size_t)T * k;
    const int nrp = k * nkr, np = nrp + nks;
    const uint32_t dropped = dec_dropped_slots(ids, t, k);
    auto add_planes = [&](f32x4 &acc, const auto &hv, const auto &use) {
#pragma unroll
        for (int i = 0; i < (int)(sizeof(use) / sizeof(use[0])); ++i) {
            const f32x4 v = use[i] ? f32x4{f16_lo(hv[i][0]), f16_hi(hv[i][0]), f16_lo(hv[i][1]), f16_hi(hv[i][1])}
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += v[e];
        }
    };
    // the four lanes' sums in lane order, + the residual, out in bf16 and
    // into LDS as the next layer reads it
    auto finish = [&](f32x4 acc, int quad, int q, int c, u32x2 r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float s1 = __shfl_down(acc[e], 1, WAVE);
            const float s2 = __shfl_down(acc[e], 2, WAVE);
            const float s3 = __shfl_down(acc[e], 3, WAVE);
            acc[e] = ((acc[e] + s1) + s2) + s3;
        }
        if (q == 0) {
            if (res) {
                acc[0] += bf16_lo(r[0]);
                acc[1] += bf16_hi(r[0]);
                acc[2] += bf16_lo(r[1]);
                acc[3] += bf16_hi(r[1]);
            }
            const u32x2 o = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            *(u32x2 *)(out + (size_t)t * H + c) = o;
            float *x = xq + (c - c0);
            x[0] = bf16_lo(o[0]);
            x[1] = bf16_hi(o[0]);
            x[2] = bf16_lo(o[1]);
            x[3] = bf16_hi(o[1]);
        }
    };
    const int nquad = H4 / 4;
    if (nquad == 256 / CB_SPLIT && np <= CB_SPLIT * MAXF) {
        // H = 1024 (one quad per four threads), one batch of up to 32
        // planes: straight-line code, the planes and the residual first, then
        // the W values of the first 64 experts, all in flight together (no
        // load is conditional, so waiting for the planes does not wait for W)
        const int quad = tid / CB_SPLIT, q = tid % CB_SPLIT;
        const int c = c0 + quad * 4;
        u32x2 hv[MAXF];
        bool use[MAXF];
        dec_plane_loads<MAXF>(hv, use, yp, ysp, true, q, np, nrp, nkr, dropped, P, T, t, k, H, c);
        const u32x2 r = *(const u32x2 *)(res ? res + (size_t)t * H + c : yp);  // (used only with res)
        asm volatile("" ::: "memory");  // the W loads after the planes (they complete in issue order)
        static_assert(CL_GPT * 4 * CL_SUBS == 256, "a quarter of a 1024-column row");
#pragma unroll
        for (int i = 0; i < CL_EPT; ++i) {
            const float *wr = nrw + (size_t)min(ex + 16 * i, nE - 1) * H + c0 + 4 * sub;
#pragma unroll
            for (int j = 0; j < CL_GPT; ++j) wv[i][j] = *(const f32x4 *)(wr + 4 * CL_SUBS * j);
        }
        pre = true;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        add_planes(acc, hv, use);
        finish(acc, quad, q, c, r);
    } else {
        for (int qd0 = 0; qd0 < nquad; qd0 += 256 / CB_SPLIT) {
            const int quad = qd0 + tid / CB_SPLIT, q = tid % CB_SPLIT;
            const bool lq = quad < nquad;
            const int c = c0 + (lq ? quad : 0) * 4;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int p0 = q; p0 < np; p0 += CB_SPLIT * MAXL) {
                u32x2 hv[MAXL];
                bool use[MAXL];
                dec_plane_loads<MAXL>(hv, use, yp, ysp, lq, p0, np, nrp, nkr, dropped, P, T, t, k, H, c);
                add_planes(acc, hv, use);
            }
            const u32x2 r = *(const u32x2 *)(res ? res + (size_t)t * H + c : yp);
            if (lq) finish(acc, quad, q, c, r);
        }
    }
    __syncthreads();
    float *zp = nzp + ((size_t)g * T + t) * nE;
    const float *xs = xq + 4 * sub;
    for (int e0 = 0; e0 < nE; e0 += CL_EPT * 16) {
        float z[CL_EPT];
#pragma unroll
        for (int i = 0; i < CL_EPT; ++i) z[i] = 0.f;
        if (pre && e0 == 0) {
#pragma unroll
            for (int j = 0; j < CL_GPT; ++j) {
                const f32x4 xv = *(const f32x4 *)(xs + 4 * CL_SUBS * j);
#pragma unroll
                for (int i = 0; i < CL_EPT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) z[i] = fmaf(xv[r], wv[i][j][r], z[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < CL_EPT; ++i) {
                const float *wr = nrw + (size_t)min(e0 + ex + 16 * i, nE - 1) * H + c0 + 4 * sub;
                for (int cc = 0; cc < H4; cc += 4 * CL_SUBS) {
                    const f32x4 w4 = *(const f32x4 *)(wr + cc);
                    const f32x4 xv = *(const f32x4 *)(xs + cc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) z[i] = fmaf(xv[r], w4[r], z[i]);
                }
            }
        }
        // the sixteen partials in a fixed butterfly (the same sum in every lane)
#pragma unroll
        for (int i = 0; i < CL_EPT; ++i) {
#pragma unroll
            for (int o = 1; o < CL_SUBS; o <<= 1) z[i] += __shfl_xor(z[i], o, WAVE);
            const int e = e0 + ex + 16 * i;
            if (sub == 0 && e < nE) zp[e] = z[i];
        }
    }
}

// ---------------------------------------------------------------- launcher

static bool dec_topp_on(float p) { return p > 0.f && p < 1.f; }

bool decode_supported(int H, int E, int k, int I, int Ish, int sh_bits)
{
    static_assert(DEC_MAXT == DEC_CHUNK_TOKENS, "one launch takes one chunk of the batch");
    if (E > 256 || k > DEC_MAXK) return false;
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
    a.pscale = d.pscale;
    a.zp = d.z;
    a.rb = d.rb;
    a.n_group = d.n_group;
    a.topk_group = d.topk_group;
    a.rsf = d.rsf;
    a.top_p = d.top_p;
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
    a.ebits = d.ebits;
    a.sgq = d.sgq;
    a.suq = d.suq;
    a.sdq = d.sdq;
    a.sgs = d.sgs;
    a.sus = d.sus;
    a.sds = d.sds;
    a.Ish = d.Ish;
    a.sh_bits = d.sh_bits;
    a.yp = d.y;
    a.ysp = d.shp;

    hipError_t e;
    if (!d.experts_only && !d.logits_given) {
        const int grid = ((d.E + 15) / 16) * ((d.T + 15) / 16) * LG_NP;
        hipLaunchKernelGGL(k_dec_logits, dim3(grid), dim3(256), 0, st, d.x, d.rw, d.T, d.H, d.E, d.z);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    // expert units; the grid is padded to whole groups of 32 workgroups (the
    // XCD-aware placement permutes within such groups)
    const int nsh = d.sh_bits ? (d.Ish / DX_ROWS) * dx_token_halves(d.T) : 0;
    const int nunits = nsh + d.E * (d.I / DX_ROWS);
    const int grid = (nunits + 31) / 32 * 32;
    if (d.ev0) {
        e = hipEventRecord(d.ev0, st);
        if (e != hipSuccess) return e;
    }
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(grid), dim3(DX_THREADS), 0, st, a, nunits); };
    const bool sh8 = d.sh_bits == 8;
    auto pick = [&](auto mixc) {
        constexpr bool MX = decltype(mixc)::value;
        if (d.E <= 64)
            sh8 ? go(k_dec_expert<true, 1, MX>) : go(k_dec_expert<false, 1, MX>);
        else if (d.E <= 128)
            sh8 ? go(k_dec_expert<true, 2, MX>) : go(k_dec_expert<false, 2, MX>);
        else
            sh8 ? go(k_dec_expert<true, 4, MX>) : go(k_dec_expert<false, 4, MX>);
    };
    if (d.ebits) pick(std::true_type{});
    else pick(std::false_type{});
    e = hipGetLastError();
    if (e == hipSuccess && d.ev1) e = hipEventRecord(d.ev1, st);
    if (e != hipSuccess || d.experts_only) return e;
    if (d.nrw) {
        hipLaunchKernelGGL(k_dec_combine_logits, dim3(d.T * 4), dim3(256), (size_t)(d.H / 4) * sizeof(float), st, d.y,
                           d.I / DX_ROWS, d.shp, d.sh_bits ? d.Ish / DX_ROWS : 0, d.res, (uint16_t *)d.out, d.T, d.H,
                           d.k, d.nrw, d.nE, d.nz, dec_topp_on(d.top_p) ? d.ids : nullptr);
        return hipGetLastError();
    }
    const long nthreads = (long)d.T * (d.H / 4) * CB_SPLIT;
    hipLaunchKernelGGL(k_dec_combine, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, st, d.y,
                       d.I / DX_ROWS, d.shp, d.sh_bits ? d.Ish / DX_ROWS : 0, d.res, d.out, d.T, d.H, d.k,
                       d.out_f32, dec_topp_on(d.top_p) ? d.ids : nullptr);
    return hipGetLastError();
}

}  // namespace moe

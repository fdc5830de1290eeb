// ffn.hip -- grouped GEMMs of the SwiGLU experts on int4 (or int8) per-row weights.
//
// Batch-union (colibri README, "What's implemented"): the pairs are grouped by
// expert, so one tile of rows reads one expert's weights once and applies them
// to every row routed to it.  Weights are per-row symmetric with one f32 scale
// per row (colibri-nano README, "Converting a checkpoint yourself"); an
// expert's three matrices are gate [I][H], up [I][H], down [H][I].
//
// Both GEMMs run on bf16 matrix cores (v_mfma_f32_16x16x32_bf16) with f32
// accumulation.  A rows (activations) are staged through LDS; B rows (weights)
// are staged through LDS as raw packed bytes and unpacked to bf16 in registers
// right before the MFMA.  int4 values become q + 136 (one AND-OR per pair of
// values, see unpack_int4x8); the constant is removed in the epilogue as
// 136 * sum(A row), a sum taken from the same bf16 values the MFMA consumes.
// int8 values are converted exactly.  The per-row weight scale, SiLU * up
// (gate/up kernel) and the per-pair combine weight rsf * w (down kernel) are
// applied in the epilogue.
//
// The intermediate h = silu(g) * u is stored in f32.  The down kernel feeds it
// to the bf16 matrix cores as an exact two-term split h = hi + lo (hi = bf16(h),
// lo = bf16(h - hi)), two MFMAs per unpacked weight fragment: a single bf16
// rounding of h would leave a 2^-9 relative error on every product, about 1e-2
// of the output RMS at the tails of a large batch.
//
// Tiles.  A launch covers every (m-tile, n-tile) of every expert without
// reading the histogram back to the host: the grid is an upper bound
// (ceil(rows/BM) + experts m-tile slots, times n-tiles) and each workgroup
// finds its expert and first row from the offsets; surplus workgroups exit.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int FF_BK = 64;             // reduction columns per stage
constexpr int FF_LDA = FF_BK + 8;     // LDS A row, bf16 elements (144 B)


// Find this workgroup's expert, first sorted row and row count for m-tile
// slot `slot`; returns false when the slot is beyond the last tile.
template <int BM>
__device__ __forceinline__ bool find_tile(const FfnArgs &a, int slot, int &e, int &row0, int &rows)
{
    __shared__ int st[3];
    if (a.offsets == nullptr) {
        e = 0;
        row0 = slot * BM;
        rows = min(BM, a.M - row0);
        return rows > 0;
    }
    const int tid = threadIdx.x;
    if (tid < WAVE) {
        // lane l covers experts [4l, 4l+4)
        int cnt[4], tiles[4], mine = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ee = tid * 4 + q;
            cnt[q] = (ee < a.E) ? a.offsets[ee + 1] - a.offsets[ee] : 0;
            tiles[q] = (cnt[q] + BM - 1) / BM;
            mine += tiles[q];
        }
        // inclusive scan of per-lane tile counts
        int incl = mine;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const int v = __shfl_up(incl, o, WAVE);
            if (tid >= o) incl += v;
        }
        const int total = __shfl(incl, WAVE - 1, WAVE);
        int pre = incl - mine;
        if (tid == 0) st[0] = -1;
        if (slot < total) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (slot >= pre && slot < pre + tiles[q]) {
                    const int ee = tid * 4 + q;
                    st[0] = ee;
                    st[1] = a.offsets[ee] + (slot - pre) * BM;
                    st[2] = min(BM, cnt[q] - (slot - pre) * BM);
                }
                pre += tiles[q];
            }
        }
    }
    __syncthreads();
    e = st[0];
    row0 = st[1];
    rows = st[2];
    return e >= 0;
}

// MODE 0: gate/up + SwiGLU -> f32 h [rows][N];  MODE 1: down -> f32 y [rows][N] * pscale;
// MODE 2: gate/up raw integer-weight sums (no scale, no activation) -> f32
// [rows][0:N] (gate) and [rows][N:2N] (up), for the exactness test.
template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_ffn(FfnArgs a)
{
    constexpr int NMAT = (MODE == 1) ? 1 : 2;
    constexpr int BKB = FF_BK * WBITS / 8;        // bytes of a B row per stage
    constexpr int LDB = BKB + 16;                 // LDS B row stride in bytes
    constexpr int BROWS = NMAT * BN;
    constexpr int A_CHUNKS = BM * FF_BK / 8;      // 16-byte chunks of A per stage
    constexpr int B_CPR = BKB / 16;               // 16-byte chunks per B row per stage
    constexpr int B_CHUNKS = BROWS * B_CPR;
    constexpr int A_PT = (A_CHUNKS + 255) / 256;  // per thread
    constexpr int B_PT = (B_CHUNKS + 255) / 256;
    constexpr int MB = BM / WM / 16;
    constexpr int NB = BN / WN / 16;
    constexpr int AW = (MODE == 1) ? 2 : 1;       // 16-byte loads per 8-element A chunk (f32 h: 2)
    constexpr int NPLANE = (MODE == 1) ? 2 : 1;   // bf16 planes of A in LDS (hi, lo)
    static_assert(WM * WN == 4, "four waves");
    static_assert(MB >= 1 && NB >= 1, "wave tile");

    __shared__ __attribute__((aligned(16))) uint16_t sA[NPLANE * BM * FF_LDA];
    __shared__ __attribute__((aligned(16))) uint8_t sB[BROWS * LDB];
    __shared__ float sRow[BM];

    const int NT = a.N / BN;
    const int slot = blockIdx.x / NT;
    const int nt = blockIdx.x % NT;
    int e, row0, rows;
    if (!find_tile<BM>(a, slot, e, row0, rows)) return;
    const int n0 = nt * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // A source rows for this thread's chunks (fixed across stages)
    const uint8_t *asrc[A_PT];  // bytes; A elements are bf16 (gate/up) or f32 (down)
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        const int c = tid + i * 256;
        const int m = c / 8;
        asrc[i] = nullptr;
        if (c < A_CHUNKS && m < rows) {
            const int r = row0 + m;
            const int src = a.gather ? a.gather[r] / a.kdiv : r;
            asrc[i] = (const uint8_t *)a.A + ((size_t)src * a.lda + (c % 8) * 8) * (AW * 2);
        }
    }
    const uint8_t *bsrc[B_PT];
    const size_t brow_bytes = (size_t)a.K * WBITS / 8;
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
        const int c = tid + i * 256;
        bsrc[i] = nullptr;
        if (c < B_CHUNKS) {
            const int rr = c / B_CPR, cc = c % B_CPR;
            const int mat = rr / BN, n = rr % BN;
            const uint8_t *q = (mat == 0) ? a.q0 : a.q1;
            bsrc[i] = q + (size_t)e * a.qstride + (size_t)(n0 + n) * brow_bytes + cc * 16;
        }
    }

    u32x4 ra[A_PT][AW], rb[B_PT];
    float rsum[A_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) rsum[i] = 0.f;

    auto load_stage = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PT; ++i)
#pragma unroll
            for (int h = 0; h < AW; ++h)
                ra[i][h] = asrc[i] ? *(const u32x4 *)(asrc[i] + (size_t)kt * FF_BK * AW * 2 + h * 16)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < B_PT; ++i)
            if (bsrc[i]) rb[i] = *(const u32x4 *)(bsrc[i] + kt * BKB);
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int c = tid + i * 256;
            if (c < A_CHUNKS) {
                float s = 0.f;
                u32x4 v, vlo;
                if constexpr (MODE == 1) {
                    // eight f32 -> bf16 hi and bf16 lo planes
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        uint32_t pr[2], pl[2];
#pragma unroll
                        for (int e2 = 0; e2 < 2; ++e2) {
                            const float f = __uint_as_float(ra[i][d / 2][(d % 2) * 2 + e2]);
                            const uint32_t hb = f32_to_bf16(f);
                            const float hf = __uint_as_float(hb << 16);
                            const uint32_t lb = f32_to_bf16(f - hf);
                            s += hf + __uint_as_float(lb << 16);
                            pr[e2] = hb;
                            pl[e2] = lb;
                        }
                        v[d] = pr[0] | (pr[1] << 16);
                        vlo[d] = pl[0] | (pl[1] << 16);
                    }
                } else {
                    v = ra[i][0];
#pragma unroll
                    for (int d = 0; d < 4; ++d) s += bf16_lo(v[d]) + bf16_hi(v[d]);
                }
                rsum[i] += s;
                if constexpr (WBITS == 4) {
                    v = interleave_bf16x8(v);
                    if constexpr (MODE == 1) vlo = interleave_bf16x8(vlo);
                }
                *(u32x4 *)(sA + (c / 8) * FF_LDA + (c % 8) * 8) = v;
                if constexpr (MODE == 1) *(u32x4 *)(sA + BM * FF_LDA + (c / 8) * FF_LDA + (c % 8) * 8) = vlo;
            }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int c = tid + i * 256;
            if (c < B_CHUNKS) *(u32x4 *)(sB + (c / B_CPR) * LDB + (c % B_CPR) * 16) = rb[i];
        }
    };

    f32x4 acc[NMAT][MB][NB];
#pragma unroll
    for (int x = 0; x < NMAT; ++x)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[x][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = a.K / FF_BK;
    load_stage(0);
    store_stage();
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) load_stage(kt + 1);
#pragma unroll
        for (int ks = 0; ks < FF_BK / 32; ++ks) {
            u32x4 af[NPLANE][MB];
#pragma unroll
            for (int pl = 0; pl < NPLANE; ++pl)
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    af[pl][i] = *(const u32x4 *)(sA + pl * BM * FF_LDA +
                                                 (wm * (BM / WM) + i * 16 + (lane & 15)) * FF_LDA + ks * 32 +
                                                 (lane >> 4) * 8);
#pragma unroll
            for (int x = 0; x < NMAT; ++x)
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const uint8_t *bp = sB + (x * BN + wn * (BN / WN) + j * 16 + (lane & 15)) * LDB;
                    u32x4 bf;
                    if (WBITS == 4) {
                        bf = unpack_int4x8(*(const uint32_t *)(bp + ks * 16 + (lane >> 4) * 4));
                    } else {
                        bf = unpack_int8x8(*(const u32x2 *)(bp + ks * 32 + (lane >> 4) * 8));
                    }
#pragma unroll
                    for (int pl = 0; pl < NPLANE; ++pl)
#pragma unroll
                        for (int i = 0; i < MB; ++i) acc[x][i][j] = mfma_bf16(af[pl][i], bf, acc[x][i][j]);
                }
        }
        __syncthreads();
        if (kt + 1 < KT) {
            store_stage();
            __syncthreads();
        }
    }

    // row sums of A: the 8 threads of a row are 8 consecutive lanes
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        float s = rsum[i];
        s += __shfl_xor(s, 1, WAVE);
        s += __shfl_xor(s, 2, WAVE);
        s += __shfl_xor(s, 4, WAVE);
        const int c = tid + i * 256;
        if (c < A_CHUNKS && (c % 8) == 0) sRow[c / 8] = s;
    }
    __syncthreads();

    const float bias = (WBITS == 4) ? INT4_BIAS : 0.f;
    const float *sc0 = a.s0 + (size_t)e * a.sstride;
    const float *sc1 = (MODE != 1) ? a.s1 + (size_t)e * a.sstride : nullptr;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + r;
            if (m >= rows) continue;
            const float corr = bias * sRow[m];
            const int row = row0 + m;
            if constexpr (MODE == 0) {
                float *o = (float *)a.out + (size_t)row * a.ldo;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
                    const float g = (acc[0][i][j][r] - corr) * sc0[n];
                    const float u = (acc[1][i][j][r] - corr) * sc1[n];
                    o[n] = silu(g) * u;
                }
            } else if constexpr (MODE == 2) {
                float *o = (float *)a.out + (size_t)row * a.ldo;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
                    o[n] = acc[0][i][j][r] - corr;
                    o[a.N + n] = acc[1][i][j][r] - corr;
                }
            } else {
                float *o = (float *)a.out + (size_t)row * a.ldo;
                const float ps = (a.pscale && a.pair_of_row) ? a.pscale[a.pair_of_row[row]] : 1.f;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
                    o[n] = (acc[0][i][j][r] - corr) * sc0[n] * ps;
                }
            }
        }
}

// ------------------------------------------------------------------ launchers

// m-tile row count for a regime: mean rows per group decides
int ffn_bm(int rows, int groups)
{
    const int mean = groups > 0 ? rows / groups : rows;
    if (mean < 24) return 16;
    if (mean < 96) return 64;
    return 128;
}

template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
static hipError_t launch_one(const FfnArgs &a, int slots, hipStream_t st)
{
    const int NT = a.N / BN;
    const long grid = (long)slots * NT;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((k_ffn<MODE, WBITS, BM, BN, WM, WN>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

// slots = upper bound on m-tiles over all groups
template <int MODE, int WBITS>
static hipError_t launch_mode(const FfnArgs &a, int rows_total, int groups, hipStream_t st)
{
    const int bm = ffn_bm(rows_total, groups);
    const int ng = a.offsets ? groups : 1;
    const int slots = (rows_total + bm - 1) / bm + (a.offsets ? min(ng, rows_total) : 0);
    if constexpr (MODE != 1) {
        if (bm == 16) return launch_one<MODE, WBITS, 16, 64, 1, 4>(a, slots, st);
        if (bm == 64) return launch_one<MODE, WBITS, 64, 64, 2, 2>(a, slots, st);
        return launch_one<MODE, WBITS, 128, 64, 2, 2>(a, slots, st);
    } else {
        if (bm == 16) return launch_one<MODE, WBITS, 16, 64, 1, 4>(a, slots, st);
        if (bm == 64) return launch_one<MODE, WBITS, 64, 128, 2, 2>(a, slots, st);
        return launch_one<MODE, WBITS, 128, 128, 2, 2>(a, slots, st);
    }
}

hipError_t launch_ffn(int mode, int wbits, const FfnArgs &a, int rows_total, int groups, hipStream_t st)
{
    if (mode == 2) return launch_mode<2, 4>(a, rows_total, groups, st);
    if (mode == 0) return wbits == 4 ? launch_mode<0, 4>(a, rows_total, groups, st)
                                     : launch_mode<0, 8>(a, rows_total, groups, st);
    return wbits == 4 ? launch_mode<1, 4>(a, rows_total, groups, st) : launch_mode<1, 8>(a, rows_total, groups, st);
}

}  // namespace moe

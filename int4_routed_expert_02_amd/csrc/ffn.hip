// ffn.hip -- grouped GEMMs of the SwiGLU experts on int4 (or int8) per-row weights.
//
// Batch-union (colibri README, "What's implemented"): the pairs are grouped by
// expert, so one tile of rows reads one expert's weights once and applies them
// to every row routed to it.  Weights are per-row symmetric with one f32 scale
// per row (colibri-nano README, "Converting a checkpoint yourself"); an
// expert's three matrices are gate [I][H], up [I][H], down [H][I].
//
// Gate/up runs on bf16 matrix cores (v_mfma_f32_16x16x32_bf16, the
// activations' own format), down on f16 matrix cores (v_mfma_f32_16x16x32_f16)
// with h = silu(g) * u carried in f16; both accumulate in f32.  Weights are
// unpacked in registers right before the MFMA, with an OR of exponent bits:
// int4 becomes q + 136 in bf16 or q + 1032 in f16, int8 becomes q + 1152 in
// f16 (gate/up converts int8 exactly to bf16).  The constant times the A row
// sum is taken out again, either by one more MFMA against a constant fragment
// or from row sums of the same 16-bit values the MFMA consumes.  The per-row
// weight scale, SiLU * up (gate/up) and the per-pair combine weight rsf * w
// (down) are applied in the epilogue.
//
// h in f16 rounds each value with a 2^-11 relative error, a quarter of one
// bf16 rounding (which alone left about 1e-2 of the output RMS at the tails
// of a large batch); f16 holds |h| up to 65504.  The gate/up kernel writes h
// already in the k-slot order the down kernel's int4 unpack uses.
//
// Tiles of 64 and 128 rows (k_ffn3) are 128 output columns wide, gate and up
// of the same 128 intermediate rows in one workgroup; a wave holds up to
// 64 x 64 outputs per matrix, so each unpacked weight fragment feeds up to
// four MFMAs.  Tiles of 16 rows, and widths that are not a multiple of 128,
// use the register-staged k_ffn.
//
// Tiles.  A launch covers every (m-tile, n-tile) of every expert without
// reading the histogram back to the host: the grid is an upper bound
// (ceil(rows/BM) + experts m-tile slots, times n-tiles) and each workgroup
// finds its expert and first row from the offsets; surplus workgroups exit.
#include "ffn_common.h"

namespace moe {

// MODE 0: gate/up + SwiGLU -> h as f16 [M][N] (see hpos);
// MODE 1: down -> f32 y [rows][N] * pscale, A = that f16 h, f16 matrix cores;
// MODE 2: gate/up raw integer-weight sums (no scale, no activation) -> f32
// [rows][0:N] (gate) and [rows][N:2N] (up), for the exactness test.
template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
struct FfShape {
    static constexpr int NMAT = (MODE == 1) ? 1 : 2;
    static constexpr int BKB = FF_BK * WBITS / 8;  // bytes of a B row per stage
    static constexpr int LDB = BKB + 16;           // LDS B row stride in bytes
    static constexpr int ABUF = BM * FF_LDA;       // bf16 elements of one A buffer
    static constexpr int BBUF = NMAT * BN * LDB;   // bytes of one B buffer
};

// One (m-tile, n-tile) of expert e: rows [row0, row0 + rows), columns
// [n0, n0 + BN), weights in the WBITS format; sA / sB / sRow: the kernel's LDS.
template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
__device__ __forceinline__ void ffn_tile(const FfnArgs &a, int e, int row0, int rows, int n0, uint16_t *sA,
                                         uint8_t *sB, float *sRow)
{
    constexpr int NMAT = (MODE == 1) ? 1 : 2;
    constexpr int NPLANE = 1;
    constexpr bool F16 = (MODE == 1);             // A is f16 h, weights unpack to f16
    constexpr int BKB = FF_BK * WBITS / 8;        // bytes of a B row per stage
    constexpr int LDB = BKB + 16;                 // LDS B row stride in bytes
    constexpr int BROWS = NMAT * BN;
    constexpr int A_CHUNKS = NPLANE * BM * FF_BK / 8;  // 16-byte chunks of A per stage
    constexpr int B_CPR = BKB / 16;               // 16-byte chunks per B row per stage
    constexpr int B_CHUNKS = BROWS * B_CPR;
    constexpr int A_PT = (A_CHUNKS + 255) / 256;  // per thread
    constexpr int B_PT = (B_CHUNKS + 255) / 256;
    constexpr int MB = BM / WM / 16;
    constexpr int NB = BN / WN / 16;
    constexpr int ABUF = NPLANE * BM * FF_LDA;    // bf16 elements of one A buffer
    constexpr int BBUF = BROWS * LDB;             // bytes of one B buffer
    static_assert(WM * WN == 4, "four waves");
    static_assert(MB >= 1 && NB >= 1, "wave tile");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // A source of this thread's chunks (fixed across stages): chunk c is
    // (plane, row m, 8-column group c % 8)
    const uint16_t *asrc[A_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        const int c = tid + i * 256;
        const int pl = c / (BM * 8), m = (c / 8) % BM;
        asrc[i] = nullptr;
        if (c < A_CHUNKS && m < rows) {
            const int r = row0 + m;
            const int src = a.gather ? a.gather[r] / a.kdiv : r;
            asrc[i] = (const uint16_t *)a.A + (size_t)pl * a.M * a.lda + (size_t)src * a.lda + (c % 8) * 8;
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

    u32x4 ra[A_PT], rb[B_PT];
    float rsum[A_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) rsum[i] = 0.f;

    auto load_stage = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PT; ++i)
            ra[i] = asrc[i] ? *(const u32x4 *)(asrc[i] + (size_t)kt * FF_BK) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < B_PT; ++i)
            if (bsrc[i]) rb[i] = *(const u32x4 *)(bsrc[i] + (size_t)kt * BKB);
    };
    auto store_stage = [&](int buf) {
        uint16_t *dA = sA + buf * ABUF;
        uint8_t *dB = sB + buf * BBUF;
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int c = tid + i * 256;
            if (c < A_CHUNKS) {
                u32x4 v = ra[i];
                float s = 0.f;
#pragma unroll
                for (int d = 0; d < 4; ++d) s += F16 ? f16_lo(v[d]) + f16_hi(v[d]) : bf16_lo(v[d]) + bf16_hi(v[d]);
                rsum[i] += s;
                // gate/up: the activations take the int4 k-slot order here;
                // down: h is stored in that order already
                if (WBITS == 4 && MODE != 1) v = interleave_bf16x8(v);
                *(u32x4 *)(dA + (c / 8) * FF_LDA + (c % 8) * 8) = v;
            }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int c = tid + i * 256;
            if (c < B_CHUNKS) *(u32x4 *)(dB + (c / B_CPR) * LDB + (c % B_CPR) * 16) = rb[i];
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
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_stage(kt + 1);
        const uint16_t *cA = sA + buf * ABUF;
        const uint8_t *cB = sB + buf * BBUF;
#pragma unroll
        for (int ks = 0; ks < FF_BK / 32; ++ks) {
            u32x4 af[NPLANE][MB];
#pragma unroll
            for (int pl = 0; pl < NPLANE; ++pl)
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    af[pl][i] = *(const u32x4 *)(cA + pl * BM * FF_LDA +
                                                 (wm * (BM / WM) + i * 16 + (lane & 15)) * FF_LDA + ks * 32 +
                                                 (lane >> 4) * 8);
#pragma unroll
            for (int x = 0; x < NMAT; ++x)
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const uint8_t *bp = cB + (x * BN + wn * (BN / WN) + j * 16 + (lane & 15)) * LDB;
                    u32x4 bf;
                    if (WBITS == 4) {
                        const uint32_t w = *(const uint32_t *)(bp + ks * 16 + (lane >> 4) * 4);
                        bf = F16 ? unpack_int4x8_f16(w) : unpack_int4x8(w);
                    } else if (WBITS == 2) {
                        const uint32_t w = *(const uint16_t *)(bp + ks * 8 + (lane >> 4) * 2);
                        bf = F16 ? unpack_int2x8<0x6400u>(w) : unpack_int2x8<0x4300u>(w);
                    } else {
                        const u32x2 w = *(const u32x2 *)(bp + ks * 32 + (lane >> 4) * 8);
                        bf = F16 ? unpack_int8x8_f16(w) : unpack_int8x8(w);
                    }
#pragma unroll
                    for (int pl = 0; pl < NPLANE; ++pl)
#pragma unroll
                        for (int i = 0; i < MB; ++i)
                            acc[x][i][j] = F16 ? mfma_f16(af[pl][i], bf, acc[x][i][j])
                                               : mfma_bf16(af[pl][i], bf, acc[x][i][j]);
                }
        }
        if (kt + 1 < KT) store_stage(buf ^ 1);  // the other buffer: last read before the previous barrier
        __syncthreads();
    }

    // row sums of A: the 8 threads of a row are 8 consecutive lanes
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        float s = rsum[i];
        s += __shfl_xor(s, 1, WAVE);
        s += __shfl_xor(s, 2, WAVE);
        s += __shfl_xor(s, 4, WAVE);
        rsum[i] = s;
    }
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        const int c = tid + i * 256;
        if (c < A_CHUNKS && (c % 8) == 0) sRow[c / 8] = rsum[i];
    }
    __syncthreads();

    const float bias = F16 ? (WBITS == 4 ? INT4_F16_BIAS : WBITS == 2 ? INT2_F16_BIAS : INT8_F16_BIAS)
                           : (WBITS == 4 ? INT4_BIAS : WBITS == 2 ? INT2_BIAS : 0.f);
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
                _Float16 *oh = (_Float16 *)a.out + (size_t)row * a.ldo;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
                    const float g = (acc[0][i][j][r] - corr) * sc0[n];
                    const float u = (acc[1][i][j][r] - corr) * sc1[n];
                    oh[hpos<WBITS>(n)] = (_Float16)(silu(g) * u);
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
                const int pr = a.pair_of_row ? a.pair_of_row[row] : row;
                const float ps = (a.pscale && a.pair_of_row) ? a.pscale[pr] : 1.f;
                const size_t orow = a.out_by_pair ? (size_t)pr : (size_t)row;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
                    const float v = (acc[0][i][j][r] - corr) * sc0[n] * ps;
                    if (a.out_f16)
                        ((uint16_t *)a.out)[orow * a.ldo + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
                    else
                        ((float *)a.out)[orow * a.ldo + n] = v;
                }
            }
        }
}

template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256, 2) void k_ffn(FfnArgs a)
{
    using S = FfShape<MODE, WBITS, BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * S::ABUF];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2 * S::BBUF];
    __shared__ float sRow[BM];
    // XCD-aware placement: workgroup b runs on XCD b % 8; the NT n-tiles of
    // m-tile slot s get workgroups on XCD s % 8, so the slot's activation rows
    // are fetched into one L2 and re-read from there
    const int NT = a.N / BN;
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int nt = q % NT;
    const int slot = (q / NT) * 8 + xcd;
    int e, row0, rows;
    if (!find_tile<BM>(a, slot, e, row0, rows)) return;
    ffn_tile<MODE, WBITS, BM, BN, WM, WN>(a, e, row0, rows, nt * BN, sA, sB, sRow);
}

// A family whose experts are int4 or int2 each (a.ebits): the tile's expert
// decides which body runs; the LDS is sized for int4, the larger stage.
template <int MODE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256, 2) void k_ffn_mix(FfnArgs a)
{
    using S = FfShape<MODE, 4, BM, BN, WM, WN>;
    static_assert(FfShape<MODE, 2, BM, BN, WM, WN>::BBUF <= S::BBUF, "int2 stage fits the int4 one");
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * S::ABUF];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2 * S::BBUF];
    __shared__ float sRow[BM];
    const int NT = a.N / BN;
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int nt = q % NT;
    const int slot = (q / NT) * 8 + xcd;
    int e, row0, rows;
    if (!find_tile<BM>(a, slot, e, row0, rows)) return;
    if (a.ebits[e] == 2)
        ffn_tile<MODE, 2, BM, BN, WM, WN>(a, e, row0, rows, nt * BN, sA, sB, sRow);
    else
        ffn_tile<MODE, 4, BM, BN, WM, WN>(a, e, row0, rows, nt * BN, sA, sB, sRow);
}

// ------------------------------------------------------------------ pipelined tiles (64 and 128 rows)

// Tiles of 64 or 128 rows run a deeper pipeline: global memory is copied
// straight into a ring of LDS stages (global_load_lds, 16 bytes per lane), so
// loads in flight hold no registers and staging costs no vector instructions.
// Three stages, or two when a stage exceeds 24 KB (int8 gate/up at 128
// rows), so that two workgroups fit in a compute unit's 160 KB.  Each wave's copy fills 1 KB of LDS contiguously:
//  - A (16-bit rows of 64 columns = 8 chunks of 16 bytes) is stored with the
//    chunk slot XOR-swizzled by (row % 8), which makes the fragment reads
//    conflict-free;
//  - B rows are raw packed weight bytes.
// The four waves share the tile's rows and split its 128 columns (32 each),
// so one unpacked weight fragment feeds BM / 16 MFMAs.  Gate/up unpacks its
// weights in natural k order (the activations are used as they are); down
// uses the k-slot order h is written in.  The unpack offset is removed with
// one extra MFMA per 16-row block and k-step against a constant fragment
// holding minus the offset: wave w takes the row blocks i = w (mod 4) and the
// results are shared through LDS in the epilogue.

// one weight fragment (8 k values of one output column) from its LDS bytes
template <int MODE, int WBITS>
__device__ __forceinline__ u32x4 weight_fragment(const uint8_t *bp)
{
    if constexpr (WBITS == 4) {
        const uint32_t w = *(const uint32_t *)bp;
        return MODE == 1 ? unpack_int4x8_f16(w) : unpack_int4x8_nat(w);
    } else if constexpr (WBITS == 2) {
        const uint32_t w = *(const uint16_t *)bp;
        return MODE == 1 ? unpack_int2x8<0x6400u>(w) : unpack_int2x8<0x4300u>(w);
    } else {
        const u32x2 w = *(const u32x2 *)bp;
        return MODE == 1 ? unpack_int8x8_f16(w) : unpack_int8x8_bf16o(w);
    }
}

// One (m-tile, n-tile) of expert e in the WBITS format; smem3 / sCor: the
// kernel's LDS (the stage ring, dynamic, and the row corrections).  RS: the
// row sums of A come precomputed (a.rsum) instead of from an MFMA against a
// constant fragment at every k-step (which every n-tile of a row block would
// repeat).
template <int MODE, int WBITS, int BM, int BN = 128, bool RS = false>
__device__ __forceinline__ void ffn3_tile(const FfnArgs &a, int e, int row0, int rows, int n0, uint8_t *smem3,
                                          float *sCor)
{
    using C = Ff3<MODE, WBITS, BM, BN>;
    constexpr int NMAT = C::NMAT, BKB = C::BKB;
    constexpr bool F16 = (MODE == 1);   // down: A is f16 h, weights unpack to f16
    constexpr int MB = BM / 16;         // 16-row blocks, all in every wave
    constexpr int NB = BN / 4 / 16;     // 16-column blocks per wave and matrix
    constexpr int CB = MB / 4;          // offset-correction blocks per wave
    static_assert(MB % 4 == 0, "row blocks split evenly over the waves");
    static_assert(!RS || WBITS != 2, "precomputed row sums: int4 and int8 families");
    const int tid = threadIdx.x, lane = tid & 63, wn = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wn);  // the same, known wave-uniform

    // LDS swizzles of the 64-k stages, so that the fragment reads of 16
    // consecutive lanes hit distinct banks: A rows (128 bytes, 16 rows per
    // read) hold 16-byte chunk c at slot c ^ ((row >> 1) & 7); int4 B rows (32
    // bytes) swap their two chunks when (row >> 3) & 1, int8 B rows (64 bytes)
    // XOR the chunk with (row >> 2) & 3; int2 rows are one chunk.
    auto aswz = [](int r) { return (r >> 1) & 7; };
    auto bswz = [](int r) { return BKB == 32 ? (r >> 3) & 1 : BKB == 64 ? (r >> 2) & 3 : 0; };
    // this lane's source for each of its wave's copies (fixed across stages)
    const uint8_t *src[C::PER_WAVE];
    int dst[C::PER_WAVE];  // byte offset of the wave's 1 KB block within a stage
#pragma unroll
    for (int j = 0; j < C::PER_WAVE; ++j) {
        const int l = wn + 4 * j;  // copy index within the stage
        dst[j] = l * 1024;
        if (l < C::A_LOADS) {
            const int r = l * 8 + lane / 8;  // tile row
            const int chunk = (lane % 8) ^ aswz(r);
            const int rr = r < rows ? r : 0;  // padded rows read row 0 (outputs discarded)
            const int srow = a.gather ? a.gather[row0 + rr] / a.kdiv : row0 + rr;
            src[j] = (const uint8_t *)a.A + ((size_t)srow * a.lda + chunk * 8) * 2;
        } else {
            const int lb = l < C::A_LOADS + C::B_LOADS ? l - C::A_LOADS : 0;  // a padding copy repeats B copy 0
            const int cpr = BKB / 16;                     // 16-byte chunks per B row per stage
            const int br = lb * (64 / cpr) + lane / cpr;  // B row within the stage
            const int mat = br / BN, n = br % BN;
            const uint8_t *qm = (mat == 0) ? a.q0 : a.q1;
            src[j] = qm + (size_t)e * a.qstride + (size_t)(n0 + n) * (size_t)a.K * WBITS / 8 +
                     ((lane % cpr) ^ bswz(br)) * 16;
        }
    }
    // Copy j < A_LOADS / 4 of every wave is an A copy (8 rows).  Only the
    // first AJ of them are issued: rows past 32 AJ are never read.  The ring
    // is laid out for the tile's valid rows: a stage holds 4 AJ KB of A, then
    // the B copies, and the ring takes as many such stages as the space
    // reserved for NST full-height stages holds (more weight bytes in flight
    // when a group has fewer rows than the tile height).
    auto issue = [&](int kt, auto ajc, auto nsc) {
        constexpr int AJ = decltype(ajc)::value, NS = decltype(nsc)::value;
        constexpr int ABY = 4 * AJ * 1024, SBY = ABY + (C::LOADS - C::A_LOADS) * 1024;
        uint8_t *base = smem3 + (kt % NS) * SBY;
#pragma unroll
        for (int j = 0; j < C::PER_WAVE; ++j) {
            if (j >= AJ && j < C::A_LOADS / 4) continue;
            const bool isa = j < C::A_LOADS / 4;
            const size_t adv = isa ? (size_t)kt * FF_BK * 2 : (size_t)kt * BKB;
            lds_copy16(src[j] + adv, base + (isa ? dst[j] : ABY + dst[j] - C::A_BYTES));
        }
    };

    // The products run as W x A^T (weights are the MFMA's first operand), so
    // a lane ends up holding four consecutive output columns of one row.
    f32x4 acc[NMAT][MB][NB];
    f32x4 cor[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) cor[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NMAT; ++x)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[x][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // minus the unpack offset as a constant operand: bf16 -136 / -130 / -128, f16 -1032 / -1026 / -1152
    constexpr uint32_t CW = F16 ? (WBITS == 4 ? 0xE408E408u : WBITS == 2 ? 0xE402E402u : 0xE480E480u)
                                : (WBITS == 4 ? 0xC308C308u : WBITS == 2 ? 0xC302C302u : 0xC300C300u);
    const u32x4 cneg = u32x4{CW, CW, CW, CW};
    auto mma = [](u32x4 x, u32x4 y, f32x4 c) { return F16 ? mfma_f16(x, y, c) : mfma_bf16(x, y, c); };

    const int KT = a.K / FF_BK;
    // The k loop, specialised on MV, the number of 16-row blocks holding valid
    // rows: rows past the tile's last 32-row group are not copied, and blocks
    // past its last row take no fragment reads and no MFMAs (a group's last
    // tile is often mostly padding).
    auto kloop = [&](auto mvc) {
        constexpr int MV = decltype(mvc)::value;
        constexpr int AJ = (MV + 1) / 2;                       // A copies per wave and stage
        constexpr int PW = C::PER_WAVE - (C::A_LOADS / 4 - AJ);  // copies per wave and stage
        constexpr int ABY = 4 * AJ * 1024, SBY = ABY + (C::LOADS - C::A_LOADS) * 1024;  // compact stage
        constexpr int NS_FIT = C::RING / SBY, NS_CNT = 2 + 63 / PW;
        constexpr int NS = NS_FIT < NS_CNT ? (NS_FIT < 8 ? NS_FIT : 8) : (NS_CNT < 8 ? NS_CNT : 8);
        static_assert(NS >= C::NST && PW * (NS - 2) < 64, "ring");
        const IntC<AJ> ajc;
        const IntC<NS> nsc;
#pragma unroll
        for (int s0 = 0; s0 < NS - 1; ++s0)
            if (s0 < KT) issue(s0, ajc, nsc);
        for (int kt = 0; kt < KT; ++kt) {
            // stage kt has landed once at most the later stages' copies are outstanding
            wait_stages<PW, NS - 2>(KT - 1 - kt);
            ring_barrier();  // every wave's copies of stage kt are in LDS; stage kt - 1 is free
            if (kt + NS - 1 < KT) issue(kt + NS - 1, ajc, nsc);
            const uint8_t *sa = smem3 + (kt % NS) * SBY;
            const uint8_t *sb = sa + ABY;
#pragma unroll
            for (int ks = 0; ks < FF_BK / 32; ++ks) {
                u32x4 af[MV];
#pragma unroll
                for (int i = 0; i < MV; ++i) {
                    const int r = i * 16 + (lane & 15);
                    const int chunk = ks * 4 + (lane >> 4);
                    af[i] = *(const u32x4 *)(sa + r * 128 + ((chunk ^ aswz(r)) * 16));
                }
                // (the correction blocks depend on the wave, so their fragments
                // are read again rather than picked from af by a run-time index;
                // a block past the valid ones is skipped, by a wave-uniform test)
                if constexpr (!RS) {
#pragma unroll
                    for (int c = 0; c < CB; ++c) {
                        if (4 * c >= MV) break;
                        if (4 * c + 3 >= MV && wu + 4 * c >= MV) continue;
                        const int r = (wn + 4 * c) * 16 + (lane & 15);
                        const int chunk = ks * 4 + (lane >> 4);
                        cor[c] = mma(cneg, *(const u32x4 *)(sa + r * 128 + ((chunk ^ aswz(r)) * 16)), cor[c]);
                    }
                }
#pragma unroll
                for (int x = 0; x < NMAT; ++x)
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const int br = x * BN + wn * (BN / 4) + j * 16 + (lane & 15);
                        const int bo = ks * (BKB / 2) + (lane >> 4) * (WBITS / 2) * 2;  // byte in the row
                        const u32x4 bf = weight_fragment<MODE, WBITS>(sb + br * BKB +
                                                                      (((bo >> 4) ^ bswz(br)) << 4) + (bo & 15));
#pragma unroll
                        for (int i = 0; i < MV; ++i) acc[x][i][j] = mma(bf, af[i], acc[x][i][j]);
                    }
            }
        }
    };
    // Tiles of few valid rows with int4 weights take 128-k stages instead
    // (kloop128): a weight copy is then 16 rows x 64 bytes, half the
    // requests per weight byte of the 32-byte rows above (the request rate,
    // not the bytes, limits the copies of a weight-bound tile), and the
    // compact stage of the valid rows still leaves two stages in the ring.
    // Lane l of a copy of block b loads row l % 16 of the block, bytes
    // 16 (l / 16) .. + 16 of the stage's 64; global_load_lds puts it at 16 l,
    // so the wave that multiplies block b reads its own 16 bytes back with
    // one conflict-free LDS read.  k-slots: lane group g holds k = 32 g + v of
    // the stage, MFMA j takes v = 8 j .. 8 j + 7; the A fragment of lane
    // (row, g) for j is the 16-byte chunk 4 g + j of the row (256-byte rows,
    // chunk slots XOR-swizzled by the row's low four bits).
    auto kloop128 = [&](auto mvc) {
        constexpr int MV = decltype(mvc)::value;
        constexpr int NBLK = NMAT * BN / 16;               // 16-row weight blocks of the tile
        constexpr int BJ = NBLK / 4;                        // weight copies per wave and stage
        constexpr int PW = MV + BJ;                         // copies per wave and stage (MV of A)
        constexpr int ABY = MV * 4 * 1024, SBY = ABY + NBLK * 1024;
        constexpr int NS_FIT = C::RING / SBY, NS_CNT = 2 + 63 / PW;
        constexpr int NS = NS_FIT < NS_CNT ? (NS_FIT < 8 ? NS_FIT : 8) : (NS_CNT < 8 ? NS_CNT : 8);
        static_assert(NS >= 2 && PW * (NS - 2) < 64, "ring");
        const int KT2 = a.K / 128;
        const uint8_t *as[MV];
#pragma unroll
        for (int j = 0; j < MV; ++j) {
            const int c = wn + 4 * j;  // copy c: rows 4c .. 4c + 3
            const int r = 4 * c + lane / 16;
            const int rr = r < rows ? r : 0;
            const int srow = a.gather ? a.gather[row0 + rr] / a.kdiv : row0 + rr;
            as[j] = (const uint8_t *)a.A + ((size_t)srow * a.lda + (((lane & 15) ^ (r & 15)) * 8)) * 2;
        }
        const uint8_t *bs[BJ];
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
            const int b = wn + 4 * j;  // block b: matrix b / (BN / 16), rows 16 (b % (BN / 16)) ..
            const uint8_t *qm = (b / (BN / 16) == 0) ? a.q0 : a.q1;
            const int n = (b % (BN / 16)) * 16 + (lane & 15);
            bs[j] = qm + (size_t)e * a.qstride + (size_t)(n0 + n) * (size_t)(a.K / 2) + (lane >> 4) * 16;
        }
        auto issue2 = [&](int kt) {
            uint8_t *base = smem3 + (kt % NS) * SBY;
#pragma unroll
            for (int j = 0; j < MV; ++j) lds_copy16(as[j] + (size_t)kt * 256, base + (wn + 4 * j) * 1024);
#pragma unroll
            for (int j = 0; j < BJ; ++j) lds_copy16(bs[j] + (size_t)kt * 64, base + ABY + (wn + 4 * j) * 1024);
        };
#pragma unroll
        for (int s0 = 0; s0 < NS - 1; ++s0)
            if (s0 < KT2) issue2(s0);
        for (int kt = 0; kt < KT2; ++kt) {
            wait_stages<PW, NS - 2>(KT2 - 1 - kt);
            ring_barrier();
            if (kt + NS - 1 < KT2) issue2(kt + NS - 1);
            const uint8_t *sa = smem3 + (kt % NS) * SBY;
            // this wave's weight blocks: matrix x, column block wn * NB + j
            u32x4 bw[NMAT][NB];
#pragma unroll
            for (int x = 0; x < NMAT; ++x)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    bw[x][j] = *(const u32x4 *)(sa + ABY + (x * (BN / 16) + wn * NB + j) * 1024 + lane * 16);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int chunk = 4 * (lane >> 4) + jj;
                u32x4 af[MV];
#pragma unroll
                for (int i = 0; i < MV; ++i) {
                    const int r = i * 16 + (lane & 15);
                    af[i] = *(const u32x4 *)(sa + r * 256 + ((chunk ^ (r & 15)) * 16));
                }
                if constexpr (!RS) {
#pragma unroll
                    for (int c = 0; c < CB; ++c) {
                        if (4 * c >= MV) break;
                        if (4 * c + 3 >= MV && wu + 4 * c >= MV) continue;
                        const int r = (wn + 4 * c) * 16 + (lane & 15);
                        cor[c] = mma(cneg, *(const u32x4 *)(sa + r * 256 + ((chunk ^ (r & 15)) * 16)), cor[c]);
                    }
                }
#pragma unroll
                for (int x = 0; x < NMAT; ++x)
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const u32x4 bf = F16 ? unpack_int4x8_f16(bw[x][j][jj]) : unpack_int4x8_nat(bw[x][j][jj]);
#pragma unroll
                        for (int i = 0; i < MV; ++i) acc[x][i][j] = mma(bf, af[i], acc[x][i][j]);
                    }
            }
        }
    };
    const int mv = (rows + 15) / 16;  // 1 .. MB
    if constexpr (WBITS == 4 && MB == 8) {
        if (a.K % 128 == 0 && mv <= 5) {
            switch (mv) {
            case 1: kloop128(IntC<1>{}); break;
            case 2: kloop128(IntC<2>{}); break;
            case 3: kloop128(IntC<3>{}); break;
            case 4: kloop128(IntC<4>{}); break;
            default: kloop128(IntC<5>{}); break;
            }
            goto epilogue;
        }
    }
    if constexpr (WBITS == 4 && MB == 4 && MODE == 1) {
        // the down GEMM's 64-row tiles: 128-k stages throughout (its 64-k
        // stages carry too few MFMAs per barrier and per LDS round trip)
        if (a.K % 128 == 0) {
            switch (mv) {
            case 1: kloop128(IntC<1>{}); break;
            case 2: kloop128(IntC<2>{}); break;
            case 3: kloop128(IntC<3>{}); break;
            default: kloop128(IntC<4>{}); break;
            }
            goto epilogue;
        }
    }
    if constexpr (MB == 4) {
        switch (mv) {
        case 1: kloop(IntC<1>{}); break;
        case 2: kloop(IntC<2>{}); break;
        case 3: kloop(IntC<3>{}); break;
        default: kloop(IntC<4>{}); break;
        }
    } else {
        static_assert(MB == 8, "64- or 128-row tiles");
        switch (mv) {
        case 1: kloop(IntC<1>{}); break;
        case 2: kloop(IntC<2>{}); break;
        case 3: kloop(IntC<3>{}); break;
        case 4: kloop(IntC<4>{}); break;
        case 5: kloop(IntC<5>{}); break;
        case 6: kloop(IntC<6>{}); break;
        case 7: kloop(IntC<7>{}); break;
        default: kloop(IntC<8>{}); break;
        }
    }

epilogue:
    // Epilogue.  Lane l holds, for block (i, j), row m = 16 i + l % 16 and the
    // columns 4 (l / 16) .. 4 (l / 16) + 3 of its 16 x 16 block; the offset
    // correction of every row comes back from sCor.
    if constexpr (RS) {
        // minus the unpack offset times the row's sum: MODE 0/2 one sum per
        // source row of A, MODE 1 rsum_parts partials added in order
        constexpr float CF = F16 ? (WBITS == 4 ? -1032.f : -1152.f) : (WBITS == 4 ? -136.f : -128.f);
        for (int m = tid; m < rows; m += 256) {
            const int row = row0 + m;
            float sum = 0.f;
            if constexpr (MODE == 1) {
                const float *pp = a.rsum + (size_t)row * a.rsum_parts;
                for (int p = 0; p < a.rsum_parts; ++p) sum += pp[p];
            } else {
                sum = a.rsum[a.gather ? a.gather[row] / a.kdiv : row];
            }
            sCor[m] = CF * sum;
        }
    } else {
#pragma unroll
        for (int c = 0; c < CB; ++c)
            if (lane < 16) sCor[(wn + 4 * c) * 16 + lane] = cor[c][0];
    }
    const int mloc = lane & 15;
    const int nloc = wn * (BN / 4) + 4 * (lane >> 4);
    const size_t sbase = (size_t)e * a.sstride + n0 + nloc;
    if constexpr (MODE == 0) {
        // h = silu(g) * u in f16, staged in LDS in natural column order
        // (8-byte writes), then copied out as whole rows with the down
        // kernel's k-slot order applied on the way
        constexpr int HP = BN * 2 + 16;  // LDS row pitch in bytes
        static_assert(BM * HP <= C::NST * C::STAGE, "the h tile fits in the stage ring");
        f32x4 sg[NB], su[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            sg[j] = *(const f32x4 *)(a.s0 + sbase + j * 16);
            su[j] = *(const f32x4 *)(a.s1 + sbase + j * 16);
        }
        __syncthreads();  // every wave is done reading the stage ring; sCor is complete
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const float c = sCor[i * 16 + mloc];
            uint8_t *hrow = smem3 + (i * 16 + mloc) * HP + nloc * 2;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float g = (acc[0][i][j][r] + c) * sg[j][r];
                    const float u = (acc[1][i][j][r] + c) * su[j][r];
                    h[r] = fast_silu(g) * u;
                }
                *(u32x2 *)(hrow + j * 32) = u32x2{pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3])};
            }
        }
        __syncthreads();
        constexpr int CPR = BN * 2 / 16;  // 16-byte chunks per row
        for (int ci = tid; ci < BM * CPR; ci += 256) {
            const int m = ci / CPR, ch = ci % CPR;
            if (m >= rows) continue;
            u32x4 v = *(const u32x4 *)(smem3 + m * HP + ch * 16);
            // (128-column tiles: a row's sixteen chunks are consecutive lanes)
            if (BN == 128 && a.hsum) {
                // the row's sum over the tile's columns of the f16 values the
                // down GEMM reads: a lane's eight in order, then the row's
                // sixteen lanes by a fixed butterfly
                float hs = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    hs += (float)__builtin_bit_cast(_Float16, (uint16_t)(v[q] & 0xFFFFu));
                    hs += (float)__builtin_bit_cast(_Float16, (uint16_t)(v[q] >> 16));
                }
#pragma unroll
                for (int o = 1; o < CPR; o <<= 1) hs += __shfl_xor(hs, o, WAVE);
                if (ch == 0) a.hsum[(size_t)(row0 + m) * (a.N / BN) + n0 / BN] = hs;
            }
            if (WBITS == 4) v = interleave_bf16x8(v);
            *(u32x4 *)((uint16_t *)a.out + (size_t)(row0 + m) * a.ldo + n0 + ch * 8) = v;
        }
    } else {
        f32x4 sv[NB];
        if constexpr (MODE == 1) {
#pragma unroll
            for (int j = 0; j < NB; ++j) sv[j] = *(const f32x4 *)(a.s0 + sbase + j * 16);
        }
        __syncthreads();  // sCor is complete
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int m = i * 16 + mloc;
            if (m >= rows) continue;
            const int row = row0 + m;
            const float c = sCor[m];
            const size_t o = (size_t)row * a.ldo + n0 + nloc;
            if constexpr (MODE == 2) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    *(f32x4 *)((float *)a.out + o + j * 16) = acc[0][i][j] + c;
                    *(f32x4 *)((float *)a.out + o + a.N + j * 16) = acc[1][i][j] + c;
                }
            } else {
                const int pr = a.pair_of_row ? a.pair_of_row[row] : row;
                const float ps = (a.pscale && a.pair_of_row) ? a.pscale[pr] : 1.f;
                const size_t ob = a.out_by_pair ? (size_t)pr * a.ldo + n0 + nloc : o;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    f32x4 v;
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = (acc[0][i][j][q] + c) * sv[j][q] * ps;
                    if (a.out_f16)
                        *(u32x2 *)((uint16_t *)a.out + ob + j * 16) = u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
                    else
                        *(f32x4 *)((float *)a.out + ob + j * 16) = v;
                }
            }
        }
    }
}

template <int MODE, int WBITS, int BM, int BN = 128, bool RS = false>
__global__ __launch_bounds__(256, 2) void k_ffn3(FfnArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem3[];
    __shared__ float sCor[BM];
    const int NT = a.N / BN;
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int nt = q % NT;
    const int slot = (q / NT) * 8 + xcd;
    int e, row0, rows;
    if (!find_tile<BM>(a, slot, e, row0, rows)) return;
    ffn3_tile<MODE, WBITS, BM, BN, RS>(a, e, row0, rows, nt * BN, smem3, sCor);
}

// A family whose experts are int4 or int2 each (a.ebits): the tile's expert
// picks the body; the dynamic LDS holds the larger ring.
template <int MODE, int BM>
__global__ __launch_bounds__(256, 2) void k_ffn3_mix(FfnArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem3[];
    __shared__ float sCor[BM];
    const int NT = a.N / Ff3<MODE, 4, BM>::BN;
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int nt = q % NT;
    const int slot = (q / NT) * 8 + xcd;
    int e, row0, rows;
    if (!find_tile<BM>(a, slot, e, row0, rows)) return;
    if (a.ebits[e] == 2)
        ffn3_tile<MODE, 2, BM>(a, e, row0, rows, nt * Ff3<MODE, 2, BM>::BN, smem3, sCor);
    else
        ffn3_tile<MODE, 4, BM>(a, e, row0, rows, nt * Ff3<MODE, 4, BM>::BN, smem3, sCor);
}

template <int MODE, int BM>
static hipError_t launch_three_mix(const FfnArgs &a, int slots, hipStream_t st)
{
    const int NT = a.N / 128;
    const long grid = (long)((slots + 7) / 8 * 8) * NT;
    if (grid <= 0) return hipSuccess;
    using C4 = Ff3<MODE, 4, BM>;
    using C2 = Ff3<MODE, 2, BM>;
    const size_t l4 = (size_t)C4::RING, l2 = (size_t)C2::RING;  // the larger ring of the two formats
    hipLaunchKernelGGL((k_ffn3_mix<MODE, BM>), dim3((unsigned)grid), dim3(256), l4 > l2 ? l4 : l2, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ launchers

// m-tile row count.  Few rows per group: 16-row tiles.  Otherwise 128-row
// tiles where they fill the chip's 512 workgroup slots (two per compute
// unit): their estimated count (a group adds half a tile on average) fills at
// least 90% of a round and no round is less than half full; else 64.  Padded
// row blocks cost no MFMAs, so larger tiles mostly save weight re-reads.  The
// int4 down GEMM always takes 64-row tiles (measured never slower: its stage
// is small and the extra workgroups hide its short k loop's prologue).
int ffn_bm(int mode, int wbits, int rows, int groups, int nt)
{
    const int mean = groups > 0 ? rows / groups : rows;
    if (mean < 24) return 16;
    // the int4 down GEMM of a narrow output (fewer than 32 128-column tiles)
    // takes 64-row tiles, its stage being small and more workgroups hiding the
    // short k loop's prologue; a wide one (H = 6144) follows the rule below,
    // which reads each expert's weights fewer times
    if (mode == 1 && wbits == 4 && nt < 32) return 64;
    // a single group of at least 1024 rows (the shared expert) takes 128-row
    // tiles even where they leave slots free: it runs beside the routed
    // experts on the second stream, whose workgroups take those slots (the
    // GLM-class layer's shared gate/up: 1.832 -> 1.816 ms, three alternating
    // pairs on one box)
    if (groups == 1 && rows >= 1024) return 128;
    const long t128 = ((long)rows / 128 + (groups > 1 ? groups / 2 : 0)) * nt;
    const long slots = 512;
    if (t128 < slots * 9 / 10) return 64;
    const long rem = t128 % slots;
    if (rem != 0 && rem < slots / 2 && t128 < 4 * slots) return 64;
    return 128;
}

template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
static hipError_t launch_one(const FfnArgs &a, int slots, hipStream_t st)
{
    const int NT = a.N / BN;
    const long grid = (long)((slots + 7) / 8 * 8) * NT;  // whole groups of 8 slots (see the placement)
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((k_ffn<MODE, WBITS, BM, BN, WM, WN>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int MODE, int WBITS, int BM, int BN = 128>
static hipError_t launch_three(const FfnArgs &a, int slots, hipStream_t st)
{
    const int NT = a.N / BN;
    const long grid = (long)((slots + 7) / 8 * 8) * NT;
    if (grid <= 0) return hipSuccess;
    const size_t lds = (size_t)Ff3<MODE, WBITS, BM, BN>::RING;
    if (a.rsum)
        hipLaunchKernelGGL((k_ffn3<MODE, WBITS, BM, BN, true>), dim3((unsigned)grid), dim3(256), lds, st, a);
    else
        hipLaunchKernelGGL((k_ffn3<MODE, WBITS, BM, BN, false>), dim3((unsigned)grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

// slots = upper bound on m-tiles over all groups.  Output tiles are 128
// columns wide when N allows (64 otherwise); rows per tile by the mean rows
// per group.
template <int MODE, int WBITS>
static hipError_t launch_mode(const FfnArgs &a, int rows_total, int groups, hipStream_t st)
{
    const int bm = ffn_bm(MODE, WBITS, rows_total, groups, a.N % 128 == 0 ? a.N / 128 : a.N / 64);
    const int ng = a.offsets ? groups : 1;
    const int slots = (rows_total + bm - 1) / bm + (a.offsets ? min(ng, rows_total) : 0);
    if (a.N % 128 == 0) {
        if (bm == 16) return launch_one<MODE, WBITS, 16, 128, 1, 4>(a, slots, st);
        if (bm == 64) {
            // the int4 down GEMM of a wide output: 256-column tiles halve the
            // re-reads of its activation rows (per tile as many bytes as its
            // weights); measured faster at H = 6144, slower at H = 1024 (half
            // the workgroups, two instead of three per compute unit)
            if (MODE == 1 && WBITS == 4 && a.N % 256 == 0 && a.N >= 4096)
                return launch_three<MODE, WBITS, 64, 256>(a, slots, st);
            return launch_three<MODE, WBITS, 64>(a, slots, st);
        }
        if constexpr (MODE == 1 && WBITS == 4)
            if (a.N % 256 == 0 && a.N >= 4096) return launch_three<MODE, WBITS, 128, 256>(a, slots, st);
        return launch_three<MODE, WBITS, 128>(a, slots, st);
    }
    if (bm == 16) return launch_one<MODE, WBITS, 16, 64, 1, 4>(a, slots, st);
    if (bm == 64) return launch_one<MODE, WBITS, 64, 64, 2, 2>(a, slots, st);
    return launch_one<MODE, WBITS, 128, 64, 4, 1>(a, slots, st);
}

// ------------------------------------------------- int8 activations (Q8_0-style)
//
// The integer-dot form of the expert matmuls (colibri README, "What's
// implemented": int8 activations against int8 or int4 weights): rows hold
// int8 activation codes with one f32 scale per 32 codes along k, weights int4
// or int8 codes with one f32 scale per row.  Each 32-wide k block is one
// v_mfma_i32_16x16x32_i8 (an exact integer sum), converted and added into f32
// with the row's block scale; the weight row scale comes in the epilogue.
// Int4 weights enter the MFMA as code << 4, sixteen times the code, exact in
// int8 and in the i32 sums; the 1/16 joins the weight scale.  Operands as in
// k_ffn: activations first (a lane ends with four rows of one column).
// MODE 0: gate/up + SwiGLU -> h as f32 [rows][N]; MODE 1: down -> f32
// [rows][N] * pscale.  Staging: registers to a double-buffered LDS tile, the
// rows' two block scales of a stage beside it.

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int FQ_BK = 64;           // k per stage (two blocks)
constexpr int FQ_LDA = FQ_BK + 16;  // LDS A row in bytes (80: the 8-byte fragment reads spread over the banks)

// eight int4 codes (element 2c in the low nibble of byte c) -> eight bytes,
// byte j = code j << 4
__device__ __forceinline__ u32x2 unpack_int4x8_i8(uint32_t w)
{
    const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
    return u32x2{__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u)};
}

__device__ __forceinline__ i32x4 mfma_i8(u32x2 a, u32x2 b)
{
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b),
                                                 i32x4{0, 0, 0, 0}, 0, 0, 0);
}

template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256, 2) void k_ffn_q8(FfnArgs a)
{
    constexpr int NMAT = (MODE == 0) ? 2 : 1;
    constexpr int BKB = FQ_BK * WBITS / 8;  // bytes of a B row per stage
    constexpr int LDB = BKB + 16;
    constexpr int BROWS = NMAT * BN;
    constexpr int A_CHUNKS = BM * FQ_BK / 16;  // 16-byte chunks of A per stage (four per row)
    constexpr int B_CPR = BKB / 16;
    constexpr int B_CHUNKS = BROWS * B_CPR;
    constexpr int A_PT = (A_CHUNKS + 255) / 256;
    constexpr int B_PT = (B_CHUNKS + 255) / 256;
    constexpr int MB = BM / WM / 16;
    constexpr int NB = BN / WN / 16;
    static_assert(WM * WN == 4, "four waves");
    static_assert(MB >= 1 && NB >= 1 && BM <= 256, "wave tile");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * FQ_LDA];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BROWS * LDB];
    __shared__ __attribute__((aligned(16))) float sD[2][2][BM];  // [buffer][block of the stage][row]

    // XCD-aware placement as in k_ffn
    const int NT = a.N / BN;
    const int xcd = blockIdx.x & 7, qq = blockIdx.x >> 3;
    const int nt = qq % NT;
    const int slot = (qq / NT) * 8 + xcd;
    int e, row0, rows;
    if (!find_tile<BM>(a, slot, e, row0, rows)) return;
    const int n0 = nt * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int KB = a.K / 32;  // scale blocks per row

    const int8_t *asrc[A_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        const int c = tid + i * 256, m = c / 4;
        asrc[i] = nullptr;
        if (c < A_CHUNKS && m < rows) {
            const int r = row0 + m;
            const int src = a.gather ? a.gather[r] / a.kdiv : r;
            asrc[i] = (const int8_t *)a.A + (size_t)src * a.lda + (c % 4) * 16;
        }
    }
    const float *dsrc = nullptr;
    if (tid < rows) {
        const int r = row0 + tid;
        const int src = a.gather ? a.gather[r] / a.kdiv : r;
        dsrc = a.ad + (size_t)src * KB;
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

    u32x4 ra[A_PT], rb[B_PT];
    u32x2 rd = u32x2{0u, 0u};
    auto load_stage = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PT; ++i)
            ra[i] = asrc[i] ? *(const u32x4 *)(asrc[i] + (size_t)kt * FQ_BK) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < B_PT; ++i)
            if (bsrc[i]) rb[i] = *(const u32x4 *)(bsrc[i] + (size_t)kt * BKB);
        if (tid < BM) rd = dsrc ? *(const u32x2 *)(dsrc + 2 * kt) : u32x2{0u, 0u};
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int c = tid + i * 256;
            if (c < A_CHUNKS) *(u32x4 *)(sA[buf] + (c / 4) * FQ_LDA + (c % 4) * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int c = tid + i * 256;
            if (c < B_CHUNKS) *(u32x4 *)(sB[buf] + (c / B_CPR) * LDB + (c % B_CPR) * 16) = rb[i];
        }
        if (tid < BM) {
            sD[buf][0][tid] = __uint_as_float(rd[0]);
            sD[buf][1][tid] = __uint_as_float(rd[1]);
        }
    };

    f32x4 acc[NMAT][MB][NB];
#pragma unroll
    for (int x = 0; x < NMAT; ++x)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[x][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = a.K / FQ_BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_stage(kt + 1);
        const uint8_t *cA = sA[buf];
        const uint8_t *cB = sB[buf];
#pragma unroll
        for (int ks = 0; ks < FQ_BK / 32; ++ks) {
            u32x2 af[MB];
            f32x4 dsc[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int mr = wm * (BM / WM) + i * 16;
                af[i] = *(const u32x2 *)(cA + (mr + (lane & 15)) * FQ_LDA + ks * 32 + (lane >> 4) * 8);
                dsc[i] = *(const f32x4 *)(&sD[buf][ks][mr + (lane >> 4) * 4]);
            }
#pragma unroll
            for (int x = 0; x < NMAT; ++x)
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const uint8_t *bp = cB + (x * BN + wn * (BN / WN) + j * 16 + (lane & 15)) * LDB;
                    const u32x2 bf = WBITS == 4 ? unpack_int4x8_i8(*(const uint32_t *)(bp + ks * 16 + (lane >> 4) * 4))
                                                : *(const u32x2 *)(bp + ks * 32 + (lane >> 4) * 8);
#pragma unroll
                    for (int i = 0; i < MB; ++i) {
                        const i32x4 p = mfma_i8(af[i], bf);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[x][i][j][r] = fmaf((float)p[r], dsc[i][r], acc[x][i][j][r]);
                    }
                }
        }
        if (kt + 1 < KT) store_stage(buf ^ 1);  // the other buffer: last read before the previous barrier
        __syncthreads();
    }

    const float wq = WBITS == 4 ? 0.0625f : 1.f;  // int4 codes entered as code << 4
    const float *sc0 = a.s0 + (size_t)e * a.sstride;
    const float *sc1 = (MODE == 0) ? a.s1 + (size_t)e * a.sstride : nullptr;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + r;
            if (m >= rows) continue;
            const int row = row0 + m;
            float *o = (float *)a.out + (size_t)row * a.ldo;
            if constexpr (MODE == 0) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
                    const float g = acc[0][i][j][r] * (sc0[n] * wq);
                    const float u = acc[1][i][j][r] * (sc1[n] * wq);
                    o[n] = silu(g) * u;
                }
            } else {
                const float ps = (a.pscale && a.pair_of_row) ? a.pscale[a.pair_of_row[row]] : 1.f;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
                    o[n] = acc[0][i][j][r] * (sc0[n] * wq) * ps;
                }
            }
        }
}

template <int MODE, int WBITS, int BM, int BN, int WM, int WN>
static hipError_t launch_q8(const FfnArgs &a, int slots, hipStream_t st)
{
    const int NT = a.N / BN;
    const long grid = (long)((slots + 7) / 8 * 8) * NT;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((k_ffn_q8<MODE, WBITS, BM, BN, WM, WN>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

// 64-row tiles once the groups average 24 rows, else 16; 64 output columns.
template <int MODE, int WBITS>
static hipError_t launch_q8_mode(const FfnArgs &a, int rows_total, int groups, hipStream_t st)
{
    const int ng = a.offsets ? groups : 1;
    const bool big = rows_total >= 24 * ng;
    const int bm = big ? 64 : 16;
    const int slots = (rows_total + bm - 1) / bm + (a.offsets ? min(ng, rows_total) : 0);
    if (big) return launch_q8<MODE, WBITS, 64, 64, 2, 2>(a, slots, st);
    return launch_q8<MODE, WBITS, 16, 64, 1, 4>(a, slots, st);
}

hipError_t launch_ffn_q8(int mode, int wbits, const FfnArgs &a, int rows_total, int groups, hipStream_t st)
{
    if (mode == 0) return wbits == 4 ? launch_q8_mode<0, 4>(a, rows_total, groups, st)
                                     : launch_q8_mode<0, 8>(a, rows_total, groups, st);
    return wbits == 4 ? launch_q8_mode<1, 4>(a, rows_total, groups, st) : launch_q8_mode<1, 8>(a, rows_total, groups, st);
}

template <int MODE, int BM, int BN, int WM, int WN>
static hipError_t launch_mix(const FfnArgs &a, int slots, hipStream_t st)
{
    const int NT = a.N / BN;
    const long grid = (long)((slots + 7) / 8 * 8) * NT;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((k_ffn_mix<MODE, BM, BN, WM, WN>), dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

// int4/int2 families: the register-staged tiles, 16 or 64 rows by the mean
// rows per expert, 64 columns.
int ffn_bm(int mode, int wbits, int rows, int groups, int nt);

bool ffn3_taken(int mode, int wbits, int rows_total, int groups, int N)
{
    return N % 128 == 0 && ffn_bm(mode, wbits, rows_total, groups, N / 128) != 16;
}

// f32 sum of each bf16 row (K values, rows lda elements apart): one wave per
// row, 16-byte loads where the rows allow them; a lane adds its values in
// order, the wave by a fixed butterfly.
__global__ __launch_bounds__(256) void k_rowsum_bf16(const uint16_t *__restrict__ A, int lda, int rows, int K,
                                                      float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t *r = A + (size_t)row * lda;
    auto bf = [](uint32_t u) { return __uint_as_float(u << 16); };
    float sum = 0.f;
    const int K8 = (lda & 7) ? 0 : K / 8 * 8;
    for (int k = lane * 8; k < K8; k += WAVE * 8) {
        const u32x4 v = *(const u32x4 *)(r + k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            sum += bf(v[q] & 0xFFFFu);
            sum += bf(v[q] >> 16);
        }
    }
    for (int k = K8 + lane; k < K; k += WAVE) sum += bf(r[k]);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) sum += __shfl_xor(sum, o, WAVE);
    if (lane == 0) out[row] = sum;
}

hipError_t launch_rowsum_bf16(const uint16_t *A, int lda, int rows, int K, float *out, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rowsum_bf16, dim3((rows + 3) / 4), dim3(256), 0, st, A, lda, rows, K, out);
    return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mix_mode(const FfnArgs &a, int rows_total, int groups, hipStream_t st)
{
    if (a.N % 128 == 0) {
        // the pipelined tiles where the int4 path would take them
        const int bm = ffn_bm(MODE, 4, rows_total, groups, a.N / 128);
        const int slots = (rows_total + bm - 1) / bm + min(groups, rows_total);
        if (bm == 64) return launch_three_mix<MODE, 64>(a, slots, st);
        if (MODE == 0 && bm == 128) return launch_three_mix<0, 128>(a, slots, st);
    }
    const bool big = rows_total >= 24 * groups;
    const int bm = big ? 64 : 16;
    const int slots = (rows_total + bm - 1) / bm + min(groups, rows_total);
    if (big) return launch_mix<MODE, 64, 64, 2, 2>(a, slots, st);
    return launch_mix<MODE, 16, 64, 1, 4>(a, slots, st);
}

hipError_t launch_ffn(int mode, int wbits, const FfnArgs &a, int rows_total, int groups, hipStream_t st)
{
    if (a.ebits) {
        if (!a.offsets || mode == 2) return hipErrorInvalidValue;
        return mode == 0 ? launch_mix_mode<0>(a, rows_total, groups, st) : launch_mix_mode<1>(a, rows_total, groups, st);
    }
    if (mode == 2) return launch_mode<2, 4>(a, rows_total, groups, st);
    if (mode == 0) return wbits == 4 ? launch_mode<0, 4>(a, rows_total, groups, st)
                                     : launch_mode<0, 8>(a, rows_total, groups, st);
    return wbits == 4 ? launch_mode<1, 4>(a, rows_total, groups, st) : launch_mode<1, 8>(a, rows_total, groups, st);
}

}  // namespace moe

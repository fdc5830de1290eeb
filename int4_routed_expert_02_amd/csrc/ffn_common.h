// ffn_common.h -- pieces shared by the grouped-GEMM kernels of the experts
// (ffn.hip): tile lookup, the h column order, LDS copies and
// counted waits.
#pragma once

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int FF_BK = 64;           // reduction columns per stage
constexpr int FF_LDA = FF_BK + 8;   // LDS A row, bf16 elements (144 B: conflict-free fragment reads)

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

// Position of column j of an h row in its stored order: with int4 down weights
// each 8-group is stored as (j0, j4, j1, j5, j2, j6, j3, j7), the k-slot order
// of unpack_int4x8.
template <int WBITS>
__device__ __forceinline__ int hpos(int j)
{
    return WBITS == 4 ? (j & ~7) | ((j & 3) << 1) | ((j >> 2) & 1) : j;
}

template <int N>
struct IntC {
    static constexpr int value = N;
};

template <int MODE, int WBITS, int BM, int BN_ = 128>
struct Ff3 {
    static constexpr int NMAT = (MODE == 1) ? 1 : 2;
    static constexpr int BN = BN_;  // output columns per matrix
    static constexpr int BKB = FF_BK * WBITS / 8;      // B bytes per row per stage
    static constexpr int A_BYTES = BM * FF_BK * 2;     // per stage
    static constexpr int B_BYTES = NMAT * BN * BKB;
    static constexpr int A_LOADS = A_BYTES / 1024;     // wave copies per stage
    static constexpr int B_LOADS = B_BYTES / 1024;
    // padding copies (a B copy repeated into a spare 1 KB) so that every wave
    // issues the same number: int2 down has 8 + 2
    static constexpr int PAD_LOADS = (4 - (A_LOADS + B_LOADS) % 4) % 4;
    static constexpr int LOADS = A_LOADS + B_LOADS + PAD_LOADS;
    static constexpr int STAGE = LOADS * 1024;
    static_assert(LOADS % 4 == 0, "copies split evenly over the four waves");
    static constexpr int PER_WAVE = LOADS / 4;
    // ring stages: three, or two where three would not leave room for two
    // workgroups per compute unit (deeper rings measured slower)
    static constexpr int NST = STAGE <= 24 * 1024 ? 3 : 2;
    static_assert(PER_WAVE * (NST - 2) < 64, "vmcnt range");
    // LDS of the ring (the launch's dynamic LDS); tiles of fewer valid rows
    // lay out more, smaller stages in it.  The int4 down GEMM of 64-row tiles
    // gets room for two of its 128-k stages: 48 KB for 128 columns (three
    // workgroups still fit a compute unit, as many as its registers allow),
    // 64 KB for 256
    static constexpr int RING = (MODE == 1 && BM == 64 && WBITS == 4) ? (BN == 256 ? 64 : 48) * 1024 : NST * STAGE;
};

__device__ __forceinline__ void lds_copy16(const void *g, void *l)
{
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)g,
                                     (void __attribute__((address_space(3))) *)l, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));  // gfx9 encoding
}

// Wait until at most min(later, L) stages of PW copies each are outstanding:
// the stages after the one about to be read that were issued (fewer than L
// near the end of the k loop).
template <int PW, int L>
__device__ __forceinline__ void wait_stages(int later)
{
    if constexpr (L == 0) {
        wait_vm<0>();
    } else {
        if (later >= L) wait_vm<PW * L>();
        else wait_stages<PW, L - 1>(later);
    }
}

// Workgroup barrier of the stage ring.  It waits for this wave's LDS reads
// (lgkmcnt 0) but not for its global-to-LDS copies in flight, which the
// counted wait_vm before it has already settled for the stage about to be
// read; the memory clobber keeps the compiler from moving memory accesses
// across it.  (__syncthreads would also drain every copy in flight, leaving
// the ring only one stage ahead.)
__device__ __forceinline__ void ring_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace moe

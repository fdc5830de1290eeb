// permute.hip -- batch-union grouping of the (token, expert) pairs by expert.
//
// The colibri README ("What's implemented", batch-union MoE) reads each unique
// expert once and applies it to every position routed to it.  Here that is a
// stable counting sort of the pairs p = t*k + j by expert id:
//   counts[e], offsets[e] (exclusive scan), sorted[offsets[e] + rank] = p,
//   inv[p] = sorted row of p,
// where rank = number of earlier pairs (smaller p) routed to the same expert.
// Ranks come from ordered counting -- per-block histograms, a scan over blocks,
// and within a block wave ballots over the pairs in order -- never from atomic
// position counters, so the permutation is bit-exact and deterministic.
#include "moe_device.h"

namespace moe {

// Block histograms of `chunk` consecutive pairs each (used when the caller has
// ids but no histograms from the router).
__global__ __launch_bounds__(256) void k_pair_hist(const int32_t *__restrict__ ids, int P, int E, int chunk,
                                                   int32_t *__restrict__ bcounts)
{
    __shared__ int32_t hist[256];
    for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
    __syncthreads();
    const int p0 = blockIdx.x * chunk;
    const int p1 = min(P, p0 + chunk);
    for (int p = p0 + threadIdx.x; p < p1; p += 256)
        if (ids[p] >= 0) atomicAdd(&hist[ids[p]], 1);  // (-1: a pair dropped by adaptive top-p)
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) bcounts[(size_t)blockIdx.x * E + e] = hist[e];
}

// Lanes of this wave whose 8-bit key equals mine (E <= 256).
__device__ __forceinline__ uint64_t match_key(int key, bool active)
{
    uint64_t m = __ballot(active);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool on = (key >> bit) & 1;
        const uint64_t b = __ballot(active && on);
        m &= on ? b : ~b;
    }
    return active ? m : 0ull;
}

// grid = nblocks; block b owns pairs [b*chunk, min(P, (b+1)*chunk)).
__global__ __launch_bounds__(256) void k_scatter(const int32_t *__restrict__ ids, const int32_t *__restrict__ bcounts,
                                                 int nblocks, int P, int E, int chunk, int32_t *__restrict__ counts,
                                                 int32_t *__restrict__ offsets, int32_t *__restrict__ sorted,
                                                 int32_t *__restrict__ inv)
{
    __shared__ int32_t base[256];     // first free position of each expert for this block
    __shared__ int32_t wcnt[4][256];  // per-wave counts of the current step
    __shared__ int32_t scan[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;

    // totals and this block's prefix over earlier blocks, one expert per
    // thread; sixteen blocks' counts in flight at a time (integer sums, so the
    // grouping does not change them)
    int total = 0, before = 0;
    if (tid < E) {
        constexpr int QB = 16;
        for (int q0 = 0; q0 < nblocks; q0 += QB) {
            int c[QB];
#pragma unroll
            for (int i = 0; i < QB; ++i) c[i] = q0 + i < nblocks ? bcounts[(size_t)(q0 + i) * E + tid] : 0;
#pragma unroll
            for (int i = 0; i < QB; ++i) {
                total += c[i];
                if (q0 + i < b) before += c[i];
            }
        }
    }
    // exclusive scan of totals over experts (E <= 256): Hillis-Steele in LDS
    scan[tid] = (tid < E) ? total : 0;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int v = (tid >= o) ? scan[tid - o] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        const int excl = scan[tid] - total;
        base[tid] = excl + before;
        if (b == 0) {
            counts[tid] = total;
            offsets[tid] = excl;
            if (tid == E - 1) offsets[E] = scan[tid];
        }
    }
    __syncthreads();

    const int p0 = b * chunk;
    const int p1 = min(P, p0 + chunk);
    for (int s0 = p0; s0 < p1; s0 += 256) {
        const int p = s0 + tid;
        const int idr = p < p1 ? ids[p] : 0;
        const bool act = p < p1 && idr >= 0;  // (-1: a pair dropped by adaptive top-p, no row)
        const int id = act ? idr : 0;
        if (p < p1 && idr < 0) inv[p] = -1;
        const uint64_t same = match_key(id, act);
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int rank_w = __popcll(same & lt);
        const int cnt_w = __popcll(same);
        for (int e = tid; e < 4 * 256; e += 256) (&wcnt[0][0])[e] = 0;
        __syncthreads();
        if (act && rank_w == 0) wcnt[wave][id] = cnt_w;  // the lowest lane of each key writes
        __syncthreads();
        if (act) {
            int r = rank_w;
            for (int w2 = 0; w2 < wave; ++w2) r += wcnt[w2][id];
            const int pos = base[id] + r;
            sorted[pos] = p;
            inv[p] = pos;
        }
        __syncthreads();
        if (tid < E) base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
        __syncthreads();
    }
}

hipError_t launch_pair_hist(const int32_t *ids, int P, int E, int chunk, int nblocks, int32_t *bcounts,
                            hipStream_t st)
{
    hipLaunchKernelGGL(k_pair_hist, dim3(nblocks), dim3(256), 0, st, ids, P, E, chunk, bcounts);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t *ids, const int32_t *bcounts, int nblocks, int P, int E, int chunk,
                          int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *inv, hipStream_t st)
{
    hipLaunchKernelGGL(k_scatter, dim3(nblocks), dim3(256), 0, st, ids, bcounts, nblocks, P, E, chunk, counts,
                       offsets, sorted, inv);
    return hipGetLastError();
}

}  // namespace moe

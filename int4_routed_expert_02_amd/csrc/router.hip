// router.hip -- router logits, sigmoid+bias selection, combine weights, per-block
// expert histograms.
//
// The router is a sigmoid router whose per-expert bias only decides selection
// (Colibri-Nano model card, "Architecture": sigmoid+bias router with
// DeepSeek-V3-style aux-loss-free balancing), optionally group-limited
// ("noaux_tc" in the colibri README's "What's implemented" list).
//
// Logits.  z = x . W_e with x in bf16 and W in f32.  Each f32 weight is split
// exactly into three bf16 parts (w = hi + mid + lo: 8 + 8 + 8 significant
// bits), so every product x * part is exact in f32 and the dot product runs on
// bf16 matrix cores with f32 accumulation at three times the bf16 cost.  The K
// (hidden) dimension may be split over workgroups; the partial sums are added
// in a fixed order by the selection kernel, so results are deterministic.
//
// Selection.  One wavefront per token.  A lane holds up to four experts' scores
// (lane l holds experts [l*EPL, (l+1)*EPL)); arg-max reductions across the wave
// break ties toward the lower expert id.  The K-split partial logits are added
// in split order, so results do not depend on timing.
#include "moe_device.h"
#include "moe_select.h"

namespace moe {

constexpr int RT_TB = 64;   // tokens per logits tile
constexpr int RT_EB = 64;   // experts per logits tile
constexpr int RT_BK = 64;   // hidden columns per k-step
constexpr int RT_LDA = RT_BK + 8;  // padded LDS row (bf16 elements)

// Split one f32 into three bf16 bit patterns whose exact sum is the input.
__device__ __forceinline__ void split3(float w, uint32_t &hi, uint32_t &mid, uint32_t &lo)
{
    uint32_t u = __float_as_uint(w);
    uint32_t h = u & 0xFFFF0000u;
    float r1 = w - __uint_as_float(h);
    uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
    float r2 = r1 - __uint_as_float(m);
    hi = h >> 16;
    mid = m >> 16;
    lo = __float_as_uint(r2) >> 16;  // r2 has at most 8 significant bits: exact
}

// grid: (ceil(T/RT_TB) * ceil(E/RT_EB), KS).  zpart[ks][t][e] f32.  Global
// loads run two k-steps ahead of the matrix cores (two register sets, used in
// turn), so a workgroup waits for memory once rather than once per k-step.
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t *__restrict__ x, const float *__restrict__ W,
                                                       float *__restrict__ zpart, int T, int H, int E, int ksteps_per_split,
                                                       int32_t *__restrict__ clear, int clear_n)
{
    if (clear && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < clear_n; i += 256) clear[i] = 0;
    __shared__ uint16_t sA[RT_TB * RT_LDA];
    __shared__ uint16_t sB[3][RT_EB * RT_LDA];

    const int n_eb = (E + RT_EB - 1) / RT_EB;
    const int tb = blockIdx.x / n_eb;
    const int eb = blockIdx.x % n_eb;
    const int ks = blockIdx.y;
    const int t0 = tb * RT_TB, e0 = eb * RT_EB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, each 32 tokens x 32 experts

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // x: 64 rows x 64 bf16 = 512 chunks of 16 B, 2 per thread;
    // W: 64 experts x 64 f32 = 1024 chunks of 4 floats, 4 per thread
    struct Regs {
        u32x4 x[2];
        f32x4 w[4];
    };
    auto gload = [&](Regs &r, int kt) {
        const int k0 = kt * RT_BK;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int chunk = tid + c * 256;
            const int t = t0 + (chunk >> 3);
            r.x[c] = t < T ? *(const u32x4 *)(x + (size_t)t * H + k0 + (chunk & 7) * 8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int chunk = tid + c * 256;
            const int e = e0 + (chunk >> 4);
            r.w[c] = e < E ? *(const f32x4 *)(W + (size_t)e * H + k0 + (chunk & 15) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto lstore = [&](const Regs &r) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int chunk = tid + c * 256;
            *(u32x4 *)(sA + (chunk >> 3) * RT_LDA + (chunk & 7) * 8) = r.x[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int chunk = tid + c * 256;
            const int row = chunk >> 4, cc = chunk & 15;
            uint32_t h[4], m[4], l[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split3(r.w[c][i], h[i], m[i], l[i]);
            *(u32x2 *)(sB[0] + row * RT_LDA + cc * 4) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
            *(u32x2 *)(sB[1] + row * RT_LDA + cc * 4) = u32x2{m[0] | (m[1] << 16), m[2] | (m[3] << 16)};
            *(u32x2 *)(sB[2] + row * RT_LDA + cc * 4) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
        }
    };
    auto compute = [&]() {
#pragma unroll
        for (int kk = 0; kk < RT_BK; kk += 32) {
            const int ko = kk + (lane >> 4) * 8;
            u32x4 av[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) av[i] = *(const u32x4 *)(sA + (wm * 32 + i * 16 + (lane & 15)) * RT_LDA + ko);
#pragma unroll
            for (int p = 0; p < 3; ++p) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x4 bv = *(const u32x4 *)(sB[p] + (wn * 32 + j * 16 + (lane & 15)) * RT_LDA + ko);
#pragma unroll
                    for (int i = 0; i < 2; ++i) acc[i][j] = mfma_bf16(av[i], bv, acc[i][j]);
                }
            }
        }
    };
    // one k-step from register set r, which then fetches k-step kt + 2
    auto step = [&](Regs &r, int kt, int kend) {
        lstore(r);
        __syncthreads();
        if (kt + 2 < kend) gload(r, kt + 2);
        compute();
        __syncthreads();
    };

    const int kbeg = ks * ksteps_per_split, kend = kbeg + ksteps_per_split;
    Regs ra, rb;
    gload(ra, kbeg);
    if (kbeg + 1 < kend) gload(rb, kbeg + 1);
    for (int kt = kbeg; kt < kend; kt += 2) {
        step(ra, kt, kend);
        if (kt + 1 < kend) step(rb, kt + 1, kend);
    }
    float *zp = zpart + (size_t)ks * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int t = t0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
                int e = e0 + wn * 32 + j * 16 + (lane & 15);
                if (t < T && e < E) zp[(size_t)t * E + e] = acc[i][j][r];
            }
}

constexpr int SEL_TOKENS = 4;  // tokens per workgroup: one wave per token

// One wave per token.  Writes ids, w, gap and optionally pair_scale (rsf * w
// per pair).  When sbcounts is given, each workgroup adds the expert histogram
// of its SEL_TOKENS tokens into sbcounts[superblock][E], a superblock being
// sb_tokens consecutive tokens (integer atomics: the totals do not depend on
// the order of the additions).
template <int EPL>
__global__ __launch_bounds__(256) void k_router_select(const float *__restrict__ zpart, int KS,
                                                       const float *__restrict__ bias, int T, int E, int k,
                                                       int n_group, int topk_group, float rsf,
                                                       int32_t *__restrict__ ids, float *__restrict__ w,
                                                       float *__restrict__ gap, float *__restrict__ pair_scale,
                                                       int32_t *__restrict__ sbcounts, int sb_tokens, float top_p)
{
    __shared__ int32_t hist[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += 256) hist[e] = 0;
    __syncthreads();

    const int t = blockIdx.x * SEL_TOKENS + wave;
    if (t < T) {
        float s[EPL], b[EPL], z[EPL];
        bool ok[EPL];
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            ok[q] = lane * EPL + q < E;
            z[q] = 0.f;
        }
        // partial logits added in plane order; eight planes' loads in flight at once
        constexpr int PB = 8;
        for (int p0 = 0; p0 < KS; p0 += PB) {
            float v[PB][EPL];
#pragma unroll
            for (int i = 0; i < PB; ++i)
#pragma unroll
                for (int q = 0; q < EPL; ++q)
                    v[i][q] = (p0 + i < KS && ok[q]) ? zpart[((size_t)(p0 + i) * T + t) * E + lane * EPL + q] : 0.f;
#pragma unroll
            for (int i = 0; i < PB; ++i)
#pragma unroll
                for (int q = 0; q < EPL; ++q)
                    if (p0 + i < KS) z[q] += v[i][q];
        }
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            s[q] = ok[q] ? 1.0f / (1.0f + expf(-z[q])) : 0.f;
            b[q] = ok[q] ? s[q] + bias[lane * EPL + q] : -INFINITY;
        }
        select_token<EPL>(s, b, ok, lane, t, E, k, n_group, topk_group, rsf, ids, w, gap, pair_scale, hist, top_p);
    }
    __syncthreads();
    if (sbcounts) {
        const int sb = (blockIdx.x * SEL_TOKENS) / sb_tokens;
        for (int e = tid; e < E; e += 256)
            if (hist[e]) atomicAdd(&sbcounts[(size_t)sb * E + e], hist[e]);
    }
}

// ------------------------------------------------------------------ bias update

// Aux-loss-free balancing after a step (Colibri-Nano model card,
// "Architecture": sigmoid+bias router with DeepSeek-V3-style aux-loss-free
// balancing).  Reading (the pages give no rule): bias[e] += gamma *
// sign(mean - counts[e]) with mean = sum(counts) / E, compared exactly as
// E * counts[e] against the sum; an expert exactly at the mean keeps its
// bias.  One workgroup: the sum in int64, then one f32 addition per expert.
__global__ __launch_bounds__(256) void k_bias_update(int E, const int32_t *__restrict__ counts,
                                                     float *__restrict__ bias, float gamma)
{
    __shared__ long long part[256];
    long long s = 0;
    for (int e = threadIdx.x; e < E; e += 256) s += counts[e];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
        __syncthreads();
    }
    const long long total = part[0];
    for (int e = threadIdx.x; e < E; e += 256) {
        const long long load = (long long)E * counts[e];
        if (load < total) bias[e] = bias[e] + gamma;
        else if (load > total) bias[e] = bias[e] - gamma;
    }
}

hipError_t launch_bias_update(int E, const int32_t *counts, float *bias, float gamma, hipStream_t st)
{
    hipLaunchKernelGGL(k_bias_update, dim3(1), dim3(256), 0, st, E, counts, bias, gamma);
    return hipGetLastError();
}

// ------------------------------------------------------------------ launchers

// K splits of the logits: the smallest divisor of the k-step count that gives
// at least 512 workgroups (two per compute unit), else one k-step each
int router_ks(int T, int H, int E)
{
    const int ksteps = H / RT_BK;
    const int tiles = ((T + RT_TB - 1) / RT_TB) * ((E + RT_EB - 1) / RT_EB);
    int ks = 1;
    for (int c = 1; c <= ksteps; ++c) {
        if (ksteps % c) continue;
        ks = c;
        if (tiles * c >= 512) break;
    }
    return ks;
}

int router_select_blocks(int T) { return (T + SEL_TOKENS - 1) / SEL_TOKENS; }

// tokens per permutation superblock: about 1024 pairs, a multiple of SEL_TOKENS
int superblock_tokens(int k)
{
    int t = (1024 / k) / SEL_TOKENS * SEL_TOKENS;
    return t < SEL_TOKENS ? SEL_TOKENS : t;
}

hipError_t launch_router(const uint16_t *x, const float *W, const float *bias, int T, int H, int E, int k,
                         int n_group, int topk_group, float rsf, float top_p, float *zpart, int KS, int32_t *ids,
                         float *w, float *gap, float *pair_scale, int32_t *sbcounts, hipStream_t st)
{
    const int ksteps = H / RT_BK;
    const int sbt = superblock_tokens(k);
    const int nsb = (T + sbt - 1) / sbt;
    dim3 g1(((T + RT_TB - 1) / RT_TB) * ((E + RT_EB - 1) / RT_EB), KS);
    hipLaunchKernelGGL(k_router_logits, g1, dim3(256), 0, st, x, W, zpart, T, H, E, ksteps / KS, sbcounts,
                       sbcounts ? nsb * E : 0);
    const int nb = router_select_blocks(T);
    if (E <= 64)
        hipLaunchKernelGGL(k_router_select<1>, dim3(nb), dim3(256), 0, st, zpart, KS, bias, T, E, k, n_group,
                           topk_group, rsf, ids, w, gap, pair_scale, sbcounts, sbt, top_p);
    else if (E <= 128)
        hipLaunchKernelGGL(k_router_select<2>, dim3(nb), dim3(256), 0, st, zpart, KS, bias, T, E, k, n_group,
                           topk_group, rsf, ids, w, gap, pair_scale, sbcounts, sbt, top_p);
    else
        hipLaunchKernelGGL(k_router_select<4>, dim3(nb), dim3(256), 0, st, zpart, KS, bias, T, E, k, n_group,
                           topk_group, rsf, ids, w, gap, pair_scale, sbcounts, sbt, top_p);
    return hipGetLastError();
}

}  // namespace moe

// combine.hip -- weighted sum of a token's routed expert outputs plus the shared
// expert (and optionally the layer input).
//
// The routed terms carry routed_scaling_factor * w (DeepSeek-V3-style router
// with routed_scaling_factor, colibri README "What's implemented"); the shared
// expert is always applied with weight 1 (NanoColibri README: a fat
// always-resident shared expert).  The k routed terms are added in ascending j
// order, then the shared term, then the residual: a fixed order, so the result
// does not depend on scheduling.  The layer's own routed and shared output
// rows are f16 (each rounded once); those of the split API f32.
#include "moe_device.h"

namespace moe {

// Four consecutive values of a routed or shared output row: f32, or f16.
__device__ __forceinline__ f32x4 ld4(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ f32x4 ld4(const uint16_t *p)
{
    const u32x2 h = *(const u32x2 *)p;
    return f32x4{f16_lo(h[0]), f16_hi(h[0]), f16_lo(h[1]), f16_hi(h[1])};
}

// one thread per 4 consecutive columns of one token; YT: the element type of
// the routed and shared output rows; B > 0: routed rows in pair order (row p
// of pair p), no row address waits for inv (read only to skip dropped
// pairs), so a batch of B rows' loads is issued before any is used; B = 0:
// rows in sorted order (row inv[p]).
template <typename YT, int B>
__global__ __launch_bounds__(256) void k_combine(const YT *__restrict__ y, const int32_t *__restrict__ inv,
                                                 const float *__restrict__ topk_w, float rsf,
                                                 const YT *__restrict__ sh, const uint16_t *__restrict__ res,
                                                 void *__restrict__ out, int T, int H, int k, int out_f32)
{
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int cpt = H / 4;
    if (idx >= (long)T * cpt) return;
    const int t = (int)(idx / cpt);
    const int c = (int)(idx % cpt) * 4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (B > 0) {
        for (int j0 = 0; j0 < k; j0 += B) {
            f32x4 v[B];
            int iv[B];
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const int p = t * k + (j0 + i < k ? j0 + i : 0);
                v[i] = ld4(y + (size_t)p * H + c);
                iv[i] = inv[p];
            }
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const int p = t * k + j0 + i;
                if (j0 + i >= k || iv[i] < 0) continue;  // past top_k, or a pair dropped by adaptive top-p
                const float coef = topk_w ? rsf * topk_w[p] : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += coef * v[i][e];
            }
        }
    } else {
        for (int j = 0; j < k; ++j) {
            const int p = t * k + j;
            if (inv[p] < 0) continue;  // a pair dropped by adaptive top-p
            const float coef = topk_w ? rsf * topk_w[p] : 1.f;
            const f32x4 v = ld4(y + (size_t)inv[p] * H + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += coef * v[i];
        }
    }
    if (sh) {
        const f32x4 v = ld4(sh + (size_t)t * H + c);
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
        u32x2 o = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *(u32x2 *)((uint16_t *)out + (size_t)t * H + c) = o;
    }
}

hipError_t launch_combine(const void *y, const int32_t *inv, const float *topk_w, float rsf, const void *sh,
                          const uint16_t *res, void *out, int T, int H, int k, int out_f32, int y_f16, int y_by_pair,
                          hipStream_t st)
{
    const long n = (long)T * (H / 4);
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (grid == 0) return hipSuccess;
    auto go = [&](auto kern, auto yt) {
        using YT = decltype(yt);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, (const YT *)y, inv, topk_w, rsf, (const YT *)sh, res,
                           out, T, H, k, out_f32);
    };
    // pair order: batches of 2, 4 or 8 rows by top_k
    const int b = !y_by_pair ? 0 : k <= 2 ? 2 : k <= 4 ? 4 : 8;
    if (y_f16) {
        if (b == 2) go(k_combine<uint16_t, 2>, uint16_t{});
        else if (b == 4) go(k_combine<uint16_t, 4>, uint16_t{});
        else if (b == 8) go(k_combine<uint16_t, 8>, uint16_t{});
        else go(k_combine<uint16_t, 0>, uint16_t{});
    } else {
        if (b == 2) go(k_combine<float, 2>, float{});
        else if (b == 4) go(k_combine<float, 4>, float{});
        else if (b == 8) go(k_combine<float, 8>, float{});
        else go(k_combine<float, 0>, float{});
    }
    return hipGetLastError();
}

}  // namespace moe

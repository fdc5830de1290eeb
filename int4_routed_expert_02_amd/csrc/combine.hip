// combine.hip -- weighted sum of a token's routed expert outputs plus the shared
// expert (and optionally the layer input).
//
// The routed terms carry routed_scaling_factor * w (DeepSeek-V3-style router
// with routed_scaling_factor, colibri README "What's implemented"); the shared
// expert is always applied with weight 1 (NanoColibri README: a fat
// always-resident shared expert).  The k routed terms are added in ascending j
// order, then the shared term, then the residual: a fixed order, so the result
// does not depend on scheduling.
#include "moe_device.h"

namespace moe {

// one thread per 4 consecutive columns of one token
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ y, const int32_t *__restrict__ inv,
                                                 const float *__restrict__ topk_w, float rsf,
                                                 const float *__restrict__ sh, const uint16_t *__restrict__ res,
                                                 void *__restrict__ out, int T, int H, int k, int out_f32)
{
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int cpt = H / 4;
    if (idx >= (long)T * cpt) return;
    const int t = (int)(idx / cpt);
    const int c = (int)(idx % cpt) * 4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int p = t * k + j;
        if (inv[p] < 0) continue;  // a pair dropped by adaptive top-p
        const float coef = topk_w ? rsf * topk_w[p] : 1.f;
        const f32x4 v = *(const f32x4 *)(y + (size_t)inv[p] * H + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += coef * v[i];
    }
    if (sh) {
        const f32x4 v = *(const f32x4 *)(sh + (size_t)t * H + c);
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

hipError_t launch_combine(const float *y, const int32_t *inv, const float *topk_w, float rsf, const float *sh,
                          const uint16_t *res, void *out, int T, int H, int k, int out_f32, hipStream_t st)
{
    const long n = (long)T * (H / 4);
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(k_combine, dim3(grid), dim3(256), 0, st, y, inv, topk_w, rsf, sh, res, out, T, H, k, out_f32);
    return hipGetLastError();
}

}  // namespace moe

// quant.hip -- per-row symmetric quantiser and packer: f32 or bf16 rows ->
// int4 (packed, two per byte) or int8 codes with one f32 scale per row.
//
// The container keeps expert weights per-row symmetric with f32 scales in a
// sibling .qs tensor (colibri-nano README, "Converting a checkpoint
// yourself"; colibri README, "What's implemented": int8 and packed int4
// quantisation kernels with per-row scales).  The pages give no formula; the
// reading used here: scale = max|w| / qmax (qmax = 7 for int4, 127 for int8),
// code = the nearest integer to w / scale with ties to even, clamped to
// [-qmax, qmax]; an all-zero row gets scale 0 and codes 0.  Both divisions
// are correctly rounded f32 (__fdiv_rn) and the rounding is v_rndne, so each
// code is decided exactly as a plain f32 implementation decides it.  Int4
// packing: element 2c in the low nibble of byte c, two's complement.
//
// One wave per row, four rows per workgroup.  The row is read twice (its
// maximum, then its codes; the second pass mostly hits the cache) and its
// codes written once: HBM-bound.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int QZ_ROWS = 4;  // rows (waves) per workgroup

template <bool BF16>
__device__ __forceinline__ float qz_load1(const void *src, size_t i)
{
    if constexpr (BF16) return bf16_to_f32(((const uint16_t *)src)[i]);
    else return ((const float *)src)[i];
}

// eight consecutive values starting at element i (16-byte aligned)
template <bool BF16>
__device__ __forceinline__ void qz_load8(const void *src, size_t i, float (&v)[8])
{
    if constexpr (BF16) {
        const u32x4 d = *(const u32x4 *)((const uint16_t *)src + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_lo(d[j]);
            v[2 * j + 1] = bf16_hi(d[j]);
        }
    } else {
        const f32x4 a = *(const f32x4 *)((const float *)src + i);
        const f32x4 b = *(const f32x4 *)((const float *)src + i + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = b[j];
        }
    }
}

// vec: every row starts 16-byte aligned and cols % 8 == 0, so groups of
// eight values are loaded and stored as vectors; other shapes go value by value
template <bool BF16, int BITS>
__global__ __launch_bounds__(256) void k_quantize_rows(const void *__restrict__ src, long rows, int cols,
                                                       uint8_t *__restrict__ q, float *__restrict__ qs, int vec)
{
    constexpr float QMAX = (BITS == 4) ? 7.0f : 127.0f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long r = (long)blockIdx.x * QZ_ROWS + wave;
    if (r >= rows) return;  // wave-uniform
    const size_t base = (size_t)r * cols;
    const int ng = vec ? cols / 8 : 0;  // groups of eight on the vector path
    const int tail0 = ng * 8;

    float amax = 0.0f;
    for (int g = lane; g < ng; g += WAVE) {
        float v[8];
        qz_load8<BF16>(src, base + (size_t)g * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
    for (int c = tail0 + lane; c < cols; c += WAVE) amax = fmaxf(amax, fabsf(qz_load1<BF16>(src, base + c)));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));

    const float scale = __fdiv_rn(amax, QMAX);
    if (lane == 0) qs[r] = scale;
    auto code = [&](float w) -> uint32_t {
        if (amax == 0.0f) return 0u;
        const float v = fminf(fmaxf(rintf(__fdiv_rn(w, scale)), -QMAX), QMAX);
        return (uint32_t)(int)v;
    };

    uint8_t *qrow = q + (size_t)r * (BITS == 4 ? cols / 2 : cols);
    for (int g = lane; g < ng; g += WAVE) {
        float v[8];
        qz_load8<BF16>(src, base + (size_t)g * 8, v);
        if constexpr (BITS == 4) {
            uint32_t p = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) p |= (code(v[j]) & 0xFu) << (4 * j);
            *(uint32_t *)(qrow + (size_t)g * 4) = p;
        } else {
            uint32_t p0 = 0, p1 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p0 |= (code(v[j]) & 0xFFu) << (8 * j);
                p1 |= (code(v[4 + j]) & 0xFFu) << (8 * j);
            }
            *(u32x2 *)(qrow + (size_t)g * 8) = u32x2{p0, p1};
        }
    }
    if constexpr (BITS == 4) {
        for (int b = tail0 / 2 + lane; b < cols / 2; b += WAVE) {
            const uint32_t lo = code(qz_load1<BF16>(src, base + 2 * b));
            const uint32_t hi = code(qz_load1<BF16>(src, base + 2 * b + 1));
            qrow[b] = (uint8_t)((lo & 0xFu) | ((hi & 0xFu) << 4));
        }
    } else {
        for (int c = tail0 + lane; c < cols; c += WAVE) qrow[c] = (uint8_t)(code(qz_load1<BF16>(src, base + c)) & 0xFFu);
    }
}

hipError_t launch_quantize(const void *src, int src_bf16, long rows, int cols, int bits, void *q, float *qs,
                           hipStream_t st)
{
    const int vec = (cols % 8 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)q % 16) == 0) ? 1 : 0;
    const long blocks = (rows + QZ_ROWS - 1) / QZ_ROWS;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(QZ_ROWS * WAVE);
    uint8_t *qb = (uint8_t *)q;
    if (src_bf16) {
        if (bits == 4) hipLaunchKernelGGL((k_quantize_rows<true, 4>), grid, block, 0, st, src, rows, cols, qb, qs, vec);
        else hipLaunchKernelGGL((k_quantize_rows<true, 8>), grid, block, 0, st, src, rows, cols, qb, qs, vec);
    } else {
        if (bits == 4) hipLaunchKernelGGL((k_quantize_rows<false, 4>), grid, block, 0, st, src, rows, cols, qb, qs, vec);
        else hipLaunchKernelGGL((k_quantize_rows<false, 8>), grid, block, 0, st, src, rows, cols, qb, qs, vec);
    }
    return hipGetLastError();
}

}  // namespace moe

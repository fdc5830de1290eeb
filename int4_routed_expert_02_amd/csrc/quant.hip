// quant.hip -- per-row symmetric quantiser and packer: f32 or bf16 rows ->
// int4 (packed, two per byte) or int8 codes with one f32 scale per row.
//
// The container keeps expert weights per-row symmetric with f32 scales in a
// sibling .qs tensor (colibri-nano README, "Converting a checkpoint
// yourself"; colibri README, "What's implemented": int8 and packed int4
// quantisation kernels with per-row scales).  The pages give no formula; the
// reading used here: scale = max|w| / qmax (qmax = 7 for int4, 127 for int8),
// code = the nearest integer to w / scale with ties to even, clamped to
// [-qmax, qmax]; an all-zero row gets scale 0 and codes 0.  The scale is a
// correctly rounded f32 division and every code equals the nearest integer
// (v_rndne, ties to even) of the correctly rounded quotient, so each code is
// decided exactly as a plain f32 implementation decides it (see qz_code).  Int4
// packing: element 2c in the low nibble of byte c, two's complement.
//
// One wave per row, four rows per workgroup, HBM-bound.  Rows of up to
// 64 x QZ_RG groups of eight values are read once: each lane keeps its groups
// in registers while the row maximum is reduced.  Longer or unaligned rows
// are read twice (maximum, then codes).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int QZ_ROWS = 4;  // rows (waves) per workgroup
constexpr int QZ_RG = 16;   // register-held groups of eight values per lane (rows up to 8192)

// The code of w: the nearest integer to the correctly rounded quotient w /
// scale (ties to even), clamped to [-qmax, qmax].  t = w * inv (inv the
// correctly rounded 1 / scale) is within 1.5 * 2^-23 * |t| <= 2.3e-5 of that
// quotient for |t| <= 127.5, so rint(t) is the same integer unless t lies
// within that distance of a half-integer; there (about one value in 8000)
// the correctly rounded division decides.  That bound needs a normal scale:
// below 2^-126 (rows whose max|w| is under qmax * 2^-126) 1 / scale loses
// precision and below 2^-128 it overflows to infinity, so such rows (a
// wave-uniform case) take the division for every value.
__device__ __forceinline__ uint32_t qz_code(float w, float scale, float inv, float qmax)
{
    float k;
    if (scale < 0x1p-126f) {
        k = rintf(__fdiv_rn(w, scale));
    } else {
        const float t = w * inv;
        k = rintf(t);
        if (fabsf(fabsf(t - k) - 0.5f) < 0x1p-14f) k = rintf(__fdiv_rn(w, scale));
    }
    return (uint32_t)(int)fminf(fmaxf(k, -qmax), qmax);
}

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
    uint8_t *qrow = q + (size_t)r * (BITS == 4 ? cols / 2 : cols);

    if (vec && ng <= WAVE * QZ_RG) {
        // one pass: group g = lane + 64 j stays in registers (raw bits)
        constexpr int RW = BF16 ? 4 : 8;  // 32-bit words per group
        uint32_t raw[QZ_RG][RW];
#pragma unroll
        for (int j = 0; j < QZ_RG; ++j) {
            const int g = lane + WAVE * j;
            if (g < ng) {
                if constexpr (BF16) {
                    const u32x4 d = *(const u32x4 *)((const uint16_t *)src + base + (size_t)g * 8);
#pragma unroll
                    for (int w = 0; w < 4; ++w) raw[j][w] = d[w];
                } else {
                    const u32x4 a = *(const u32x4 *)((const float *)src + base + (size_t)g * 8);
                    const u32x4 b = *(const u32x4 *)((const float *)src + base + (size_t)g * 8 + 4);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        raw[j][w] = a[w];
                        raw[j][4 + w] = b[w];
                    }
                }
            }
        }
        auto values = [&](int j, float (&v)[8]) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if constexpr (BF16) {
                    v[2 * w] = bf16_lo(raw[j][w]);
                    v[2 * w + 1] = bf16_hi(raw[j][w]);
                } else {
                    v[w] = __uint_as_float(raw[j][w]);
                    v[4 + w] = __uint_as_float(raw[j][4 + w]);
                }
            }
        };
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < QZ_RG; ++j) {
            if (lane + WAVE * j < ng) {
                float v[8];
                values(j, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
        const float scale = __fdiv_rn(amax, QMAX);
        const float inv = __frcp_rn(scale);
        if (lane == 0) qs[r] = scale;
#pragma unroll
        for (int j = 0; j < QZ_RG; ++j) {
            const int g = lane + WAVE * j;
            if (g >= ng) continue;
            float v[8];
            values(j, v);
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = amax == 0.0f ? 0u : qz_code(v[i], scale, inv, QMAX);
            if constexpr (BITS == 4) {
                uint32_t p = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) p |= (c[i] & 0xFu) << (4 * i);
                *(uint32_t *)(qrow + (size_t)g * 4) = p;
            } else {
                uint32_t p0 = 0, p1 = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p0 |= (c[i] & 0xFFu) << (8 * i);
                    p1 |= (c[4 + i] & 0xFFu) << (8 * i);
                }
                *(u32x2 *)(qrow + (size_t)g * 8) = u32x2{p0, p1};
            }
        }
        return;
    }

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
    const float inv = __frcp_rn(scale);
    if (lane == 0) qs[r] = scale;
    auto code = [&](float w) -> uint32_t { return amax == 0.0f ? 0u : qz_code(w, scale, inv, QMAX); };

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

// ------------------------------------------------- Q8_0-style activation codes
//
// Int8 activations for the integer-dot expert matmuls (colibri README, "What's
// implemented": Q8_0-style int8 activations).  Reading: blocks of 32
// consecutive values along a row; d = max|v| / 127 and each code the nearest
// integer to v / d (ties to even) inside [-127, 127], both divisions correctly
// rounded f32; an all-zero block has d = 0 and codes 0.  One thread per
// block: its 32 values are read as 16-byte vectors, the codes written as two.

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void k_quant_act_q8(const void *__restrict__ src, long nblocks,
                                                      int8_t *__restrict__ q, float *__restrict__ d)
{
    const long b = (long)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
    if (BF16) {
        const u32x4 *s = (const u32x4 *)((const uint16_t *)src + b * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 w = s[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        }
    } else {
        const f32x4 *s = (const f32x4 *)((const float *)src + b * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 w = s[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * i + j] = w[j];
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float dd = __fdiv_rn(amax, 127.f);
    u32x4 out[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float c = 0.f;
            if (amax != 0.f) c = fminf(fmaxf(rintf(__fdiv_rn(v[4 * i + j], dd)), -127.f), 127.f);
            word |= ((uint32_t)(int)c & 0xFFu) << (8 * j);
        }
        out[i / 4][i % 4] = word;
    }
    u32x4 *o = (u32x4 *)(q + b * 32);
    o[0] = out[0];
    o[1] = out[1];
    d[b] = dd;
}

hipError_t launch_quant_act_q8(const void *src, int src_bf16, long rows, int cols, int8_t *q, float *d,
                               hipStream_t st)
{
    const long nblocks = rows * (cols / 32);
    if (nblocks <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((nblocks + 255) / 256);
    if (src_bf16)
        hipLaunchKernelGGL(k_quant_act_q8<true>, dim3(grid), dim3(256), 0, st, src, nblocks, q, d);
    else
        hipLaunchKernelGGL(k_quant_act_q8<false>, dim3(grid), dim3(256), 0, st, src, nblocks, q, d);
    return hipGetLastError();
}

}  // namespace moe

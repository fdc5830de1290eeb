// moe_device.h -- device helpers shared by the gfx950 kernels of this library.
//
// Matrix-core operands: v_mfma_f32_16x16x32_bf16 takes, per lane, 8 bf16 of A
// (row = lane % 16) and 8 bf16 of B (column = lane % 16); lane group g = lane / 16
// owns a fixed set of 8 k-slots, the same set in A and B.  The accumulator
// holds D[4*g + r][lane % 16] in element r.  Any one-to-one assignment of
// actual k indices to the k-slots is valid as long as A and B use the same one;
// the int4 path below uses that freedom to make the weight unpack cheap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// the same shape with f16 operands (v_mfma_f32_16x16x32_f16)
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)v); }
__device__ __forceinline__ float f16_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// two f32 -> packed f16 pair, each rounded to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// round to nearest even (finite values)
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Eight packed int4 values -> eight bf16 holding q + 136, in k-slot order
// (e0,e4),(e1,e5),(e2,e6),(e3,e7) where e_j is nibble j of w.
// Flipping bit 3 of a nibble turns two's complement q into the offset value
// n = q + 8 in [0, 15]; the bf16 with bit pattern 0x4300 | n is exactly
// 128 + n.  Per pair of values: a shift and one 3-input bit operation
// (keep the nibble bits of (w >> s) ^ 0x0008_0008, elsewhere 0x4300_4300).
// The caller removes the constant 136 from the dot product with
// 136 * (sum of the A row).
constexpr float INT4_BIAS = 136.0f;

__device__ __forceinline__ u32x4 unpack_int4x8(uint32_t w)
{
    u32x4 r;
    r[0] = ((w ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    r[1] = (((w >> 4) ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    r[2] = (((w >> 8) ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    r[3] = (((w >> 12) ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    return r;
}

// Natural k order forms for bf16 operands whose activations are not
// reordered (k-slot pairs (e0,e1),(e2,e3),(e4,e5),(e6,e7)):
//  - int4: byte j of w and of w >> 4 hold nibbles 2j and 2j+1 in their low
//    bits; a byte permute places them in the two halves, then the same bit
//    operation as unpack_int4x8 gives q + 136;
//  - int8: b = q + 128 (bit 7 flipped) converted byte-wise to f32 is exact,
//    and so are its upper halves as bf16; the caller removes 128 * (row sum).
constexpr float INT8_BF16_BIAS = 128.0f;

__device__ __forceinline__ u32x4 unpack_int4x8_nat(uint32_t w)
{
    const uint32_t u = w >> 4;
    u32x4 r;
    // selector: byte 0 <- byte j of w, byte 2 <- byte j of u, bytes 1 and 3 <- 0
    r[0] = ((__builtin_amdgcn_perm(u, w, 0x0C040C00u) ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    r[1] = ((__builtin_amdgcn_perm(u, w, 0x0C050C01u) ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    r[2] = ((__builtin_amdgcn_perm(u, w, 0x0C060C02u) ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    r[3] = ((__builtin_amdgcn_perm(u, w, 0x0C070C03u) ^ 0x00080008u) & 0x000F000Fu) | 0x43004300u;
    return r;
}

__device__ __forceinline__ u32x4 unpack_int8x8_bf16o(u32x2 w)
{
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const uint32_t t = w[d] ^ 0x80808080u;
        const float f0 = (float)(t & 0xFFu), f1 = (float)((t >> 8) & 0xFFu);
        const float f2 = (float)((t >> 16) & 0xFFu), f3 = (float)(t >> 24);
        // the upper halves of (f0, f1) and of (f2, f3)
        r[2 * d] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        r[2 * d + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    return r;
}

// f16 forms of the same unpacks, for the down GEMM, whose activations h are
// f16.  The f16 with bit pattern 0x6400 | m is exactly 1024 + m for m < 1024:
//  - int4: nibble n = q + 8 gives q + 1032, k-slot order as unpack_int4x8;
//  - int8: byte b = q + 128 (bit 7 flipped) gives q + 1152, natural order,
//    one byte permute per pair (the 0x64 bytes come from a constant).
// The caller removes the constant with (its bias) * (sum of the A row).
constexpr float INT4_F16_BIAS = 1032.0f;
constexpr float INT2_BIAS = 130.0f;       // int2 code + 130 in bf16
constexpr float INT2_F16_BIAS = 1026.0f;  // int2 code + 1026 in f16

// Eight packed int2 codes (element j in bits 2j..2j+1 of w, two's complement)
// -> four pairs of 16-bit values 2^e + (code + 2) in natural order: the field
// XOR 2 is code + 2 (0..3), ORed into the mantissa of 128 (bf16, hi =
// 0x4300) or 1024 (f16, hi = 0x6400).  Pair i holds elements 2i (low half)
// and 2i + 1: t = w | w << 14 puts element 2i + 1 sixteen bits above 2i.
template <uint32_t HI>
__device__ __forceinline__ u32x4 unpack_int2x8(uint32_t w)
{
    const uint32_t t = (w & 0xFFFFu) | ((w & 0xFFFFu) << 14);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (((t >> (4 * i)) & 0x00030003u) ^ 0x00020002u) | (HI | (HI << 16));
    return r;
}
constexpr float INT8_F16_BIAS = 1152.0f;

__device__ __forceinline__ u32x4 unpack_int4x8_f16(uint32_t w)
{
    u32x4 r;
    r[0] = ((w ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
    r[1] = (((w >> 4) ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
    r[2] = (((w >> 8) ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
    r[3] = (((w >> 12) ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
    return r;
}

__device__ __forceinline__ u32x4 unpack_int8x8_f16(u32x2 w)
{
    const uint32_t f0 = w[0] ^ 0x80808080u, f1 = w[1] ^ 0x80808080u;
    u32x4 r;
    // selector bytes: 0..3 pick bytes of the second operand, 4..7 of the first
    r[0] = __builtin_amdgcn_perm(0x64646464u, f0, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(0x64646464u, f0, 0x04030402u);
    r[2] = __builtin_amdgcn_perm(0x64646464u, f1, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(0x64646464u, f1, 0x04030402u);
    return r;
}

// The matching A-side order: eight consecutive bf16 x0..x7 held as dwords
// d = {x0x1, x2x3, x4x5, x6x7} become {x0x4, x1x5, x2x6, x3x7}.
__device__ __forceinline__ u32x4 interleave_bf16x8(u32x4 d)
{
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
    return r;
}

// Eight int8 values (two dwords, natural order) -> eight exact bf16.
__device__ __forceinline__ u32x4 unpack_int8x8(u32x2 w)
{
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        int32_t v = (int32_t)w[d];
        float f0 = (float)((v << 24) >> 24);
        float f1 = (float)((v << 16) >> 24);
        float f2 = (float)((v << 8) >> 24);
        float f3 = (float)(v >> 24);
        // small integers are exact in bf16: take the upper halves
        r[2 * d] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
        r[2 * d + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
    }
    return r;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// z * sigmoid(z) with the hardware reciprocal (about 1 ulp): for epilogues
__device__ __forceinline__ float fast_silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ float wave_sum_f32(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

}  // namespace moe

/*
 * synth.c -- seeded synthetic inputs for one MoE FFN layer.
 *
 * This file draws random numbers and lays them out in the container format:
 * nothing else.  It holds none of the layer's arithmetic (no dot products, no
 * sigmoid, no selection, no dequantisation), so the CPU oracle and the HIP
 * path can both consume its output without sharing any part of the method.
 *
 * Generator: xoshiro256** (Blackman & Vigna, "Scrambled linear pseudorandom
 * number generators", 2018) whose 256-bit state is filled by SplitMix64
 * (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
 * 2014).  Every row of every tensor has its own stream, keyed by
 * (seed, layer, tensor id, row), so rows can be generated in parallel and a
 * tensor's content never depends on the thread count or on the memory layout
 * it is written into.
 *
 * Formats written (the colibri-nano README, "Converting a checkpoint
 * yourself": per-row symmetric quantisation with f32 scales in a sibling .qs
 * tensor):
 *   - packed int4: a row of `cols` signed 4-bit values takes cols/2 bytes;
 *     element 2c sits in the low nibble of byte c and element 2c+1 in the
 *     high nibble, two's complement;
 *   - int8: one signed byte per element;
 *   - bf16: the upper 16 bits of an IEEE binary32 after round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t sm64_next(uint64_t *x)
{
    uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

typedef struct { uint64_t s[4]; } xo256;

static inline uint64_t rotl64(uint64_t v, int k) { return (v << k) | (v >> (64 - k)); }

static inline uint64_t xo_next(xo256 *r)
{
    const uint64_t out = rotl64(r->s[1] * 5u, 7) * 9u;
    const uint64_t t = r->s[1] << 17;
    r->s[2] ^= r->s[0];
    r->s[3] ^= r->s[1];
    r->s[1] ^= r->s[2];
    r->s[0] ^= r->s[3];
    r->s[2] ^= t;
    r->s[3] = rotl64(r->s[3], 45);
    return out;
}

/* One stream per (seed, layer, tensor, row).  Each key is folded in through
 * its own SplitMix64 step so that neighbouring keys give unrelated states. */
static void xo_seed(xo256 *r, uint64_t seed, uint64_t layer, uint64_t tensor, uint64_t row)
{
    uint64_t x = seed;
    uint64_t k = sm64_next(&x);
    x = k ^ (layer * 0xD1B54A32D192ED03ull);
    k = sm64_next(&x);
    x = k ^ (tensor * 0x8CB92BA72F3D8DD7ull);
    k = sm64_next(&x);
    x = k ^ (row * 0xABC98388FB8FAC03ull + 0x632BE59BD9B4E019ull);
    for (int i = 0; i < 4; ++i) r->s[i] = sm64_next(&x);
}

/* uniform in [0, 1) with 53 random bits */
static inline double u01(xo256 *r) { return (double)(xo_next(r) >> 11) * 0x1.0p-53; }

/* uniform integer in [0, n) from 32 random bits by multiply-shift
 * (Lemire, "Fast random integer generation in an interval", 2019, without the
 * rejection step; the bias is below n / 2^32). */
static inline uint32_t below(uint32_t r32, uint32_t n) { return (uint32_t)(((uint64_t)r32 * n) >> 32); }

/* Box-Muller pair: two independent N(0,1) draws */
static inline void normal_pair(xo256 *r, double *a, double *b)
{
    double u1 = ((double)(xo_next(r) >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    double u2 = u01(r);
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *a = rad * cos(th);
    *b = rad * sin(th);
}

static inline uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* rows x cols f32 values ~ N(mean, std^2), one stream per row. */
void synth_normal_f32(uint64_t seed, int32_t layer, int32_t tensor, int64_t rows, int64_t cols,
                      float mean, float stdv, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        xo256 g;
        xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)r);
        float *o = out + r * cols;
        for (int64_t c = 0; c < cols; c += 2) {
            double a, b;
            normal_pair(&g, &a, &b);
            o[c] = (float)(mean + stdv * a);
            if (c + 1 < cols) o[c + 1] = (float)(mean + stdv * b);
        }
    }
}

/* rows x cols bf16 values: an f32 N(0,1) draw rounded to nearest even. */
void synth_normal_bf16(uint64_t seed, int32_t layer, int32_t tensor, int64_t rows, int64_t cols,
                       float stdv, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        xo256 g;
        xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)r);
        uint16_t *o = out + r * cols;
        for (int64_t c = 0; c < cols; c += 2) {
            double a, b;
            normal_pair(&g, &a, &b);
            o[c] = f32_to_bf16_bits((float)(stdv * a));
            if (c + 1 < cols) o[c + 1] = f32_to_bf16_bits((float)(stdv * b));
        }
    }
}

/* n f32 values ~ U(lo, hi) in one stream (row 0). */
void synth_uniform_f32(uint64_t seed, int32_t layer, int32_t tensor, int64_t n, float lo, float hi,
                       float *out)
{
    xo256 g;
    xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, 0);
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * u01(&g));
}

/* rows x cols signed 4-bit values, uniform over [-qmax, qmax], packed two per
 * byte (element 2c in the low nibble).  `dst_row_bytes` is the distance between
 * consecutive output rows, so a tensor can be written into a strided block
 * (an expert's three matrices stored back to back). */
void synth_int4_packed(uint64_t seed, int32_t layer, int32_t tensor, int64_t rows, int64_t cols,
                       int32_t qmax, uint8_t *out, int64_t dst_row_bytes, int64_t rows_per_block,
                       int64_t block_stride_bytes)
{
    const uint32_t span = (uint32_t)(2 * qmax + 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        xo256 g;
        xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)r);
        uint8_t *o = out + (r / rows_per_block) * block_stride_bytes + (r % rows_per_block) * dst_row_bytes;
        for (int64_t c = 0; c < cols / 2; ++c) {
            uint64_t w = xo_next(&g);
            int32_t lo = (int32_t)below((uint32_t)w, span) - qmax;
            int32_t hi = (int32_t)below((uint32_t)(w >> 32), span) - qmax;
            o[c] = (uint8_t)(((uint32_t)lo & 0xFu) | (((uint32_t)hi & 0xFu) << 4));
        }
    }
}

/* rows x cols int8 values uniform over [-qmax, qmax], strided like above. */
void synth_int8(uint64_t seed, int32_t layer, int32_t tensor, int64_t rows, int64_t cols, int32_t qmax,
                int8_t *out, int64_t dst_row_bytes, int64_t rows_per_block, int64_t block_stride_bytes)
{
    const uint32_t span = (uint32_t)(2 * qmax + 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        xo256 g;
        xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)r);
        int8_t *o = out + (r / rows_per_block) * block_stride_bytes + (r % rows_per_block) * dst_row_bytes;
        for (int64_t c = 0; c < cols; c += 2) {
            uint64_t w = xo_next(&g);
            o[c] = (int8_t)((int32_t)below((uint32_t)w, span) - qmax);
            if (c + 1 < cols) o[c + 1] = (int8_t)((int32_t)below((uint32_t)(w >> 32), span) - qmax);
        }
    }
}

/* f32 scales ~ U(lo, hi), one per row, written with a stride so the scales of
 * an expert's three matrices can sit back to back. */
void synth_scales(uint64_t seed, int32_t layer, int32_t tensor, int64_t rows, float lo, float hi,
                  float *out, int64_t rows_per_block, int64_t block_stride_floats)
{
    xo256 g;
    xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, 0);
    for (int64_t r = 0; r < rows; ++r)
        out[(r / rows_per_block) * block_stride_floats + (r % rows_per_block)] =
            (float)(lo + (hi - lo) * u01(&g));
}

/* a uniformly random permutation of 0..n-1 (Fisher-Yates). */
void synth_permutation(uint64_t seed, int32_t layer, int32_t tensor, int32_t n, int32_t *out)
{
    xo256 g;
    xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, 0);
    for (int32_t i = 0; i < n; ++i) out[i] = i;
    for (int32_t i = n - 1; i > 0; --i) {
        int32_t j = (int32_t)below((uint32_t)(xo_next(&g) >> 32), (uint32_t)(i + 1));
        int32_t t = out[i];
        out[i] = out[j];
        out[j] = t;
    }
}

/* small-integer bf16 values uniform over [-vmax, vmax] (exact in bf16). */
void synth_small_int_bf16(uint64_t seed, int32_t layer, int32_t tensor, int64_t rows, int64_t cols,
                          int32_t vmax, uint16_t *out)
{
    const uint32_t span = (uint32_t)(2 * vmax + 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        xo256 g;
        xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)r);
        for (int64_t c = 0; c < cols; ++c) {
            int32_t v = (int32_t)below((uint32_t)(xo_next(&g) >> 32), span) - vmax;
            out[r * cols + c] = f32_to_bf16_bits((float)v);
        }
    }
}

/* raw 64-bit outputs of one stream, for the generator's own reference test */
void synth_raw_u64(uint64_t seed, int32_t layer, int32_t tensor, int64_t row, int64_t n, uint64_t *out)
{
    xo256 g;
    xo_seed(&g, seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)row);
    for (int64_t i = 0; i < n; ++i) out[i] = xo_next(&g);
}

/*
 * oracle_moe.c -- plain CPU oracle for one MoE FFN layer forward pass.
 *
 * TEST INFRASTRUCTURE: see oracle_moe.h for who may call it, what it follows
 * and its precision rules.  Loops are written in the order the method is
 * described -- route, group the pairs by expert, run each expert's FFN on its
 * rows, run the shared expert, combine -- with no blocking or fusion.
 */
#include "oracle_moe.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define O_OK 0
#define O_ERR_NULL (-1)
#define O_ERR_SHAPE (-2)
#define O_ERR_NOMEM (-7)

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the following oracle calls from this thread (n >= 1); the
 * results do not depend on it (no reduction is split across threads). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- formats */

float oracle_bf16_to_f32(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* round to nearest, ties to even (finite inputs) */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Packed int4 reading (the pages say only "packed int4, per-row scales"):
 * element 2c is the low nibble of byte c, element 2c+1 the high nibble, both
 * two's complement, so nibble 0x8 decodes to -8. */
void oracle_unpack_int4_row(const uint8_t *row, int32_t cols, int32_t *vals)
{
    for (int32_t c = 0; c < cols; ++c) {
        uint32_t byte = row[c / 2];
        uint32_t nib = (c % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
        vals[c] = (nib >= 8u) ? (int32_t)nib - 16 : (int32_t)nib;
    }
}

/* Packed int2 (see oracle_weights.expert_bits): element 4c + j in bits
 * 2j..2j+1 of byte c, two's complement. */
void oracle_unpack_int2_row(const uint8_t *row, int32_t cols, int32_t *vals)
{
    for (int32_t c = 0; c < cols; ++c) {
        uint32_t f = ((uint32_t)row[c / 4] >> (2 * (c % 4))) & 3u;
        vals[c] = (f >= 2u) ? (int32_t)f - 4 : (int32_t)f;
    }
}

void oracle_pack_int4_row(const int32_t *vals, int32_t cols, uint8_t *row)
{
    for (int32_t c = 0; c < cols; c += 2) {
        uint32_t lo = (uint32_t)vals[c] & 0xFu;
        uint32_t hi = (c + 1 < cols) ? ((uint32_t)vals[c + 1] & 0xFu) : 0u;
        row[c / 2] = (uint8_t)(lo | (hi << 4));
    }
}

/* Per-row symmetric dequantisation: w = q * scale, one f32 scale per row
 * (colibri-nano README, "Converting a checkpoint yourself"). */
void oracle_dequant_row(const void *q, int32_t bits, const float *scale, int32_t cols, float *out)
{
    const float s = scale[0];
    if (bits == 2) {
        for (int32_t c = 0; c < cols; ++c) {
            uint32_t f = ((uint32_t)((const uint8_t *)q)[c / 4] >> (2 * (c % 4))) & 3u;
            int32_t v = (f >= 2u) ? (int32_t)f - 4 : (int32_t)f;
            out[c] = (float)v * s;
        }
    } else if (bits == 4) {
        const uint8_t *row = (const uint8_t *)q;
        for (int32_t c = 0; c < cols; ++c) {
            uint32_t byte = row[c / 2];
            uint32_t nib = (c % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
            int32_t v = (nib >= 8u) ? (int32_t)nib - 16 : (int32_t)nib;
            out[c] = (float)v * s;
        }
    } else {
        const int8_t *row = (const int8_t *)q;
        for (int32_t c = 0; c < cols; ++c) out[c] = (float)row[c] * s;
    }
}

/* ---------------------------------------------------------------- quantiser */

/* See oracle_moe.h for the reading.  Rows are independent, so they are split
 * across threads; each row is done in column order. */
int oracle_quantize_rows(const void *src, int32_t src_bf16, int64_t rows, int32_t cols, int32_t bits, void *q,
                         float *qs)
{
    if (rows < 0 || cols <= 0 || (bits != 4 && bits != 8) || (bits == 4 && cols % 2)) return O_ERR_SHAPE;
    if (rows == 0) return O_OK;
    if (!src || !q || !qs) return O_ERR_NULL;
    const float qmax = (bits == 4) ? 7.0f : 127.0f;
    const int64_t row_bytes = (bits == 4) ? cols / 2 : cols;
    int failed = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float *w = (float *)malloc((size_t)cols * sizeof(float));
        int32_t *code = (int32_t *)malloc((size_t)cols * sizeof(int32_t));
        if (!w || !code) {
            free(w);
            free(code);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        /* the row in f32 */
        for (int32_t c = 0; c < cols; ++c)
            w[c] = src_bf16 ? oracle_bf16_to_f32(((const uint16_t *)src)[r * cols + c])
                            : ((const float *)src)[r * cols + c];
        /* its largest magnitude and the scale */
        float amax = 0.0f;
        for (int32_t c = 0; c < cols; ++c)
            if (fabsf(w[c]) > amax) amax = fabsf(w[c]);
        const float scale = amax / qmax;
        /* the codes: nearest integer, ties to even, inside [-qmax, qmax] */
        for (int32_t c = 0; c < cols; ++c) {
            if (amax == 0.0f) {
                code[c] = 0;
                continue;
            }
            float v = nearbyintf(w[c] / scale);
            if (v > qmax) v = qmax;
            if (v < -qmax) v = -qmax;
            code[c] = (int32_t)v;
        }
        qs[r] = scale;
        if (bits == 4) {
            oracle_pack_int4_row(code, cols, (uint8_t *)q + r * row_bytes);
        } else {
            int8_t *out = (int8_t *)q + r * row_bytes;
            for (int32_t c = 0; c < cols; ++c) out[c] = (int8_t)code[c];
        }
        free(w);
        free(code);
    }
    return failed ? O_ERR_NOMEM : O_OK;
}

/* One block of Q8_0-style activation codes: the rule above with qmax 127 over
 * the n values of v (see ORACLE_ACT_Q8 in oracle_moe.h). */
static float q8_block(const float *v, int32_t n, int8_t *q)
{
    float amax = 0.0f;
    for (int32_t c = 0; c < n; ++c)
        if (fabsf(v[c]) > amax) amax = fabsf(v[c]);
    const float d = amax / 127.0f;
    for (int32_t c = 0; c < n; ++c) {
        if (amax == 0.0f) {
            q[c] = 0;
            continue;
        }
        float t = nearbyintf(v[c] / d);
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        q[c] = (int8_t)t;
    }
    return d;
}

static void q8_row(const float *v, int32_t n, int8_t *q, float *d)
{
    for (int32_t b = 0; b < n / 32; ++b) d[b] = q8_block(v + 32 * b, 32, q + 32 * b);
}

int oracle_quantize_act_q8(const void *src, int32_t src_bf16, int64_t rows, int32_t cols, int8_t *q, float *d)
{
    if (rows < 0 || cols <= 0 || cols % 32) return O_ERR_SHAPE;
    if (rows == 0) return O_OK;
    if (!src || !q || !d) return O_ERR_NULL;
    int failed = 0;
#pragma omp parallel
    {
        float *v = (float *)malloc((size_t)cols * sizeof(float));
        if (!v) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < rows; ++r) {
                for (int32_t c = 0; c < cols; ++c)
                    v[c] = src_bf16 ? oracle_bf16_to_f32(((const uint16_t *)src)[r * cols + c])
                                    : ((const float *)src)[r * cols + c];
                q8_row(v, cols, q + r * cols, d + r * (cols / 32));
            }
        }
        free(v);
    }
    return failed ? O_ERR_NOMEM : O_OK;
}

/* ---------------------------------------------------------------- bias update */

int oracle_bias_update(int32_t E, const int32_t *counts, const float *bias_in, float gamma, float *bias_out)
{
    if (E <= 0) return O_ERR_SHAPE;
    if (!counts || !bias_in || !bias_out) return O_ERR_NULL;
    int64_t total = 0;
    for (int32_t e = 0; e < E; ++e) total += counts[e];
    for (int32_t e = 0; e < E; ++e) {
        const int64_t load = (int64_t)E * counts[e];  /* E times this expert's load, against E times the mean */
        if (load < total)
            bias_out[e] = bias_in[e] + gamma;  /* under-loaded: more likely to be selected */
        else if (load > total)
            bias_out[e] = bias_in[e] - gamma;  /* over-loaded: less likely */
        else
            bias_out[e] = bias_in[e];
    }
    return O_OK;
}

/* row r of expert e of a matrix family with `cols` columns */
static const void *qrow(const oracle_qmat *m, int32_t bits, int32_t e, int64_t r, int32_t cols)
{
    int64_t row_bytes = (bits == 4) ? cols / 2 : (bits == 2) ? cols / 4 : cols;
    return (const uint8_t *)m->q + (int64_t)e * m->q_stride_bytes + r * row_bytes;
}

/* the weight format of routed expert e */
static int32_t rbits(const oracle_weights *wt, int32_t e) { return wt->expert_bits ? wt->expert_bits[e] : 4; }

static const float *qscale(const oracle_qmat *m, int32_t e, int64_t r)
{
    return m->qs + (int64_t)e * m->qs_stride_floats + r;
}

static double dot_f64(const float *a, const float *b, int32_t n)
{
    double acc = 0.0;
    for (int32_t i = 0; i < n; ++i) acc += (double)a[i] * (double)b[i];
    return acc;
}

static void widen_row(const uint16_t *x, int32_t n, float *out)
{
    for (int32_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(x[i]);
}

static int check_shape(const oracle_shape *sh)
{
    if (!sh) return O_ERR_NULL;
    if (sh->T < 0 || sh->H <= 0 || sh->E <= 0 || sh->top_k <= 0 || sh->I <= 0) return O_ERR_SHAPE;
    if (sh->top_k > sh->E) return O_ERR_SHAPE;
    if (sh->H % 2 || sh->I % 2) return O_ERR_SHAPE;
    if (sh->shared_bits != 0 && sh->shared_bits != 4 && sh->shared_bits != 8) return O_ERR_SHAPE;
    if (sh->shared_bits && (sh->I_shared <= 0 || sh->I_shared % 2)) return O_ERR_SHAPE;
    if (sh->n_group <= 0 || sh->E % sh->n_group) return O_ERR_SHAPE;
    if (sh->topk_group <= 0 || sh->topk_group > sh->n_group) return O_ERR_SHAPE;
    if (sh->n_group > 1 && sh->E / sh->n_group < 2) return O_ERR_SHAPE;
    if (sh->top_k > sh->topk_group * (sh->E / sh->n_group)) return O_ERR_SHAPE;
    if (sh->top_p != sh->top_p || (sh->top_p > 0.f && sh->top_p < 1.f && sh->top_k > 256)) return O_ERR_SHAPE;
    if ((sh->flags & ORACLE_ACT_Q8) && (sh->H % 32 || sh->I % 32 || (sh->shared_bits && sh->I_shared % 32)))
        return O_ERR_SHAPE;
    return O_OK;
}

/* ---------------------------------------------------------------- router */

/* Logits z = x . W_e (W one row per expert), scores s = 1/(1+exp(-z)), and
 * the selection score b = s + bias: the bias is added after the sigmoid and is
 * used only to choose experts (model card "Architecture": sigmoid+bias router,
 * DeepSeek-V3-style aux-loss-free balancing). */
static void token_scores(const oracle_shape *sh, const float *xf, const float *W, const float *bias,
                         float *z, float *s, float *b)
{
    for (int32_t e = 0; e < sh->E; ++e) {
        float ze = (float)dot_f64(xf, W + (int64_t)e * sh->H, sh->H);
        float se = (float)(1.0 / (1.0 + exp(-(double)ze)));
        z[e] = ze;
        s[e] = se;
        b[e] = se + bias[e];
    }
}

/* Selection for one token.
 * Group-limited ("noaux_tc", colibri README "What's implemented"), read as:
 * experts split into n_group contiguous groups; a group's score is the sum of
 * its two largest b; the topk_group best groups are kept (ties -> lower group
 * id); experts of the other groups cannot be chosen.
 * Then the top_k largest b among the allowed experts, ties -> lower expert id,
 * listed in descending b.  Weights are the unbiased scores of the chosen
 * experts divided by their sum (normalised sigmoid scores); the routed scaling
 * factor is applied later, in the combine. */
/* Adaptive expert top-p (colibri README, "Got a better machine", the
 * `--topp 0.7` knob: adaptive expert top-p, less expert traffic).  The pages
 * give no formula; the reading here is nucleus selection over the routing
 * weights: rank the k selections by weight (descending; equal weights, the
 * lower id first), keep the shortest prefix of that ranking whose weights
 * add up to at least p (the running sum in f32, in rank order, as the kernel
 * decides it), drop the rest (id -1, weight 0) and renormalise the kept
 * weights: w_j = s_j / (sum of the kept s). */
static void apply_top_p(float p, int32_t k, const float *s, int32_t *ids, float *w)
{
    int32_t ord[256];
    for (int32_t j = 0; j < k; ++j) ord[j] = j;
    for (int32_t a = 0; a < k; ++a) /* selection sort by (w desc, id asc) */
        for (int32_t c = a + 1; c < k; ++c) {
            const int32_t x = ord[a], y = ord[c];
            if (w[y] > w[x] || (w[y] == w[x] && ids[y] < ids[x])) {
                ord[a] = y;
                ord[c] = x;
            }
        }
    float mass = 0.f;
    int32_t keep = 0;
    while (keep < k && mass < p) mass += w[ord[keep++]];
    unsigned char kept[256] = {0};
    double ks = 0.0;
    for (int32_t r = 0; r < keep; ++r) {
        kept[ord[r]] = 1;
        ks += (double)s[ids[ord[r]]];
    }
    for (int32_t j = 0; j < k; ++j) {
        if (kept[j]) {
            w[j] = (float)((double)s[ids[j]] / ks);
        } else {
            ids[j] = -1;
            w[j] = 0.f;
        }
    }
}

static void token_select(const oracle_shape *sh, const float *s, const float *b, int32_t *ids, float *w,
                         float *gap, float *ggap, unsigned char *allowed, float *gscore, unsigned char *gkept)
{
    const int32_t E = sh->E, k = sh->top_k;
    float group_gap = INFINITY;
    for (int32_t e = 0; e < E; ++e) allowed[e] = 1;
    if (sh->n_group > 1 && sh->topk_group < sh->n_group) {
        const int32_t Eg = E / sh->n_group;
        for (int32_t g = 0; g < sh->n_group; ++g) {
            /* two largest b of the group */
            float b1 = -INFINITY, b2 = -INFINITY;
            for (int32_t e = g * Eg; e < (g + 1) * Eg; ++e) {
                if (b[e] > b1) {
                    b2 = b1;
                    b1 = b[e];
                } else if (b[e] > b2) {
                    b2 = b[e];
                }
            }
            gscore[g] = b1 + b2;
            gkept[g] = 0;
        }
        float last_kept = 0.f;
        for (int32_t r = 0; r < sh->topk_group; ++r) {
            int32_t best = -1;
            for (int32_t g = 0; g < sh->n_group; ++g)
                if (!gkept[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
            gkept[best] = 1;
            last_kept = gscore[best];
        }
        float first_dropped = -INFINITY;
        for (int32_t g = 0; g < sh->n_group; ++g)
            if (!gkept[g] && gscore[g] > first_dropped) first_dropped = gscore[g];
        group_gap = last_kept - first_dropped;
        for (int32_t e = 0; e < E; ++e) allowed[e] = gkept[e / Eg];
    }
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
            if (allowed[e] && (best < 0 || b[e] > b[best])) best = e;
        ids[j] = best;
        allowed[best] = 0; /* taken */
    }
    float next = -INFINITY;
    int any = 0;
    for (int32_t e = 0; e < E; ++e)
        if (allowed[e] && (!any || b[e] > next)) {
            next = b[e];
            any = 1;
        }
    if (gap) *gap = any ? b[ids[k - 1]] - next : INFINITY;
    if (ggap) *ggap = group_gap;
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) sum += (double)s[ids[j]];
    for (int32_t j = 0; j < k; ++j) w[j] = (float)((double)s[ids[j]] / sum);
    if (sh->top_p > 0.f && sh->top_p < 1.f) apply_top_p(sh->top_p, k, s, ids, w);
}

int oracle_router_scores(const oracle_shape *sh, const uint16_t *hidden, const float *W, const float *bias,
                         float *z, float *s, float *b)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!hidden || !W || !bias) return O_ERR_NULL;
    const int32_t E = sh->E, H = sh->H;
    int fail = 0;
#pragma omp parallel
    {
        float *xf = malloc(sizeof(float) * H);
        float *tz = malloc(sizeof(float) * E * 3);
        if (!xf || !tz) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int32_t t = 0; t < sh->T; ++t) {
                widen_row(hidden + (int64_t)t * H, H, xf);
                token_scores(sh, xf, W, bias, tz, tz + E, tz + 2 * E);
                if (z) memcpy(z + (int64_t)t * E, tz, sizeof(float) * E);
                if (s) memcpy(s + (int64_t)t * E, tz + E, sizeof(float) * E);
                if (b) memcpy(b + (int64_t)t * E, tz + 2 * E, sizeof(float) * E);
            }
        }
        free(xf);
        free(tz);
    }
    return fail ? O_ERR_NOMEM : O_OK;
}

/* route a list of tokens (all when tokens == NULL); outputs indexed by list position */
static int route_tokens(const oracle_shape *sh, const uint16_t *hidden, const float *W, const float *bias,
                        const int32_t *tokens, int32_t n, int32_t *ids, float *w, float *gap, float *ggap)
{
    const int32_t E = sh->E, H = sh->H, k = sh->top_k;
    int fail = 0;
#pragma omp parallel
    {
        float *xf = malloc(sizeof(float) * H);
        float *tz = malloc(sizeof(float) * E * 3);
        unsigned char *allowed = malloc((size_t)E);
        float *gscore = malloc(sizeof(float) * sh->n_group);
        unsigned char *gkept = malloc((size_t)sh->n_group);
        if (!xf || !tz || !allowed || !gscore || !gkept) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int32_t i = 0; i < n; ++i) {
                int32_t t = tokens ? tokens[i] : i;
                widen_row(hidden + (int64_t)t * H, H, xf);
                token_scores(sh, xf, W, bias, tz, tz + E, tz + 2 * E);
                token_select(sh, tz + E, tz + 2 * E, ids + (int64_t)i * k, w + (int64_t)i * k,
                             gap ? gap + i : NULL, ggap ? ggap + i : NULL, allowed, gscore, gkept);
            }
        }
        free(xf);
        free(tz);
        free(allowed);
        free(gscore);
        free(gkept);
    }
    return fail ? O_ERR_NOMEM : O_OK;
}

int oracle_router(const oracle_shape *sh, const uint16_t *hidden, const float *W, const float *bias,
                  int32_t *ids, float *w, float *gap, float *ggap)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!hidden || !W || !bias || !ids || !w) return O_ERR_NULL;
    return route_tokens(sh, hidden, W, bias, NULL, sh->T, ids, w, gap, ggap);
}

/* ----------------------------------------------------------- permutation */

/* Batch-union grouping (colibri README "What's implemented": each unique
 * expert of the batch is read once and applied to every position routed to
 * it): a stable counting sort of the pairs p = t*k + j by expert id, so the
 * rows of one expert are contiguous and in ascending pair order. */
int oracle_permute(const oracle_shape *sh, const int32_t *ids, int32_t *counts, int32_t *offsets,
                   int32_t *sorted, int32_t *inv)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!ids || !counts || !offsets || !sorted || !inv) return O_ERR_NULL;
    const int64_t P = (int64_t)sh->T * sh->top_k;
    for (int32_t e = 0; e < sh->E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] == -1) continue; /* dropped by adaptive top-p */
        if (ids[p] < 0 || ids[p] >= sh->E) return O_ERR_SHAPE;
        counts[ids[p]] += 1;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < sh->E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = malloc(sizeof(int32_t) * sh->E);
    if (!fill) return O_ERR_NOMEM;
    for (int32_t e = 0; e < sh->E; ++e) fill[e] = offsets[e];
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] == -1) {
            inv[p] = -1;
            continue;
        }
        int32_t pos = fill[ids[p]]++;
        sorted[pos] = (int32_t)p;
        inv[p] = pos;
    }
    free(fill);
    return O_OK;
}

/* ------------------------------------------------------------ expert FFN */

/* SwiGLU expert (activation from the benchmark spec; the pages say only
 * that an expert has three matrices): g = x.Wg_i, u = x.Wu_i,
 * h_i = silu(g)*u with silu(z) = z/(1+exp(-z)), y_c = h.Wd_c. */
/* Q8_0-style dot of a quantised activation row with weight row r of expert
 * e: s_w * sum_b d_b * (sum over block b of q * code), block sums in integers. */
static double q8_dot(const int8_t *q, const float *d, const oracle_qmat *m, int32_t bits, int32_t e, int64_t r,
                     int32_t n, int32_t *codes)
{
    const void *row = qrow(m, bits, e, r, n);
    if (bits == 4) {
        oracle_unpack_int4_row((const uint8_t *)row, n, codes);
    } else if (bits == 2) {
        oracle_unpack_int2_row((const uint8_t *)row, n, codes);
    } else {
        for (int32_t c = 0; c < n; ++c) codes[c] = ((const int8_t *)row)[c];
    }
    double acc = 0.0;
    for (int32_t b = 0; b < n / 32; ++b) {
        int64_t isum = 0;
        for (int32_t c = 32 * b; c < 32 * b + 32; ++c) isum += (int64_t)q[c] * codes[c];
        acc += (double)d[b] * (double)isum;
    }
    return (double)*qscale(m, e, r) * acc;
}

/* The expert with Q8_0-style activations: x and then h (as f32) quantised per
 * 32-block, every dot as q8_dot; the SwiGLU as in ffn_one. */
static void ffn_one_q8(const float *xf, int32_t H, int32_t I, int32_t bits, const oracle_qmat *gate,
                       const oracle_qmat *up, const oracle_qmat *down, int32_t e, float *h, float *y)
{
    const int32_t n = H > I ? H : I;
    int8_t *q = malloc((size_t)n);
    float *d = malloc(sizeof(float) * (size_t)(n / 32));
    int32_t *codes = malloc(sizeof(int32_t) * (size_t)n);
    q8_row(xf, H, q, d);
    for (int32_t i = 0; i < I; ++i) {
        float g = (float)q8_dot(q, d, gate, bits, e, i, H, codes);
        float u = (float)q8_dot(q, d, up, bits, e, i, H, codes);
        h[i] = (float)((double)g / (1.0 + exp(-(double)g)) * (double)u);
    }
    q8_row(h, I, q, d);
    for (int32_t c = 0; c < H; ++c) y[c] = (float)q8_dot(q, d, down, bits, e, c, I, codes);
    free(q);
    free(d);
    free(codes);
}

static void ffn_one(const float *xf, int32_t H, int32_t I, int32_t bits, const oracle_qmat *gate,
                    const oracle_qmat *up, const oracle_qmat *down, int32_t e, float *h, float *wrow, float *y,
                    int q8)
{
    if (q8) {
        ffn_one_q8(xf, H, I, bits, gate, up, down, e, h, y);
        return;
    }
    for (int32_t i = 0; i < I; ++i) {
        oracle_dequant_row(qrow(gate, bits, e, i, H), bits, qscale(gate, e, i), H, wrow);
        float g = (float)dot_f64(xf, wrow, H);
        oracle_dequant_row(qrow(up, bits, e, i, H), bits, qscale(up, e, i), H, wrow);
        float u = (float)dot_f64(xf, wrow, H);
        h[i] = (float)((double)g / (1.0 + exp(-(double)g)) * (double)u);
    }
    for (int32_t c = 0; c < H; ++c) {
        oracle_dequant_row(qrow(down, bits, e, c, I), bits, qscale(down, e, c), I, wrow);
        y[c] = (float)dot_f64(h, wrow, I);
    }
}

static int32_t expert_of_row(const int32_t *offsets, int32_t E, int32_t r)
{
    int32_t lo = 0, hi = E - 1; /* largest e with offsets[e] <= r */
    while (lo < hi) {
        int32_t mid = (lo + hi + 1) / 2;
        if (offsets[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    while (lo + 1 < E && offsets[lo + 1] <= r) ++lo; /* skip empty experts sharing the offset */
    return lo;
}

int oracle_expert_ffn(const oracle_shape *sh, const uint16_t *hidden, const oracle_weights *wt,
                      const int32_t *offsets, const int32_t *sorted, const float *pair_scale, float *y_pairs)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!hidden || !wt || !offsets || !sorted || !y_pairs) return O_ERR_NULL;
    const int32_t H = sh->H, I = sh->I, k = sh->top_k, E = sh->E;
    const int32_t rows = offsets[E];
    const int32_t wmax = H > I ? H : I;
    int fail = 0;
#pragma omp parallel
    {
        float *xf = malloc(sizeof(float) * H);
        float *h = malloc(sizeof(float) * I);
        float *wrow = malloc(sizeof(float) * wmax);
        if (!xf || !h || !wrow) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int32_t r = 0; r < rows; ++r) {
                int32_t e = expert_of_row(offsets, E, r);
                int32_t p = sorted[r];
                int32_t t = p / k;
                float *y = y_pairs + (int64_t)r * H;
                widen_row(hidden + (int64_t)t * H, H, xf);
                ffn_one(xf, H, I, rbits(wt, e), &wt->gate, &wt->up, &wt->down, e, h, wrow, y,
                        (sh->flags & ORACLE_ACT_Q8) != 0);
                if (pair_scale) {
                    const double c = (double)pair_scale[p];
                    for (int32_t j = 0; j < H; ++j) y[j] = (float)((double)y[j] * c);
                }
            }
        }
        free(xf);
        free(h);
        free(wrow);
    }
    return fail ? O_ERR_NOMEM : O_OK;
}

/* the shared expert on a list of tokens (all when tokens == NULL) */
static int shared_tokens(const oracle_shape *sh, const uint16_t *hidden, const oracle_weights *wt,
                         const int32_t *tokens, int32_t n, float *out)
{
    const int32_t H = sh->H, I = sh->I_shared;
    if (sh->shared_bits == 0) {
        memset(out, 0, sizeof(float) * (size_t)n * H);
        return O_OK;
    }
    const int32_t wmax = H > I ? H : I;
    int fail = 0;
#pragma omp parallel
    {
        float *xf = malloc(sizeof(float) * H);
        float *h = malloc(sizeof(float) * I);
        float *wrow = malloc(sizeof(float) * wmax);
        if (!xf || !h || !wrow) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int32_t i = 0; i < n; ++i) {
                int32_t t = tokens ? tokens[i] : i;
                widen_row(hidden + (int64_t)t * H, H, xf);
                ffn_one(xf, H, I, sh->shared_bits, &wt->sh_gate, &wt->sh_up, &wt->sh_down, 0, h, wrow,
                        out + (int64_t)i * H, (sh->flags & ORACLE_ACT_Q8) != 0);
            }
        }
        free(xf);
        free(h);
        free(wrow);
    }
    return fail ? O_ERR_NOMEM : O_OK;
}

int oracle_shared_ffn(const oracle_shape *sh, const uint16_t *hidden, const oracle_weights *wt, float *out)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!hidden || !wt || !out) return O_ERR_NULL;
    return shared_tokens(sh, hidden, wt, NULL, sh->T, out);
}

/* --------------------------------------------------------------- combine */

/* out_t = sum over j (ascending) of c_j * y_{t,j} + shared_t (+ x_t), with
 * c_j = routed_scaling_factor * w_j: the scaling factor multiplies the routed
 * terms only; the shared expert is ungated (weight 1). One rounding to f32. */
int oracle_combine(const oracle_shape *sh, const float *y_pairs, const int32_t *inv, const float *topk_w,
                   const float *shared_out, const uint16_t *residual, float *out)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!y_pairs || !inv || !out) return O_ERR_NULL;
    const int32_t H = sh->H, k = sh->top_k;
    const double rsf = (double)sh->routed_scaling_factor;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < sh->T; ++t) {
        for (int32_t c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int64_t p = (int64_t)t * k + j;
                if (inv[p] < 0) continue; /* a pair dropped by adaptive top-p */
                double coef = topk_w ? rsf * (double)topk_w[p] : 1.0;
                acc += coef * (double)y_pairs[(int64_t)inv[p] * H + c];
            }
            if (shared_out) acc += (double)shared_out[(int64_t)t * H + c];
            if (residual) acc += (double)oracle_bf16_to_f32(residual[(int64_t)t * H + c]);
            out[(int64_t)t * H + c] = (float)acc;
        }
    }
    return O_OK;
}

/* ----------------------------------------------------------- whole layer */

int oracle_layer_forward(const oracle_shape *sh, const oracle_weights *wt, const uint16_t *hidden, float *out,
                         int32_t *ids_out, float *w_out, float *gap_out, float *ggap_out)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!wt || !hidden || !out) return O_ERR_NULL;
    const int64_t T = sh->T, k = sh->top_k, H = sh->H, P = T * k;
    if (T == 0) return O_OK;
    int32_t *ids = malloc(sizeof(int32_t) * P);
    float *w = malloc(sizeof(float) * P);
    int32_t *counts = malloc(sizeof(int32_t) * sh->E);
    int32_t *offsets = malloc(sizeof(int32_t) * (sh->E + 1));
    int32_t *sorted = malloc(sizeof(int32_t) * P);
    int32_t *inv = malloc(sizeof(int32_t) * P);
    float *y = malloc(sizeof(float) * P * H);
    float *shout = malloc(sizeof(float) * T * H);
    if (!ids || !w || !counts || !offsets || !sorted || !inv || !y || !shout) {
        st = O_ERR_NOMEM;
        goto done;
    }
    st = oracle_router(sh, hidden, wt->router_w, wt->router_bias, ids, w, gap_out, ggap_out);
    if (!st) st = oracle_permute(sh, ids, counts, offsets, sorted, inv);
    if (!st) st = oracle_expert_ffn(sh, hidden, wt, offsets, sorted, NULL, y);
    if (!st) st = oracle_shared_ffn(sh, hidden, wt, shout);
    if (!st)
        st = oracle_combine(sh, y, inv, w, sh->shared_bits ? shout : NULL,
                            (sh->flags & ORACLE_ADD_RESIDUAL) ? hidden : NULL, out);
    if (!st && ids_out) memcpy(ids_out, ids, sizeof(int32_t) * P);
    if (!st && w_out) memcpy(w_out, w, sizeof(float) * P);
done:
    free(ids);
    free(w);
    free(counts);
    free(offsets);
    free(sorted);
    free(inv);
    free(y);
    free(shout);
    return st;
}

int oracle_layer_tokens(const oracle_shape *sh, const oracle_weights *wt, const uint16_t *hidden,
                        const int32_t *tokens, int32_t n, const int32_t *ids_in, const float *w_in, float *out)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!wt || !hidden || !tokens || !out) return O_ERR_NULL;
    if ((ids_in == NULL) != (w_in == NULL)) return O_ERR_NULL;
    const int32_t H = sh->H, I = sh->I, k = sh->top_k;
    for (int32_t i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= sh->T) return O_ERR_SHAPE;
    int32_t *ids = malloc(sizeof(int32_t) * ((size_t)n * k + 1));
    float *w = malloc(sizeof(float) * ((size_t)n * k + 1));
    float *shout = malloc(sizeof(float) * ((size_t)n * H + 1));
    if (!ids || !w || !shout) {
        st = O_ERR_NOMEM;
        goto done;
    }
    if (ids_in) {
        for (int32_t i = 0; i < n; ++i)
            for (int32_t j = 0; j < k; ++j) {
                ids[(int64_t)i * k + j] = ids_in[(int64_t)tokens[i] * k + j];
                w[(int64_t)i * k + j] = w_in[(int64_t)tokens[i] * k + j];
            }
    } else {
        st = route_tokens(sh, hidden, wt->router_w, wt->router_bias, tokens, n, ids, w, NULL, NULL);
        if (st) goto done;
    }
    st = shared_tokens(sh, hidden, wt, tokens, n, shout);
    if (st) goto done;
    {
        const double rsf = (double)sh->routed_scaling_factor;
        const int32_t wmax = H > I ? H : I;
        int fail = 0;
#pragma omp parallel
        {
            float *xf = malloc(sizeof(float) * H);
            float *h = malloc(sizeof(float) * I);
            float *wrow = malloc(sizeof(float) * wmax);
            float *y = malloc(sizeof(float) * (size_t)k * H);
            if (!xf || !h || !wrow || !y) {
#pragma omp atomic write
                fail = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int32_t i = 0; i < n; ++i) {
                    int32_t t = tokens[i];
                    widen_row(hidden + (int64_t)t * H, H, xf);
                    for (int32_t j = 0; j < k; ++j)
                        if (ids[(int64_t)i * k + j] >= 0) /* (-1: dropped by adaptive top-p) */
                            ffn_one(xf, H, I, rbits(wt, ids[(int64_t)i * k + j]), &wt->gate, &wt->up, &wt->down,
                                    ids[(int64_t)i * k + j], h, wrow,
                                    y + (int64_t)j * H, (sh->flags & ORACLE_ACT_Q8) != 0);
                    for (int32_t c = 0; c < H; ++c) {
                        double acc = 0.0;
                        for (int32_t j = 0; j < k; ++j)
                            if (ids[(int64_t)i * k + j] >= 0)
                                acc += rsf * (double)w[(int64_t)i * k + j] * (double)y[(int64_t)j * H + c];
                        if (sh->shared_bits) acc += (double)shout[(int64_t)i * H + c];
                        if (sh->flags & ORACLE_ADD_RESIDUAL) acc += (double)xf[c];
                        out[(int64_t)i * H + c] = (float)acc;
                    }
                }
            }
            free(xf);
            free(h);
            free(wrow);
            free(y);
        }
        if (fail) st = O_ERR_NOMEM;
    }
done:
    free(ids);
    free(w);
    free(shout);
    return st;
}

/* Brute force: every expert's FFN on every token, weighted by a dense [T][E]
 * coefficient mask that holds rsf*w at the routed experts and 0 elsewhere. */
int oracle_layer_forward_dense(const oracle_shape *sh, const oracle_weights *wt, const uint16_t *hidden,
                               float *out)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!wt || !hidden || !out) return O_ERR_NULL;
    const int32_t T = sh->T, E = sh->E, H = sh->H, I = sh->I, k = sh->top_k;
    if (T == 0) return O_OK;
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)T * k);
    float *w = malloc(sizeof(float) * (size_t)T * k);
    double *mask = calloc((size_t)T * E, sizeof(double));
    float *shout = malloc(sizeof(float) * (size_t)T * H);
    if (!ids || !w || !mask || !shout) {
        st = O_ERR_NOMEM;
        goto done;
    }
    st = oracle_router(sh, hidden, wt->router_w, wt->router_bias, ids, w, NULL, NULL);
    if (st) goto done;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j)
            if (ids[(int64_t)t * k + j] >= 0) /* (-1: dropped by adaptive top-p) */
                mask[(int64_t)t * E + ids[(int64_t)t * k + j]] =
                    (double)sh->routed_scaling_factor * (double)w[(int64_t)t * k + j];
    st = oracle_shared_ffn(sh, hidden, wt, shout);
    if (st) goto done;
    {
        const int32_t wmax = H > I ? H : I;
        int fail = 0;
#pragma omp parallel
        {
            float *xf = malloc(sizeof(float) * H);
            float *h = malloc(sizeof(float) * I);
            float *wrow = malloc(sizeof(float) * wmax);
            float *y = malloc(sizeof(float) * (size_t)E * H);
            if (!xf || !h || !wrow || !y) {
#pragma omp atomic write
                fail = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int32_t t = 0; t < T; ++t) {
                    widen_row(hidden + (int64_t)t * H, H, xf);
                    for (int32_t e = 0; e < E; ++e)
                        ffn_one(xf, H, I, rbits(wt, e), &wt->gate, &wt->up, &wt->down, e, h, wrow, y + (int64_t)e * H,
                                (sh->flags & ORACLE_ACT_Q8) != 0);
                    for (int32_t c = 0; c < H; ++c) {
                        double acc = 0.0;
                        for (int32_t e = 0; e < E; ++e)
                            acc += mask[(int64_t)t * E + e] * (double)y[(int64_t)e * H + c];
                        if (sh->shared_bits) acc += (double)shout[(int64_t)t * H + c];
                        if (sh->flags & ORACLE_ADD_RESIDUAL) acc += (double)xf[c];
                        out[(int64_t)t * H + c] = (float)acc;
                    }
                }
            }
            free(xf);
            free(h);
            free(wrow);
            free(y);
        }
        if (fail) st = O_ERR_NOMEM;
    }
done:
    free(ids);
    free(w);
    free(mask);
    free(shout);
    return st;
}

/* Unscaled integer sums sum_h x_h * q_{i,h} of each sorted row's expert, for
 * inputs whose exact products and sums fit a double: the integer-exact check. */
int oracle_gateup_int_sums(const oracle_shape *sh, const uint16_t *hidden, const oracle_weights *wt,
                           const int32_t *offsets, const int32_t *sorted, double *g, double *u)
{
    int st = check_shape(sh);
    if (st) return st;
    if (!hidden || !wt || !offsets || !sorted || !g || !u) return O_ERR_NULL;
    const int32_t H = sh->H, I = sh->I, k = sh->top_k, E = sh->E;
    const int32_t rows = offsets[E];
    int fail = 0;
#pragma omp parallel
    {
        int32_t *qv = malloc(sizeof(int32_t) * H);
        float *xf = malloc(sizeof(float) * H);
        if (!qv || !xf) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int32_t r = 0; r < rows; ++r) {
                int32_t e = expert_of_row(offsets, E, r);
                int32_t t = sorted[r] / k;
                widen_row(hidden + (int64_t)t * H, H, xf);
                for (int32_t i = 0; i < I; ++i) {
                    double ag = 0.0, au = 0.0;
                    oracle_unpack_int4_row((const uint8_t *)qrow(&wt->gate, 4, e, i, H), H, qv);
                    for (int32_t h = 0; h < H; ++h) ag += (double)xf[h] * (double)qv[h];
                    oracle_unpack_int4_row((const uint8_t *)qrow(&wt->up, 4, e, i, H), H, qv);
                    for (int32_t h = 0; h < H; ++h) au += (double)xf[h] * (double)qv[h];
                    g[(int64_t)r * I + i] = ag;
                    u[(int64_t)r * I + i] = au;
                }
            }
        }
        free(qv);
        free(xf);
    }
    return fail ? O_ERR_NOMEM : O_OK;
}

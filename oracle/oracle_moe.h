/*
 * oracle_moe.h -- plain CPU oracle for one MoE FFN layer forward pass.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP library never
 * includes, links or calls anything here, and this file shares no code,
 * header, table or constant with it.
 *
 * What it computes is the exact f32 dequant path of the colibri-nano README
 * ("Knobs", the IDOT=0 row: the integer-dot kernels switched off select an
 * exact f32 dequantised matmul) applied to the layer the pages describe:
 *   - a sigmoid router whose per-expert bias only decides selection
 *     (Colibri-Nano model card, "Architecture": sigmoid+bias router with
 *     DeepSeek-V3-style aux-loss-free balancing; colibri README, "What's
 *     implemented": DeepSeek-V3-style sigmoid router, noaux_tc,
 *     routed_scaling_factor, shared expert);
 *   - batch-union routing: each unique expert is applied to every position
 *     routed to it (colibri README, "What's implemented", batch-union MoE);
 *   - experts of three matrices (colibri README at 0d2fb6f, "Never wait for
 *     the disk twice") stored per-row symmetric: packed int4 or int8 rows
 *     with one f32 scale per row in a sibling .qs tensor (colibri-nano
 *     README, "Converting a checkpoint yourself");
 *   - a shared expert applied to every token (NanoColibri README, model
 *     table: top-2 of 64 plus a 2048-wide shared expert).
 * Modes beside it: adaptive expert top-p (oracle_shape.top_p), Q8_0-style
 * int8 activations with integer block sums (ORACLE_ACT_Q8: the integer-dot
 * kernels of the same README), and int2 cold-tail experts
 * (oracle_weights.expert_bits).
 * The readings taken where the pages are silent (activation, tie order,
 * group score, normalisation, nibble order, top-p rule, activation blocks,
 * int2 layout) are stated at each function or field.
 *
 * Precision: x is widened from bf16 exactly; weights are dequantised as the
 * f32 product q * qs; every dot product is accumulated in double and rounded
 * once to f32; every stored intermediate is f32.  Work is split across
 * threads only over independent outputs, so results do not depend on the
 * thread count.
 *
 * Parity pins (what fixes each function other than itself) are listed in the
 * test suite; none of the functions below is "parity unpinned".
 */
#ifndef ORACLE_MOE_H
#define ORACLE_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_ADD_RESIDUAL 2u
/* Q8_0-style int8 activations (colibri README, "What's implemented": the
 * integer-dot kernels take int8 activations).  Reading: the input row of
 * every expert matmul (x for gate and up, h for down) is cut into blocks of 32
 * consecutive elements along the contraction axis; each block gets
 * d = max|v| / 127 (f32 division) and codes q = the nearest integer to v / d
 * (f32 division, ties to even, inside [-127, 127]; an all-zero block has
 * d = 0 and codes 0), the rule of oracle_quantize_rows per block.  A dot is
 * s_w * sum over blocks of d * (sum of q * weight code), the inner sums in
 * integers.  h enters as f32.  H, I and I_shared must be multiples of 32. */
#define ORACLE_ACT_Q8 4u

typedef struct {
    int32_t T;            /* tokens */
    int32_t H;            /* hidden size */
    int32_t E;            /* routed experts */
    int32_t top_k;        /* experts per token */
    int32_t I;            /* routed intermediate size */
    int32_t I_shared;     /* shared intermediate size */
    int32_t shared_bits;  /* 0 (no shared expert), 4 or 8 */
    int32_t n_group;      /* expert groups for group-limited selection (1 = off) */
    int32_t topk_group;   /* groups kept */
    float routed_scaling_factor;
    uint32_t flags;       /* ORACLE_ADD_RESIDUAL: the combine adds the layer input; ORACLE_ACT_Q8 */
    float top_p;          /* adaptive expert top-p, 0 < top_p < 1; any other value keeps all top_k */
} oracle_shape;

/* One quantised matrix family: expert e's rows start at q + e*q_stride_bytes
 * and its scales at qs + e*qs_stride_floats.  Row r of an int4 matrix with
 * `cols` columns is cols/2 bytes; of an int8 matrix, cols bytes. */
typedef struct {
    const void *q;
    const float *qs;
    int64_t q_stride_bytes;
    int64_t qs_stride_floats;
} oracle_qmat;

typedef struct {
    const float *router_w;     /* [E][H] */
    const float *router_bias;  /* [E] */
    oracle_qmat gate, up;      /* int4 [E][I][H/2], scales [E][I] */
    oracle_qmat down;          /* int4 [E][H][I/2], scales [E][H] */
    oracle_qmat sh_gate, sh_up, sh_down; /* shared expert, E = 1, int4 or int8 */
    /* [E] per routed expert: 4 (packed int4) or 2 (packed int2, the cold-tail
     * experts: the colibri-nano README lists, among the checkpoint tools it
     * leaves out, one that stores the rarely routed experts in int2; the
     * colibri README, "What's implemented", has packed int2 with per-row
     * scales, dequantised on use).  Reading: element 4c + j of a row in
     * bits 2j..2j+1 of byte c, two's complement (-2..1), one f32 scale per
     * row, the row cols/4 bytes; an int2 expert's matrices sit where an int4
     * expert's would (same expert stride, the first half of each).  NULL: all
     * int4. */
    const uint8_t *expert_bits;
} oracle_weights;

/* format helpers (the pins of the packed layout) */
float oracle_bf16_to_f32(uint16_t bits);
uint16_t oracle_f32_to_bf16(float f);
void oracle_unpack_int4_row(const uint8_t *row, int32_t cols, int32_t *vals);
void oracle_unpack_int2_row(const uint8_t *row, int32_t cols, int32_t *vals);
void oracle_pack_int4_row(const int32_t *vals, int32_t cols, uint8_t *row);
void oracle_dequant_row(const void *q, int32_t bits, const float *scale, int32_t cols, float *out);

/* router logits z, scores s = sigmoid(z) and selection scores b = s + bias, each [T][E] (nullable) */
int oracle_router_scores(const oracle_shape *sh, const uint16_t *hidden, const float *W, const float *bias,
                         float *z, float *s, float *b);
/* ids [T][k] (descending b), w [T][k] normalised (sum 1, before the routed scaling factor),
 * gap [T] = b_(k) - b_(k+1), ggap [T] = G_(keep) - G_(keep+1) (+inf when undefined); gap/ggap nullable */
int oracle_router(const oracle_shape *sh, const uint16_t *hidden, const float *W, const float *bias,
                  int32_t *ids, float *w, float *gap, float *ggap);
/* counts [E], offsets [E+1], sorted [T*k] (pair index p = t*k + j), inv [T*k] */
int oracle_permute(const oracle_shape *sh, const int32_t *ids, int32_t *counts, int32_t *offsets,
                   int32_t *sorted, int32_t *inv);
/* y_pairs [T*k][H] in sorted order; pair_scale [T*k] indexed by pair (nullable = 1) */
int oracle_expert_ffn(const oracle_shape *sh, const uint16_t *hidden, const oracle_weights *wt,
                      const int32_t *offsets, const int32_t *sorted, const float *pair_scale,
                      float *y_pairs);
/* shared expert output [T][H] (zeros when shared_bits == 0) */
int oracle_shared_ffn(const oracle_shape *sh, const uint16_t *hidden, const oracle_weights *wt, float *out);
/* out [T][H] = sum_j coef_j * y_pairs[inv[t*k+j]] + shared_out[t] + residual[t];
 * coef_j = rsf * topk_w[t][j] when topk_w is given, else 1 (pre-scaled pairs). */
int oracle_combine(const oracle_shape *sh, const float *y_pairs, const int32_t *inv, const float *topk_w,
                   const float *shared_out, const uint16_t *residual, float *out);
/* the whole layer, f32 output [T][H]; ids/w/gap/ggap nullable diagnostics */
int oracle_layer_forward(const oracle_shape *sh, const oracle_weights *wt, const uint16_t *hidden, float *out,
                         int32_t *ids, float *w, float *gap, float *ggap);
/* the layer for a subset of tokens: out [n][H] for tokens[0..n); routing is
 * the oracle's own unless ids/w are given ([T][k], as from a router) */
int oracle_layer_tokens(const oracle_shape *sh, const oracle_weights *wt, const uint16_t *hidden,
                        const int32_t *tokens, int32_t n, const int32_t *ids, const float *w, float *out);
/* brute force: every expert on every token, weighted by a dense [T][E] mask */
int oracle_layer_forward_dense(const oracle_shape *sh, const oracle_weights *wt, const uint16_t *hidden,
                               float *out);
/* gate/up pre-activations of one sorted row's expert, unscaled integer sums
 * sum_h x*q (no scale), for the integer-exact check: g,u [T*k][I] in sorted order */
int oracle_gateup_int_sums(const oracle_shape *sh, const uint16_t *hidden, const oracle_weights *wt,
                           const int32_t *offsets, const int32_t *sorted, double *g, double *u);

/* Per-row symmetric quantiser (colibri-nano README, "Converting a checkpoint
 * yourself": per-row symmetric quantisation with f32 scales in a sibling .qs
 * tensor; colibri README, "What's implemented": int8 and packed int4
 * quantisation kernels with per-row scales).  The pages give no formula; the
 * plain reading taken here, per row of `cols` values w (f32, or bf16 widened
 * exactly when src_bf16 != 0):
 *   amax  = max |w|                        (exact)
 *   scale = amax / qmax                    (f32 division, round to nearest
 *                                           even; qmax = 7 for int4, 127 for
 *                                           int8)
 *   q     = clamp(rint(w / scale), -qmax, qmax)   (f32 division, then round
 *                                           half to even, as numpy does)
 * An all-zero row gets scale 0 and codes 0.  Codes are stored in the packed
 * layout of oracle_pack_int4_row (int4, cols even, rows of cols/2 bytes) or as
 * int8 rows.  Inputs must be finite.  Returns 0, or -2 for a bad shape. */
/* Q8_0-style activation codes (see ORACLE_ACT_Q8): rows x cols (cols % 32 ==
 * 0) f32 or bf16 (src_bf16) values -> q [rows][cols] int8 and d
 * [rows][cols/32] f32. */
int oracle_quantize_act_q8(const void *src, int32_t src_bf16, int64_t rows, int32_t cols, int8_t *q, float *d);

int oracle_quantize_rows(const void *src, int32_t src_bf16, int64_t rows, int32_t cols, int32_t bits, void *q,
                         float *qs);

/* Aux-loss-free load balancing, the training-side step after the histogram
 * (Colibri-Nano model card, "Architecture": sigmoid+bias router with
 * DeepSeek-V3-style aux-loss-free balancing; the README's repository layout
 * lists aux-loss-free balancing under train/).  The pages give no rule; the
 * reading is the published DeepSeek-V3 one: after a step, every expert's bias
 * moves by gamma toward balance,
 *   bias[e] += gamma * sign(mean - counts[e]),  mean = sum(counts) / E,
 * with the comparison taken exactly in integers (E * counts[e] against the
 * sum) and no change for an expert exactly at the mean.  Each update is one
 * f32 addition.  bias_out may equal bias_in.  Returns 0, -1 or -2. */
int oracle_bias_update(int32_t E, const int32_t *counts, const float *bias_in, float gamma, float *bias_out);

int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif

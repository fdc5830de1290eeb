/*
 * moe.h -- C ABI of the int4 routed-expert MoE layer forward pass on MI355X (gfx950).
 *
 * One Mixture-of-Experts FFN layer as Colibri-Nano and the colibri engine
 * define it:
 *   - a sigmoid router with an aux-loss-free selection bias (Colibri-Nano model
 *     card, "Architecture": sigmoid+bias router, DeepSeek-V3-style aux-loss-free
 *     balancing; colibri README, "What's implemented": DeepSeek-V3-style sigmoid
 *     router with noaux_tc and routed_scaling_factor, shared expert);
 *   - batch-union routing: the pairs are grouped by expert so each unique expert
 *     is read once and applied to every position routed to it (colibri README,
 *     "What's implemented": batch-union MoE);
 *   - SwiGLU experts of three matrices (colibri README at 0d2fb6f, "Never wait for
 *     the disk twice": an expert's three matrices are stored adjacent) whose
 *     weights are per-row symmetric packed int4 with one f32 scale per row in a
 *     sibling .qs tensor (colibri-nano README, "Converting a checkpoint
 *     yourself");
 *   - an always-resident shared expert (NanoColibri README, model table) in int4
 *     or int8 (colibri-nano README: int4 experts, int8 dense);
 *   - a weighted combine scaled by routed_scaling_factor.
 *
 * Conventions for every call below
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps none of them after the call's work completes and allocates nothing.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream).  Calls return as soon as the work is enqueued; they never
 *     synchronise and never read device memory back to the host.
 *   - Shapes and pointers are validated on the host before anything is
 *     enqueued: a call that returns an error has enqueued nothing.
 *   - T == 0 is a no-op that returns MOE_OK.
 *   - Results are deterministic: the same inputs give the same bits, run to run.
 *   - Calls that share a workspace on different streams race; one workspace per
 *     stream.
 *
 * Layouts (row-major, C order)
 *   hidden     [T][H] bf16 (raw bits, moe_bf16)
 *   router_w   [E][H] f32, one row per expert;  router_bias [E] f32
 *   int4 matrix with `rows` x `cols`: rows of cols/2 bytes, element 2c in the
 *              low nibble of byte c, element 2c+1 in the high nibble, two's
 *              complement; int8: rows of cols signed bytes.  One f32 scale per
 *              row; the weight is q * scale.
 *   gate, up   per expert [I][H]  (row = intermediate channel, columns = hidden)
 *   down       per expert [H][I]  (row = output channel, columns = intermediate)
 *   Expert e of a matrix family starts at q + e*q_stride_bytes with its scales at
 *   qs + e*qs_stride_floats, so the three matrices of an expert may be stored
 *   back to back.  q pointers and q strides must be multiples of 16 bytes; qs
 *   pointers and strides multiples of 4 floats.
 *   Pairs: p = t*top_k + j is token t's j-th chosen expert (j in descending
 *   selection-score order).  Sorted rows r list the pairs grouped by expert in
 *   ascending expert id, pairs of one expert in ascending p.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)       /* inconsistent shape */
#define MOE_ERR_UNSUPPORTED (-3) /* legal shape the gfx950 kernels do not cover */
#define MOE_ERR_WORKSPACE (-4)   /* workspace too small */
#define MOE_ERR_ALIGN (-5)       /* misaligned pointer or stride */
#define MOE_ERR_HIP (-6)         /* a HIP launch failed */

/* moe_shape.flags */
#define MOE_OUT_F32 1u      /* out is f32 [T][H]; otherwise bf16 [T][H] rounded to nearest even */
#define MOE_ADD_RESIDUAL 2u /* moe_layer_forward adds the layer input to the output */
#define MOE_EXPERT_INT8 4u  /* moe_expert_ffn: gate/up/down are int8 rows (the shared expert of an
                               int8 dense stack); otherwise packed int4 */
#define MOE_STAGE_GATEUP_ONLY 0x200u /* moe_expert_ffn, profiling: run only the gate/up + SwiGLU kernel
                               (h stays in the workspace; y_pairs is not written) */
#define MOE_STAGE_EXPERTS_ONLY 0x400u /* moe_layer_forward(_profiled), profiling, small-batch regime only
                               (else MOE_ERR_UNSUPPORTED): run only the expert kernel, from the router
                               logits a previous full call with the same shape, weights, input and ws
                               left in ws; out is not written */
#define MOE_LOGITS_GIVEN 0x800u /* moe_layer_forward(_chain), small-batch regime only (else
                               MOE_ERR_UNSUPPORTED): this call's router logits are already in ws, written
                               there by the previous layer's moe_layer_forward_chain; the logits kernel
                               is not run (the selection is, from those logits) */
#define MOE_ACT_Q8 0x1000u /* moe_layer_forward(_profiled): Q8_0-style int8 activations for the expert
                               matmuls (colibri README, "What's implemented": the integer-dot kernels take
                               int8 activations).  The input row of every expert matmul (x for gate and up,
                               h for down, h taken in f32) is cut into blocks of 32 along the contraction
                               axis; each block gets d = max|v| / 127 and codes as moe_quantize_act_q8
                               gives; a dot is s_w * sum over blocks of d * (integer sum of code products).
                               Always the tiled kernels (v_mfma_i32_16x16x32_i8); the router is unchanged.
                               moe_expert_ffn and moe_layer_forward_chain return MOE_ERR_UNSUPPORTED */
#define MOE_EXPERT_MIXED 0x2000u /* routed experts in int4 or int2 per weights->expert_bits, in both regimes
                               (the small-batch kernel loads an int2 expert's rows at half the bytes and
                               unpacks them to the int4 path's operand bits); with MOE_ACT_Q8 or
                               MOE_TEST_GATEUP_SUMS: MOE_ERR_UNSUPPORTED */
#define MOE_REGIME_TILED 0x4000u /* moe_layer_forward(_profiled, _noalloc): take the tiled grouped-GEMM kernels at
                               any T (the small-batch weight-streaming kernels are otherwise chosen for
                               the shapes moe_layer_routing names); for measuring the two regimes side by
                               side.  With MOE_STAGE_EXPERTS_ONLY, MOE_LOGITS_GIVEN or in a chained call:
                               MOE_ERR_UNSUPPORTED */
#define MOE_REGIME_SMALL 0x8000u /* moe_layer_forward(_profiled, _noalloc): take the small-batch kernels at any T,
                               in chunks of 32 tokens (each chunk streams its experts' weights again), for a
                               shape they serve (top_k <= 16, H % 1024 == 0, I and I_shared % 512 == 0),
                               else MOE_ERR_UNSUPPORTED; with MOE_REGIME_TILED or MOE_ACT_Q8:
                               MOE_ERR_UNSUPPORTED.  For measuring the two regimes side by side */
#define MOE_TEST_GATEUP_SUMS 0x100u /* moe_expert_ffn, testing only: write the raw integer-weight sums
                               sum_h x*q of gate into y_pairs[r][0:I] and of up into y_pairs[r][I:2I]
                               (no scale, no activation, no down projection); needs 2*I <= H, int4 */

/* workspace kinds for moe_workspace_bytes */
#define MOE_WS_PERMUTE 1
#define MOE_WS_EXPERT_FFN 2
#define MOE_WS_LAYER 3

typedef uint16_t moe_bf16; /* raw bfloat16 bits */

typedef struct {
    int32_t T;          /* tokens in the batch, >= 0 */
    int32_t H;          /* hidden size */
    int32_t E;          /* routed experts */
    int32_t top_k;      /* experts per token, 1 <= top_k <= E */
    int32_t I;          /* routed expert intermediate size */
    int32_t I_shared;   /* shared expert intermediate size (ignored when shared_bits == 0) */
    int32_t shared_bits;/* 0 = no shared expert, 4 = int4, 8 = int8 */
    int32_t n_group;    /* groups for group-limited selection; 1 = plain top-k */
    int32_t topk_group; /* groups kept, 1 <= topk_group <= n_group */
    float routed_scaling_factor; /* multiplies the routed terms (not the shared expert) */
    uint32_t flags;     /* MOE_OUT_F32 | MOE_ADD_RESIDUAL */
    float top_p;        /* adaptive expert top-p (colibri README, the --topp knob): with 0 < top_p < 1
                           each token keeps only the shortest prefix of its top_k selections ranked by
                           combine weight (descending; equal weights, the lower id first) whose f32
                           running weight reaches top_p, renormalised over the kept ones; dropped slots
                           read id -1, weight 0 and cost no expert work.  Any other value keeps all
                           top_k (0 is the plain router); NaN is MOE_ERR_SHAPE */
} moe_shape;

typedef struct {
    const void *q;            /* packed int4 (u8) or int8 rows */
    const float *qs;          /* one f32 scale per row */
    int64_t q_stride_bytes;   /* expert-to-expert distance in q (0 for a single expert) */
    int64_t qs_stride_floats; /* expert-to-expert distance in qs */
} moe_qmat;

typedef struct {
    const float *router_w;    /* [E][H] f32 */
    const float *router_bias; /* [E] f32; selection only */
    moe_qmat gate, up, down;  /* routed experts, int4 */
    moe_qmat sh_gate, sh_up, sh_down; /* shared expert (E = 1), int4 or int8 per shared_bits */
    /* with MOE_EXPERT_MIXED: device [E] u8, each routed expert's format, 4 (packed int4) or 2
     * (packed int2: the rarely routed experts, which the colibri-nano README's checkpoint tools store in int2; colibri
     * README, "What's implemented": packed int2 with per-row scales).  Int2: element 4c + j of a row
     * in bits 2j..2j+1 of byte c, two's complement, rows of cols/4 bytes, one f32 scale per row; an
     * int2 expert's gate, up and down start where an int4 expert's would (same strides), so its
     * matrices take the first half of each region.  Ignored without the flag. */
    const uint8_t *expert_bits;
} moe_weights;

/*
 * moe_router -- router scores, selection and combine weights.
 * Defined by: Colibri-Nano model card, "Architecture" (sigmoid+bias router,
 * DeepSeek-V3-style aux-loss-free balancing) and colibri README, "What's
 * implemented" (noaux_tc group-limited selection, routed_scaling_factor).
 *   z[t,e] = sum_h x[t,h] * W[e,h] (f32),  s = 1/(1+exp(-z)),  b = s + bias.
 *   n_group > 1: groups are contiguous blocks of E/n_group experts; a group
 *   scores the sum of its two largest b; the topk_group best groups are kept
 *   (ties -> lower group id).  top_k largest b among kept experts, ties ->
 *   lower id, listed by descending b.  topk_w[t,j] = s_j / sum_j s_j (sums to
 *   1; the routed scaling factor is applied by moe_expert_ffn / moe_combine).
 * Out: topk_ids [T][top_k] i32, topk_w [T][top_k] f32, sel_gap [T] f32
 *   (nullable): the smaller of b_(k) - b_(k+1) and, when groups are dropped,
 *   G_(keep) - G_(keep+1); it measures how close the token's selection is to a tie.
 * The GPU kernels need H % 128 == 0, I % 64 == 0, I_shared % 64 == 0, E <= 256,
 * top_k <= 64 and n_group <= 64 (else MOE_ERR_UNSUPPORTED; every call checks).
 * Workspace: the K-split partial logits (the router splits the H-long dot
 * products over workgroups and adds the slices in a fixed order, so it needs
 * scratch that the caller owns like every other buffer);
 * moe_workspace_bytes(shape, MOE_WS_PERMUTE) covers it.
 */
int moe_router(const moe_shape *shape, const moe_bf16 *hidden, const float *router_w, const float *router_bias,
               int32_t *topk_ids, float *topk_w, float *sel_gap, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_permute -- group the T*top_k pairs by expert (batch-union; colibri README,
 * "What's implemented").  A stable counting sort by expert id:
 *   counts[e] = #pairs routed to e;  offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e];
 *   sorted_pairs[r] = the pair at sorted row r (pairs of one expert ascending);
 *   inv_pos[p] = the sorted row of pair p.
 * Positions come from ordered ranks, not atomics, so the result is bit-exact.
 * topk_ids must hold ids in [0, E) (not checked on the device).
 * Out: counts [E], offsets [E+1], sorted_pairs [T*top_k], inv_pos [T*top_k], all i32.
 * Workspace: moe_workspace_bytes(shape, MOE_WS_PERMUTE).
 */
int moe_permute(const moe_shape *shape, const int32_t *topk_ids, int32_t *counts, int32_t *offsets,
                int32_t *sorted_pairs, int32_t *inv_pos, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn -- the routed experts on their sorted rows.
 * Defined by: colibri README at 0d2fb6f, "Never wait for the disk twice" (an
 * expert is three matrices, stored adjacent, read once per step for every
 * position routed to it) and colibri README (older revision), "What's
 * implemented" (batch-union MoE; per-row int4 weights dequantised on use);
 * the activation between the matrices is SwiGLU (the pages name only the
 * three matrices; gate, up and down is the plainest reading).
 * For sorted row r of expert e (offsets[e] <= r < offsets[e+1]), pair
 * p = sorted_pairs[r], token t = p / top_k:
 *   g_i = sg_i * sum_h x[t,h] q_gate[e,i,h],  u_i likewise with up,
 *   h_i = silu(g_i) * u_i with silu(z) = z / (1 + exp(-z))  (SwiGLU),
 *   y_pairs[r, c] = pair_scale[p] * sd_c * sum_i h_i q_down[e,c,i].
 * pair_scale is indexed by pair and nullable (then 1).  Computed on matrix
 * cores: x and the int4 values are exact in bf16, products accumulate in f32,
 * h is rounded to f16 (nearest even) before the down projection, which runs
 * on f16 matrix cores.
 * The shared expert runs through this call as E = 1, top_k = 1 with
 * offsets = {0, T}, sorted_pairs = identity and gate/up/down = the shared
 * matrices (shape.I = I_shared; set MOE_EXPERT_INT8 for int8 rows).  gate and
 * up must use the same expert stride.
 * Out: y_pairs [T*top_k][H] f32 in sorted order.
 * Needs H % 128 == 0 and I % 64 == 0.  Workspace: moe_workspace_bytes(shape, MOE_WS_EXPERT_FFN).
 */
int moe_expert_ffn(const moe_shape *shape, const moe_bf16 *hidden, const moe_weights *weights,
                   const int32_t *offsets, const int32_t *sorted_pairs, const float *pair_scale,
                   float *y_pairs, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_combine -- the weighted sum of a token's expert outputs plus the shared
 * expert (colibri README (older revision), "What's implemented": the router's
 * weights scaled by routed_scaling_factor, and the shared expert; Colibri-Nano
 * model card, "Architecture": an always-resident shared expert beside the
 * routed ones):
 *   out[t,c] = sum over j ascending of coef(t,j) * y_pairs[inv_pos[t*top_k+j], c]
 *              + shared_out[t,c] + residual[t,c]
 * with coef = routed_scaling_factor * topk_w[t,j] when topk_w is given, else 1
 * (pairs already scaled).  shared_out [T][H] f32 and residual [T][H] bf16 are
 * nullable.  out is f32 or bf16 per MOE_OUT_F32.
 */
int moe_combine(const moe_shape *shape, const float *y_pairs, const int32_t *inv_pos, const float *topk_w,
                const float *shared_out, const moe_bf16 *residual, void *out, void *stream);

/*
 * moe_layer_forward -- the whole layer: router, permutation, routed experts,
 * shared expert, combine (and the input added back when MOE_ADD_RESIDUAL).
 * Defined by the calls above together: Colibri-Nano model card, "Architecture"
 * (a sigmoid-routed MoE layer with a shared expert), colibri README (older
 * revision), "What's implemented" (router, batch-union, shared expert, scaled
 * combine) and colibri README at 0d2fb6f, "Never wait for the disk twice"
 * (the per-token expert path).  Routed experts must be packed int4 (or int4
 * and int2 with MOE_EXPERT_MIXED); MOE_EXPERT_INT8 is MOE_ERR_UNSUPPORTED here.
 * out: [T][H] f32 or bf16 per MOE_OUT_F32.  Inside the layer the routed and
 * shared output rows (in the small-batch regime each 128-row unit's partial
 * rows) are carried in f16, each value rounded once to nearest even (so
 * |value| must stay below 65504), and summed in f32 in a fixed order.  The
 * regime (small-batch weight streaming or tiled grouped GEMM) is chosen from
 * the shape and T, as moe_layer_routing describes.  In the tiled
 * regime the shared expert runs on a second stream of the current device
 * (created on first use, default priority), forked from and joined back to
 * `stream` with events, so the call stays ordered on `stream` and a captured
 * graph gets two branches; for H >= 2048 the input's row sums are computed
 * there first and the routed GEMMs wait for them by one more event.  Calls
 * from several host threads are serialised around these events.
 * Workspace: moe_workspace_bytes(shape, MOE_WS_LAYER).
 */
int moe_layer_forward(const moe_shape *shape, const moe_weights *weights, const moe_bf16 *hidden, void *out,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * moe_layer_forward_chain -- one layer of a stacked small-batch decode step
 * whose output is the next layer's input (the layers of a model run one after
 * another, each on the previous one's output: colibri README, "What's
 * implemented", the faithful model forward).  It runs the layer as
 * moe_layer_forward does; when next_weights is given, the layer's combine also
 * computes the next layer's router logits of the output row it has just
 * written, into next_ws, so the next call passes MOE_LOGITS_GIVEN and skips
 * its logits kernel.  The call's own output equals the unchained call's bit
 * for bit when its router logits are the same (always for the first layer of
 * a step, which computes them itself).  The logits it leaves for the next
 * layer are the same f32 sums added in another order, so the next layer's
 * combine weights can differ from the unchained call's by f32 rounding
 * (about 1e-7) and its selection only at a near tie.
 *   shape, weights, hidden, out, ws  as for moe_layer_forward; out must be bf16
 *               (no MOE_OUT_F32): it is what the next layer reads
 *   next_shape  the next layer's shape: same T and H, small-batch regime
 *   next_weights  nullable: the next layer's weights (only router_w is read);
 *               NULL runs this layer unchained (the last layer of a step)
 *   next_ws     the next layer's MOE_WS_LAYER workspace (next_ws_bytes bytes)
 * Errors: as moe_layer_forward; MOE_ERR_UNSUPPORTED if either layer is not in
 * the small-batch regime, out is f32 or MOE_STAGE_EXPERTS_ONLY is set with a
 * next layer; MOE_ERR_SHAPE if T or H differ.
 */
int moe_layer_forward_chain(const moe_shape *shape, const moe_weights *weights, const moe_bf16 *hidden, void *out,
                            void *ws, size_t ws_bytes, const moe_shape *next_shape, const moe_weights *next_weights,
                            void *next_ws, size_t next_ws_bytes, void *stream);

/*
 * moe_layer_forward_noalloc -- moe_layer_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Instead of a caller workspace it uses the
 * library's own scratch, a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that each GPU the library runs on holds until the process ends;
 * the call allocates nothing (no hipMalloc, no stream or event creation: in
 * the tiled regime the shared expert runs on `stream` too).  Results are
 * those of moe_layer_forward, bit for bit.
 *   shape, weights, hidden, out, stream  as for moe_layer_forward
 * Errors: as moe_layer_forward; MOE_ERR_WORKSPACE when the shape's layer
 * workspace, moe_workspace_bytes(shape, MOE_WS_LAYER), exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (checked before anything is enqueued);
 * MOE_ERR_UNSUPPORTED with MOE_STAGE_EXPERTS_ONLY or MOE_LOGITS_GIVEN (they
 * read a previous call's workspace); MOE_ERR_HIP if the scratch's device
 * address cannot be had.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (every kernel of the layer writes what it later reads, so
 * no clearing is needed): calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_forward_noalloc(const moe_shape *shape, const moe_weights *weights, const moe_bf16 *hidden, void *out,
                              void *stream);

/* moe_layer_forward with two HIP events (hipEvent_t as void*, nullable) recorded
 * on `stream` immediately before and after the expert gate/up kernel: the
 * grouped gate/up + SwiGLU GEMM of the routed experts (tiled regime) or the
 * gate/up weight stream of routed and shared experts (small-batch regime).
 * For measuring that kernel inside a real layer pass; results are identical
 * to moe_layer_forward. */
int moe_layer_forward_profiled(const moe_shape *shape, const moe_weights *weights, const moe_bf16 *hidden,
                               void *out, void *ws, size_t ws_bytes, void *stream, void *ev_start, void *ev_stop);

/* Bytes of workspace a call needs for this shape (0 for an invalid shape). */
size_t moe_workspace_bytes(const moe_shape *shape, int which);

/* Host-side validation only (no device work): MOE_OK or the status a call would return. */
int moe_validate_shape(const moe_shape *shape);

/* A static string naming a status code. */
const char *moe_status_string(int status);

/* The layer-forward workspace also exposes, for inspection after a call, the
 * routing it computed: moe_layer_routing(ws, shape, ...) returns device
 * pointers into ws (ids [T][k], w [T][k], offsets [E+1], sorted [T*k]).
 * Pointers stay valid until the workspace is reused.  In the small-batch
 * regime each expert kernel gathers its own pairs and no sorted list is
 * materialised: offsets and sorted_pairs are then returned as NULL.  That
 * regime serves T <= 64 (at most two chunks of 32 tokens: the measured
 * crossover with the tiled kernels lies between 64 and 96 tokens at the Nano
 * shape), top_k <= 16, H % 1024 == 0, I % 512 == 0 and I_shared % 512 == 0,
 * unless MOE_REGIME_TILED or MOE_REGIME_SMALL decides; MOE_ACT_Q8 always
 * takes the tiled kernels.  Chained calls
 * (moe_layer_forward_chain), MOE_LOGITS_GIVEN and MOE_STAGE_EXPERTS_ONLY need
 * T <= 32 (one chunk), else MOE_ERR_UNSUPPORTED. */
int moe_layer_routing(const moe_shape *shape, void *ws, size_t ws_bytes, int32_t **topk_ids, float **topk_w,
                      int32_t **offsets, int32_t **sorted_pairs);

/* ---- the step before the path: the per-row symmetric quantiser and packer ----
 *
 * moe_quantize_rows turns `rows` rows of `cols` values into the container
 * format the layer reads: per-row symmetric codes with one f32 scale per row
 * in a sibling .qs array (colibri-nano README, "Converting a checkpoint
 * yourself"; colibri README, "What's implemented": int8 and packed int4
 * quantisation kernels with per-row scales).  The pages give no formula; per
 * row, with qmax = 7 (bits 4) or 127 (bits 8):
 *   scale = max|w| / qmax                 (f32, correctly rounded)
 *   code  = clamp(nearest integer to w / scale, ties to even, -qmax, qmax)
 * and an all-zero row gets scale 0 and codes 0.  Inputs must be finite, and
 * a nonzero row's scale must not underflow to 0 (max|w| >= qmax * 2^-149);
 * subnormal scales are fine.
 *
 *   src         device, [rows][cols], f32 (src_format MOE_SRC_F32) or bf16
 *               bits (MOE_SRC_BF16), row-major, no padding
 *   q           device, [rows][cols/2] bytes for bits 4 (element 2c in the low
 *               nibble of byte c, two's complement; cols must be even) or
 *               [rows][cols] int8 for bits 8
 *   qs          device, [rows] f32 scales
 * The caller owns every buffer; the call only enqueues on `stream`.
 * Returns MOE_OK (rows == 0 is a no-op), MOE_ERR_SHAPE (rows < 0, cols <= 0,
 * bits not 4 or 8, odd cols for bits 4, unknown src_format), MOE_ERR_NULL,
 * MOE_ERR_ALIGN (src or qs not aligned to its element size) or MOE_ERR_HIP.
 * 16-byte aligned rows with cols % 8 == 0 take the vector path. */
#define MOE_SRC_F32 0
#define MOE_SRC_BF16 1
int moe_quantize_rows(const void *src, int32_t src_format, int64_t rows, int32_t cols, int32_t bits, void *q,
                      float *qs, void *stream);

/* ---- Q8_0-style activation codes (the MOE_ACT_Q8 mode's quantiser) ----
 *
 * moe_quantize_act_q8 cuts each of `rows` rows of `cols` values into blocks of
 * 32 and writes, per block (colibri README, "What's implemented": Q8_0-style
 * int8 activations; the pages give no formula, the reading is the weight
 * quantiser's rule per block):
 *   d    = max|v| / 127                    (f32, correctly rounded)
 *   code = clamp(nearest integer to v / d, ties to even, -127, 127)
 * and an all-zero block gets d = 0 and codes 0.  Inputs must be finite.
 *   src   device, [rows][cols] f32 (MOE_SRC_F32) or bf16 bits (MOE_SRC_BF16),
 *         16-byte aligned, row-major, no padding
 *   q     device, [rows][cols] int8 codes, 16-byte aligned
 *   d     device, [rows][cols/32] f32 block scales
 * The caller owns every buffer; the call only enqueues on `stream`.
 * Returns MOE_OK (rows == 0 is a no-op), MOE_ERR_SHAPE (rows < 0, cols <= 0,
 * cols % 32 != 0, unknown src_format), MOE_ERR_NULL, MOE_ERR_ALIGN or
 * MOE_ERR_HIP. */
int moe_quantize_act_q8(const void *src, int32_t src_format, int64_t rows, int32_t cols, int8_t *q, float *d,
                        void *stream);

/* ---- the training-side step after the histogram: aux-loss-free balancing ----
 *
 * moe_bias_update moves each expert's router bias (the bias that only decides
 * selection) by gamma toward balance, from the expert counts of a step
 * (Colibri-Nano model card, "Architecture": sigmoid+bias router with
 * DeepSeek-V3-style aux-loss-free balancing).  The pages give no rule; the
 * reading is the published DeepSeek-V3 one:
 *   router_bias[e] += gamma * sign(mean - counts[e]),  mean = sum(counts) / E,
 * the comparison taken exactly in integers (E * counts[e] against the sum),
 * no change for an expert exactly at the mean, one f32 addition each.
 *
 *   counts       device, [E] int32, e.g. the counts output of moe_permute
 *                (or a sum of several steps' counts)
 *   router_bias  device, [E] f32, updated in place
 * Enqueues one small kernel on `stream`.  Returns MOE_OK, MOE_ERR_SHAPE
 * (E < 1), MOE_ERR_NULL, MOE_ERR_ALIGN (pointers not 4-byte aligned) or
 * MOE_ERR_HIP. */
int moe_bias_update(int32_t E, const int32_t *counts, float *router_bias, float gamma, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

// moe_launch.h -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct FfnArgs {
    const void *A;  // rows: bf16 activations (gate/up) or f16 h (down)
    int lda;
    const int32_t *gather;
    int kdiv;
    const int32_t *pair_of_row;
    const int32_t *offsets;
    int E;
    int M;
    const uint8_t *q0;
    const float *s0;
    const uint8_t *q1;
    const float *s1;
    int64_t qstride;
    int64_t sstride;
    int K;
    int N;
    void *out;
    int ldo;
    const float *pscale;
    const float *ad;  // Q8 mode: f32 scale of every 32 activation codes, [rows of A][K/32]
    const uint8_t *ebits;  // per-expert format (4 or 2) of a mixed family, or null (all WBITS)
    int out_f16;           // MODE 1: output rows in f16 (rounded to nearest even) instead of f32
    int out_by_pair;       // MODE 1: row r is written at row pair_of_row[r] (pair order) instead of r
    // Row sums of A, precomputed (null: the kernels take them with an MFMA
    // per k-step): MODE 0/2 one f32 per source row of A (indexed like A, by
    // gather / kdiv); MODE 1 rsum_parts partials per row, added in order.
    const float *rsum;
    int rsum_parts;
    // MODE 0 (pipelined tiles): where set, the sum of each h row's f16
    // values over the tile's columns, [rows][N / 128] (partials of the down
    // GEMM's rsum)
    float *hsum;
};

// small-batch regime (decode.hip)
struct DecLaunch {
    const uint16_t *x;
    const float *rw, *rb;
    int T, H, E, k, n_group, topk_group;
    float rsf, top_p;
    int32_t *ids;
    float *w, *gap, *pscale;
    float *z;  // [DEC_LOGIT_PLANES][T][E] partial router logits (scratch)
    const uint8_t *gq, *uq, *dq;
    const float *gs, *us, *ds;
    int64_t qstride, dqstride, sstride, dsstride;
    int I;
    const uint8_t *ebits;  // [E] each routed expert's format, 4 or 2 (packed int2); null: all int4
    const uint8_t *sgq, *suq, *sdq;
    const float *sgs, *sus, *sds;
    int Ish, sh_bits;
    uint16_t *y, *shp;  // f16 partial outputs: [I/128][T*k][H] routed, [I_shared/128][T][H] shared
    const uint16_t *res;
    void *out;
    int out_f32;
    hipEvent_t ev0, ev1;  // nullable: recorded around the expert kernel
    int experts_only;     // launch only the expert kernel (router logits already in z)
    int logits_given;     // z already holds this step's router logits (written by the previous layer's combine)
    // chained next layer (used when nrw is set): its router logits, taken from
    // this layer's bf16 output, into its workspace's planes nz
    const float *nrw;
    int nE;
    float *nz;
};
constexpr int DEC_LOGIT_PLANES = 4;  // partial-logit planes of the small-batch router
constexpr int DEC_CHUNK_ROWS = 128;  // intermediate rows per small-batch expert unit (one output plane each)
constexpr int DEC_CHUNK_TOKENS = 32; // tokens per small-batch launch (a larger batch runs in chunks)
// shapes the small-batch kernels serve (any T, in chunks of DEC_CHUNK_TOKENS)
bool decode_supported(int H, int E, int k, int I, int Ish, int sh_bits);
hipError_t launch_decode(const DecLaunch &d, hipStream_t st);

int router_ks(int T, int H, int E);
int router_select_blocks(int T);
int superblock_tokens(int k);
hipError_t launch_router(const uint16_t *x, const float *W, const float *bias, int T, int H, int E, int k,
                         int n_group, int topk_group, float rsf, float top_p, float *zpart, int KS, int32_t *ids,
                         float *w, float *gap, float *pair_scale, int32_t *sbcounts, hipStream_t st);
hipError_t launch_pair_hist(const int32_t *ids, int P, int E, int chunk, int nblocks, int32_t *bcounts,
                            hipStream_t st);
hipError_t launch_scatter(const int32_t *ids, const int32_t *bcounts, int nblocks, int P, int E, int chunk,
                          int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *inv, hipStream_t st);
hipError_t launch_ffn(int mode, int wbits, const FfnArgs &a, int rows_total, int groups, hipStream_t st);
// Whether launch_ffn (no mixed family) takes the pipelined tiles, which use
// rsum and write hsum, for this shape.
bool ffn3_taken(int mode, int wbits, int rows_total, int groups, int N);
// f32 sum of each bf16 row of A (rows x K, row stride lda elements).
hipError_t launch_rowsum_bf16(const uint16_t *A, int lda, int rows, int K, float *out, hipStream_t st);
// Q8_0-style int8 activations (A = int8 codes, ad = their block scales);
// mode 0 writes h as f32, mode 1 the down rows
hipError_t launch_ffn_q8(int mode, int wbits, const FfnArgs &a, int rows_total, int groups, hipStream_t st);
hipError_t launch_quant_act_q8(const void *src, int src_bf16, long rows, int cols, int8_t *q, float *d,
                               hipStream_t st);
hipError_t launch_bias_update(int E, const int32_t *counts, float *bias, float gamma, hipStream_t st);
hipError_t launch_quantize(const void *src, int src_bf16, long rows, int cols, int bits, void *q, float *qs,
                           hipStream_t st);
// y and sh in f32, or (y_f16) both in f16; y rows in sorted order (row inv[p]
// for pair p), or (y_by_pair) in pair order (row p)
hipError_t launch_combine(const void *y, const int32_t *inv, const float *topk_w, float rsf, const void *sh,
                          const uint16_t *res, void *out, int T, int H, int k, int out_f32, int y_f16, int y_by_pair,
                          hipStream_t st);

}  // namespace moe

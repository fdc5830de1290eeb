// moe_select.h -- per-token expert selection of the sigmoid+bias router, one
// wavefront per token.
//
// Scores s = sigmoid(z) and selection scores b = s + bias arrive spread over
// the wave (lane l holds experts [l*EPL, (l+1)*EPL)).  The bias only decides
// selection (Colibri-Nano model card, "Architecture": sigmoid+bias router,
// DeepSeek-V3-style aux-loss-free balancing); the weights are the unbiased
// scores of the chosen experts normalised to sum 1.  Group-limited selection
// ("noaux_tc", colibri README "What's implemented"): groups are contiguous
// blocks of E/n_group experts scored by the sum of their two largest b, the
// topk_group best groups stay eligible.  Ties go to the lower id throughout.
#pragma once

#include "moe_device.h"

namespace moe {

struct ArgMax {
    float v;
    int i;
};

// larger value wins; equal values -> lower index; index < 0 means empty
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b)
{
    if (b.i < 0) return a;
    if (a.i < 0) return b;
    if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
    return a;
}

// c ranks strictly before d (an empty d ranks last)
__device__ __forceinline__ bool beats(ArgMax c, ArgMax d)
{
    return c.i >= 0 && (d.i < 0 || c.v > d.v || (c.v == d.v && c.i < d.i));
}

__device__ __forceinline__ ArgMax wave_argmax(ArgMax a)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        ArgMax b;
        b.v = __shfl_xor(a.v, o, WAVE);
        b.i = __shfl_xor(a.i, o, WAVE);
        a = better(a, b);
    }
    return a;
}

// Select top_k experts for token t from this wave's scores and write ids,
// weights (and rsf * w when pair_scale is given), the tie gap and, when hist
// is given, the LDS expert histogram.  All 64 lanes must call it together.
template <int EPL>
__device__ __forceinline__ void select_token(float (&s)[EPL], float (&b)[EPL], bool (&ok)[EPL], int lane, int t,
                                             int E, int k, int n_group, int topk_group, float rsf,
                                             int32_t *__restrict__ ids, float *__restrict__ w,
                                             float *__restrict__ gap, float *__restrict__ pair_scale,
                                             int32_t *hist, float top_p)
{
    float ggap = INFINITY;
    if (n_group > 1 && topk_group < n_group) {
        const int Eg = E / n_group;
        float my_g = -INFINITY;  // lane g holds group g's score
        const int lpg = Eg / EPL;  // lanes per group when groups cover whole lanes
        if (Eg % EPL == 0 && (lpg & (lpg - 1)) == 0) {
            // each lane's own top two, then a top-two merge across the lpg
            // lanes of its group (xor partners stay inside the group)
            ArgMax m1{-INFINITY, -1}, m2{-INFINITY, -1};
#pragma unroll
            for (int q = 0; q < EPL; ++q) {
                const ArgMax c{b[q], lane * EPL + q};
                if (!ok[q]) continue;
                if (beats(c, m1)) {
                    m2 = m1;
                    m1 = c;
                } else if (beats(c, m2)) {
                    m2 = c;
                }
            }
            for (int o = 1; o < lpg; o <<= 1) {
                ArgMax o1, o2;
                o1.v = __shfl_xor(m1.v, o, WAVE);
                o1.i = __shfl_xor(m1.i, o, WAVE);
                o2.v = __shfl_xor(m2.v, o, WAVE);
                o2.i = __shfl_xor(m2.i, o, WAVE);
                if (beats(o1, m1)) {
                    m2 = beats(m1, o2) ? m1 : o2;
                    m1 = o1;
                } else {
                    m2 = beats(o1, m2) ? o1 : m2;
                }
            }
            const float gsc = m1.v + m2.v;
            const float gv = __shfl(gsc, (lane < n_group ? lane : 0) * lpg, WAVE);
            if (lane < n_group) my_g = gv;
        } else
        for (int g = 0; g < n_group; ++g) {
            ArgMax m1{-INFINITY, -1};
#pragma unroll
            for (int q = 0; q < EPL; ++q) {
                int e = lane * EPL + q;
                if (ok[q] && e / Eg == g) m1 = better(m1, ArgMax{b[q], e});
            }
            m1 = wave_argmax(m1);
            ArgMax m2{-INFINITY, -1};
#pragma unroll
            for (int q = 0; q < EPL; ++q) {
                int e = lane * EPL + q;
                if (ok[q] && e / Eg == g && e != m1.i) m2 = better(m2, ArgMax{b[q], e});
            }
            m2 = wave_argmax(m2);
            if (lane == g) my_g = m1.v + m2.v;
        }
        bool kept = false;
        float last_kept = 0.f;
        for (int r = 0; r < topk_group; ++r) {
            ArgMax m = (lane < n_group && !kept) ? ArgMax{my_g, lane} : ArgMax{-INFINITY, -1};
            m = wave_argmax(m);
            if (lane == m.i) kept = true;
            last_kept = m.v;
        }
        ArgMax d = (lane < n_group && !kept) ? ArgMax{my_g, lane} : ArgMax{-INFINITY, -1};
        d = wave_argmax(d);
        ggap = last_kept - d.v;
        const uint64_t kept_mask = __ballot(kept);
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            int e = lane * EPL + q;
            if (ok[q] && !((kept_mask >> (e / Eg)) & 1ull)) ok[q] = false;
        }
    }
    // top-k by repeated arg-max over the allowed experts
    float ssum = 0.f;
    float sel_s = 0.f;  // lane j keeps the unbiased score and the id of selection j
    int sel_id = -1;
    float bk = 0.f;
    for (int j = 0; j < k; ++j) {
        ArgMax m{-INFINITY, -1};
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (ok[q]) m = better(m, ArgMax{b[q], lane * EPL + q});
        m = wave_argmax(m);
        bk = m.v;
        float own = 0.f;
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (lane * EPL + q == m.i) {
                ok[q] = false;
                own = s[q];
            }
        const float sj = __shfl(own, m.i / EPL, WAVE);
        ssum += sj;
        if (lane == j) {
            sel_s = sj;
            sel_id = m.i;
        }
    }
    // the best remaining allowed score, for the tie gap
    ArgMax nx{-INFINITY, -1};
#pragma unroll
    for (int q = 0; q < EPL; ++q)
        if (ok[q]) nx = better(nx, ArgMax{b[q], lane * EPL + q});
    nx = wave_argmax(nx);
    float wj = lane < k ? sel_s / ssum : 0.f;
    bool keep = lane < k;
    if (top_p > 0.f && top_p < 1.f) {
        // adaptive expert top-p: rank the k selections by weight (descending,
        // equal weights the lower id first), keep those whose running mass
        // before them (f32, summed in rank order) is below p, renormalise
        int rank = 0;
        for (int i = 0; i < k; ++i) {
            const float wi = __shfl(wj, i, WAVE);
            const int ii = __shfl(sel_id, i, WAVE);
            if (lane < k && i != lane && (wi > wj || (wi == wj && ii < sel_id))) ++rank;
        }
        float mass = 0.f, before = 0.f;
        for (int r = 0; r < k; ++r) {
            const uint64_t at = __ballot(lane < k && rank == r);
            const float wr = __shfl(wj, (int)__builtin_ctzll(at), WAVE);
            if (lane < k && rank == r) before = mass;
            mass += wr;
        }
        keep = lane < k && before < top_p;
        float ks = keep ? sel_s : 0.f;  // the kept scores' sum (a wave sum; order immaterial at 1e-7)
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ks += __shfl_xor(ks, o, WAVE);
        wj = keep ? sel_s / ks : 0.f;
    }
    if (lane < k) {
        ids[(size_t)t * k + lane] = keep ? sel_id : -1;
        w[(size_t)t * k + lane] = wj;
        if (pair_scale) pair_scale[(size_t)t * k + lane] = rsf * wj;
        if (hist && keep) atomicAdd(&hist[sel_id], 1);
    }
    if (lane == 0 && gap) {
        const float g1 = nx.i >= 0 ? bk - nx.v : INFINITY;
        gap[t] = fminf(g1, ggap);
    }
}

}  // namespace moe

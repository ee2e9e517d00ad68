// Per-token top-k routing, shared by the routing kernel and the fused
// small-batch front end: one wave64 owns one token, holds its E scores in
// registers and selects with cross-lane reductions.
#pragma once
#include "common.h"

namespace moe {

// (value, index) order: a ranks before b when larger, ties to the lower index.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Arg-best of the wave: every lane ends with the winning (value, index).
__device__ __forceinline__ void wave_argbest(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o, 64);
        const int oi = __shfl_xor(i, o, 64);
        if (beats(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// Largest two of the wave (values only), every lane ends with (m1, m2).
__device__ __forceinline__ void wave_top2(float& m1, float& m2) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float a1 = __shfl_xor(m1, o, 64), a2 = __shfl_xor(m2, o, 64);
        const float n1 = fmaxf(m1, a1);
        const float n2 = fmaxf(fminf(m1, a1), fmaxf(m2, a2));
        m1 = n1; m2 = n2;
    }
}

// ----------------------------------------------------------------------------
// One wave per token.  Lane l holds experts e = l + 64*i, i < EPL (E <= 64*EPL).
// SCORING 0: key = logit; 1: grouped sigmoid.
// ----------------------------------------------------------------------------
// Routes one token (its E logits at lr) with the whole wave; lane j < k
// ends with the j-th pick's expert in *id and its weight in *wt.
template <int EPL, int SCORING>
__device__ __forceinline__ void route_token(const float* __restrict__ lr, int E, int k, int n_groups,
                                            int topk_groups, const float* __restrict__ sel_bias, int renormalize,
                                            float route_scale, int lane, int* id, float* wt) {
    const float NEG = -__builtin_inff();

    float key[EPL];     // selection keys (-inf: absent or taken)
    float sc[EPL];      // softmax: logit; sigmoid: unbiased score s
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        const float l = e < E ? lr[e] : 0.0f;
        if (SCORING == 0) {
            sc[i] = l;
            key[i] = e < E ? l : NEG;
        } else {
            // sigmoid in fp64, rounded once to fp32
            const float s = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(l))));
            sc[i] = s;
            const float b = sel_bias ? (e < E ? sel_bias[e] : 0.0f) : 0.0f;
            key[i] = e < E ? s + b : NEG;
        }
    }

    if (SCORING == 1) {
        // group score = sum of the two largest keys of each group; keep the
        // topk_groups best groups (ties to the lower group index)
        const int gsz = E / n_groups;
        float mine = NEG;                    // lane g keeps the score of group g
        for (int g = 0; g < n_groups; ++g) {
            float m1 = NEG, m2 = NEG;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                if (e < E && e / gsz == g) {
                    const float v = key[i];
                    if (v > m1) { m2 = m1; m1 = v; } else if (v > m2) { m2 = v; }
                }
            }
            wave_top2(m1, m2);
            if (lane == g) mine = gsz >= 2 ? m1 + m2 : m1;
        }
        // group g is kept iff fewer than topk_groups groups rank before it
        int r = 0;
        for (int h = 0; h < n_groups; ++h) {
            const float other = __shfl(mine, h, 64);
            r += (h != lane) && beats(other, h, mine, lane);
        }
        const uint64_t keep = __ballot(lane < n_groups && r < topk_groups);
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((keep >> (e / gsz)) & 1ull)) key[i] = NEG;
        }
    }

    // k rounds of arg-best; the winner is removed from its owner lane
    float selv = 0.0f;   // lane j (< k) keeps the j-th pick's score
    int seli = 0;
    float vfirst = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = NEG;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (key[i] != NEG && beats(key[i], e, bv, bi)) { bv = key[i]; bi = e; }
        }
        wave_argbest(bv, bi);
        // owner fetches the pick's score and removes it
        float s_pick = 0.0f;
        if ((bi & 63) == lane) {
            const int i = bi >> 6;
#pragma unroll
            for (int q = 0; q < EPL; ++q)
                if (q == i) { s_pick = sc[q]; key[q] = NEG; }
        }
        s_pick = __shfl(s_pick, bi & 63, 64);
        if (j == 0) vfirst = s_pick;
        if (lane == j) { selv = s_pick; seli = bi; }
    }

    // weights in fp64, one rounding to fp32
    double wj = 0.0, den = 0.0;
    if (SCORING == 0) {
        const double lmax = static_cast<double>(vfirst);
        wj = lane < k ? exp(static_cast<double>(selv) - lmax) : 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j) den += __shfl(wj, j, 64);
        } else {
            double part = 0.0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                if (e < E) part += exp(static_cast<double>(sc[i]) - lmax);
            }
            // fixed-order tree over lanes
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
            den = part;
        }
        wj = wj / den;
    } else {
        wj = lane < k ? static_cast<double>(selv) : 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j) den += __shfl(wj, j, 64);
            wj = wj / den;
        }
        wj *= static_cast<double>(route_scale);
    }
    *id = seli;
    *wt = static_cast<float>(wj);
}


}  // namespace moe

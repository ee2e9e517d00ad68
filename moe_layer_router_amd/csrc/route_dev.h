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

// One step of a DPP reduction: take (value, index) from the lane the DPP
// control names when it beats ours (lanes without a source keep their own).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_best_step(float& v, int& i) {
    const float ov = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                           false));
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xF, false);
    if (beats(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Arg-best of the wave, returned wave-uniform: DPP row shifts by 1, 2, 4, 8
// leave each 16-lane row's best in its lane 15, row broadcasts 15 and 31
// carry them to lane 63, which v_readlane reads.  (value, index) under
// `beats` is a total order, so the result does not depend on the tree.
__device__ __forceinline__ void wave_argbest(float& v, int& i) {
    dpp_best_step<0x111, 0xF>(v, i);   // row_shr:1
    dpp_best_step<0x112, 0xF>(v, i);   // row_shr:2
    dpp_best_step<0x114, 0xF>(v, i);   // row_shr:4
    dpp_best_step<0x118, 0xF>(v, i);   // row_shr:8
    dpp_best_step<0x142, 0xA>(v, i);   // row_bcast:15 into rows 1 and 3
    dpp_best_step<0x143, 0xC>(v, i);   // row_bcast:31 into rows 2 and 3
    v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    i = __builtin_amdgcn_readlane(i, 63);
}

// value of lane j (j wave-uniform)
__device__ __forceinline__ float lane_f(float v, int j) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}
__device__ __forceinline__ double lane_d(double v, int j) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), j);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), j);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
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
            const float other = lane_f(mine, h);
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
        s_pick = lane_f(s_pick, bi & 63);
        if (j == 0) vfirst = s_pick;
        if (lane == j) { selv = s_pick; seli = bi; }
    }

    // weights in fp64, one rounding to fp32
    double wj = 0.0, den = 0.0;
    if (SCORING == 0) {
        const double lmax = static_cast<double>(vfirst);
        wj = lane < k ? exp(static_cast<double>(selv) - lmax) : 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j) den += lane_d(wj, j);
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
            for (int j = 0; j < k; ++j) den += lane_d(wj, j);
            wj = wj / den;
        }
        wj *= static_cast<double>(route_scale);
    }
    *id = seli;
    *wt = static_cast<float>(wj);
}


}  // namespace moe

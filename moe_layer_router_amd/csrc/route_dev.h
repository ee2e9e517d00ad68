// Per-token top-k routing: route_token (one wave64 per token; the routing
// kernel and the front-end launches) and route_token_row (four tokens per
// wave, one per 16-lane row; the fused router kernel).  The lanes hold the
// token's E scores in registers and select with cross-lane reductions.
#pragma once
#include "common.h"

namespace moe {

// (value, index) order: a ranks before b when larger, ties to the lower index.
// Non-short-circuit operators and the selects below keep the selection
// code branch-free (one compare chain and v_cndmask per candidate).
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
    return (va > vb) | ((va == vb) & (ia < ib));
}

// One step of a DPP reduction: take (value, index) from the lane the DPP
// control names when it beats ours (lanes without a source keep their own).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_best_step(float& v, int& i) {
    const float ov = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                           false));
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xF, false);
    const bool take = beats(ov, oi, v, i);
    v = take ? ov : v;
    i = take ? oi : i;
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
            const bool take = (key[i] != NEG) & beats(key[i], e, bv, bi);
            bv = take ? key[i] : bv;
            bi = take ? e : bi;
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


// ----------------------------------------------------------------------------
// Four tokens per wave: the token of a 16-lane row (a DPP row) is routed by
// that row alone, so one instruction stream selects for four tokens.  Lane
// sub = lane % 16 of the row holds experts e = sub + 16 i, i < EPL
// (E <= 16 EPL).  The selection is the same as route_token's: `beats` is a
// total order, so the reduction tree does not change the picks.
// ----------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ int row_dpp(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float row_dpp_f(float x) {
    return __builtin_bit_cast(float, row_dpp<CTRL>(__builtin_bit_cast(int, x)));
}

// One combining step: the partner lane's (value, index, payload) when it
// beats ours.  Every source of the controls below is inside the row.
template <int CTRL>
__device__ __forceinline__ void row_best_step(float& v, int& i, float& s) {
    const float ov = row_dpp_f<CTRL>(v), os = row_dpp_f<CTRL>(s);
    const int oi = row_dpp<CTRL>(i);
    const bool take = beats(ov, oi, v, i);
    v = take ? ov : v;
    i = take ? oi : i;
    s = take ? os : s;
}

// Best (value, index) of the row, with the payload s of the lane that held
// it, in every lane of the row.  Rotations by 8 and 4 and the quad
// permutations xor 2 and xor 1 combine disjoint lane sets at each step, so
// each lane ends with the best of all 16.
__device__ __forceinline__ void row_argbest(float& v, int& i, float& s) {
    row_best_step<0x128>(v, i, s);   // row_ror:8
    row_best_step<0x124>(v, i, s);   // row_ror:4
    row_best_step<0x4E>(v, i, s);    // quad_perm [2, 3, 0, 1]
    row_best_step<0xB1>(v, i, s);    // quad_perm [1, 0, 3, 2]
}

// Largest two values of the row (the same disjoint combining steps).
template <int CTRL>
__device__ __forceinline__ void row_top2_step(float& m1, float& m2) {
    const float a1 = row_dpp_f<CTRL>(m1), a2 = row_dpp_f<CTRL>(m2);
    const float n1 = fmaxf(m1, a1);
    const float n2 = fmaxf(fminf(m1, a1), fmaxf(m2, a2));
    m1 = n1;
    m2 = n2;
}
__device__ __forceinline__ void row_top2(float& m1, float& m2) {
    row_top2_step<0x128>(m1, m2);
    row_top2_step<0x124>(m1, m2);
    row_top2_step<0x4E>(m1, m2);
    row_top2_step<0xB1>(m1, m2);
}

// value of lane j of this lane's row
__device__ __forceinline__ float row_lane_f(float v, int lane, int j) { return __shfl(v, (lane & ~15) + j, 64); }
__device__ __forceinline__ double row_lane_d(double v, int lane, int j) { return __shfl(v, (lane & ~15) + j, 64); }

// Routes the token of this lane's row (its E logits at lr).  Lane j < k of
// the row ends with the j-th pick's expert in *id and its weight in *wt.
// Grouped scoring needs n_groups <= 16 (lane g of the row keeps group g's
// score).  Every lane of the wave must call it (the steps are cross-lane).
template <int EPL, int SCORING>
__device__ __forceinline__ void route_token_row(const float* __restrict__ lr, int E, int k, int n_groups,
                                                int topk_groups, const float* __restrict__ sel_bias,
                                                int renormalize, float route_scale, int lane, int* id, float* wt) {
    const float NEG = -__builtin_inff();
    const int sub = lane & 15;

    float key[EPL];     // selection keys (-inf: absent or taken)
    float sc[EPL];      // softmax: logit; sigmoid: unbiased score s
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = sub + 16 * i;
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
        float mine = NEG;                    // lane g of the row keeps group g's score
        for (int g = 0; g < n_groups; ++g) {
            float m1 = NEG, m2 = NEG;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = sub + 16 * i;
                if (e < E && e / gsz == g) {
                    const float v = key[i];
                    if (v > m1) { m2 = m1; m1 = v; } else if (v > m2) { m2 = v; }
                }
            }
            row_top2(m1, m2);
            if (sub == g) mine = gsz >= 2 ? m1 + m2 : m1;
        }
        int r = 0;
        for (int h = 0; h < n_groups; ++h) {
            const float other = row_lane_f(mine, lane, h);
            r += (h != sub) && beats(other, h, mine, sub);
        }
        const uint32_t keep =
            static_cast<uint32_t>(__ballot(sub < n_groups && r < topk_groups) >> (lane & ~15)) & 0xFFFFu;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = sub + 16 * i;
            if (e < E && !((keep >> (e / gsz)) & 1u)) key[i] = NEG;
        }
    }

    // k rounds of arg-best; every lane of the row learns the pick and its
    // score, and the owner removes it
    float selv = 0.0f;   // lane j (< k) of the row keeps the j-th pick's score
    int seli = 0;
    float vfirst = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = NEG, bs = 0.0f;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = sub + 16 * i;
            const bool take = (key[i] != NEG) & beats(key[i], e, bv, bi);
            bv = take ? key[i] : bv;
            bi = take ? e : bi;
            bs = take ? sc[i] : bs;
        }
        row_argbest(bv, bi, bs);
        const int own = (bi & 15) == sub ? bi >> 4 : -1;
#pragma unroll
        for (int q = 0; q < EPL; ++q) key[q] = q == own ? NEG : key[q];
        if (j == 0) vfirst = bs;
        if (sub == j) { selv = bs; seli = bi; }
    }

    // weights in fp64, one rounding to fp32
    double wj = 0.0, den = 0.0;
    if (SCORING == 0) {
        const double lmax = static_cast<double>(vfirst);
        wj = sub < k ? exp(static_cast<double>(selv) - lmax) : 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j) den += row_lane_d(wj, lane, j);
        } else {
            double part = 0.0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = sub + 16 * i;
                if (e < E) part += exp(static_cast<double>(sc[i]) - lmax);
            }
            // fixed-order tree over the row
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
            den = part;
        }
        wj = wj / den;
    } else {
        wj = sub < k ? static_cast<double>(selv) : 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j) den += row_lane_d(wj, lane, j);
            wj = wj / den;
        }
        wj *= static_cast<double>(route_scale);
    }
    *id = seli;
    *wt = static_cast<float>(wj);
}

}  // namespace moe

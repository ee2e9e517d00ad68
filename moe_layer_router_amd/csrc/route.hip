// Router projection and top-k routing.
//
// The router gate scores every token against the routed experts and keeps the
// top-k (Qwen 3.5 page, MoE paragraph of the model description); the Qwen 3.5
// roadmap item asks for the top-k selection to run where the scores are,
// without a round trip: here one wave64 owns one token, holds its E scores in
// registers and selects with cross-lane reductions, so logits are read once
// and ids/weights written once.
#include "common.h"

namespace moe {

// ----------------------------------------------------------------------------
// logits[t, e] = sum_d x[t, d] * Wr[e, d]  in fp64 (bf16 x fp32 products are
// exact in fp64), rounded once to fp32.  One block per token; x[t] is staged
// in LDS; each wave takes experts e = wave, wave + 4, ...; lanes split D and
// reduce in a fixed order.
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            int T, int D, int E,
                                                            float* __restrict__ logits) {
    extern __shared__ float xs[];
    const int t = blockIdx.x;
    const uint16_t* xr = x + static_cast<int64_t>(t) * D;
    for (int d = threadIdx.x; d < D; d += blockDim.x) xs[d] = bf16_to_f32(xr[d]);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int e = wave; e < E; e += nw) {
        const float* w = wr + static_cast<int64_t>(e) * D;
        double acc = 0.0;
        for (int d = lane; d < D; d += 64) acc += static_cast<double>(xs[d]) * static_cast<double>(w[d]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
        if (lane == 0) logits[static_cast<int64_t>(t) * E + e] = static_cast<float>(acc);
    }
}

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
template <int EPL, int SCORING>
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int n_groups, int topk_groups,
                                                         const float* __restrict__ sel_bias,
                                                         int renormalize, float route_scale,
                                                         int* __restrict__ ids, float* __restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* lr = logits + static_cast<int64_t>(t) * E;
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
    if (lane < k) {
        ids[static_cast<int64_t>(t) * k + lane] = seli;
        wout[static_cast<int64_t>(t) * k + lane] = static_cast<float>(wj);
    }
}

template <int EPL>
static void launch_topk(int scoring, dim3 g, dim3 b, hipStream_t s, const float* logits, int T, int E, int k,
                        int ng, int tg, const float* bias, int renorm, float scale, int* ids, float* w) {
    if (scoring == 0)
        hipLaunchKernelGGL((route_topk_kernel<EPL, 0>), g, b, 0, s, logits, T, E, k, ng, tg, bias, renorm, scale, ids, w);
    else
        hipLaunchKernelGGL((route_topk_kernel<EPL, 1>), g, b, 0, s, logits, T, E, k, ng, tg, bias, renorm, scale, ids, w);
}

int32_t route_topk_launch(const float* logits, int T, int E, int k, int scoring, int n_groups, int topk_groups,
                          const float* sel_bias, int renormalize, float route_scale, int* ids, float* w,
                          hipStream_t s) {
    if (T == 0) return MOE_OK;
    const dim3 block(256), grid(static_cast<unsigned>(ceil_div(T, 4)));
    const int epl = static_cast<int>(ceil_div(E, 64));
    if (epl <= 1) launch_topk<1>(scoring, grid, block, s, logits, T, E, k, n_groups, topk_groups, sel_bias, renormalize, route_scale, ids, w);
    else if (epl <= 2) launch_topk<2>(scoring, grid, block, s, logits, T, E, k, n_groups, topk_groups, sel_bias, renormalize, route_scale, ids, w);
    else if (epl <= 4) launch_topk<4>(scoring, grid, block, s, logits, T, E, k, n_groups, topk_groups, sel_bias, renormalize, route_scale, ids, w);
    else if (epl <= 8) launch_topk<8>(scoring, grid, block, s, logits, T, E, k, n_groups, topk_groups, sel_bias, renormalize, route_scale, ids, w);
    else launch_topk<16>(scoring, grid, block, s, logits, T, E, k, n_groups, topk_groups, sel_bias, renormalize, route_scale, ids, w);
    return moe_launch_status();
}

int32_t router_logits_launch(const uint16_t* x, const float* wr, int T, int D, int E, float* logits,
                             hipStream_t s) {
    if (T == 0) return MOE_OK;
    hipLaunchKernelGGL(router_logits_kernel, dim3(T), dim3(256), D * sizeof(float), s, x, wr, T, D, E, logits);
    return moe_launch_status();
}

}  // namespace moe

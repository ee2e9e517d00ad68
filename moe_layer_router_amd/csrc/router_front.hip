// Router projection fused with top-k routing and the FP8 quantization of x.
//
// The router gate scores every token against the routed experts (Qwen 3.5
// TPU page, MoE paragraph of the model description), and the page's roadmap
// item asks for the top-k selection to happen where the scores are computed
// instead of moving the logits between units.  Here one workgroup takes 32
// tokens against all E experts:
//   1. logits[t, e] = x[t] . Wr[e] on the matrix cores.  x is bf16; each
//      fp32 router weight is split exactly into three bf16 pieces
//      (hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid, which has at most
//      8 significant bits), so every product x * piece is exact in fp32 and
//      v_mfma_f32_32x32x16_bf16 only adds: the logits carry nothing but fp32
//      accumulation rounding.  The weight rows are the first operand, so lane
//      (token l % 32) ends with 16 experts of its token per 32-expert tile.
//   2. The tile's logits go to LDS (and to the logits buffer); each wave then
//      routes 8 of the tokens with the wave-per-token top-k (route_token).
//   3. The same tokens' x rows are quantized to FP8 (one scale per row or
//      per 128 elements), the rows being fresh in L2.
// Used by moe_forward for batches above the decode sizes when it is given
// no logits (large batches spread over T / 32 workgroups), and by
// moe_router_front.
#include "quant_dev.h"
#include "route_dev.h"

namespace moe {

typedef __bf16 v8bf_r __attribute__((ext_vector_type(8)));
typedef float v16f_r __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_r __attribute__((ext_vector_type(4)));

constexpr int kRouterTokens = 32;
constexpr int kRouterMaxE = 512;

struct RouterArgs {
    const uint16_t* x;
    const float* wr;
    int T, D, E, k;
    int n_groups, topk_groups;
    const float* sel_bias;
    int renormalize;
    float route_scale;
    float* logits;             // [T, E]
    int* ids;                  // [T, k]
    float* w;                  // [T, k]
    uint8_t* xq;               // codes [T, D] (FP8) or [T, D/2] (MXFP4); NULL for bf16 layers
    void* xs;                  // fp32 scales [T] or [T, D/128], or E8M0 bytes [T, D/32]
};

// w == hi + mid + lo exactly, each piece a bf16 (see the file comment).
__device__ __forceinline__ void split3(const float (&w)[8], v8bf_r& hi, v8bf_r& mid, v8bf_r& lo) {
    uint16_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = f32_to_bf16(w[i]);
        const float r1 = w[i] - bf16_to_f32(h[i]);       // exact
        m[i] = f32_to_bf16(r1);
        l[i] = f32_to_bf16(r1 - bf16_to_f32(m[i]));     // exact, and exactly a bf16
    }
    hi = __builtin_bit_cast(v8bf_r, h);
    mid = __builtin_bit_cast(v8bf_r, m);
    lo = __builtin_bit_cast(v8bf_r, l);
}

// EPT: 32-expert tiles per wave (E <= 128 * EPT); EPL: experts per lane in
// the top-k (E <= 64 * EPL); GROUP: -1 (bf16 layer, x not quantized), 0 (per
// row), 128 (1x128 groups).
template <int EPT, int EPL, int SCORING, int GROUP>
__global__ void __launch_bounds__(256) router_front_kernel(const RouterArgs p) {
    constexpr int LD = EPT * 128 + 1;                 // LDS row stride (floats)
    __shared__ float s_lg[kRouterTokens][LD];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kRouterTokens;
    const int r = lane & 31, kh = lane >> 5;

    // Lane (r, kh) supplies, for K step s and 16-wide chunk c, the elements
    // [64 s + 32 kh + 8 c, +8) of its token row and of its expert rows: both
    // operands use the same K positions, so the products pair up.
    const int tok = min(t0 + r, p.T - 1);               // rows past T read the last token (not stored)
    const uint16_t* xr = p.x + static_cast<int64_t>(tok) * p.D + kh * 32;
    const float* wrow[EPT];
    bool tile_on[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int et = wave + 4 * j;
        tile_on[j] = et * 32 < p.E;
        const int e = et * 32 + r;
        wrow[j] = p.wr + static_cast<int64_t>(e < p.E ? e : 0) * p.D + kh * 32;
    }
    v16f_r acc[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[j] = v16f_r{};

    const int nsteps = p.D >> 6;
    for (int s = 0; s < nsteps; ++s) {
        const int ko = s * 64;
        u32x4_r xa[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) xa[c] = *reinterpret_cast<const u32x4_r*>(xr + ko + 8 * c);
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (!tile_on[j]) continue;                    // wave-uniform
            float4 wf[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) wf[q] = *reinterpret_cast<const float4*>(wrow[j] + ko + 4 * q);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float w8[8] = {wf[2 * c].x, wf[2 * c].y, wf[2 * c].z, wf[2 * c].w,
                                     wf[2 * c + 1].x, wf[2 * c + 1].y, wf[2 * c + 1].z, wf[2 * c + 1].w};
                v8bf_r hi, mid, lo;
                split3(w8, hi, mid, lo);
                const v8bf_r xb = __builtin_bit_cast(v8bf_r, xa[c]);
                // smallest pieces first
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, xb, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, xb, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, xb, acc[j], 0, 0, 0);
            }
        }
    }

    // lane (r, kh): token r, register v holds expert 8 (v / 4) + 4 kh + v % 4 of the tile
    const bool tok_ok = t0 + r < p.T;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (!tile_on[j]) continue;
        const int ebase = (wave + 4 * j) * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int e0 = ebase + 8 * g + 4 * kh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = e0 + i;
                if (e < p.E) {
                    s_lg[r][e] = acc[j][4 * g + i];
                    if (tok_ok) p.logits[static_cast<int64_t>(t0 + r) * p.E + e] = acc[j][4 * g + i];
                }
            }
        }
    }
    __syncthreads();

    // top-k of each token, one wave per token, from the logits in LDS
    for (int tt = wave; tt < kRouterTokens; tt += 4) {
        const int t = t0 + tt;
        if (t >= p.T) break;
        int id;
        float wt;
        route_token<EPL, SCORING>(&s_lg[tt][0], p.E, p.k, p.n_groups, p.topk_groups, p.sel_bias, p.renormalize,
                                  p.route_scale, lane, &id, &wt);
        if (lane < p.k) {
            p.ids[static_cast<int64_t>(t) * p.k + lane] = id;
            p.w[static_cast<int64_t>(t) * p.k + lane] = wt;
        }
    }

    // FP8 codes of the same tokens' x rows
    if constexpr (GROUP >= 0) {
        for (int tt = wave; tt < kRouterTokens; tt += 4) {
            const int t = t0 + tt;
            if (t >= p.T) break;
            quant_x_row<GROUP>(p.x, p.D, t, p.xq, p.xs, lane);
        }
    }
}

template <int EPT, int EPL, int SCORING>
static void router_launch_group(int group, dim3 g, hipStream_t s, const RouterArgs& a) {
    if (group < 0) hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, -1>), g, dim3(256), 0, s, a);
    else if (group == 0) hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, 0>), g, dim3(256), 0, s, a);
    else if (group == 32) hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, 32>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, 128>), g, dim3(256), 0, s, a);
}

template <int EPT, int EPL>
static void router_launch_scoring(int scoring, int group, dim3 g, hipStream_t s, const RouterArgs& a) {
    if (scoring == MOE_SCORING_SOFTMAX) router_launch_group<EPT, EPL, 0>(group, g, s, a);
    else router_launch_group<EPT, EPL, 1>(group, g, s, a);
}

bool router_front_ok(int E, int D) { return E <= kRouterMaxE && D % 64 == 0; }

// group: -1 (no x quantization), 0, 128 or 32 (MXFP4).  The caller has validated the
// layer (router_front_ok, routing limits).
int32_t router_front_launch(const moe_layer_desc* L, const void* x, int T, int group, float* logits, int* ids,
                            float* w, uint8_t* xq, float* xs, hipStream_t s) {
    if (T == 0) return MOE_OK;
    RouterArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.wr = L->router_w;
    a.T = T;
    a.D = L->D;
    a.E = L->E;
    a.k = L->top_k;
    a.n_groups = L->n_groups;
    a.topk_groups = L->topk_groups;
    a.sel_bias = L->sel_bias;
    a.renormalize = L->renormalize;
    a.route_scale = L->route_scale;
    a.logits = logits;
    a.ids = ids;
    a.w = w;
    a.xq = xq;
    a.xs = xs;
    const dim3 g(static_cast<unsigned>(ceil_div(T, kRouterTokens)));
    const int E = L->E;
    if (E <= 64) router_launch_scoring<1, 1>(L->scoring, group, g, s, a);
    else if (E <= 128) router_launch_scoring<1, 2>(L->scoring, group, g, s, a);
    else if (E <= 256) router_launch_scoring<2, 4>(L->scoring, group, g, s, a);
    else router_launch_scoring<4, 8>(L->scoring, group, g, s, a);
    return moe_launch_status();
}

}  // namespace moe

// Front end: routing and FP8 quantization of x in one launch (any batch),
// and the one-workgroup permutation.
//
// At a few dozen tokens the routing, the three permutation steps and the FP8
// quantization of x each move a few KB; as five separate launches they cost
// more in launch latency and dependent round trips than in work (the Qwen
// 3.5 roadmap item asks for top-k to run next to the scores, and the MI300X
// page tunes small-batch latency).  Here:
//   token_front_kernel: one workgroup of two waves per token; wave 0 routes
//     the token (route_token, shared with the routing kernel), wave 1
//     quantizes its x row (the row-quantization arithmetic), in parallel and
//     spread over T CUs (every batch size uses it);
//   permute_small_kernel: the permutation of up to 256 tokens' distinct
//     picks by one workgroup (perm_dev.h: token masks, ranks by mask bits
//     below the token) in place of the three launches of the general one.
//     In the weight-streaming path the gate/up GEMM builds the same
//     permutation itself and this launch is not needed.
#include "perm_dev.h"
#include "quant_dev.h"
#include "route_dev.h"

namespace moe {

constexpr int kFrontWaves = 16;
constexpr int kFrontMaxT = 64;
constexpr int kFrontMaxRows = kFrontMaxT * (MOE_MAX_TOPK + 1);
// the one-workgroup permutation also serves batches up to this many tokens
// (routed by the other launches) in place of the three-launch one
constexpr int kPermSmallMaxT = 256;

struct FrontArgs {
    const float* logits;
    const uint16_t* x;
    int T, D, E, k, n_shared;
    int n_groups, topk_groups;
    const float* sel_bias;
    int renormalize;
    float route_scale;
    int block_m, max_rows;
    int* ids;
    float* w;
    int* counts;
    int* offsets;
    int* sorted;
    int* bexp;
    int* inv;
    uint8_t* xq;               // FP8 modes: codes [T, D]; NULL for bf16
    float* xs;                 // scales [T] or [T, D/128]
};

// GROUP: -1 (bf16 layer, no quantization), 0 (per row), 128 (1x128), 32 (MXFP4).
template <int EPL, int SCORING, int GROUP>
__global__ void __launch_bounds__(128) token_front_kernel(const FrontArgs p) {
    const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave == 0) {
        int id;
        float wt;
        route_token<EPL, SCORING>(p.logits + static_cast<int64_t>(t) * p.E, p.E, p.k, p.n_groups, p.topk_groups,
                                  p.sel_bias, p.renormalize, p.route_scale, lane, &id, &wt);
        if (lane < p.k) {
            p.ids[t * p.k + lane] = id;
            p.w[t * p.k + lane] = wt;
        }
    } else if constexpr (GROUP >= 0) {
        quant_x_row<GROUP>(p.x, p.D, t, p.xq, p.xs, lane);
    }
}

// MW: 32-token words of each expert's token mask (T <= 32 MW).
template <int MW>
__global__ void __launch_bounds__(kFrontWaves * 64) permute_small_kernel(const FrontArgs p) {
    __shared__ int s_e[32 * MW * MOE_MAX_TOPK];         // expert of each pick (-1: no row)
    __shared__ PermShared<MW> s_perm;
    perm_build<MW, kFrontWaves * 64>(p.ids, p.T, p.k, p.E, p.n_shared, p.block_m, p.max_rows, s_perm, s_e, nullptr,
                                     PermOut{p.counts, p.offsets, p.sorted, p.bexp, p.inv}, true);
}

template <int EPL, int SCORING>
static void front_group(int group, const FrontArgs& a, hipStream_t s) {
    const dim3 g(static_cast<unsigned>(a.T)), b(128);
    if (group < 0) hipLaunchKernelGGL((token_front_kernel<EPL, SCORING, -1>), g, b, 0, s, a);
    else if (group == 0) hipLaunchKernelGGL((token_front_kernel<EPL, SCORING, 0>), g, b, 0, s, a);
    else if (group == 32) hipLaunchKernelGGL((token_front_kernel<EPL, SCORING, 32>), g, b, 0, s, a);
    else hipLaunchKernelGGL((token_front_kernel<EPL, SCORING, 128>), g, b, 0, s, a);
}

template <int EPL>
static void front_scoring(int scoring, int group, const FrontArgs& a, hipStream_t s) {
    if (scoring == MOE_SCORING_SOFTMAX) front_group<EPL, 0>(group, a, s);
    else front_group<EPL, 1>(group, a, s);
}

bool front_small_ok(int T, int k, int n_shared) {
    return T >= 1 && T <= kFrontMaxT && T * (k + n_shared) <= kFrontMaxRows;
}

static void front_tokens(const moe_layer_desc* L, const FrontArgs& a, hipStream_t s) {
    const int group = L->quant == MOE_QUANT_NONE_BF16 ? -1
                      : L->quant == MOE_QUANT_BLOCK128_FP8 ? 128 : L->quant == MOE_QUANT_MXFP4 ? 32 : 0;
    const int epl = static_cast<int>(ceil_div(L->E, 64));
    if (epl <= 1) front_scoring<1>(L->scoring, group, a, s);
    else if (epl <= 2) front_scoring<2>(L->scoring, group, a, s);
    else if (epl <= 4) front_scoring<4>(L->scoring, group, a, s);
    else if (epl <= 8) front_scoring<8>(L->scoring, group, a, s);
    else front_scoring<16>(L->scoring, group, a, s);
}

// Routing and x quantization only (ids, w, xq, xs), for any T >= 1.
int32_t front_route_quant_launch(const moe_layer_desc* L, const void* x, const float* logits, int T, int* ids,
                                 float* w, uint8_t* xq, float* xs, hipStream_t s) {
    FrontArgs a{};
    a.logits = logits;
    a.x = static_cast<const uint16_t*>(x);
    a.T = T;
    a.D = L->D;
    a.E = L->E;
    a.k = L->top_k;
    a.n_shared = L->n_shared;
    a.n_groups = L->n_groups;
    a.topk_groups = L->topk_groups;
    a.sel_bias = L->sel_bias;
    a.renormalize = L->renormalize;
    a.route_scale = L->route_scale;
    a.ids = ids;
    a.w = w;
    a.xq = xq;
    a.xs = xs;
    front_tokens(L, a, s);
    return moe_launch_status();
}

// The one-workgroup permutation alone, for ids routed by another launch with
// distinct picks per token (moe_forward's own routing) and T <= 256: one
// launch in place of the three of the general permutation.
bool permute_small_ok(int T, int k, int n_shared) {
    return T >= 1 && T <= kPermSmallMaxT && T * (k + n_shared) <= kPermSmallMaxT * (MOE_MAX_TOPK + 1);
}

int32_t permute_small_launch(const int* ids, int T, int k, int E, int n_shared, int block_m, int max_rows,
                             int* counts, int* offsets, int* sorted, int* bexp, int* inv, hipStream_t s) {
    FrontArgs a{};
    a.ids = const_cast<int*>(ids);
    a.T = T;
    a.E = E;
    a.k = k;
    a.n_shared = n_shared;
    a.block_m = block_m;
    a.max_rows = max_rows;
    a.counts = counts;
    a.offsets = offsets;
    a.sorted = sorted;
    a.bexp = bexp;
    a.inv = inv;
    hipLaunchKernelGGL(permute_small_kernel<kPermSmallMaxT / 32>, dim3(1), dim3(kFrontWaves * 64), 0, s, a);
    return moe_launch_status();
}

}  // namespace moe

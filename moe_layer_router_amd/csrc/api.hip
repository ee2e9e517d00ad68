// C ABI: argument validation, workspace carving and the fused forward.
// Every check runs on the host before anything is enqueued (moe_forward
// checks the limits of all of its kernels before the first launch).
#include "common.h"
#include "perm_dev.h"

#include <atomic>
#include <mutex>

namespace moe {
int32_t route_topk_launch(const float* logits, int T, int E, int k, int scoring, int n_groups, int topk_groups,
                          const float* sel_bias, int renormalize, float route_scale, int* ids, float* w,
                          hipStream_t s);
int32_t router_logits_launch(const uint16_t* x, const float* wr, int T, int D, int E, float* logits,
                             hipStream_t s);
size_t permute_scratch_bytes(int T, int k, int n_shared, int E);
int32_t permute_align_launch(const int* ids, int T, int k, int E, int n_shared, int block_m, int max_rows,
                             int* counts, int* offsets, int* sorted_ids, int* block_expert, int* inv_perm,
                             void* scratch, hipStream_t s);
int32_t quant_wrows_launch(const uint16_t* w, int64_t M, int K, bool blocked, uint8_t* q, float* scale,
                           hipStream_t s);
int32_t quant_rows_launch(const uint16_t* x, int64_t M, int K, int group, const int* valid_rows, uint8_t* q,
                          float* scale, hipStream_t s, bool blocked = false, const int* skip_ids = nullptr,
                          int skip_id = 0);
int32_t quant_mx_rows_launch(const uint16_t* x, int64_t M, int K, const int* valid_rows, bool blocked,
                             const int* skip_ids, int skip_id, uint8_t* q, uint8_t* scale, hipStream_t s);
int32_t quant_wblock_launch(const uint16_t* w, int64_t n_mats, int N, int K, bool blocked, uint8_t* q, float* scale,
                            hipStream_t s);
bool front_small_ok(int T, int k, int n_shared);
bool permute_small_ok(int T, int k, int n_shared);
int32_t permute_small_launch(const int* ids, int T, int k, int E, int n_shared, int block_m, int max_rows,
                             int* counts, int* offsets, int* sorted, int* bexp, int* inv, hipStream_t s);
int32_t front_route_quant_launch(const moe_layer_desc* L, const void* x, const float* logits, int T, int* ids,
                                 float* w, uint8_t* xq, float* xs, hipStream_t s);
int32_t stream_gateup_fused_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T,
                                   const int* ids, int max_rows, const PermOut& pout, void* act, hipStream_t s);
bool stream_fused_perm_ok(int T);
int32_t gemm_gateup_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T, int block_m,
                           int64_t max_rows, const int* sorted_ids, const int* block_expert, const int* offsets,
                           const int* counts, void* act, hipStream_t s);
int32_t gemm_down_launch(const moe_layer_desc* L, const void* act, const float* act_scale, int T, int block_m,
                         int64_t max_rows, const int* block_expert, const int* offsets, const int* counts,
                         void* out_perm, hipStream_t s, bool act_blocked = false);
int32_t combine_launch(const void* out_perm, int out_dtype, const int* inv_perm, const float* topk_w, int T,
                       int k, int n_shared, int D, uint16_t* y, hipStream_t s);
bool router_front_ok(int E, int D);
int64_t router_front_scratch_bytes(int E, int D);
int32_t router_front_launch(const moe_layer_desc* L, const void* x, int T, int group, float* logits, int* ids,
                            float* w, uint8_t* xq, float* xs, void* scratch, hipStream_t s);
int64_t ep_payload_row_bytes(int D, int format);
int32_t ep_pack_launch(const uint16_t* x, int T, int D, int format, uint8_t* payload, hipStream_t s);
int32_t ep_unpack_launch(const uint8_t* payload, int T, int D, int format, uint16_t* x, hipStream_t s);
}  // namespace moe

using namespace moe;

namespace {

constexpr int64_t kAlign = 256;

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int64_t max_rows_of(int64_t T, int64_t k, int64_t E, int64_t n_sh, int64_t B) {
    const int64_t A = T * (k + n_sh);
    const int64_t Ep = E + n_sh;
    int64_t blocks = (A + Ep * (B - 1)) / B;
    if (blocks > A) blocks = A;
    return blocks * B;
}

// block_m 16 selects the weight-streaming kernels (a wave carries up to 64
// rows of an expert at a time); 32/64/128/256 the LDS-tiled ones.
constexpr int kStreamMaxT = 64;          // the automatic choice streams at or below this batch

bool block_m_ok(int block_m) {
    return block_m == 16 || block_m == 32 || block_m == 64 || block_m == 128 || block_m == 192 || block_m == 256;
}

int32_t check_routing(int E, int k, int scoring, int n_groups, int topk_groups) {
    MOE_CHECK_ARG(E > 0 && k > 0 && k <= E);
    MOE_CHECK_ARG(scoring == MOE_SCORING_SOFTMAX || scoring == MOE_SCORING_SIGMOID_GROUPED);
    MOE_CHECK_SUP(k <= MOE_MAX_TOPK && E <= MOE_MAX_EXPERTS);
    if (scoring == MOE_SCORING_SIGMOID_GROUPED) {
        MOE_CHECK_ARG(n_groups > 0 && E % n_groups == 0 && topk_groups > 0 && topk_groups <= n_groups);
        MOE_CHECK_ARG(k <= topk_groups * (E / n_groups));
        MOE_CHECK_SUP(n_groups <= MOE_MAX_GROUPS);
    }
    return MOE_OK;
}

// Shapes the layer's kernels cover.
int32_t check_layer(const moe_layer_desc* L) {
    MOE_CHECK_ARG(L != nullptr);
    MOE_CHECK_ARG(L->D > 0 && L->I > 0 && L->E > 0 && (L->n_shared == 0 || L->n_shared == 1));
    int32_t st = check_routing(L->E, L->top_k, L->scoring, L->n_groups, L->topk_groups);
    if (st != MOE_OK) return st;
    MOE_CHECK_SUP(L->E + L->n_shared <= MOE_MAX_EXPERTS);
    MOE_CHECK_ARG(L->quant == MOE_QUANT_NONE_BF16 || L->quant == MOE_QUANT_PTPC_FP8 ||
                  L->quant == MOE_QUANT_BLOCK128_FP8 || L->quant == MOE_QUANT_MXFP4);
    MOE_CHECK_ARG(L->w13 != nullptr && L->w2 != nullptr);
    if (L->quant != MOE_QUANT_NONE_BF16) MOE_CHECK_ARG(L->w13_scale != nullptr && L->w2_scale != nullptr);
    MOE_CHECK_ARG(L->weight_layout == MOE_WEIGHTS_ROWS || L->weight_layout == MOE_WEIGHTS_BLOCKED);
    MOE_CHECK_SUP(L->weight_layout == MOE_WEIGHTS_ROWS || L->quant != MOE_QUANT_NONE_BF16);
    // column tiles of the grouped GEMMs: 128 act columns, 256 output columns
    MOE_CHECK_SUP(L->I % 128 == 0 && L->D % 256 == 0);
    MOE_CHECK_SUP(L->D <= 16384 && L->I <= 16384);
    // MXFP4: each 128-byte step of the tiled GEMMs is 256 elements
    if (L->quant == MOE_QUANT_MXFP4) MOE_CHECK_SUP(L->I % 256 == 0);
    return MOE_OK;
}

// The activation format of the layer's quantizers: -1 none (bf16), 0 PTPC
// (fp32 scale per row), 128 (fp32 scale per 1x128 group), 32 (MXFP4).
int act_group(const moe_layer_desc* L) {
    switch (L->quant) {
        case MOE_QUANT_PTPC_FP8: return 0;
        case MOE_QUANT_BLOCK128_FP8: return 128;
        case MOE_QUANT_MXFP4: return 32;
        default: return -1;
    }
}

// the weight-streaming kernels (block_m 16) cover every mode; MXFP4 runs
// the LDS-tiled kernels up to 192-row tiles (the 256-row tile's scale words
// do not fit its registers); 192-row tiles exist for the quantized modes
bool block_m_ok_for(const moe_layer_desc* L, int block_m) {
    if (L->quant == MOE_QUANT_MXFP4) return block_m == 16 || block_m == 32 || block_m == 64 || block_m == 128 || block_m == 192;
    if (L->quant == MOE_QUANT_NONE_BF16 && block_m == 192) return false;   // (the 192-row tile: quantized modes)
    return block_m_ok(block_m);
}

// The LDS-tiled GEMMs address the activation rows and one expert's weights
// with 32-bit byte offsets from a 64-bit base (the weight-streaming kernels,
// block_m 16, use 64-bit addresses throughout).  Checked on the host before
// any launch of a call.
bool gemm_ranges_ok(const moe_layer_desc* L, int64_t T, int block_m, int64_t R) {
    if (block_m == 16) return true;
    const int64_t elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;   // (MXFP4: half a byte, within this)
    const int64_t lim = 1LL << 32;
    return T * L->D * elem < lim && 2LL * L->I * L->D * elem < lim &&   // gate/up
           R * L->I * elem < lim;                                        // down (its weights are half of W13)
}

struct Carver {
    int64_t off = 0;
    int64_t take(int64_t bytes) {
        const int64_t at = off;
        off += (bytes + kAlign - 1) / kAlign * kAlign;
        return at;
    }
};

void layout_of(const moe_layer_desc* L, int T, int B, moe_ws_layout* o) {
    const int64_t k = L->top_k, E = L->E, Ep = E + L->n_shared, D = L->D, I = L->I;
    const int64_t A = static_cast<int64_t>(T) * (k + L->n_shared);
    const int64_t R = max_rows_of(T, k, E, L->n_shared, B);
    const bool fp8 = L->quant != MOE_QUANT_NONE_BF16;     // any quantized mode
    const bool blk = L->quant == MOE_QUANT_BLOCK128_FP8;
    const bool mx = L->quant == MOE_QUANT_MXFP4;
    Carver c;
    o->logits = c.take(static_cast<int64_t>(T) * E * 4);
    o->topk_ids = c.take(T * k * 4);
    o->topk_w = c.take(T * k * 4);
    o->counts = c.take(Ep * 4);
    o->offsets = c.take((Ep + 1) * 4);
    o->sorted_ids = c.take(R * 4);
    o->block_expert = c.take(R / B * 4);
    o->inv_perm = c.take(A * 4);
    if (mx) {
        o->xq = c.take(static_cast<int64_t>(T) * D / 2);
        o->xs = c.take(static_cast<int64_t>(T) * D / 32);
    } else {
        o->xq = fp8 ? c.take(static_cast<int64_t>(T) * D) : -1;
        o->xs = fp8 ? c.take(static_cast<int64_t>(T) * (blk ? D / 128 : 1) * 4) : -1;
    }
    o->act = c.take(R * I * 2);
    if (mx) {
        o->aq = c.take(R * I / 2);
        o->as = c.take(R * I / 32);
    } else {
        o->aq = fp8 ? c.take(R * I) : -1;
        o->as = fp8 ? c.take(R * (blk ? I / 128 : 1) * 4) : -1;
    }
    o->out_perm = c.take(R * D * (fp8 ? 2 : 4));
    o->scratch = c.take(static_cast<int64_t>(permute_scratch_bytes(T, static_cast<int>(k), L->n_shared,
                                                                    static_cast<int>(E))));
    // the router weight prepared for the fused router kernel (layers that
    // carry a router weight and that kernel can take)
    o->router = L->router_w && router_front_ok(L->E, L->D) ? c.take(router_front_scratch_bytes(L->E, L->D)) : -1;
    o->total = c.off;
    o->max_rows = R;
    o->block_m = B;
}

}  // namespace

extern "C" {

const char* moe_status_str(int32_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or mode";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int32_t moe_router_logits(const void* x_bf16, const float* router_w, int32_t T, int32_t D, int32_t E,
                          float* logits, void* stream) {
    MOE_CHECK_ARG(T >= 0 && D > 0 && E > 0);
    MOE_CHECK_SUP(D <= MOE_MAX_ROUTER_D);
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(x_bf16 && router_w && logits);
    return router_logits_launch(static_cast<const uint16_t*>(x_bf16), router_w, T, D, E, logits,
                                as_stream(stream));
}

int32_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t scoring, int32_t n_groups,
                       int32_t topk_groups, const float* sel_bias, int32_t renormalize, float route_scale,
                       int32_t* topk_ids, float* topk_w, void* stream) {
    MOE_CHECK_ARG(T >= 0);
    const int32_t st = check_routing(E, k, scoring, n_groups, topk_groups);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(logits && topk_ids && topk_w);
    return route_topk_launch(logits, T, E, k, scoring, n_groups, topk_groups, sel_bias, renormalize, route_scale,
                             topk_ids, topk_w, as_stream(stream));
}

size_t moe_router_front_workspace_size(const moe_layer_desc* L) {
    if (check_layer(L) != MOE_OK || !router_front_ok(L->E, L->D)) return 0;
    return static_cast<size_t>(router_front_scratch_bytes(L->E, L->D));
}

int32_t moe_router_front(const moe_layer_desc* L, const void* x_bf16, int32_t T, float* logits,
                         int32_t* topk_ids, float* topk_w, uint8_t* xq, float* xs, void* workspace,
                         size_t workspace_bytes, void* stream) {
    int32_t st = check_layer(L);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(T >= 0 && L->router_w != nullptr);
    MOE_CHECK_SUP(router_front_ok(L->E, L->D));
    if (T == 0) return MOE_OK;
    const bool fp8 = L->quant != MOE_QUANT_NONE_BF16;
    MOE_CHECK_ARG(x_bf16 && logits && topk_ids && topk_w && workspace);
    MOE_CHECK_ARG(reinterpret_cast<uintptr_t>(workspace) % 16 == 0);
    if (fp8) MOE_CHECK_ARG(xq && xs);
    if (static_cast<int64_t>(workspace_bytes) < router_front_scratch_bytes(L->E, L->D)) return MOE_ERR_WORKSPACE;
    return router_front_launch(L, x_bf16, T, act_group(L), logits, topk_ids, topk_w, fp8 ? xq : nullptr,
                               fp8 ? xs : nullptr, workspace, as_stream(stream));
}

int64_t moe_permute_max_rows(int32_t T, int32_t k, int32_t E, int32_t n_shared, int32_t block_m) {
    if (T < 0 || k <= 0 || E <= 0 || n_shared < 0 || n_shared > 1 || block_m <= 0) return -1;
    return max_rows_of(T, k, E, n_shared, block_m);
}

size_t moe_permute_scratch_bytes(int32_t T, int32_t k, int32_t n_shared, int32_t E) {
    if (T < 0 || k <= 0 || E <= 0 || n_shared < 0 || n_shared > 1) return 0;
    return permute_scratch_bytes(T, k, n_shared, E);
}

int32_t moe_permute_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t n_shared,
                          int32_t block_m, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_ids,
                          int32_t* block_expert, int32_t* inv_perm, void* scratch, void* stream) {
    MOE_CHECK_ARG(T >= 0 && k > 0 && E > 0 && (n_shared == 0 || n_shared == 1));
    MOE_CHECK_ARG(block_m >= 1 && block_m <= 1024);
    MOE_CHECK_SUP(E + n_shared <= MOE_MAX_EXPERTS);
    const int64_t R = max_rows_of(T, k, E, n_shared, block_m);
    MOE_CHECK_SUP(static_cast<int64_t>(T) * (k + n_shared) < (1LL << 30) && R < (1LL << 30));
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(topk_ids && expert_counts && expert_offsets && sorted_ids && block_expert && inv_perm && scratch);
    return permute_align_launch(topk_ids, T, k, E, n_shared, block_m, static_cast<int>(R), expert_counts,
                                expert_offsets, sorted_ids, block_expert, inv_perm, scratch, as_stream(stream));
}

int32_t moe_quant_ptpc_fp8(const void* x_bf16, int64_t M, int32_t K, int32_t group, const int32_t* valid_rows,
                           uint8_t* q, float* scale, void* stream) {
    MOE_CHECK_ARG(M >= 0 && K > 0 && (group == 0 || group == 128));
    MOE_CHECK_SUP(K % 8 == 0 && K <= 16384 && (group == 0 || K % 128 == 0));
    MOE_CHECK_SUP(M < (1LL << 31) * 4);
    if (M == 0) return MOE_OK;
    MOE_CHECK_ARG(x_bf16 && q && scale);
    return quant_rows_launch(static_cast<const uint16_t*>(x_bf16), M, K, group, valid_rows, q, scale,
                             as_stream(stream));
}

int32_t moe_quant_mxfp4(const void* x_bf16, int64_t M, int32_t K, const int32_t* valid_rows, uint8_t* q,
                        uint8_t* scale, void* stream) {
    MOE_CHECK_ARG(M >= 0 && K > 0);
    MOE_CHECK_SUP(K % 128 == 0 && K <= 65536);
    MOE_CHECK_SUP(M < (1LL << 31) * 4);
    if (M == 0) return MOE_OK;
    MOE_CHECK_ARG(x_bf16 && q && scale);
    return quant_mx_rows_launch(static_cast<const uint16_t*>(x_bf16), M, K, valid_rows, false, nullptr, 0, q, scale,
                                as_stream(stream));
}

int32_t moe_quant_weight_mxfp4(const void* w_bf16, int64_t n_mats, int32_t N, int32_t K, int32_t layout, uint8_t* q,
                               uint8_t* scale, void* stream) {
    MOE_CHECK_ARG(n_mats >= 0 && N > 0 && K > 0);
    MOE_CHECK_ARG(layout == MOE_WEIGHTS_ROWS || layout == MOE_WEIGHTS_BLOCKED);
    MOE_CHECK_SUP(K % 128 == 0 && K <= 65536);
    const bool blocked = layout == MOE_WEIGHTS_BLOCKED;
    if (blocked) MOE_CHECK_SUP(N % 16 == 0 && K % 256 == 0);
    if (n_mats == 0) return MOE_OK;
    MOE_CHECK_ARG(w_bf16 && q && scale);
    return quant_mx_rows_launch(static_cast<const uint16_t*>(w_bf16), n_mats * N, K, nullptr, blocked, nullptr, 0, q,
                                scale, as_stream(stream));
}

int32_t moe_quant_weight_fp8(const void* w_bf16, int64_t n_mats, int32_t N, int32_t K, int32_t quant,
                             int32_t layout, uint8_t* q, float* scale, void* stream) {
    MOE_CHECK_ARG(n_mats >= 0 && N > 0 && K > 0);
    MOE_CHECK_ARG(quant == MOE_QUANT_PTPC_FP8 || quant == MOE_QUANT_BLOCK128_FP8);
    MOE_CHECK_ARG(layout == MOE_WEIGHTS_ROWS || layout == MOE_WEIGHTS_BLOCKED);
    const bool blocked = layout == MOE_WEIGHTS_BLOCKED;
    if (blocked) MOE_CHECK_SUP(N % 16 == 0 && K % 128 == 0);
    if (n_mats == 0) return MOE_OK;
    MOE_CHECK_ARG(w_bf16 && q && scale);
    if (quant == MOE_QUANT_PTPC_FP8) {
        MOE_CHECK_SUP(K % 8 == 0 && K <= 16384);
        return quant_wrows_launch(static_cast<const uint16_t*>(w_bf16), n_mats * N, K, blocked, q, scale,
                                  as_stream(stream));
    }
    MOE_CHECK_SUP(N % 128 == 0 && K % 128 == 0);
    MOE_CHECK_SUP(n_mats * (N / 128) * (K / 128) < (1LL << 31));
    return quant_wblock_launch(static_cast<const uint16_t*>(w_bf16), n_mats, N, K, blocked, q, scale,
                               as_stream(stream));
}

int32_t moe_grouped_gemm_gateup_silu(const moe_layer_desc* L, const void* a, const float* a_scale, int32_t T,
                                     int32_t block_m, const int32_t* sorted_ids, const int32_t* block_expert,
                                     const int32_t* expert_offsets, const int32_t* expert_counts, void* act_bf16,
                                     void* stream) {
    int32_t st = check_layer(L);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(T >= 0);
    MOE_CHECK_SUP(block_m_ok_for(L, block_m));
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(a && sorted_ids && block_expert && expert_offsets && act_bf16);
    MOE_CHECK_ARG(L->quant == MOE_QUANT_NONE_BF16 || a_scale);
    const int64_t R = max_rows_of(T, L->top_k, L->E, L->n_shared, block_m);
    MOE_CHECK_SUP(gemm_ranges_ok(L, T, block_m, R));
    return gemm_gateup_launch(L, a, a_scale, T, block_m, R, sorted_ids, block_expert, expert_offsets, expert_counts,
                              act_bf16,
                              as_stream(stream));
}

int32_t moe_grouped_gemm_down(const moe_layer_desc* L, const void* act, const float* act_scale, int32_t T,
                              int32_t block_m, const int32_t* block_expert, const int32_t* expert_offsets,
                              const int32_t* expert_counts, void* out_perm, void* stream) {
    int32_t st = check_layer(L);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(T >= 0);
    MOE_CHECK_SUP(block_m_ok_for(L, block_m));
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(act && block_expert && expert_offsets && out_perm);
    MOE_CHECK_ARG(L->quant == MOE_QUANT_NONE_BF16 || act_scale);
    const int64_t R = max_rows_of(T, L->top_k, L->E, L->n_shared, block_m);
    MOE_CHECK_SUP(gemm_ranges_ok(L, T, block_m, R));
    return gemm_down_launch(L, act, act_scale, T, block_m, R, block_expert, expert_offsets, expert_counts, out_perm,
                            as_stream(stream));
}

int32_t moe_unpermute_combine(const void* out_perm, int32_t out_dtype, const int32_t* inv_perm,
                              const float* topk_w, int32_t T, int32_t k, int32_t n_shared, int32_t D,
                              void* y_bf16, void* stream) {
    MOE_CHECK_ARG(T >= 0 && k > 0 && D > 0 && (n_shared == 0 || n_shared == 1));
    MOE_CHECK_ARG(out_dtype == 0 || out_dtype == 1);
    MOE_CHECK_SUP(D % 8 == 0);
    MOE_CHECK_SUP(k + n_shared <= MOE_MAX_TOPK + 1);   // rows a token gathers: the widest kernel instance has 17 row slots
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(out_perm && inv_perm && topk_w && y_bf16);
    return combine_launch(out_perm, out_dtype, inv_perm, topk_w, T, k, n_shared, D, static_cast<uint16_t*>(y_bf16),
                          as_stream(stream));
}

int32_t moe_default_block_m(const moe_layer_desc* L, int32_t T) {
    if (!L || L->E <= 0 || T < 0) return 64;
    const int64_t rows = static_cast<int64_t>(T) * (L->top_k + L->n_shared);
    const int64_t per_expert = rows / (L->E + L->n_shared);
    // small batches stream the weights in every mode (MXFP4 on the Qwen3-235B
    // decode shape, T = 16 / 32 / 48 / 64: 100 / 126 / 158 / 160 us with
    // 32-row tiles, 90 / 115 / 135 / 145 us streaming)
    if (T <= kStreamMaxT) return 16;
    // A few dozen rows per expert: the weight-streaming kernels (every
    // active expert's weights read once per 64 of its rows) beat 32-row
    // tiles (the Qwen3-30B-A3B-shaped batch, 16 rows per expert:
    // 0.163 -> 0.158 ms).
    if (L->quant != MOE_QUANT_MXFP4 && per_expert <= 24) return 16;
    // 32-row tiles of pads are skipped, so a tall tile costs little beyond
    // the expert's rows and reads each weight tile once per 256 rows; an
    // expert of fewer than ~224 rows fits one 192-row tile with less idle
    // MFMA work per streamed weight byte (the DeepSeek-R1-shaped layer:
    // 3.19 -> 3.03 ms).  MXFP4 keeps the 128-row tile (its taller tiles
    // exceed the register budget).
    if (L->quant == MOE_QUANT_MXFP4 && per_expert >= 48) return 128;
    if (per_expert >= 96) return L->quant != MOE_QUANT_NONE_BF16 && per_expert < 224 ? 192 : 256;
    if (per_expert >= 48) return 128;
    return 32;
}

size_t moe_forward_workspace_size(const moe_layer_desc* L, int32_t T, int32_t block_m) {
    if (check_layer(L) != MOE_OK || T < 0) return 0;
    if (block_m == 0) block_m = moe_default_block_m(L, T);
    if (!block_m_ok_for(L, block_m)) return 0;
    moe_ws_layout o;
    layout_of(L, T, block_m, &o);
    if (!gemm_ranges_ok(L, T, block_m, o.max_rows)) return 0;
    return static_cast<size_t>(o.total);
}

int32_t moe_workspace_layout(const moe_layer_desc* L, int32_t T, int32_t block_m, moe_ws_layout* out) {
    int32_t st = check_layer(L);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(T >= 0 && out);
    if (block_m == 0) block_m = moe_default_block_m(L, T);
    MOE_CHECK_SUP(block_m_ok_for(L, block_m));
    layout_of(L, T, block_m, out);
    MOE_CHECK_SUP(gemm_ranges_ok(L, T, block_m, out->max_rows));
    return MOE_OK;
}

int32_t moe_forward(const moe_layer_desc* L, const void* x_bf16, const float* logits_or_null, int32_t T,
                    int32_t block_m, void* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
    int32_t st = check_layer(L);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(T >= 0);
    if (block_m == 0) block_m = moe_default_block_m(L, T);
    MOE_CHECK_SUP(block_m_ok_for(L, block_m));
    const int64_t A = static_cast<int64_t>(T) * (L->top_k + L->n_shared);
    MOE_CHECK_SUP(A < (1LL << 30));
    if (T == 0) return MOE_OK;
    if (!logits_or_null) {
        MOE_CHECK_ARG(L->router_w != nullptr);
        MOE_CHECK_SUP(L->D <= MOE_MAX_ROUTER_D);
    }
    MOE_CHECK_ARG(x_bf16 && y_bf16 && workspace);
    MOE_CHECK_ARG(reinterpret_cast<uintptr_t>(workspace) % kAlign == 0);
    moe_ws_layout o;
    layout_of(L, T, block_m, &o);
    MOE_CHECK_SUP(gemm_ranges_ok(L, T, block_m, o.max_rows));
    if (static_cast<int64_t>(workspace_bytes) < o.total) return MOE_ERR_WORKSPACE;

    hipStream_t s = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    auto at = [&](int64_t off) { return static_cast<void*>(ws + off); };
    const int k = L->top_k, E = L->E, Ep = E + L->n_shared;
    const bool fp8 = L->quant != MOE_QUANT_NONE_BF16;     // any quantized mode (FP8 or MXFP4)
    const int group = act_group(L);

    // Without logits: batches that take the small-batch front end run the
    // per-token fp64 router projection first; larger ones route in the fused
    // router kernel (projection on the matrix cores, top-k and x
    // quantization in the same launch).
    const bool small_front = block_m == 16 && front_small_ok(T, k, L->n_shared);
    // the weight-streaming gate/up GEMM builds the permutation itself
    const bool perm_in_gemm = block_m == 16 && stream_fused_perm_ok(T);
    const bool fused_router = !logits_or_null && !small_front && router_front_ok(E, L->D);
    float* lg = static_cast<float*>(at(o.logits));
    const float* logits = logits_or_null;
    if (!logits && !fused_router) {
        if ((st = router_logits_launch(static_cast<const uint16_t*>(x_bf16), L->router_w, T, L->D, E, lg, s)) != MOE_OK)
            return st;
        logits = lg;
    }
    int* ids = static_cast<int*>(at(o.topk_ids));
    float* w = static_cast<float*>(at(o.topk_w));
    int* offsets = static_cast<int*>(at(o.offsets));
    int* sorted = static_cast<int*>(at(o.sorted_ids));
    int* bexp = static_cast<int*>(at(o.block_expert));
    int* inv = static_cast<int*>(at(o.inv_perm));
    const void* a = fp8 ? at(o.xq) : x_bf16;
    const float* a_scale = fp8 ? static_cast<float*>(at(o.xs)) : nullptr;
    {
        // routing and x quantization in one launch (with the router
        // projection when there are no logits), then the permutation: inside
        // the weight-streaming gate/up GEMM up to 256 tokens, else one
        // workgroup up to 256 tokens (the routing's picks are distinct per
        // token), else the multi-kernel one
        uint8_t* xq = fp8 ? static_cast<uint8_t*>(at(o.xq)) : nullptr;
        float* xs = fp8 ? static_cast<float*>(at(o.xs)) : nullptr;
        if (fused_router) {
            if ((st = router_front_launch(L, x_bf16, T, group, lg, ids, w, xq, xs, at(o.router), s)) != MOE_OK)
                return st;
        } else if ((st = front_route_quant_launch(L, x_bf16, logits, T, ids, w, xq, xs, s)) != MOE_OK) {
            return st;
        }
        if (perm_in_gemm)
            st = MOE_OK;
        else if (permute_small_ok(T, k, L->n_shared))
            st = permute_small_launch(ids, T, k, E, L->n_shared, block_m, static_cast<int>(o.max_rows),
                                      static_cast<int*>(at(o.counts)), offsets, sorted, bexp, inv, s);
        else
            st = permute_align_launch(ids, T, k, E, L->n_shared, block_m, static_cast<int>(o.max_rows),
                                      static_cast<int*>(at(o.counts)), offsets, sorted, bexp, inv, at(o.scratch), s);
        if (st != MOE_OK) return st;
    }
    void* act = at(o.act);
    int* counts = static_cast<int*>(at(o.counts));
    if (perm_in_gemm)
        st = stream_gateup_fused_launch(L, a, a_scale, T, ids, static_cast<int>(o.max_rows),
                                        PermOut{counts, offsets, sorted, bexp, inv}, act, s);
    else
        st = gemm_gateup_launch(L, a, a_scale, T, block_m, o.max_rows, sorted, bexp, offsets, counts, act, s);
    if (st != MOE_OK) return st;
    const void* act_in = act;
    const float* act_scale = nullptr;
    // the streaming down GEMM reads act codes stored in 16-row x 128-byte
    // blocks (whole lines per load, as for the weights); max_rows is a
    // multiple of 16 there.  The tiled down GEMM never reads a pad row's
    // codes or scale (it is given the expert counts), so pad rows are not
    // quantized for it.
    const bool aq_blocked = fp8 && block_m == 16;
    if (fp8) {
        if (group == 32) {
            st = quant_mx_rows_launch(static_cast<const uint16_t*>(act), o.max_rows, L->I, offsets + Ep, aq_blocked,
                                      block_m == 16 ? nullptr : sorted, T * (k + L->n_shared),
                                      static_cast<uint8_t*>(at(o.aq)), static_cast<uint8_t*>(at(o.as)), s);
        } else {
            st = quant_rows_launch(static_cast<const uint16_t*>(act), o.max_rows, L->I, group, offsets + Ep,
                                   static_cast<uint8_t*>(at(o.aq)), static_cast<float*>(at(o.as)), s, aq_blocked,
                                   block_m == 16 ? nullptr : sorted, T * (k + L->n_shared));
        }
        if (st != MOE_OK) return st;
        act_in = at(o.aq);
        act_scale = static_cast<float*>(at(o.as));
    }
    void* outp = at(o.out_perm);
    if ((st = gemm_down_launch(L, act_in, act_scale, T, block_m, o.max_rows, bexp, offsets, counts, outp, s,
                               aq_blocked)) != MOE_OK)
        return st;
    return combine_launch(outp, fp8 ? 1 : 0, inv, w, T, k, L->n_shared, L->D, static_cast<uint16_t*>(y_bf16), s);
}

}  // extern "C"

// Workspace of moe_forward_noalloc: device memory the library owns for the
// life of the process, one copy per GPU (the loader places the array on every
// device the code object is loaded on).  In host code `scratch` names only
// the host-side stand-in of the array; its device address comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array (the current device: the
// one the caller's stream belongs to).
int32_t scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return MOE_ERR_HIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}
}  // namespace

extern "C" {

int32_t moe_forward_noalloc(const moe_layer_desc* L, const void* x_bf16, const float* logits_or_null, int32_t T,
                            int32_t block_m, void* y_bf16, void* stream) {
    int32_t st = check_layer(L);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(T >= 0);
    if (T == 0) return MOE_OK;
    const size_t need = moe_forward_workspace_size(L, T, block_m);
    if (need > static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
    // need == 0 (a block_m or shape the kernels do not cover): moe_forward
    // reports it before launching anything
    return moe_forward(L, x_bf16, logits_or_null, T, block_m, y_bf16, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int64_t moe_ep_payload_bytes(int32_t D, int32_t format) {
    if (D <= 0 || D % 128 || D > 65536) return -1;
    return ep_payload_row_bytes(D, format);
}

int32_t moe_ep_pack_payload(const void* x_bf16, int32_t T, int32_t D, int32_t format, uint8_t* payload,
                            void* stream) {
    MOE_CHECK_ARG(T >= 0);
    MOE_CHECK_SUP(moe_ep_payload_bytes(D, format) > 0);
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(x_bf16 && payload);
    return ep_pack_launch(static_cast<const uint16_t*>(x_bf16), T, D, format, payload, as_stream(stream));
}

int32_t moe_ep_unpack_payload(const uint8_t* payload, int32_t T, int32_t D, int32_t format, void* x_bf16,
                              void* stream) {
    MOE_CHECK_ARG(T >= 0);
    MOE_CHECK_SUP(moe_ep_payload_bytes(D, format) > 0);
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(x_bf16 && payload);
    return ep_unpack_launch(payload, T, D, format, static_cast<uint16_t*>(x_bf16), as_stream(stream));
}

}  // extern "C"

/*
 * moe.h -- C ABI of the fused Mixture-of-Experts layer forward for one
 * AMD Instinct MI355X (gfx950) that holds every expert.
 *
 * The layer (pages it follows):
 *   - "Systems engineering playbook: optimizing Qwen 3.5 397B MoE on Ironwood
 *     TPU7x" (Google Developers Blog): a router gate scores each token against
 *     the routed experts and keeps the top-k of a soft-max distribution, plus
 *     one always-executed shared expert (model description, MoE paragraph);
 *     routing metadata is a [tokens, k] array of expert ids and one of top-k
 *     weights (expert-parallel routing item); token rows are gathered into a
 *     contiguous per-expert buffer (SparseCore permutation item); a grouped
 *     GEMM packs gate and up projections in one tile with SwiGLU fused and
 *     processes each expert's variable token count in bounded slices (GMM V2
 *     item); expert outputs are gathered back and reduced per token
 *     (SparseCore unpermutation item).
 *   - "Unleashing Computational Power: Ultimate Latency Optimization of Qwen3
 *     and Qwen3-VL on AMD MI300X Series" (LMSYS blog), 2.1.1 "GEMM
 *     Quantization Strategy", Figure 3: PTPC-FP8, a dynamic scale per token
 *     for activations and a static scale per output channel for weights.
 *   - "Win on TCO: How AMD Instinct MI355X Achieves Cost-Competitive
 *     Distributed Inference Through SGLang with MoRI", "Hybrid FP4/FP8
 *     quantized all-to-all": FP8 blockwise quantization with one fp32 scale
 *     per 128 elements (used here for 1x128 activation groups and 128x128
 *     weight blocks of the DeepSeek-R1-shaped layer, hidden 7168, top-8).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless stated; the caller allocates and
 *     owns every buffer and keeps it alive until the stream work completes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued asynchronously on it; no entry point allocates,
 *     frees, synchronizes, or reads device memory from the host, so every
 *     call can be captured in a HIP graph.
 *   - Matrices are row-major.  GEMM operands are "NT": both the activation
 *     rows and the weight rows are contiguous along the reduction dimension.
 *   - bf16 data is passed as uint16 bit patterns (void*), FP8 as OCP e4m3fn
 *     codes (uint8).  e4m3fn conversion rounds to nearest even, keeps
 *     subnormals and the sign of zero, and saturates to +-448.
 *   - Return value: a moe_status code.  Arguments are validated on the host
 *     before anything is enqueued: an invalid call enqueues nothing.
 *     MOE_ERR_HIP reports a launch failure (hipGetLastError after launch).
 *     T = 0 (no tokens) is valid and enqueues nothing.
 *   - The only state the library keeps between calls is a per-device cache of
 *     how many workgroups of the weight-streaming kernels fit on the device
 *     at once (filled on first use, read-only afterwards) and the per-device
 *     scratch array of moe_forward_noalloc.  Entry points are thread-safe;
 *     calls that share buffers must be ordered by the caller.
 */
#ifndef MOE_LAYER_ROUTER_AMD_MOE_H
#define MOE_LAYER_ROUTER_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG  1  /* NULL pointer, non-positive size, k > E ... */
#define MOE_ERR_UNSUPPORTED  2  /* valid but outside what the kernels cover  */
#define MOE_ERR_WORKSPACE    3  /* workspace smaller than required          */
#define MOE_ERR_HIP          4  /* a HIP launch reported an error            */

/* router scoring */
#define MOE_SCORING_SOFTMAX          0  /* soft-max over the logits, top-k        */
#define MOE_SCORING_SIGMOID_GROUPED  1  /* sigmoid, group-limited top-k           */

/* expert arithmetic */
#define MOE_QUANT_NONE_BF16     0  /* bf16 operands, fp32 accumulate            */
#define MOE_QUANT_PTPC_FP8      1  /* e4m3 per-token x per-output-channel       */
#define MOE_QUANT_BLOCK128_FP8  2  /* e4m3 1x128 activations, 128x128 weights   */
#define MOE_QUANT_MXFP4         3  /* E2M1 + E8M0 per 32 along K, both operands  */

/* weight_layout (moe_layer_desc) / layout (moe_quant_weight_fp8) */
#define MOE_WEIGHTS_ROWS        0  /* row-major                                 */
#define MOE_WEIGHTS_BLOCKED     1  /* 16 rows x 128 bytes per contiguous block  */

/* expert-parallel payload formats (moe_ep_payload_bytes / pack / unpack) */
#define MOE_PAYLOAD_MXFP4       0  /* dispatch: FP4 E2M1 + E8M0 per 32          */
#define MOE_PAYLOAD_FP8_BLOCK   1  /* combine: e4m3fn + fp32 scale per 128      */

/* Limits of the library (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS   1024  /* E + n_shared                                 */
#define MOE_MAX_TOPK        16
#define MOE_MAX_GROUPS      32
#define MOE_MAX_ROUTER_D 16384  /* D of the router projection                  */

/*
 * Layer description (a host struct; its pointers are device pointers).
 *   D hidden size, I expert intermediate size, E routed experts, top_k,
 *   n_shared in {0,1}: the shared expert is expert index E, applied to every
 *   token with weight 1 (not scaled by route_scale).
 *   w13: [E+n_shared, 2I, D] -- rows 0..I-1 the gate projection, rows I..2I-1
 *        the up projection of each expert; bf16 (quant 0) or e4m3 codes;
 *        quant 3: E2M1 codes, two per byte ([E+n_shared, 2I, D/2] bytes,
 *        element 2i of a row in the low nibble of byte i).
 *   w13_scale: quant 1: [E+n_shared, 2I] fp32 per output channel;
 *              quant 2: [E+n_shared, 2I/128, D/128] fp32 per 128x128 block;
 *              quant 3: [E+n_shared, 2I, D/32] E8M0 bytes (a uint8 array
 *              passed through this pointer), one per 32 elements of a row;
 *              quant 0: NULL.
 *   w2: [E+n_shared, D, I]; w2_scale: [E+n_shared, D] or [.., D/128, I/128]
 *        (quant 3: codes [E+n_shared, D, I/2] bytes, scales [.., D, I/32]).
 *   MXFP4 (quant 3, the A4W4 FusedMoE of the MI355X MoRI page, OCP
 *   Microscaling v1.0): activations, weights and the re-quantized act are
 *   all E2M1 with an E8M0 scale 2^e per 32 elements along the reduction
 *   dimension, e = floor(log2(amax)) - 2 clamped to [-127, 127]; the matrix
 *   cores apply both scales.  I % 256 == 0; block_m 16 (weight streaming,
 *   the default up to 64 tokens), 32, 64, 128 or 192 (the LDS-tiled
 *   kernels).
 *   weight_layout: order of the bytes of each [N, K] weight matrix (w13:
 *              N = 2I, K = D; w2: N = D, K = I; K_bytes = K, or K/2 for MXFP4):
 *              MOE_WEIGHTS_ROWS    row-major, K contiguous;
 *              MOE_WEIGHTS_BLOCKED blocks of 16 rows x 128 bytes (the unit
 *              the expert GEMMs read per step), the byte (n, b) of a row at
 *              ((n/16) * (K_bytes/128) + b/128) * 2048 + o(n%16, b%128)
 *              with o(r, c) = (r/2 + 8 * (c/64)) * 128 +
 *              ((r%2) * 4 + (c%64)/16) * 16 + c%16: each 128-byte line of
 *              a block holds one 64-byte K half of two consecutive rows.
 *              Quantized modes only (N % 16 == 0, K_bytes % 128 == 0);
 *              moe_quant_weight_fp8 / moe_quant_weight_mxfp4 write it.
 *   router_w: [E, D] fp32 router gate, used by moe_forward when it is given
 *             no logits (may be NULL otherwise).
 *   sel_bias: [E] fp32 selection-only bias of grouped-sigmoid routing or NULL.
 */
typedef struct moe_layer_desc {
    int32_t D, I, E, top_k, n_shared;
    int32_t scoring, n_groups, topk_groups, renormalize;
    float route_scale;
    int32_t quant;
    int32_t weight_layout;
    const void* w13;
    const float* w13_scale;
    const void* w2;
    const float* w2_scale;
    const float* router_w;
    const float* sel_bias;
} moe_layer_desc;

/* Byte offsets of the intermediates moe_forward keeps in its workspace
 * (host struct; -1 when a buffer is not used by the layer's mode). */
typedef struct moe_ws_layout {
    int64_t logits, topk_ids, topk_w, counts, offsets, sorted_ids, block_expert,
            inv_perm, xq, xs, act, aq, as, out_perm, scratch, router, total;
    int64_t max_rows;   /* moe_permute_max_rows of the layer                 */
    int32_t block_m;    /* the block_m the layout was computed for            */
} moe_ws_layout;

/* Text of a status code (static string, never NULL). */
const char* moe_status_str(int32_t status);

/*
 * Router projection: logits[t, e] = sum_d x[t, d] * router_w[e, d]
 * (router gate of the Qwen 3.5 MoE paragraph).  x: [T, D] bf16,
 * router_w: [E, D] fp32, logits: [T, E] fp32.  Products and sums are formed
 * in fp64 and rounded once to fp32.  D <= MOE_MAX_ROUTER_D.
 */
int32_t moe_router_logits(const void* x_bf16, const float* router_w, int32_t T, int32_t D,
                          int32_t E, float* logits, void* stream);

/*
 * Top-k routing (router gate + top-k of the Qwen 3.5 MoE paragraph; the
 * grouped-sigmoid form is the DeepSeek-R1 layer's).  logits: [T, E] fp32,
 * finite.  Outputs topk_ids [T, k] int32 and topk_w [T, k] fp32, each row in
 * descending key order, ties to the lower expert index (+0 == -0).
 *   scoring 0: key = logit.  renormalize != 0: w = soft-max over the k
 *     selected logits; else w = the full soft-max probability.  n_groups,
 *     topk_groups, sel_bias, route_scale are ignored (pass 1, 1, NULL, 1).
 *   scoring 1: s = sigmoid(logit) (fp32); key = s + sel_bias[e] (NULL = 0);
 *     group score = sum of the two largest keys of each of n_groups equal
 *     groups; only the topk_groups best groups are eligible (ties to the
 *     lower group); w = s / sum(s of the picks) * route_scale (renormalize)
 *     or s * route_scale.
 * Weights are formed in fp64 and rounded once to fp32.
 * Limits: 1 <= k <= MOE_MAX_TOPK, k <= E <= MOE_MAX_EXPERTS, E % n_groups ==
 * 0, n_groups <= MOE_MAX_GROUPS, 1 <= topk_groups <= n_groups, and k not
 * above the experts of the eligible groups.
 */
int32_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t scoring,
                       int32_t n_groups, int32_t topk_groups, const float* sel_bias,
                       int32_t renormalize, float route_scale, int32_t* topk_ids, float* topk_w,
                       void* stream);

/*
 * Router projection fused with top-k routing and the FP8 quantization of x,
 * in one launch (router gate of the Qwen 3.5 MoE paragraph; the page's
 * roadmap item puts the top-k selection where the scores are computed).
 * For the layer L (L->router_w required; E <= 512, D % 256 == 0, else
 * MOE_ERR_UNSUPPORTED) and x [T, D] bf16:
 *   logits [T, E] fp32: x . router_w on the matrix cores; each fp32 weight
 *     is split exactly into three bf16 pieces, so the products are exact and
 *     only fp32 accumulation rounds (|error| within 1e-6 of sum_d
 *     |x[t, d] * router_w[e, d]|, far tighter in practice);
 *   topk_ids, topk_w [T, k]: moe_route_topk of those logits (bit for bit);
 *   FP8 layers: xq [T, D] codes and xs [T] or [T, D/128] scales, as
 *     moe_quant_ptpc_fp8 (xq, xs may be NULL for a bf16 layer).
 * moe_forward uses it when it is given no logits and T is above the
 * small-batch sizes (those project in fp64 per token, moe_router_logits).
 * workspace: device memory of moe_router_front_workspace_size(L) bytes,
 * 16-byte aligned, for the router weight split into its three pieces in the
 * kernel's load order (rewritten by every call; MOE_ERR_WORKSPACE if
 * smaller).
 */
size_t moe_router_front_workspace_size(const moe_layer_desc* L);
int32_t moe_router_front(const moe_layer_desc* L, const void* x_bf16, int32_t T, float* logits,
                         int32_t* topk_ids, float* topk_w, uint8_t* xq, float* xs, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Host-only: rows of the padded permuted buffer, an upper bound valid for any
 * routing: block_m * min(floor((A' + E'(block_m-1)) / block_m), A') with
 * A' = T(k + n_shared), E' = E + n_shared.  Returns -1 on invalid input.
 */
int64_t moe_permute_max_rows(int32_t T, int32_t k, int32_t E, int32_t n_shared, int32_t block_m);

/*
 * Stable permutation of the routed rows by expert (SparseCore permutation and
 * GMM V2 bounded slices of the Qwen 3.5 page).  Routed row (t, j) has flat
 * index t*k + j; with n_shared = 1 the shared-expert rows are expert E with
 * flat index T*k + t.  Within an expert rows keep ascending flat order; each
 * expert's segment is padded to a multiple of block_m with the sentinel
 * T*(k + n_shared).
 * Outputs (sizes with E' = E + n_shared, R = moe_permute_max_rows(...)):
 *   expert_counts [E'], expert_offsets [E'+1] (padded exclusive prefix; the
 *   last entry is the padded total), sorted_ids [R] (flat indices; sentinel
 *   in pads and past the total), block_expert [R / block_m] (expert of each
 *   block, -1 past the total), inv_perm [T*(k+n_shared)] (flat -> row).
 * Ids outside [0, E) get no row (inv_perm = -1).  block_m in [1, 1024].
 * `scratch` is device memory of moe_permute_scratch_bytes(T, k, n_shared, E)
 * bytes (contents need not be initialised).
 */
size_t moe_permute_scratch_bytes(int32_t T, int32_t k, int32_t n_shared, int32_t E);
int32_t moe_permute_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                          int32_t n_shared, int32_t block_m, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* sorted_ids, int32_t* block_expert,
                          int32_t* inv_perm, void* scratch, void* stream);

/*
 * PTPC / 1x128 FP8 quantization of bf16 rows (PTPC-FP8 of the Qwen3 MI300X
 * page, 2.1.1; the 1x128 blockwise form of the MI355X MoRI page).
 * x: [M, K] bf16.  group 0: one scale per row; group 128: one scale per 128
 * consecutive elements (K % 128 == 0).  For each group:
 *   amax = max|x|; scale = amax / 448; q = e4m3(x * (448 / amax)),
 * both divisions IEEE fp32, one fp32 multiply; amax = 0 gives scale 1.
 * Outputs q [M, K] uint8 and scale [M] or [M, K/128] fp32.
 * valid_rows: device int32 scalar or NULL; rows >= *valid_rows are left
 * untouched (used for the data-dependent row count of the permuted buffer).
 * Limits: K % 8 == 0, K <= 16384.
 */
int32_t moe_quant_ptpc_fp8(const void* x_bf16, int64_t M, int32_t K, int32_t group,
                           const int32_t* valid_rows, uint8_t* q, float* scale, void* stream);

/*
 * MXFP4 quantization of bf16 rows (OCP Microscaling v1.0; the A4W4 expert
 * arithmetic of the MI355X MoRI page, "FlyDSL FusedMoE").  x: [M, K] bf16,
 * K % 128 == 0, K <= 65536.  Per block of 32 consecutive elements of a row:
 * amax = max|x|, e = floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for
 * an all-zero block), scale byte e + 127, codes = E2M1 of x / 2^e (exact
 * division) rounded to nearest, ties to the even mantissa, saturating to
 * +-6, sign of zero kept.  Outputs q [M, K/2] (element 2i in the low nibble
 * of byte i) and scale [M, K/32] bytes.  valid_rows as in moe_quant_ptpc_fp8.
 */
int32_t moe_quant_mxfp4(const void* x_bf16, int64_t M, int32_t K, const int32_t* valid_rows, uint8_t* q,
                        uint8_t* scale, void* stream);

/*
 * Offline MXFP4 quantization of bf16 weights [n_mats, N, K] along K (the
 * reduction dimension), the arithmetic of moe_quant_mxfp4: codes q
 * [n_mats, N, K/2] bytes (layout MOE_WEIGHTS_ROWS, or MOE_WEIGHTS_BLOCKED on
 * the byte matrix: N % 16 == 0, K % 256 == 0), scale [n_mats, N, K/32] E8M0
 * bytes.
 */
int32_t moe_quant_weight_mxfp4(const void* w_bf16, int64_t n_mats, int32_t N, int32_t K, int32_t layout,
                               uint8_t* q, uint8_t* scale, void* stream);

/*
 * Offline FP8 quantization of bf16 weights [n_mats, N, K] (row n of a matrix
 * is output channel n).  quant 1 (PTPC): one scale per row, scale
 * [n_mats, N]; quant 2: one scale per 128x128 block, scale
 * [n_mats, N/128, K/128] (N, K multiples of 128).  Same arithmetic as
 * moe_quant_ptpc_fp8.  layout: MOE_WEIGHTS_ROWS or MOE_WEIGHTS_BLOCKED
 * (N % 16 == 0, K % 128 == 0) for the codes q; scales are always as above.
 */
int32_t moe_quant_weight_fp8(const void* w_bf16, int64_t n_mats, int32_t N, int32_t K,
                             int32_t quant, int32_t layout, uint8_t* q, float* scale, void* stream);

/*
 * Grouped GEMM gate/up with fused SwiGLU (GMM V2 item of the Qwen 3.5 page).
 * For every valid row r of the permuted buffer, with e = block_expert[r/block_m]
 * and token t of sorted_ids[r] (t = f / k for f < T*k, else f - T*k):
 *   [g | u] = A[t] . W13[e]^T (fp32 accumulate, dequantized by the row's
 *   activation scale and the weight scales), act[r] = bf16(silu(g) * u).
 * a: quant 0: x bf16 [T, D]; quant 1/2: codes [T, D] with a_scale [T] or
 * [T, D/128]; quant 3: codes [T, D/2] with E8M0 bytes [T, D/32] passed as
 * a_scale.  act: [R, I] bf16 where R = moe_permute_max_rows(...).
 * expert_counts (device, [E+n_shared], as moe_permute_align writes it; may
 * be NULL) lets the LDS-tiled kernels skip the 32-row tiles at the end of an
 * expert's segment that hold only pads; it must match expert_offsets.
 * Pad rows (sentinel) get act = 0, except that with expert_counts the pad
 * rows of those pad-only 32-row tiles are not written (the LDS-tiled
 * kernels; their contents are then unspecified); rows at or past
 * expert_offsets[E'] are not written.  block_m must equal the block_m of moe_permute_align and be one
 * of: 16 (weight-streaming kernels for small batches: each weight byte is
 * read once per 64 rows of its expert), 32, 64, 128, 192
 * (FP8 and MXFP4 only) or 256 (not MXFP4) (LDS-tiled kernels).  Shapes: I % 128 == 0 (MXFP4: 256) and D % 256 == 0.
 */
int32_t moe_grouped_gemm_gateup_silu(const moe_layer_desc* L, const void* a,
                                     const float* a_scale, int32_t T, int32_t block_m,
                                     const int32_t* sorted_ids, const int32_t* block_expert,
                                     const int32_t* expert_offsets, const int32_t* expert_counts,
                                     void* act_bf16, void* stream);

/*
 * Grouped GEMM down: out_perm[r] = act[r] . W2[e]^T for the valid rows
 * (dequantized by the row scale(s) and the weight scales).  Same block_m,
 * expert_counts and shape rules as moe_grouped_gemm_gateup_silu.  With
 * expert_counts the pad rows of act are never read and the pad rows of
 * out_perm are 0, or unspecified in pad-only 32-row tiles (as for act); with
 * expert_counts NULL every row of a segment is computed, so pad rows of
 * out_perm are 0 only where the pad rows of act hold zeros.  act: quant 0:
 * bf16 [R, I]; quant 1/2: codes [R, I] with act_scale [R] or [R, I/128];
 * quant 3: codes [R, I/2] with E8M0 bytes [R, I/32] passed as act_scale.
 * out_perm [R, D]: fp32 for quant 0, bf16 for quant 1/2/3.
 */
int32_t moe_grouped_gemm_down(const moe_layer_desc* L, const void* act, const float* act_scale,
                              int32_t T, int32_t block_m, const int32_t* block_expert,
                              const int32_t* expert_offsets, const int32_t* expert_counts,
                              void* out_perm, void* stream);

/*
 * Unpermute and weighted combine (SparseCore unpermutation item of the
 * Qwen 3.5 page): y[t] = bf16( sum_{j<k} w[t,j] * out_perm[inv_perm[t*k+j]]
 * + out_perm[inv_perm[T*k+t]] (shared, when n_shared = 1) ), accumulated in
 * fp32 in that order.  out_dtype 0: out_perm fp32; 1: bf16.  Rows with
 * inv_perm = -1 contribute nothing.  y: [T, D] bf16.  Limits: D % 8 == 0 and
 * k + n_shared <= MOE_MAX_TOPK + 1 (MOE_ERR_UNSUPPORTED otherwise).
 */
int32_t moe_unpermute_combine(const void* out_perm, int32_t out_dtype, const int32_t* inv_perm,
                              const float* topk_w, int32_t T, int32_t k, int32_t n_shared,
                              int32_t D, void* y_bf16, void* stream);

/*
 * block_m that moe_forward uses for block_m = 0 (chosen from T and the layer).
 */
int32_t moe_default_block_m(const moe_layer_desc* L, int32_t T);

/* Workspace bytes of moe_forward and where each intermediate lives in it. */
size_t moe_forward_workspace_size(const moe_layer_desc* L, int32_t T, int32_t block_m);
int32_t moe_workspace_layout(const moe_layer_desc* L, int32_t T, int32_t block_m,
                             moe_ws_layout* out);

/*
 * The whole layer: [router projection when logits == NULL] -> top-k ->
 * permute -> [quantize x] -> gate/up + SwiGLU -> [quantize act] -> down ->
 * combine.  x: [T, D] bf16; logits: [T, E] fp32 or NULL (then L->router_w is
 * required); y: [T, D] bf16.  block_m 0 picks moe_default_block_m.  The
 * workspace (>= moe_forward_workspace_size bytes, 256-byte aligned) holds
 * every intermediate at the offsets of moe_workspace_layout.  Every limit of
 * every kernel of the call (including the 32-bit byte ranges of the
 * LDS-tiled GEMMs: T*D, 2*I*D and max_rows*I elements of FP8 codes or bf16
 * below 4 GiB) is checked before the first launch; moe_forward_workspace_size
 * returns 0 and moe_workspace_layout MOE_ERR_UNSUPPORTED for such shapes.
 */
int32_t moe_forward(const moe_layer_desc* L, const void* x_bf16, const float* logits_or_null,
                    int32_t T, int32_t block_m, void* y_bf16, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as moe_forward; the
 * intermediates live in a device array of MOE_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU until the process ends.  The call allocates
 * nothing (its first call on a device looks up that device's copy of the
 * array).  Returns MOE_ERR_WORKSPACE, enqueueing nothing, when
 * moe_forward_workspace_size(L, T, block_m) exceeds the array (96 MiB: the
 * decode batches of the Qwen3-235B-shaped layer, D 4096, I 1536, 128 experts
 * top-8, up to T = 128, and of the DeepSeek-R1-shaped layer, D 7168, I 2048,
 * 256 + 1 experts top-8, up to T = 64).  Every call on a GPU uses that GPU's one array and
 * leaves its intermediates there: calls that overlap on one GPU (two streams,
 * two threads) race and must be ordered by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (96LL << 20)
int32_t moe_forward_noalloc(const moe_layer_desc* L, const void* x_bf16, const float* logits_or_null,
                            int32_t T, int32_t block_m, void* y_bf16, void* stream);

/*
 * Expert-parallel payloads ("Win on TCO ... MoRI", "Hybrid FP4/FP8 quantized
 * all-to-all": MXFP4 for dispatch, FP8 with one fp32 scale per 128 elements
 * for combine; 28,672 -> 11,200 bytes per token at hidden size 7168).  The
 * exchange between GPUs is not part of this library; these entries build and
 * read the per-token payload rows on one GPU.
 *
 * moe_ep_payload_bytes: host-only; bytes of one payload row for D elements,
 * or -1 when D is not a positive multiple of 128 or the format is unknown.
 *   MOE_PAYLOAD_MXFP4: D/2 bytes of FP4 E2M1 codes (OCP Microscaling v1.0;
 *     element 2i in the low nibble of byte i), then D/32 E8M0 scale bytes,
 *     one per block of 32 elements: exponent e = floor(log2(amax)) - 2
 *     clamped to [-127, 127] (byte e + 127; an all-zero block has byte 0),
 *     elements x / 2^e rounded to the nearest E2M1 value, ties to the even
 *     mantissa, saturating to +-6, sign of zero kept.
 *   MOE_PAYLOAD_FP8_BLOCK: D e4m3fn codes of the 1x128 blockwise
 *     quantization (as moe_quant_ptpc_fp8 with group 128), then D/128 fp32
 *     scales (little-endian).
 * moe_ep_pack_payload: x [T, D] bf16 -> payload [T, row bytes] (rows
 *   contiguous).  Inputs must be finite.
 * moe_ep_unpack_payload: payload -> x [T, D] bf16: MXFP4 elements exactly
 *   (code value * 2^(e) is a bf16 value); FP8 as bf16(fp32(code value *
 *   scale)).
 * Errors: NULL pointers or T < 0 -> MOE_ERR_INVALID_ARG; D not a positive
 * multiple of 128 (or above 65536) or an unknown format -> MOE_ERR_UNSUPPORTED.
 */
int64_t moe_ep_payload_bytes(int32_t D, int32_t format);
int32_t moe_ep_pack_payload(const void* x_bf16, int32_t T, int32_t D, int32_t format,
                            uint8_t* payload, void* stream);
int32_t moe_ep_unpack_payload(const uint8_t* payload, int32_t T, int32_t D, int32_t format,
                              void* x_bf16, void* stream);

/*
 * Debug validation of a forward's inputs, for callers that switch it on
 * (moe_forward never calls it; the Python binding does when MOE_VALIDATE=1).
 * The forward takes such inputs without complaint: a routed id outside
 * [0, E) gets no row (inv_perm -1), and Inf or NaN go through the
 * arithmetic as IEEE values.  Writes, on the stream, counts[0] = elements of
 * x_bf16 [T, D] that are Inf or NaN, counts[1] = the same for logits
 * [T, E] fp32, counts[2] = ids [T, k] int32 outside [0, E).  Any of x_bf16,
 * logits, ids may be NULL (its count is 0).  counts: device int32[3],
 * zeroed by the call; read it once the stream has synchronized.  Errors:
 * MOE_ERR_INVALID_ARG for counts NULL, T < 0, D <= 0 with x, E <= 0 with
 * logits or ids, k <= 0 with ids.  Nothing traps: the kernels only count.
 */
int32_t moe_validate_inputs(const void* x_bf16, int32_t T, int32_t D, const float* logits, int32_t E,
                            const int32_t* ids, int32_t k, int32_t* counts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_ROUTER_AMD_MOE_H */

// Grouped expert GEMMs on CDNA4 MFMA.
//
// GMM V2 of the Qwen 3.5 TPU page packs the gate and up projections into one
// tile, fuses SwiGLU into the matmul loop and walks each expert's variable
// row count in bounded slices.  PTPC-FP8 (Qwen3 MI300X page, 2.1.1) applies a
// per-token activation scale and a per-output-channel weight scale; the
// DeepSeek-R1 layer's blockwise FP8 (MI355X MoRI page) uses 1x128 activation
// and 128x128 weight scales.
//
// Layout of one workgroup (256 threads, 4 waves):
//   - a tile of BM permuted rows (one expert: the permutation pads every
//     expert to a multiple of BM, so block_expert gives the expert) times 256
//     weight rows (gate_up: 128 gate + the matching 128 up rows, giving 128
//     act columns; down: 256 output columns);
//   - K advances 128 bytes per step (128 e4m3 or 64 bf16 elements); A and B
//     tiles are staged through LDS, double buffered, one barrier per step;
//     rows are padded to 144 B so the 32 lanes that read one MFMA operand hit
//     distinct banks;
//   - waves split the tile 2x2 (BM = 128) or 1x4 (BM <= 64); each wave runs
//     32x32 MFMAs (v_mfma_f32_32x32x64_f8f6f4 or v_mfma_f32_32x32x16_bf16);
//   - A and B operands take the same lane -> K mapping, so the reduction is
//     exact whatever order the matrix core sums K in;
//   - the epilogue dequantizes (row scale x channel scale), applies
//     silu(g) * u for gate_up, rounds to bf16 and stores;
//   - workgroup ids are remapped so consecutive tiles (same rows, adjacent
//     weight columns) land on the same XCD and share its L2.
#include "common.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBKB = 128;      // K bytes per step
constexpr int kLdsRow = 144;   // padded LDS row (bytes)
constexpr int kBRows = 256;    // weight rows per tile

struct GemmArgs {
    const uint8_t* a;          // activation rows (bf16 or e4m3)
    int64_t a_ld;              // bytes per activation row
    const float* a_scale;      // PTPC: one per row; block: [rows, K/128]
    int a_scale_ld;            // block mode: K/128
    const int* sorted_ids;     // gate_up: flat id per permuted row (NULL: rows are direct)
    int topk, TK, sentinel;
    const int* block_expert;
    const uint8_t* w;          // [E', Nw, K] weights
    int64_t w_expert_bytes;
    const float* w_scale;      // PTPC: [E', Nw]; block: [E', Nw/128, K/128]
    int64_t ws_expert;         // floats per expert
    int ws_ld;                 // block mode: K/128
    int K;                     // reduction length (elements)
    int I;                     // gate_up: act columns; weight rows 2I
    void* out;
    int64_t out_ld;            // elements per output row
    int n_ntiles, n_tiles;
};

template <int MODE>
__device__ __forceinline__ void mfma_step(const uint8_t* a_lds, const uint8_t* b_lds, v16f& acc) {
    if constexpr (MODE == MOE_QUANT_NONE_BF16) {
        const v8bf a = *reinterpret_cast<const v8bf*>(a_lds);
        const v8bf b = *reinterpret_cast<const v8bf*>(b_lds);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    } else {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(a_lds), a1 = *reinterpret_cast<const u32x4*>(a_lds + 16);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(b_lds), b1 = *reinterpret_cast<const u32x4*>(b_lds + 16);
        const v8i a = __builtin_bit_cast(v8i, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        const v8i b = __builtin_bit_cast(v8i, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        // e4m3 x e4m3 (format selectors 0, 0), no block scaling
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
    }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

template <int MODE, bool GATEUP, int BM>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(const GemmArgs p) {
    constexpr int ELEM = MODE == MOE_QUANT_NONE_BF16 ? 2 : 1;
    constexpr int WM = BM >= 128 ? 2 : 1;
    constexpr int WN = 4 / WM;
    constexpr int WROWS = BM / WM;          // rows per wave
    constexpr int TM = WROWS / 32;
    constexpr int WCOLS = kBRows / WN;       // weight rows per wave
    constexpr int TN = WCOLS / 32;
    constexpr int G = 128 / WN;              // gate_up: gate (and up) rows per wave
    constexpr int A_LD = BM * 8 / 256;       // 16-B chunks of A per thread per step
    constexpr int KSUB = MODE == MOE_QUANT_NONE_BF16 ? 4 : 2;   // MFMAs per 128-B step
    constexpr int SUBB = kBKB / KSUB;        // bytes per MFMA K-substep
    constexpr int LANEB = SUBB / 2;          // bytes per lane per operand
    constexpr int TILE_N = GATEUP ? 128 : kBRows;
    constexpr bool BLOCKQ = MODE == MOE_QUANT_BLOCK128_FP8;
    static_assert(TM >= 1 && TN >= 2, "tile shape");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + kBRows) * kLdsRow];
    __shared__ float s_rowscale[BM];
    __shared__ float s_ascale[2][BM];
    __shared__ int s_tok[BM];

    // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous range of tiles.
    const int per = (p.n_tiles + 7) >> 3;
    const int lt = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lt >= p.n_tiles) return;
    const int mb = lt / p.n_ntiles, nt = lt - mb * p.n_ntiles;
    const int e = p.block_expert[mb];
    if (e < 0) return;
    const int m0 = mb * BM;
    const int n0 = nt * TILE_N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // rows of this tile -> activation row (token for gate_up)
    if (tid < BM) {
        int tok;
        if (p.sorted_ids) {
            const int f = p.sorted_ids[m0 + tid];
            tok = f == p.sentinel ? -1 : (f < p.TK ? f / p.topk : f - p.TK);
        } else {
            tok = m0 + tid;
        }
        s_tok[tid] = tok;
        if constexpr (MODE == MOE_QUANT_PTPC_FP8) s_rowscale[tid] = tok >= 0 ? p.a_scale[tok] : 0.0f;
    }
    __syncthreads();

    const uint8_t* a_src[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int c = tid + 256 * i;
        const int tok = s_tok[c >> 3];
        a_src[i] = tok >= 0 ? p.a + tok * p.a_ld + (c & 7) * 16 : nullptr;
    }
    const uint8_t* wexp = p.w + static_cast<int64_t>(e) * p.w_expert_bytes;
    const int64_t wrow_bytes = static_cast<int64_t>(p.K) * ELEM;
    const uint8_t* b_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + 256 * i;
        const int r = c >> 3;
        const int wr = GATEUP ? (r < 128 ? n0 + r : p.I + n0 + r - 128) : n0 + r;
        b_src[i] = wexp + wr * wrow_bytes + (c & 7) * 16;
    }
    const int nk = static_cast<int>(wrow_bytes / kBKB);

    u32x4 ra[A_LD], rb[8];
    float ras = 0.0f;
#define MOE_GLOAD(S)                                                                                     \
    do {                                                                                                 \
        const int64_t koff_ = static_cast<int64_t>(S) * kBKB;                                            \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i) ra[i] =                                         \
            a_src[i] ? *reinterpret_cast<const u32x4*>(a_src[i] + koff_) : u32x4{0, 0, 0, 0};      \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + koff_); \
        if constexpr (BLOCKQ) {                                                                          \
            if (tid < BM) {                                                                              \
                const int tok_ = s_tok[tid];                                                             \
                ras = tok_ >= 0 ? p.a_scale[static_cast<int64_t>(tok_) * p.a_scale_ld + (S)] : 0.0f;     \
            }                                                                                            \
        }                                                                                                \
    } while (0)
#define MOE_LSTORE(BUF)                                                                                  \
    do {                                                                                                 \
        uint8_t* L_ = lds[BUF];                                                                          \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i) {                                               \
            const int c_ = tid + 256 * i;                                                                \
            *reinterpret_cast<u32x4*>(L_ + (c_ >> 3) * kLdsRow + (c_ & 7) * 16) = ra[i];                 \
        }                                                                                                \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                                  \
            const int c_ = tid + 256 * i;                                                                \
            *reinterpret_cast<u32x4*>(L_ + (BM + (c_ >> 3)) * kLdsRow + (c_ & 7) * 16) = rb[i];          \
        }                                                                                                \
        if constexpr (BLOCKQ) {                                                                          \
            if (tid < BM) s_ascale[BUF][tid] = ras;                                                      \
        }                                                                                                \
    } while (0)

    // LDS row of this lane's operand rows
    int a_row[TM], b_row[TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) a_row[tm] = wm * WROWS + tm * 32 + (lane & 31);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        int r;
        if (GATEUP) r = tn < TN / 2 ? wn * G + tn * 32 : 128 + wn * G + (tn - TN / 2) * 32;
        else r = wn * WCOLS + tn * 32;
        b_row[tn] = BM + r + (lane & 31);
    }
    const int lane_k = (lane >> 5) * LANEB;

    v16f acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = v16f{};

    MOE_GLOAD(0);
    MOE_LSTORE(0);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int buf = s & 1;
        if (s + 1 < nk) MOE_GLOAD(s + 1);
        const uint8_t* L = lds[buf];
        if constexpr (!BLOCKQ) {
#pragma unroll
            for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        mfma_step<MODE>(L + a_row[tm] * kLdsRow + kk * SUBB + lane_k,
                                        L + b_row[tn] * kLdsRow + kk * SUBB + lane_k, acc[tm][tn]);
        } else {
            // one 128-element K step is one scale block: partial sums, then
            // acc += partial * a_scale(row, kb) * w_scale(n-block, kb)
            v16f part[TM][TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) part[tm][tn] = v16f{};
#pragma unroll
            for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        mfma_step<MODE>(L + a_row[tm] * kLdsRow + kk * SUBB + lane_k,
                                        L + b_row[tn] * kLdsRow + kk * SUBB + lane_k, part[tm][tn]);
            float wsc[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int wr0 = b_row[tn] - BM - (lane & 31);              // tile-local weight row
                const int wr = GATEUP ? (wr0 < 128 ? n0 + wr0 : p.I + n0 + wr0 - 128) : n0 + wr0;
                wsc[tn] = p.w_scale[e * p.ws_expert + (wr >> 7) * p.ws_ld + s];
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = wm * WROWS + tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    const float as = s_ascale[buf][row];
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) acc[tm][tn][i] += part[tm][tn][i] * (as * wsc[tn]);
                }
            }
        }
        if (s + 1 < nk) MOE_LSTORE(buf ^ 1);
        __syncthreads();
    }

#undef MOE_GLOAD
#undef MOE_LSTORE

    // ------------------------------------------------------------ epilogue
    const float* wsx = (MODE == MOE_QUANT_PTPC_FP8) ? p.w_scale + e * p.ws_expert : nullptr;
    if constexpr (GATEUP) {
        uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
        for (int tg = 0; tg < TN / 2; ++tg) {
            const int col = wn * G + tg * 32 + (lane & 31);     // act column within the tile
            float swg = 1.0f, swu = 1.0f;
            if constexpr (MODE == MOE_QUANT_PTPC_FP8) {
                swg = wsx[n0 + col];
                swu = wsx[p.I + n0 + col];
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = wm * WROWS + tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    float g = acc[tm][tg][i], u = acc[tm][tg + TN / 2][i];
                    if constexpr (MODE == MOE_QUANT_PTPC_FP8) {
                        const float rs = s_rowscale[row];
                        g = g * rs * swg;
                        u = u * rs * swu;
                    }
                    out[static_cast<int64_t>(m0 + row) * p.out_ld + n0 + col] = f32_to_bf16(silu_mul(g, u));
                }
            }
        }
    } else {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int col = wn * WCOLS + tn * 32 + (lane & 31);
            float sw = 1.0f;
            if constexpr (MODE == MOE_QUANT_PTPC_FP8) sw = wsx[n0 + col];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = wm * WROWS + tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    float v = acc[tm][tn][i];
                    if constexpr (MODE == MOE_QUANT_PTPC_FP8) v = v * s_rowscale[row] * sw;
                    const int64_t o = static_cast<int64_t>(m0 + row) * p.out_ld + n0 + col;
                    if constexpr (MODE == MOE_QUANT_NONE_BF16) static_cast<float*>(p.out)[o] = v;
                    else static_cast<uint16_t*>(p.out)[o] = f32_to_bf16(v);
                }
            }
        }
    }
}

template <int MODE, bool GATEUP>
static int32_t launch_bm(int block_m, const GemmArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(ceil_div(a.n_tiles, 8) * 8)), block(256);
    switch (block_m) {
        case 32: hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 32>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 64>), grid, block, 0, s, a); break;
        case 128:
            if constexpr (MODE == MOE_QUANT_BLOCK128_FP8) return MOE_ERR_UNSUPPORTED;
            else hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 128>), grid, block, 0, s, a);
            break;
        default: return MOE_ERR_UNSUPPORTED;
    }
    return moe_launch_status();
}

template <bool GATEUP>
static int32_t launch_mode(int quant, int block_m, const GemmArgs& a, hipStream_t s) {
    if (a.n_tiles == 0) return MOE_OK;
    switch (quant) {
        case MOE_QUANT_NONE_BF16: return launch_bm<MOE_QUANT_NONE_BF16, GATEUP>(block_m, a, s);
        case MOE_QUANT_PTPC_FP8: return launch_bm<MOE_QUANT_PTPC_FP8, GATEUP>(block_m, a, s);
        case MOE_QUANT_BLOCK128_FP8: return launch_bm<MOE_QUANT_BLOCK128_FP8, GATEUP>(block_m, a, s);
    }
    return MOE_ERR_UNSUPPORTED;
}

int32_t gemm_gateup_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T, int block_m,
                           int64_t max_rows, const int* sorted_ids, const int* block_expert, void* act,
                           hipStream_t s) {
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    GemmArgs g{};
    g.a = static_cast<const uint8_t*>(a);
    g.a_ld = static_cast<int64_t>(L->D) * elem;
    g.a_scale = a_scale;
    g.a_scale_ld = L->D / 128;
    g.sorted_ids = sorted_ids;
    g.topk = L->top_k;
    g.TK = T * L->top_k;
    g.sentinel = T * (L->top_k + L->n_shared);
    g.block_expert = block_expert;
    g.w = static_cast<const uint8_t*>(L->w13);
    g.w_expert_bytes = static_cast<int64_t>(2) * L->I * L->D * elem;
    g.w_scale = L->w13_scale;
    g.ws_expert = L->quant == MOE_QUANT_PTPC_FP8 ? 2LL * L->I
                                                  : static_cast<int64_t>(2 * L->I / 128) * (L->D / 128);
    g.ws_ld = L->D / 128;
    g.K = L->D;
    g.I = L->I;
    g.out = act;
    g.out_ld = L->I;
    g.n_ntiles = L->I / 128;
    g.n_tiles = static_cast<int>(max_rows / block_m) * g.n_ntiles;
    return launch_mode<true>(L->quant, block_m, g, s);
}

int32_t gemm_down_launch(const moe_layer_desc* L, const void* act, const float* act_scale, int block_m,
                         int64_t max_rows, const int* block_expert, void* out_perm, hipStream_t s) {
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    GemmArgs g{};
    g.a = static_cast<const uint8_t*>(act);
    g.a_ld = static_cast<int64_t>(L->I) * elem;
    g.a_scale = act_scale;
    g.a_scale_ld = L->I / 128;
    g.sorted_ids = nullptr;
    g.block_expert = block_expert;
    g.w = static_cast<const uint8_t*>(L->w2);
    g.w_expert_bytes = static_cast<int64_t>(L->D) * L->I * elem;
    g.w_scale = L->w2_scale;
    g.ws_expert = L->quant == MOE_QUANT_PTPC_FP8 ? static_cast<int64_t>(L->D)
                                                  : static_cast<int64_t>(L->D / 128) * (L->I / 128);
    g.ws_ld = L->I / 128;
    g.K = L->I;
    g.I = L->I;
    g.out = out_perm;
    g.out_ld = L->D;
    g.n_ntiles = L->D / kBRows;
    g.n_tiles = static_cast<int>(max_rows / block_m) * g.n_ntiles;
    return launch_mode<false>(L->quant, block_m, g, s);
}

}  // namespace moe

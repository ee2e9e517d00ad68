// Grouped expert GEMMs on CDNA4 MFMA.
//
// GMM V2 of the Qwen 3.5 TPU page packs the gate and up projections into one
// tile, fuses SwiGLU into the matmul loop and walks each expert's variable
// row count in bounded slices.  PTPC-FP8 (Qwen3 MI300X page, 2.1.1) applies a
// per-token activation scale and a per-output-channel weight scale; the
// DeepSeek-R1 layer's blockwise FP8 (MI355X MoRI page) uses 1x128 activation
// and 128x128 weight scales.
//
// Layout of one workgroup (256 threads, 4 waves, one workgroup per CU):
//   - a tile of BM permuted rows of one expert (the permutation pads every
//     expert to a multiple of BM) times 256 weight rows (gate_up: 128 gate
//     rows and the matching 128 up rows, giving 128 act columns; down: 256
//     output columns);
//   - K advances 128 bytes per step (128 e4m3 or 64 bf16 elements; one
//     128-element scale block in the blockwise mode).  Tiles move from global
//     memory straight into LDS (global_load_lds_dwordx4: each lane's 16 bytes
//     land at M0 + 16*lane, no register staging), two steps ahead, into three
//     LDS stages of 128-byte rows whose 16-byte chunks are XOR-swizzled by row
//     (the swizzle is applied on the global side, so the 16 lanes of an MFMA
//     operand read hit distinct banks); each wave waits for its own copies
//     with an explicit vmcnt, then one barrier per step; all MFMA operands of
//     a step are read from LDS before its MFMAs issue;
//   - waves split the tile 2x2 (BM = 128) or 1x4 (BM <= 64) and run 32x32
//     MFMAs (v_mfma_f32_32x32x64_f8f6f4 or v_mfma_f32_32x32x16_bf16); A and B
//     operands take the same lane -> K mapping, so the reduction pairs
//     matching K whatever order the matrix core sums in;
//   - pad rows read a real row and are zeroed by a row mask in the epilogue;
//   - tiles are ordered expert by expert, weight tile by weight tile, row
//     block fastest, and each XCD (workgroup id mod 8) takes a contiguous
//     range of that order: the row blocks of one expert that share a weight
//     tile run together on one XCD and share it through its L2;
//   - the epilogue dequantizes (row scale x channel scale), applies
//     silu(g) * u for gate_up, rounds to bf16 and stores.
#include "common.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;       // K bytes per step
constexpr int kBRows = 256;    // weight rows per tile

struct GemmArgs {
    const uint8_t* a;          // activation rows (bf16 or e4m3)
    int64_t a_ld;              // bytes per activation row
    const float* a_scale;      // PTPC: one per row; block: [rows, K/128]
    int a_scale_ld;            // block mode: K/128
    const int* sorted_ids;     // gate_up: flat id per permuted row (NULL: rows are direct)
    int topk, TK, sentinel;
    const int* block_expert;
    const int* offsets;        // [E'+1] padded expert offsets
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

// byte offset of (row, logical 16-byte chunk c) in a 128-byte-row LDS stage
__device__ __forceinline__ int lds_off(int row, int c) { return row * kBK + ((c ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ u32x4 lds16(const uint8_t* L, int off) { return *reinterpret_cast<const u32x4*>(L + off); }

__device__ __forceinline__ v8i cat8(u32x4 lo, u32x4 hi) {
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Global -> LDS copies.  Each lane's bytes land at M0 + size * lane; M0 must
// be wave-uniform.  Issued as inline asm so that the only waits on them are
// the explicit vmcnt_wait below (the compiler would otherwise drain every
// outstanding copy before each LDS read).  The main loop issues no other
// vector-memory instruction, so vmcnt counts exactly these copies.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr)
                 : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int MODE, bool GATEUP, int BM>
__global__ void __launch_bounds__(256, 1) grouped_gemm_kernel(const GemmArgs p) {
    constexpr int ELEM = MODE == MOE_QUANT_NONE_BF16 ? 2 : 1;
    constexpr int WM = BM >= 128 ? 2 : 1;
    constexpr int WN = 4 / WM;
    constexpr int WROWS = BM / WM;          // rows per wave
    constexpr int TM = WROWS / 32;
    constexpr int WCOLS = kBRows / WN;       // weight rows per wave
    constexpr int TN = WCOLS / 32;
    constexpr int G = 128 / WN;              // gate_up: gate (and up) rows per wave
    constexpr int A_CH = BM * 8 / 256;       // 16-byte A chunks per thread per step
    constexpr int B_CH = kBRows * 8 / 256;   // 16-byte B chunks per thread per step
    constexpr int TILE_N = GATEUP ? 128 : kBRows;
    constexpr bool BLOCKQ = MODE == MOE_QUANT_BLOCK128_FP8;
    constexpr int STAGE = (BM + kBRows) * kBK;
    static_assert(TM >= 1 && TN >= 2 && A_CH >= 1, "tile shape");

    constexpr int NSTAGE = 3;
    constexpr int A_IN = BM / 32;              // 1 KB copies (8 rows) of A per wave per step
    constexpr int B_IN = kBRows / 32;          // 1 KB copies of B per wave per step
    constexpr int SC_IN = BLOCKQ ? 1 : 0;      // blockwise: one 4-byte-lane copy of row scales
    constexpr int N_IN = A_IN + B_IN + SC_IN;  // copies per wave per step (vmcnt units)
    __shared__ __attribute__((aligned(16))) uint8_t lds[NSTAGE * STAGE];
    __shared__ float s_rowscale[BM];          // PTPC: row scale; other modes: row mask (pad rows 0)
    __shared__ __attribute__((aligned(16))) float s_ascale[NSTAGE][256];   // blockwise: row scales of a stage
    __shared__ int s_tok[BM];

    // tile order: expert-major, weight tile, then row block; XCD-contiguous
    const int per = (p.n_tiles + 7) >> 3;
    const int lt = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lt >= p.n_tiles) return;
    const int e = p.block_expert[lt / p.n_ntiles];
    if (e < 0) return;
    const int bs = p.offsets[e] / BM, nb = p.offsets[e + 1] / BM - bs;
    const int local = lt - bs * p.n_ntiles;
    const int nt = local / nb, mb = bs + local % nb;
    const int m0 = mb * BM;
    const int n0 = nt * TILE_N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    if (tid < BM) {
        int tok = m0 + tid;
        float rs = 1.0f;
        if (p.sorted_ids) {
            const int f = p.sorted_ids[m0 + tid];
            const bool pad = f == p.sentinel;
            tok = pad ? 0 : (f < p.TK ? f / p.topk : f - p.TK);
            rs = pad ? 0.0f : 1.0f;
        }
        s_tok[tid] = tok;
        if constexpr (MODE == MOE_QUANT_PTPC_FP8) rs = rs == 0.0f ? 0.0f : p.a_scale[tok];
        s_rowscale[tid] = rs;
    }
    __syncthreads();

    // Copy j of a wave fills 8 LDS rows: lane i writes row 8j' + i/8 (j' the
    // wave's j-th block of 8 rows), physical chunk i%8, which must hold the
    // logical chunk (i%8) ^ swizzle(row) of that row.
    const int crow = lane >> 3, cphys = lane & 7;
    const uint8_t* a_src[A_IN];
#pragma unroll
    for (int j = 0; j < A_IN; ++j) {
        const int r = (wave + 4 * j) * 8 + crow;
        const int c = cphys ^ ((r >> 1) & 7);
        a_src[j] = p.a + static_cast<int64_t>(s_tok[r]) * p.a_ld + c * 16;
    }
    const uint8_t* wexp = p.w + static_cast<int64_t>(e) * p.w_expert_bytes;
    const int64_t wrow_bytes = static_cast<int64_t>(p.K) * ELEM;
    uint32_t b_src[B_IN];                                   // byte offsets within the expert
#pragma unroll
    for (int j = 0; j < B_IN; ++j) {
        const int r = (wave + 4 * j) * 8 + crow;             // weight tile row
        const int c = cphys ^ (((BM + r) >> 1) & 7);
        const int wr = GATEUP ? (r < 128 ? n0 + r : p.I + n0 + r - 128) : n0 + r;
        b_src[j] = static_cast<uint32_t>(wr * wrow_bytes + c * 16);
    }
    // blockwise: wave w copies the scales of rows 64w .. 64w+63 (rows past BM
    // read row 0 into unused slots)
    const float* sc_src = nullptr;
    if constexpr (BLOCKQ) {
        const int r = wave * 64 + lane;
        sc_src = p.a_scale + static_cast<int64_t>(s_tok[r < BM ? r : 0]) * p.a_scale_ld;
    }
    const int nk = static_cast<int>(wrow_bytes / kBK);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    const uint32_t sc0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_ascale[0][0]));

    // issue the copies of K step S into LDS stage BUF (uniform M0 per copy)
    auto issue = [&](int S, int buf) {
        const int64_t ko = static_cast<int64_t>(S) * kBK;
        const uint32_t st = lds0 + buf * STAGE;
#pragma unroll
        for (int j = 0; j < A_IN; ++j)
            dma16(a_src[j] + ko, __builtin_amdgcn_readfirstlane(st + (wave + 4 * j) * 8 * kBK));
#pragma unroll
        for (int j = 0; j < B_IN; ++j)
            dma16(wexp + b_src[j] + ko, __builtin_amdgcn_readfirstlane(st + (BM + (wave + 4 * j) * 8) * kBK));
        if constexpr (BLOCKQ) dma4(sc_src + S, __builtin_amdgcn_readfirstlane(sc0 + (buf * 256 + wave * 64) * 4));
    };

    // LDS rows of this lane's operands
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
    const int h = lane >> 5;

    v16f acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = v16f{};

    // one 128-byte K step on LDS stage `buf`: all operand fragments first, then the MFMAs
    auto step = [&](int buf, int s) {
        const uint8_t* L = lds + buf * STAGE;
        if constexpr (MODE == MOE_QUANT_NONE_BF16) {
            v8bf av[4][TM], bv[4][TN];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) av[kk][tm] = __builtin_bit_cast(v8bf, lds16(L, lds_off(a_row[tm], 2 * kk + h)));
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) bv[kk][tn] = __builtin_bit_cast(v8bf, lds16(L, lds_off(b_row[tn], 2 * kk + h)));
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                    for (int tm = 0; tm < TM; ++tm)
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk][tm], bv[kk][tn], acc[tm][tn], 0, 0, 0);
        } else {
            v8i av[2][TM], bv[2][TN];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    av[kk][tm] = cat8(lds16(L, lds_off(a_row[tm], 4 * kk + 2 * h)), lds16(L, lds_off(a_row[tm], 4 * kk + 2 * h + 1)));
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    bv[kk][tn] = cat8(lds16(L, lds_off(b_row[tn], 4 * kk + 2 * h)), lds16(L, lds_off(b_row[tn], 4 * kk + 2 * h + 1)));
            }
            if constexpr (!BLOCKQ) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm)
                            // e4m3 x e4m3 (format selectors 0, 0), no block scaling
                            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[kk][tm], bv[kk][tn], acc[tm][tn],
                                                                                          0, 0, 0, 0, 0, 0);
            } else {
                // the step is one 128-element scale block:
                // acc += part * a_scale(row, kb) * w_scale(n-block, kb)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    const int wr0 = b_row[tn] - BM - (lane & 31);
                    const int wr = GATEUP ? (wr0 < 128 ? n0 + wr0 : p.I + n0 + wr0 - 128) : n0 + wr0;
                    const float wsc = p.w_scale[e * p.ws_expert + (wr >> 7) * p.ws_ld + s];
#pragma unroll
                    for (int tm = 0; tm < TM; ++tm) {
                        v16f part = v16f{};
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk)
                            part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[kk][tm], bv[kk][tn], part, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int row = wm * WROWS + tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                            acc[tm][tn][i] += part[i] * (s_ascale[buf][row] * wsc);
                        }
                    }
                }
            }
        }
    };

    // prologue: steps 0 and 1 in flight; wait for step 0
    issue(0, 0);
    if (nk > 1) {
        issue(1, 1);
        vmcnt_wait<N_IN>();
    } else {
        vmcnt_wait<0>();
    }
    __syncthreads();
    int s = 0;
    // steady state: the copies of step s + 2 go out, step s computes, then
    // this wave's copies of step s + 1 are waited for (those of s + 2 may
    // stay in flight) and the barrier publishes them and frees stage s
    for (; s + 2 < nk; ++s) {
        const int b = s % NSTAGE;
        issue(s + 2, (s + 2) % NSTAGE);
        step(b, s);
        vmcnt_wait<N_IN>();
        __syncthreads();
    }
    // last two steps (step nk-1 may already be the only one left)
    for (; s < nk; ++s) {
        step(s % NSTAGE, s);
        vmcnt_wait<0>();
        __syncthreads();
    }

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
                    const float rs = s_rowscale[row];
                    g = g * rs * swg;
                    u = u * rs * swu;
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
                    const float v = acc[tm][tn][i] * s_rowscale[row] * sw;
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
    if (block_m == 32) {
        hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 32>), grid, block, 0, s, a);
        return moe_launch_status();
    }
    // the blockwise mode keeps its partial sums and scales in registers: row
    // blocks above 32 would spill
    if constexpr (MODE != MOE_QUANT_BLOCK128_FP8) {
        if (block_m == 64) {
            hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 64>), grid, block, 0, s, a);
            return moe_launch_status();
        }
        if (block_m == 128) {
            hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 128>), grid, block, 0, s, a);
            return moe_launch_status();
        }
    }
    return MOE_ERR_UNSUPPORTED;
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

int32_t stream_gateup_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T,
                             const int* sorted_ids, const int* offsets, void* act, hipStream_t s);
int32_t stream_down_launch(const moe_layer_desc* L, const void* act, const float* act_scale, int T,
                           const int* offsets, void* out_perm, hipStream_t s);

int32_t gemm_gateup_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T, int block_m,
                           int64_t max_rows, const int* sorted_ids, const int* block_expert, const int* offsets,
                           void* act, hipStream_t s) {
    if (block_m == 16) return stream_gateup_launch(L, a, a_scale, T, sorted_ids, offsets, act, s);
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    GemmArgs g{};
    g.offsets = offsets;
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

int32_t gemm_down_launch(const moe_layer_desc* L, const void* act, const float* act_scale, int T, int block_m,
                         int64_t max_rows, const int* block_expert, const int* offsets, void* out_perm,
                         hipStream_t s) {
    if (block_m == 16) return stream_down_launch(L, act, act_scale, T, offsets, out_perm, s);
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    GemmArgs g{};
    g.offsets = offsets;
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

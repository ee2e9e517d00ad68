// Grouped expert GEMMs on CDNA4 MFMA.
//
// GMM V2 of the Qwen 3.5 TPU page packs the gate and up projections into one
// tile, fuses SwiGLU into the matmul loop and walks each expert's variable
// row count in bounded slices.  PTPC-FP8 (Qwen3 MI300X page, 2.1.1) applies a
// per-token activation scale and a per-output-channel weight scale; the
// DeepSeek-R1 layer's blockwise FP8 (MI355X MoRI page) uses 1x128 activation
// and 128x128 weight scales; MXFP4 (the MoRI page's A4W4 FusedMoE) has E2M1
// activations and weights with one E8M0 scale per 32 elements along K, which
// the matrix cores apply themselves (v_mfma_scale_f32_32x32x64_f8f6f4 with
// FP4 operands and per-lane scale bytes).
//
// One workgroup per CU (256 threads, 4 waves in a WM x WN grid) computes a
// tile of BM permuted rows of one expert (the permutation pads every expert
// to a multiple of BM) times WN x 32*TN weight rows.  Wave (wm, wn) owns
// BM/WM rows and 32*TN weight rows (gate_up: 16*TN gate rows and the
// matching up rows, so gate and up of an act column meet in one wave).
//
// Data movement.  K advances in 128-byte steps (128 e4m3 or 64 bf16
// elements; one step is one 128-element scale block in the blockwise mode).
// Operand rows move from global memory straight into LDS with
// global_load_lds_dwordx4 (lane i's 16 bytes land at M0 + 16 i): one copy
// instruction moves 8 rows x 128 contiguous bytes, so every L1-to-L2 request
// carries a whole 128-byte line; the number of such requests, not bytes, is
// what bounds the copy rate per CU.  LDS rows are 128 bytes with their
// 16-byte chunks XOR-swizzled by row (applied on the global side) so that the
// MFMA operand reads are free of bank conflicts.  NS (2 or 3) LDS stages form
// a ring; the copies of step S + NS go out in the second half of step S, as
// soon as stage S is released.
//
// Compute.  Each 128-byte step is two 64-byte half-steps of 32x32 MFMAs
// (v_mfma_f32_32x32x64_f8f6f4 or two v_mfma_f32_32x32x16_bf16).  Lane l
// supplies row (l mod 32) and bytes [32q, 32q + 32) of a half-step (q = l/32)
// for both operands, so the reduction pairs matching K whatever order the
// matrix core sums in.  Operand fragments are double-buffered in registers:
// while the MFMAs of one half-step run, the fragments of the next are read
// from LDS, and the MFMAs, LDS reads and copies are interleaved one by one
// (pinned with scheduling barriers) so that a memory instruction stalled at
// issue overlaps a running MFMA.  One wait + barrier per 128-byte step.
//
// Pad rows read a real row and are zeroed by a row mask in the epilogue;
// 32-row tiles made only of pads (known from the expert's row count) get no
// operand reads, no MFMAs and no output stores, and with two stages no
// activation copies.
// Tiles are ordered expert by expert, weight tile by weight tile, row block
// fastest, and each XCD (workgroup id mod 8) takes a contiguous range of
// that order, so the row blocks of one expert that share a weight tile run
// together on one XCD and share it through its L2.  The epilogue
// dequantizes (row scale x channel scale), applies silu(g) * u for gate_up,
// rounds to bf16 and stores through a buffer resource.
#include "common.h"

#include <type_traits>
#include <utility>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRow = 128;          // K bytes per step = LDS row width
constexpr int kLdsBudget = 150 * 1024;

// Waves per workgroup and their grid.  One wave per SIMD cannot keep enough
// LDS reads in flight to feed its MFMAs from the 128 x 256 tile below 256
// rows; the 256-row tile runs 8 waves (2 per SIMD, 2 x 4, each 128 x 64),
// which doubles the LDS read rate the CU sustains.  Row tiles of 128 use a
// 2 x 2 grid of 4 waves, smaller ones 1 x 4.  In the blockwise mode (a
// layer whose experts each see ~150 rows, so its weight tiles are used by
// one or two row blocks and stream from HBM) the 128-row tile also runs 8
// waves (2 x 4, each 64 x 64): a 128 x 256 tile whose 48 KB stages fit 3
// deep in LDS, so the weight copies get two steps to land instead of one.
// MXFP4 takes the same 8-wave 128-row tile (its 256-row tile's scale words
// do not fit the register budget of two waves per SIMD).  The quantized
// modes also have a 192-row tile (8 waves 2 x 4, each 96 x 64): more MFMA
// work per copied byte than 128 rows, and within MXFP4's register budget.
constexpr int nw_of(int mode, int bm) {
    return bm >= 192 || (bm == 128 && (mode == MOE_QUANT_BLOCK128_FP8 || mode == MOE_QUANT_MXFP4)) ? 8 : 4;
}
constexpr int wm_of(int bm) { return bm >= 128 ? 2 : 1; }

// 32-row weight tiles per wave: 4 for PTPC where the weight rows divide into
// WN x 128 (gate_up: 2I rows as WN waves x (64 gate + 64 up)); else 2 (the
// bf16 and blockwise modes keep more live registers per tile, and the
// 8-wave tile holds 128 x 64 per wave)
static int tn_of(int mode, int weight_rows, int bm) {
    if (nw_of(mode, bm) == 8) return 2;
    return (mode == MOE_QUANT_PTPC_FP8 || mode == MOE_QUANT_MXFP4) && weight_rows % ((4 / wm_of(bm)) * 128) == 0
               ? 4 : 2;
}

struct GemmArgs {
    const uint8_t* a;          // activation rows (bf16 or e4m3)
    int64_t a_ld;              // bytes per activation row
    const float* a_scale;      // PTPC: one per row; block: [rows, K/128]
    int a_scale_ld;            // block mode: K/128
    const int* sorted_ids;     // gate_up: flat id per permuted row (NULL: rows are direct)
    int topk, TK, sentinel;
    const int* block_expert;
    const int* offsets;        // [E'+1] padded expert offsets
    const int* counts;         // [E'] routed rows per expert (NULL: every row of a segment is live)
    const uint8_t* w;          // [E', Nw, K] weights
    int w_blocked;             // weights in blocks of 16 rows x 128 bytes (else row-major)
    int64_t w_expert_bytes;
    const float* w_scale;      // PTPC: [E', Nw]; block: [E', Nw/128, K/128]
    int64_t ws_expert;         // floats per expert
    int ws_ld;                 // block mode: K/128
    const uint8_t* a_mx;       // MXFP4: E8M0 scales of the activation rows [rows, K/32]
    const uint8_t* w_mx;       // MXFP4: E8M0 weight scales [E', Nw, K/32]
    int64_t w_mx_expert;       // MXFP4: scale bytes per expert
    int K;                     // reduction length (elements)
    int I;                     // gate_up: act columns; weight rows 2I
    void* out;
    int64_t out_ld;            // elements per output row
    int n_ntiles, n_tiles;     // weight tiles per row block; tiles the grid covers (row blocks of max_rows)
    int n_exp;                 // E' = E + n_shared: offsets[n_exp] is the padded row total
};

// byte offset of (row, logical 16-byte chunk c) in a 128-byte-row LDS stage
__device__ __forceinline__ int lds_off(int row, int c) { return row * kRow + ((c ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ u32x4 lds16(const uint8_t* L, int off) { return *reinterpret_cast<const u32x4*>(L + off); }

__device__ __forceinline__ v8i cat8(u32x4 lo, u32x4 hi) {
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}


// Global -> LDS copies.  Each lane's bytes land at M0 + size * lane; M0 must
// be wave-uniform.  Issued as inline asm so that the only waits on them are
// the explicit vmcnt_wait below (the compiler would otherwise drain every
// outstanding copy before each LDS read).  The main loop issues no other
// vector-memory instruction, so vmcnt counts exactly these copies.  The
// 16-byte copies take a wave-uniform 64-bit base (scalar registers) plus a
// 32-bit per-lane offset, which keeps one VGPR per copy stream.
__device__ __forceinline__ void dma16(uint32_t off, const void* base, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
}
// the same with the non-temporal policy (lines that are read once and
// should not displace reused lines in L2)
__device__ __forceinline__ void dma16_nt(uint32_t off, const void* base, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "s"(lds_addr)
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

// compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>)
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Raw buffer resource over one output tile (stride 0, byte-range checked;
// the offsets of one tile always fit in 32 bits)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), 0x7fffffff, 0x00020000);
}

template <int MODE, bool GATEUP, int BM, int TN>
__global__ void __launch_bounds__(nw_of(MODE, BM) * 64, 1) grouped_gemm_kernel(const GemmArgs p) {
    constexpr int ELEM = MODE == MOE_QUANT_NONE_BF16 ? 2 : 1;
    constexpr bool MX = MODE == MOE_QUANT_MXFP4;
    constexpr int NW = nw_of(MODE, BM), NT = NW * 64;
    constexpr int WM = wm_of(BM), WN = NW / WM;
    constexpr int TM = BM / (32 * WM);
    constexpr int WCOLS = TN * 32;              // weight rows per wave
    constexpr int NROWS = WN * WCOLS;           // weight rows per workgroup
    constexpr int HALF = WCOLS / 2;             // gate_up: gate (and up) rows per wave
    constexpr int TILE_N = GATEUP ? WN * HALF : NROWS;   // output columns per workgroup
    constexpr bool BLOCKQ = MODE == MOE_QUANT_BLOCK128_FP8;
    constexpr int STAGE = (BM + NROWS) * kRow;
    // LDS stages: 2 where that lets two workgroups share a CU (one's
    // prologue and epilogue then overlap the other's main loop), else 3 if
    // they fit
    constexpr int NS = 2 * STAGE + 4096 <= 80 * 1024 ? 2 : (3 * STAGE <= kLdsBudget ? 3 : 2);
    constexpr int A_IN = BM / (8 * NW);         // copies (8 rows x 128 B) of A per wave per step
    constexpr int B_IN = NROWS / (8 * NW);      // copies of B per wave per step
    // MXFP4: each row has 8 scale bytes (two dwords) per 128-byte step; a
    // copy moves 64 dwords, and every wave issues the same number (dwords
    // past the tile's rows land in padding slots)
    constexpr int AS_IN = MX ? (2 * BM + 64 * NW - 1) / (64 * NW) : 0;
    constexpr int WS_IN = MX ? (2 * NROWS + 64 * NW - 1) / (64 * NW) : 0;
    constexpr int N_BIG = A_IN + B_IN + (BLOCKQ ? 1 : 0) + AS_IN + WS_IN;   // copies per wave per step
    static_assert(TM >= 1 && A_IN >= 1 && B_IN >= 1 && BM % (8 * NW) == 0 && NROWS % (8 * NW) == 0 && BM <= 256 &&
                      2 * STAGE <= kLdsBudget && (!BLOCKQ || BM <= 64 * NW),
                  "tile shape");

    __shared__ __attribute__((aligned(16))) uint8_t lds[NS * STAGE];
    __shared__ float s_rowscale[BM];          // PTPC: row scale; other modes: row mask (pad rows 0)
    // blockwise: row scales of a stage (wave w copies rows 64w .. 64w + 63)
    __shared__ __attribute__((aligned(16))) float s_ascale[BLOCKQ ? NS : 1][BLOCKQ ? 64 * NW : 1];
    __shared__ int s_tok[BM];
    // PTPC: channel scales of the tile's output columns (gate_up: gate, then up)
    __shared__ __attribute__((aligned(16))) float s_chs[MODE == MOE_QUANT_PTPC_FP8 ? (GATEUP ? 2 : 1) * TILE_N : 1];
    __shared__ float s_wscale[BLOCKQ ? WN * TN : 1][BLOCKQ ? 128 : 1];   // blockwise: weight scales of the tile
    // MXFP4: the step's scale dwords, slot 2 row + half (activation rows) and
    // 2 t + half (weight row t of the tile)
    __shared__ __attribute__((aligned(16))) uint32_t s_asc[MX ? NS : 1][MX ? 64 * NW * AS_IN : 1];
    __shared__ __attribute__((aligned(16))) uint32_t s_wsc[MX ? NS : 1][MX ? 64 * NW * WS_IN : 1];

    // tile order: expert-major, weight tile, then row block; each XCD takes
    // a contiguous eighth of the tiles that hold rows (the grid covers the
    // worst case; workgroups past the real count exit at once)
    const int n_valid = p.offsets[p.n_exp] / BM * p.n_ntiles;
    const int per = (n_valid + 7) >> 3;
    const int lt = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (blockIdx.x >> 3 >= per || lt >= n_valid) return;
    const int e = p.block_expert[lt / p.n_ntiles];
    if (e < 0) return;
    const int bs = p.offsets[e] / BM, nb = p.offsets[e + 1] / BM - bs;
    const int local = lt - bs * p.n_ntiles;
    const int nt = local / nb, mb = bs + local % nb;
    const int m0 = mb * BM;
    const int n0 = nt * TILE_N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int q = lane >> 5, r32 = lane & 31;
    const int arow = wm * TM * 32;            // first tile row of this wave
    // rows of the block that hold routed rows (the expert's pads follow them)
    const int live = p.counts ? min(BM, max(0, p.offsets[e] + p.counts[e] - m0)) : BM;

    // Copy j of a wave fills 8 LDS rows of block wave + NW*j: lane i writes
    // row 8*blk + i/8, physical chunk i%8, which holds logical chunk
    // (i%8) ^ swizzle(row) of that row.
    const int crow = lane >> 3, cphys = lane & 7;
    // weight tile row t (LDS row BM + t) is row t % WCOLS of wave column t / WCOLS
    // (gate rows first, then up rows)
    const uint8_t* wexp = p.w + static_cast<int64_t>(e) * p.w_expert_bytes;
    const int64_t wrow_bytes = MX ? static_cast<int64_t>(p.K) / 2 : static_cast<int64_t>(p.K) * ELEM;
    const int nbig = static_cast<int>(wrow_bytes / kRow);   // steps; K bytes are a multiple of 128
    uint32_t b_src[B_IN];                                   // byte offsets within the expert
#pragma unroll
    for (int j = 0; j < B_IN; ++j) {
        const int t = (wave + NW * j) * 8 + crow;
        const int c = cphys ^ (((BM + t) >> 1) & 7);
        const int w = t / WCOLS, jj = t % WCOLS;
        const int wr = GATEUP ? (jj < HALF ? n0 + w * HALF + jj : p.I + n0 + w * HALF + jj - HALF) : n0 + t;
        // blocked weights: the 8 rows of a copy are half of one 2 KB block
        // (16 rows x one 128-byte step), 8 whole lines of it
        b_src[j] = static_cast<uint32_t>(p.w_blocked ? (wr >> 4) * (wrow_bytes / kRow) * 2048 + blocked_byte(wr & 15, c * 16)
                                                     : wr * wrow_bytes + c * 16);
    }
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    // weight copy j of step S into LDS stage BUF.  The 192-row tile is the
    // library's choice when an expert's rows fit about one tile, so each
    // weight line is read once: non-temporal, keeping the activation rows
    // that the expert's weight tiles share in L2 (512-expert top-10 layer
    // 1.903 -> 1.850 ms; where an expert spans several row blocks the weight
    // lines are reused and this policy made the Qwen3-235B-shaped gate/up
    // GEMM slower)
    auto issue_b = [&](int j, int S, int buf) {
        const int64_t kw = static_cast<int64_t>(S) * (p.w_blocked ? 2048 : kRow);   // step offset in the weights
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + buf * STAGE + (BM + (wave + NW * j) * 8) * kRow);
        if constexpr (BM == 192) dma16_nt(b_src[j], wexp + kw, dst);
        else dma16(b_src[j], wexp + kw, dst);
    };
    // Two stages without scale copies (PTPC and bf16): the weight copies of
    // steps 0 and 1 and a copy of the tile's row ids into LDS go out before
    // any other vector-memory access, so the weights' HBM latency overlaps
    // the row ids' round trip instead of following it.  A wave reads back
    // only the ids its own copy brought, once at most its weight copies are
    // still in flight.
    constexpr bool EARLY_B = NS == 2 && !BLOCKQ && !MX;
    if constexpr (EARLY_B) {
        if (p.sorted_ids && tid < BM)
            dma4(p.sorted_ids + m0 + tid, __builtin_amdgcn_readfirstlane(
                                              static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s_tok)) + (tid & ~63) * 4));
        for (int S = 0; S < NS; ++S)
            if (S < nbig) {
#pragma unroll
                for (int j = 0; j < B_IN; ++j) issue_b(j, S, S);
            }
        if (p.sorted_ids) {
            if (nbig >= 2) vmcnt_wait<2 * B_IN>();
            else vmcnt_wait<B_IN>();
        }
    }

    // Row tokens go to LDS before the activation copies can start.  The PTPC
    // row and channel scales are only needed by the epilogue: their loads go
    // out here but land in LDS after the main loop, so the copies do not
    // wait for them.
    constexpr bool PTPC = MODE == MOE_QUANT_PTPC_FP8;
    constexpr int CHN = PTPC ? (GATEUP ? 2 : 1) * TILE_N : 0;    // channel scales of the tile
    constexpr int CH_PER = (CHN + NT - 1) / NT;
    float rs = 0.0f, rsv = 0.0f, chv[CH_PER > 0 ? CH_PER : 1];
    if (tid < BM) {
        // rows past `live` are pads: down reads the block's first row for
        // them (no HBM traffic for pad rows) and masks them out
        int tok = tid < live ? m0 + tid : m0;
        rs = tid < live ? 1.0f : 0.0f;
        if (p.sorted_ids) {
            int f;
            if constexpr (EARLY_B) f = s_tok[tid];
            else f = p.sorted_ids[m0 + tid];
            const bool pad = f == p.sentinel;
            tok = pad ? 0 : (f < p.TK ? f / p.topk : f - p.TK);
            rs = pad ? 0.0f : 1.0f;
        }
        s_tok[tid] = tok;
        if constexpr (PTPC) rsv = p.a_scale[tok];
        else s_rowscale[tid] = rs;
    }
    if constexpr (PTPC) {
        const float* ws = p.w_scale + e * p.ws_expert;
#pragma unroll
        for (int j = 0; j < CH_PER; ++j) {
            const int i = tid + j * NT;
            chv[j] = i < CHN ? ws[i < TILE_N ? n0 + i : p.I + n0 + i - TILE_N] : 0.0f;
        }
    }
    auto publish_scales = [&]() __attribute__((always_inline)) {
        if constexpr (PTPC) {
            // (the empty asm keeps the compiler from applying the row mask,
            // and so waiting for the load, back where the load is issued)
            asm volatile("" : "+v"(rsv));
            if (tid < BM) s_rowscale[tid] = rs == 0.0f ? 0.0f : rsv;
#pragma unroll
            for (int j = 0; j < CH_PER; ++j)
                if (tid + j * NT < CHN) s_chs[tid + j * NT] = chv[j];
        }
    };
    __syncthreads();

    uint32_t a_src[A_IN];                                   // byte offsets within the activations
#pragma unroll
    for (int j = 0; j < A_IN; ++j) {
        const int r = (wave + NW * j) * 8 + crow;
        const int c = cphys ^ ((r >> 1) & 7);
        a_src[j] = static_cast<uint32_t>(static_cast<int64_t>(s_tok[r]) * p.a_ld + c * 16);
    }
    // With two stages every in-loop wait is for all outstanding copies, so a
    // wave may leave out the copies of its 8-row groups that lie in 32-row
    // tiles made only of pads (no MFMA reads them); only the prologue's wait
    // depends on how many copies a step issues.
    constexpr bool SKIP_DEAD = NS == 2;
    const int live32 = min(BM, (live + 31) & ~31);
    bool a_need[A_IN];
    int n_dead = 0;
#pragma unroll
    for (int j = 0; j < A_IN; ++j) {
        a_need[j] = __builtin_amdgcn_readfirstlane((wave + NW * j) * 8 < live32 ? 1 : 0) != 0;
        n_dead += a_need[j] ? 0 : 1;
    }
    // blockwise: wave w copies the scales of rows 64w .. 64w+63 (rows past BM
    // read row 0 into unused slots)
    const float* sc_src = nullptr;
    if constexpr (BLOCKQ) {
        const int r = wave * 64 + lane;
        sc_src = p.a_scale + static_cast<int64_t>(s_tok[r < BM ? r : 0]) * p.a_scale_ld;
    }
    // MXFP4 scale copies: lane source addresses (the step adds 8 bytes)
    const uint8_t* as_src[AS_IN > 0 ? AS_IN : 1];
    const uint8_t* ws_src[WS_IN > 0 ? WS_IN : 1];
    if constexpr (MX) {
        const int kb = p.K >> 5;                            // scale bytes per row
#pragma unroll
        for (int j = 0; j < AS_IN; ++j) {
            int d = 64 * (wave + NW * j) + lane;
            d = d < 2 * BM ? d : d % (2 * BM);
            as_src[j] = p.a_mx + static_cast<int64_t>(s_tok[d >> 1]) * kb + 4 * (d & 1);
        }
#pragma unroll
        for (int j = 0; j < WS_IN; ++j) {
            int d = 64 * (wave + NW * j) + lane;
            d = d < 2 * NROWS ? d : d % (2 * NROWS);
            const int t = d >> 1, w = t / WCOLS, jj = t % WCOLS;
            const int wr = GATEUP ? (jj < HALF ? n0 + w * HALF + jj : p.I + n0 + w * HALF + jj - HALF) : n0 + t;
            ws_src[j] = p.w_mx + e * p.w_mx_expert + static_cast<int64_t>(wr) * kb + 4 * (d & 1);
        }
    }
    const uint32_t sc0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_ascale[0][0]));
    const uint32_t asc0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_asc[0][0]));
    const uint32_t wsc0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_wsc[0][0]));

    // copy D (0 .. N_BIG-1) of step S into LDS stage BUF (uniform M0 per copy)
    auto issue_one = [&](auto D, int S, int buf) {
        constexpr int d = decltype(D)::value;
        const int64_t ko = static_cast<int64_t>(S) * kRow;
        const uint32_t st = lds0 + buf * STAGE;
        if constexpr (d < A_IN) {
            if (!SKIP_DEAD || a_need[d])
                dma16(a_src[d], p.a + ko, __builtin_amdgcn_readfirstlane(st + (wave + NW * d) * 8 * kRow));
        } else if constexpr (d < A_IN + B_IN) {
            issue_b(d - A_IN, S, buf);
        } else if constexpr (BLOCKQ && d == A_IN + B_IN) {
            dma4(sc_src + S, __builtin_amdgcn_readfirstlane(sc0 + (buf * 64 * NW + wave * 64) * 4));
        } else if constexpr (MX && d < A_IN + B_IN + AS_IN) {
            constexpr int j = d - A_IN - B_IN;
            dma4(as_src[j] + 8 * S,
                 __builtin_amdgcn_readfirstlane(asc0 + (buf * 64 * NW * AS_IN + 64 * (wave + NW * j)) * 4));
        } else if constexpr (MX) {
            constexpr int j = d - A_IN - B_IN - AS_IN;
            dma4(ws_src[j] + 8 * S,
                 __builtin_amdgcn_readfirstlane(wsc0 + (buf * 64 * NW * WS_IN + 64 * (wave + NW * j)) * 4));
        }
    };
    auto issue = [&](int S) { static_for<N_BIG>([&](auto D) { issue_one(D, S, S % NS); }); };

    // this wave's weight rows (first global row of each 32-row tile)
    auto wrow_of = [&](int w, int tn) {
        return GATEUP ? (tn < TN / 2 ? n0 + w * HALF + tn * 32 : p.I + n0 + w * HALF + (tn - TN / 2) * 32)
                      : n0 + w * WCOLS + tn * 32;
    };
    const int brow = BM + wn * WCOLS + r32;    // LDS row of this lane's weight row in tile 0

    // blockwise: the weight scales of this tile, [wave column * TN + tn][K block]
    if constexpr (BLOCKQ) {
        for (int idx = tid; idx < WN * TN * nbig; idx += NT) {
            const int t = idx / nbig, kb = idx - t * nbig;
            s_wscale[t][kb] = p.w_scale[e * p.ws_expert + (wrow_of(t / TN, t % TN) >> 7) * p.ws_ld + kb];
        }
    }

    v16f acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = v16f{};
    // Operand fragments, double-buffered in registers: set X holds the two
    // 16-byte chunks of this lane's rows for one half-step.
    u32x4 fa[2][TM][2], fb[2][TN][2];
    uint32_t asw[2][MX ? TM : 1], wsw[2][MX ? TN : 1];      // MXFP4 scale words, double-buffered like the fragments

    // Row tiles of this wave that hold at least one routed row: 32-row tiles
    // made only of pads get no operand reads and no MFMAs (their
    // accumulators stay 0).  The wave still issues its share of the weight
    // copies (other waves read them), and of the activation copies unless
    // SKIP_DEAD leaves out those of pad-only tiles.
    const int ta = __builtin_amdgcn_readfirstlane(min(TM, max(0, (live - arow + 31) >> 5)));

    // The main loop for TA live row tiles (TA is uniform over the tile's K
    // sweep, so each variant is branch-free).
    auto run = [&](auto TAc) __attribute__((always_inline)) {
        constexpr int TA = decltype(TAc)::value;
        // LDS reads per half-step (none without live rows) and MFMAs
        // (MXFP4: plus one scale word per row tile and weight tile)
        constexpr int NLF = TA > 0 ? 2 * (TA + TN) : 0;
        constexpr int NL = NLF + (MX && TA > 0 ? TA + TN : 0);
        constexpr int NM = (MODE == MOE_QUANT_NONE_BF16 || MX ? 2 : 1) * TA * TN;

        // LDS read L (0 .. NL-1) of half-step H of the step in stage BUF into
        // set X, in the order the MFMAs consume them: weight tile 0, the row
        // tiles, then the other weight tiles (the MFMAs run weight tile by
        // weight tile)
        auto load_one = [&](auto X, auto Lc, int buf, int h) {
            constexpr int l = decltype(Lc)::value, x = decltype(X)::value;
            const uint8_t* L = lds + buf * STAGE;
            if constexpr (l >= NLF) {
                // MXFP4 scale words of half-step h: the row's dword h holds
                // the scales of K blocks 4h .. 4h+3; shifted by 16 q, bytes 0
                // and 1 are this lane's blocks 4h + 2q and 4h + 2q + 1
                constexpr int i = l - NLF;
                if constexpr (i < TA) {
                    asw[x][i] = s_asc[buf][2 * (arow + i * 32 + r32) + h] >> (16 * q);
                } else {
                    wsw[x][i - TA] = s_wsc[buf][2 * (wn * WCOLS + (i - TA) * 32 + r32) + h] >> (16 * q);
                }
            } else if constexpr (l >= 2 && l < 2 + 2 * TA) {
                constexpr int tm = (l - 2) / 2, c = (l - 2) % 2;
                fa[x][tm][c] = lds16(L, lds_off(arow + tm * 32 + r32, 4 * h + 2 * q + c));
            } else {
                constexpr int lb = l < 2 ? l : l - 2 * TA;
                constexpr int tn = lb / 2, c = lb % 2;
                fb[x][tn][c] = lds16(L, lds_off(brow + tn * 32, 4 * h + 2 * q + c));
            }
        };

        // Blockwise scales.  A 128-byte step is one 128-element scale block;
        // the MFMAs accumulate straight into acc, kept in units of the current
        // block's scale a_scale(row, kb) * w_scale(n-block, kb): at the start
        // of block kb each tile's acc is multiplied by
        // (scale of block kb-1) / (scale of block kb), and after the last
        // block by that block's scale.  The lane's activation row is fixed
        // (row r32 of each row tile) and the weight scale is uniform over a
        // 32-row weight tile, so each factor is one float per (tm, tn).
        float pa[BLOCKQ ? TM : 1], pw[BLOCKQ ? TN : 1], ra[BLOCKQ ? TM : 1], rw[BLOCKQ ? TN : 1];
        auto step_scales = [&](int buf, int kb) {
            if constexpr (BLOCKQ) {
#pragma unroll
                for (int tm = 0; tm < TA; ++tm) {
                    const float a = s_ascale[buf][arow + tm * 32 + r32];
                    ra[tm] = pa[tm] * __builtin_amdgcn_rcpf(a);   // ratio to 1 ulp; the chain stays ~1e-6
                    pa[tm] = a;
                }
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    const float w = s_wscale[wn * TN + tn][kb];
                    rw[tn] = pw[tn] * __builtin_amdgcn_rcpf(w);
                    pw[tn] = w;
                }
            }
        };

        // MFMA J (0 .. NM-1) of a half-step from fragment set X; in the first
        // half of a blockwise step the tile's acc is rescaled just before its
        // first MFMA (its last MFMA of the previous step issued NM MFMAs ago)
        auto mma_one = [&](auto X, auto J, auto H0) {
            constexpr int j = decltype(J)::value, x = decltype(X)::value;
            if constexpr (MODE == MOE_QUANT_NONE_BF16) {
                constexpr int c = j / (TA * TN), tn = (j % (TA * TN)) / TA, tm = j % TA;
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fb[x][tn][c]),
                                                                      __builtin_bit_cast(v8bf, fa[x][tm][c]),
                                                                      acc[tm][tn], 0, 0, 0);
            } else if constexpr (MX) {
                // chunk c (16 bytes = 32 E2M1 elements = one scale block) of
                // both operands; format selectors 4 (FP4) for both, scale
                // byte c of each lane's shifted scale word
                constexpr int c = j / (TA * TN), tn = (j % (TA * TN)) / TA, tm = j % TA;
                const u32x4 z = {0u, 0u, 0u, 0u};
                acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    cat8(fb[x][tn][c], z), cat8(fa[x][tm][c], z), acc[tm][tn], 4, 4, c,
                    static_cast<int>(wsw[x][tn]), c, static_cast<int>(asw[x][tm]));
            } else {
                constexpr int tn = j / TA, tm = j % TA;
                if constexpr (BLOCKQ && decltype(H0)::value) {
                    const float r = ra[tm] * rw[tn];
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[tm][tn][i] *= r;
                }
                const v8i av = cat8(fa[x][tm][0], fa[x][tm][1]), bv = cat8(fb[x][tn][0], fb[x][tn][1]);
                // e4m3 x e4m3 (format selectors 0, 0), no hardware block
                // scaling: zero immediates select the unscaled
                // v_mfma_f32_32x32x64_f8f6f4 (a scale byte of 0 passed at run
                // time would mean 2^-127)
                acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[tm][tn], 0, 0, 0, 0, 0, 0);
            }
        };

        // One half-step: its MFMAs from set X, issued one at a time, each
        // followed by its share of the NL reads of the next half-step (into
        // the other set, from stage RBUF, half RH; when RD) and of the ND
        // copies [D0, D0 + ND) of step CS (when CP), so that a memory
        // instruction that stalls at issue overlaps a running MFMA.
        auto half_step = [&](auto X, auto H0, auto D0c, auto NDc, bool rd, int rbuf, int rh, bool cp, int cs) {
            constexpr int D0 = decltype(D0c)::value, ND = decltype(NDc)::value;
            using XN = std::integral_constant<int, 1 - decltype(X)::value>;
            if constexpr (NM == 0) {
                if (cp) static_for<ND>([&](auto D) {
                    issue_one(std::integral_constant<int, D0 + decltype(D)::value>{}, cs, cs % NS);
                });
            } else {
                static_for<NM>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    mma_one(X, J, H0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (rd) {
                        static_for<(j + 1) * NL / NM - j * NL / NM>([&](auto L) {
                            load_one(XN{}, std::integral_constant<int, j * NL / NM + decltype(L)::value>{}, rbuf, rh);
                        });
                    }
                    if (cp) {
                        static_for<(j + 1) * ND / NM - j * ND / NM>([&](auto D) {
                            issue_one(std::integral_constant<int, D0 + j * ND / NM + decltype(D)::value>{}, cs,
                                      cs % NS);
                        });
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
        };

        // Prologue: steps 0 .. NS-1 go out (every stage is free; with early
        // weight copies only their activation copies are left); wait for
        // step 0, then read the fragments of its first half.
        for (int S = 0; S < NS; ++S)
            if (S < nbig) {
                if constexpr (EARLY_B) static_for<A_IN>([&](auto D) { issue_one(D, S, S); });
                else issue(S);
            }
        if (EARLY_B && NS <= nbig) {
            // in flight after step 0's activation copies: those of step 1
            static_for<A_IN + 1>([&](auto Dc) {
                if (n_dead == decltype(Dc)::value) vmcnt_wait<A_IN - decltype(Dc)::value>();
            });
        } else if (NS <= nbig) {
            // wait for step 0; the copies of steps 1 .. NS-1 may stay in flight
            if constexpr (SKIP_DEAD) {
                static_for<A_IN + 1>([&](auto Dc) {
                    if (n_dead == decltype(Dc)::value) vmcnt_wait<(NS - 1) * (N_BIG - decltype(Dc)::value)>();
                });
            } else {
                vmcnt_wait<(NS - 1) * N_BIG>();
            }
        } else {
            vmcnt_wait<0>();
        }
        __syncthreads();
        static_for<NL>([&](auto L) { load_one(std::integral_constant<int, 0>{}, L, 0, 0); });
        if constexpr (BLOCKQ) {
#pragma unroll
            for (int tm = 0; tm < TA; ++tm) pa[tm] = s_ascale[0][arow + tm * 32 + r32];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) pw[tn] = s_wscale[wn * TN + tn][0];
        }

        // Step S (stage S % NS, landed and published):
        //   first half: MFMAs from set 0; read the second half of S into set
        //     1; wait until step S + 1 has landed (copies issued after it may
        //     stay in flight) and barrier: publishes S + 1 and releases stage
        //     S.
        //   second half: MFMAs from set 1; read the first half of S + 1 into
        //     set 0; issue all copies of step S + NS (into stage S), so each
        //     step's copies have NS - 1 whole steps to land (issuing half of
        //     them a half-step later, as a way to spread the copies over
        //     both halves, left those only half a step and was 5 % slower).
        using X0 = std::integral_constant<int, 0>;
        using X1 = std::integral_constant<int, 1>;
        using First = std::integral_constant<bool, true>;
        using Second = std::integral_constant<bool, false>;
        for (int S = 0; S < nbig; ++S) {
            const int buf = S % NS;
            const bool next = S + 1 < nbig;
            const bool cp2 = S + NS - 1 < nbig, cp1 = S + NS < nbig;
            step_scales(buf, S);
            half_step(X0{}, First{}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, true,
                      buf, 1, false, 0);
            if (next) {
                if (cp2) vmcnt_wait<(NS - 2) * N_BIG>();
                else vmcnt_wait<0>();
                __syncthreads();
            }
            // the reads of the next step's first half are issued even after
            // the last step (they then read an idle stage into registers no
            // MFMA uses): a branch around them would make the compiler wait
            // for every outstanding LDS read before the MFMAs that follow
            half_step(X1{}, Second{}, std::integral_constant<int, 0>{}, std::integral_constant<int, N_BIG>{}, true,
                      (S + 1) % NS, 0, cp1, S + NS);
        }
        vmcnt_wait<0>();
        if constexpr (BLOCKQ) {
#pragma unroll
            for (int tm = 0; tm < TA; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    const float r = pa[tm] * pw[tn];
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[tm][tn][i] *= r;
                }
        }
    };

    // ------------------------------------------------------------ epilogue
    // (called at the end of each main-loop variant, so that no variant's
    // accumulators meet another's at a join point)
    // TA: this wave's row tiles that hold routed rows; the tiles after them
    // hold only pads and are not written (their rows' contents are
    // unspecified: nothing reads pad rows of act or out_perm)
    auto epilogue = [&](auto TAc) __attribute__((always_inline)) {
        constexpr int TA = decltype(TAc)::value;
        // The MFMAs take the weight rows as their first operand, so lane
        // (r32, q) holds row r32 of each 32-row tile and, in register
        // i = 4g + j, output column 8g + 4q + j of each 32-column tile: four
        // consecutive columns per g.  Per row tile, each wave packs them into
        // 8 (bf16) or 16 (fp32) bytes, writes them row-major into its own LDS
        // region (rows padded by 16 bytes), reads them back as 16-byte row
        // pieces and stores whole 128-byte lines through a buffer resource
        // based at the tile's first row.  The LDS regions reuse the stages: a
        // barrier first lets every wave finish its last operand reads.
        constexpr int OBYTES = (!GATEUP && MODE == MOE_QUANT_NONE_BF16) ? 4 : 2;
        constexpr int CW = GATEUP ? HALF : WCOLS;            // output columns per wave
        constexpr int RB = CW * OBYTES;                       // bytes of one output row of the wave
        constexpr int RBP = RB + 16;                          // padded LDS row stride
        constexpr int LPR = RB / 16;                          // lanes per row on the way out
        constexpr int RPI = 64 / LPR;                         // rows per store instruction
        static_assert(64 % LPR == 0 && 32 % RPI == 0 && NW * 32 * RBP <= NS * STAGE, "epilogue layout");
        publish_scales();
        __syncthreads();
        uint8_t* reg = lds + wave * 32 * RBP;
        const int ldb = static_cast<int>(p.out_ld) * OBYTES;          // bytes per output row
        const __amdgpu_buffer_rsrc_t rsrc =
            tile_rsrc(static_cast<uint8_t*>(p.out) + static_cast<int64_t>(m0) * p.out_ld * OBYTES);
        // first output column of this wave
        const int col0 = GATEUP ? n0 + wn * HALF : n0 + wn * WCOLS;
        // channel scales of this lane's columns (tile t, group g: four
        // consecutive columns), read from LDS where they are used
        auto chs = [&](int t, int g, bool up) {
            if constexpr (MODE == MOE_QUANT_PTPC_FP8)
                return *reinterpret_cast<const float4*>(&s_chs[(up ? TILE_N : 0) + col0 - n0 + t * 32 + 8 * g + 4 * q]);
            else
                return float4{1.0f, 1.0f, 1.0f, 1.0f};
        };
    #pragma unroll
        for (int tm = 0; tm < TA; ++tm) {
            const float rs = s_rowscale[arow + tm * 32 + r32];
            // pack this row tile into the wave's region
    #pragma unroll
            for (int t = 0; t < (GATEUP ? TN / 2 : TN); ++t)
    #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
                    const float4 sa = chs(t, g, false);
                    const float sav[4] = {sa.x, sa.y, sa.z, sa.w};
    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (GATEUP) {
                            const float4 sb = chs(t, g, true);
                            const float sbv[4] = {sb.x, sb.y, sb.z, sb.w};
                            v[j] = silu_mul(acc[tm][t][4 * g + j] * rs * sav[j], acc[tm][t + TN / 2][4 * g + j] * rs * sbv[j]);
                        } else {
                            v[j] = acc[tm][t][4 * g + j] * rs * sav[j];
                        }
                    }
                    uint8_t* dst = reg + r32 * RBP + (t * 32 + 8 * g + 4 * q) * OBYTES;
                    if constexpr (OBYTES == 2) {
                        *reinterpret_cast<uint2*>(dst) = uint2{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])};
                    } else {
                        *reinterpret_cast<float4*>(dst) = float4{v[0], v[1], v[2], v[3]};
                    }
                }
            // read back 16-byte row pieces and store whole lines (the wave's
            // LDS operations complete in order, so the next row tile's writes
            // cannot overtake these reads)
    #pragma unroll
            for (int it = 0; it < 32 / RPI; ++it) {
                const int row = it * RPI + lane / LPR, ch = lane % LPR;
                const u32x4 d = *reinterpret_cast<const u32x4*>(reg + row * RBP + ch * 16);
                // non-temporal (cache policy bit 1): the output is read once, by
                // the next kernel, and should not displace the operands that
                // running tiles share through L2 (down GEMM 0.549 -> 0.537 ms,
                // blockwise layer 1.17 -> 1.11 ms)
                __builtin_amdgcn_raw_buffer_store_b128(d, rsrc, (arow + tm * 32 + row) * ldb + col0 * OBYTES + ch * 16, 0, 2);
            }
        }
    };
    static_for<TM + 1>([&](auto TAc) {
        if (ta == decltype(TAc)::value) {
            run(TAc);
            epilogue(TAc);
        }
    });
}

template <int MODE, bool GATEUP, int TN>
static int32_t launch_bm(int block_m, const GemmArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(ceil_div(a.n_tiles, 8) * 8));
    if (block_m == 32) {
        hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 32, TN>), grid, dim3(nw_of(MODE, 32) * 64), 0, s, a);
        return moe_launch_status();
    }
    {
        if (block_m == 64) {
            hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 64, TN>), grid, dim3(nw_of(MODE, 64) * 64), 0, s,
                               a);
            return moe_launch_status();
        }
        if constexpr (TN == 2 || nw_of(MODE, 128) == 4) {   // tn_of gives the 8-wave 128-row tile 2
            if (block_m == 128) {
                hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 128, TN>), grid, dim3(nw_of(MODE, 128) * 64), 0,
                                   s, a);
                return moe_launch_status();
            }
        }
        if constexpr (TN == 2 && MODE != MOE_QUANT_NONE_BF16) {
            if (block_m == 192) {
                hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 192, TN>), grid, dim3(nw_of(MODE, 192) * 64), 0,
                                   s, a);
                return moe_launch_status();
            }
        }
        if constexpr (TN == 2 && MODE != MOE_QUANT_MXFP4) {   // tn_of gives the 256-row tile 2 weight tiles per wave
            if (block_m == 256) {
                hipLaunchKernelGGL((grouped_gemm_kernel<MODE, GATEUP, 256, TN>), grid, dim3(nw_of(MODE, 256) * 64), 0,
                                   s, a);
                return moe_launch_status();
            }
        }
    }
    return MOE_ERR_UNSUPPORTED;
}

template <bool GATEUP>
static int32_t launch_mode(int quant, int tn, int block_m, const GemmArgs& a, hipStream_t s) {
    if (a.n_tiles == 0) return MOE_OK;
    switch (quant) {
        case MOE_QUANT_NONE_BF16: return launch_bm<MOE_QUANT_NONE_BF16, GATEUP, 2>(block_m, a, s);
        case MOE_QUANT_PTPC_FP8:
            return tn == 4 ? launch_bm<MOE_QUANT_PTPC_FP8, GATEUP, 4>(block_m, a, s)
                           : launch_bm<MOE_QUANT_PTPC_FP8, GATEUP, 2>(block_m, a, s);
        case MOE_QUANT_BLOCK128_FP8: return launch_bm<MOE_QUANT_BLOCK128_FP8, GATEUP, 2>(block_m, a, s);
        case MOE_QUANT_MXFP4:
            return tn == 4 ? launch_bm<MOE_QUANT_MXFP4, GATEUP, 4>(block_m, a, s)
                           : launch_bm<MOE_QUANT_MXFP4, GATEUP, 2>(block_m, a, s);
    }
    return MOE_ERR_UNSUPPORTED;
}

int32_t stream_gateup_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T,
                             const int* sorted_ids, const int* offsets, const int* counts, void* act,
                             hipStream_t s);
int32_t stream_down_launch(const moe_layer_desc* L, const void* act, const float* act_scale, int T,
                           const int* offsets, const int* counts, void* out_perm, hipStream_t s, bool act_blocked);

int32_t gemm_gateup_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T, int block_m,
                           int64_t max_rows, const int* sorted_ids, const int* block_expert, const int* offsets,
                           const int* counts, void* act, hipStream_t s) {
    if (block_m == 16) return stream_gateup_launch(L, a, a_scale, T, sorted_ids, offsets, counts, act, s);
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    // the copies address activations and one expert's weights with 32-bit
    // offsets: the C ABI has checked the byte ranges before any launch
    const bool mx = L->quant == MOE_QUANT_MXFP4;
    GemmArgs g{};
    g.offsets = offsets;
    g.counts = counts;
    g.a = static_cast<const uint8_t*>(a);
    g.a_ld = mx ? L->D / 2 : static_cast<int64_t>(L->D) * elem;
    if (mx) {
        g.a_mx = reinterpret_cast<const uint8_t*>(a_scale);
        g.w_mx = reinterpret_cast<const uint8_t*>(L->w13_scale);
        g.w_mx_expert = 2LL * L->I * (L->D / 32);
    }
    g.a_scale = a_scale;
    g.a_scale_ld = L->D / 128;
    g.sorted_ids = sorted_ids;
    g.topk = L->top_k;
    g.TK = T * L->top_k;
    g.sentinel = T * (L->top_k + L->n_shared);
    g.block_expert = block_expert;
    g.w = static_cast<const uint8_t*>(L->w13);
    g.w_blocked = L->weight_layout == MOE_WEIGHTS_BLOCKED;
    g.w_expert_bytes = mx ? static_cast<int64_t>(L->I) * L->D : static_cast<int64_t>(2) * L->I * L->D * elem;
    g.w_scale = L->w13_scale;
    g.ws_expert = L->quant == MOE_QUANT_PTPC_FP8 ? 2LL * L->I
                                                  : static_cast<int64_t>(2 * L->I / 128) * (L->D / 128);
    g.ws_ld = L->D / 128;
    g.K = L->D;
    g.I = L->I;
    g.out = act;
    g.out_ld = L->I;
    const int tn = tn_of(L->quant, 2 * L->I, block_m);
    g.n_ntiles = L->I / ((nw_of(L->quant, block_m) / wm_of(block_m)) * tn * 16);
    g.n_tiles = static_cast<int>(max_rows / block_m) * g.n_ntiles;
    g.n_exp = L->E + L->n_shared;
    return launch_mode<true>(L->quant, tn, block_m, g, s);
}

int32_t gemm_down_launch(const moe_layer_desc* L, const void* act, const float* act_scale, int T, int block_m,
                         int64_t max_rows, const int* block_expert, const int* offsets, const int* counts,
                         void* out_perm, hipStream_t s, bool act_blocked) {
    if (block_m == 16) return stream_down_launch(L, act, act_scale, T, offsets, counts, out_perm, s, act_blocked);
    if (act_blocked) return MOE_ERR_UNSUPPORTED;   // only the streaming kernel reads blocked act codes
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    const bool mx = L->quant == MOE_QUANT_MXFP4;
    GemmArgs g{};
    g.offsets = offsets;
    g.counts = counts;
    g.a = static_cast<const uint8_t*>(act);
    g.a_ld = mx ? L->I / 2 : static_cast<int64_t>(L->I) * elem;
    if (mx) {
        g.a_mx = reinterpret_cast<const uint8_t*>(act_scale);
        g.w_mx = reinterpret_cast<const uint8_t*>(L->w2_scale);
        g.w_mx_expert = static_cast<int64_t>(L->D) * (L->I / 32);
    }
    g.a_scale = act_scale;
    g.a_scale_ld = L->I / 128;
    g.sorted_ids = nullptr;
    g.block_expert = block_expert;
    g.w = static_cast<const uint8_t*>(L->w2);
    g.w_blocked = L->weight_layout == MOE_WEIGHTS_BLOCKED;
    g.w_expert_bytes = mx ? static_cast<int64_t>(L->D) * L->I / 2 : static_cast<int64_t>(L->D) * L->I * elem;
    g.w_scale = L->w2_scale;
    g.ws_expert = L->quant == MOE_QUANT_PTPC_FP8 ? static_cast<int64_t>(L->D)
                                                  : static_cast<int64_t>(L->D / 128) * (L->I / 128);
    g.ws_ld = L->I / 128;
    g.K = L->I;
    g.I = L->I;
    g.out = out_perm;
    g.out_ld = L->D;
    const int tn = tn_of(L->quant, L->D, block_m);
    g.n_ntiles = L->D / ((nw_of(L->quant, block_m) / wm_of(block_m)) * tn * 32);
    g.n_tiles = static_cast<int>(max_rows / block_m) * g.n_ntiles;
    g.n_exp = L->E + L->n_shared;
    return launch_mode<false>(L->quant, tn, block_m, g, s);
}

}  // namespace moe

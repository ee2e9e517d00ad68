// Weight-streaming grouped GEMMs for small batches (decode).
//
// With few tokens per expert the expert GEMMs are bound by reading the
// weights of the active experts once from HBM (the Qwen3 MI300X page, 2.1.2,
// finds MoE inference memory-bound; its 2.1.4 tunes CU-level load balance at
// low concurrency; the MI355X MoRI page notes that small-batch TP decode
// gives tall-skinny expert GEMMs).  Design:
//   - the work is (active expert x slice of weight rows) items, one wave per
//     item; the wave that streams the slice handles the expert's rows, up
//     to 16*MT at a time, so each weight byte is read once per 16*MT rows
//     (once in total for the small batches this path is chosen for);
//   - the grid is persistent (the workgroups that fit at once); each
//     workgroup lists the active experts (offsets[e+1] > offsets[e]) in LDS
//     and its waves walk the items so that every CU gets the same number of
//     items within one: only active experts cost time and no second, partly
//     filled round of workgroups idles most of the chip;
//   - no LDS: each lane streams 32 B of a weight row per 128-byte K step
//     straight into MFMA operand registers (v_mfma_f32_16x16x128_f8f6f4, or
//     two v_mfma_f32_16x16x32_bf16, or for MXFP4 two FP4 MFMAs with the
//     E8M0 block scales as operands), the next step's loads in flight
//     while the current step multiplies;
//   - activation rows are tiny and stay in L2.
#include "perm_dev.h"

#include <type_traits>

namespace moe {

typedef int v8i_s __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf_s __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_s __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));

struct StreamArgs {
    const uint8_t* a;          // gate_up: x / xq [T, K]; down: act / aq [R, K]
    int64_t a_ld;              // bytes per row
    int a_blocked;             // down: act codes in 16-row x 128-byte blocks (R a multiple of 16)
    const float* a_scale;      // PTPC: per row; block: [rows, K/128]
    int a_scale_ld;
    const int* sorted_ids;     // gate_up: flat ids; down: NULL (rows direct)
    int topk, TK, sentinel;
    const int* offsets;        // [E'+1] padded (multiples of 16)
    const int* counts;         // [E'] routed rows per expert (NULL: every row of a segment is live)
    const uint8_t* w;
    int w_blocked;             // weights in blocks of 16 rows x 128 bytes (else row-major)
    int64_t w_expert_bytes;
    const float* w_scale;
    int64_t ws_expert;
    int ws_ld;
    const uint8_t* a_mx;       // MXFP4: E8M0 scales of the activation rows [rows, K/32]
    const uint8_t* w_mx;       // MXFP4: E8M0 weight scales [E', Nw, K/32]
    int64_t w_mx_expert;       // MXFP4: scale bytes per expert
    int K;                     // elements
    int I;                     // gate_up act columns
    void* out;
    int64_t out_ld;
    int n_exp;                 // E'
    int nslice;                // weight slices (one wave each) per expert
    // gate_up given the routed ids instead of a permutation (T <= 256, distinct
    // picks per token): every workgroup builds the permutation in LDS, and
    // workgroup 0 writes it to `pout` for the launches that follow
    const int* ids;            // [T, topk] (NULL: sorted_ids, offsets and counts are given)
    int T, E, n_shared, max_rows;
    PermOut pout;
};

// Where an item finds its expert's rows: the given permutation (tok NULL),
// or the one built in LDS (padded and live offsets, token of each live row).
struct PermRef {
    const int* off;
    const int* live;
    const int* tok;
};
constexpr int kStreamPermMW = 8;           // mask words of the in-kernel permutation (T <= 256)

template <int MODE>
__device__ __forceinline__ void mfma16(const u32x8& a, const u32x8& b, v4f& acc) {
    if constexpr (MODE == MOE_QUANT_NONE_BF16) {
        const u32x4_s a0 = __builtin_shufflevector(a, a, 0, 1, 2, 3), a1 = __builtin_shufflevector(a, a, 4, 5, 6, 7);
        const u32x4_s b0 = __builtin_shufflevector(b, b, 0, 1, 2, 3), b1 = __builtin_shufflevector(b, b, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf_s, a0), __builtin_bit_cast(v8bf_s, b0),
                                                      acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf_s, a1), __builtin_bit_cast(v8bf_s, b1),
                                                      acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(v8i_s, a), __builtin_bit_cast(v8i_s, b),
                                                               acc, 0, 0, 0, 0, 0, 0);
    }
}

// MXFP4: a lane's 32 bytes of a 128-byte step (256 E2M1 elements per row)
// are two 16-byte pieces, elements 32q .. 32q+31 and 128+32q .. 128+32q+31
// of the step (q = lane / 16): the lane's part of two 16x16x128 MFMAs, one
// per piece C, each an aligned 32-element block with one E8M0 scale.  The
// step's 8 scale bytes of a row are two dwords; piece C takes byte q of
// dword C, shifted to byte 0 (operand byte select 0).  Format selectors 4
// (FP4) for both operands: the MFMA reads the piece's four registers.
template <int C>
__device__ __forceinline__ void mfma16_mx(const u32x4_s& a, const u32x4_s& b, uint2 as, uint2 ws, int sh, v4f& acc) {
    const u32x4_s z = {0u, 0u, 0u, 0u};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        __builtin_bit_cast(v8i_s, __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7)),
        __builtin_bit_cast(v8i_s, __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7)), acc, 4, 4, 0,
        static_cast<int>((C == 0 ? as.x : as.y) >> sh), 0, static_cast<int>((C == 0 ? ws.x : ws.y) >> sh));
}

// A lane's 32 operand bytes of one 128-byte K step: bytes [16q, 16q+16) and
// [64+16q, 64+16q+16) of its row, q = lane / 16; the second piece is HI
// bytes after the first (64 in a row-major row; 1024 in a blocked weight
// block, where each of the two loads then reads 8 whole lines).  Activation
// and weight operands use the same K mapping, so the MFMA pairs matching K.
__device__ __forceinline__ u32x8 ld32(const uint8_t* p, int hi_off) {
    const u32x4_s lo = *reinterpret_cast<const u32x4_s*>(p);
    const u32x4_s hi = *reinterpret_cast<const u32x4_s*>(p + hi_off);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}


__device__ __forceinline__ int src_row(const StreamArgs& p, bool gateup, int row, bool& valid) {
    if (!gateup) { valid = true; return row; }
    const int f = p.sorted_ids[row];
    valid = f != p.sentinel;
    return valid ? (f < p.TK ? f / p.topk : f - p.TK) : 0;
}

// TN: 16-row weight tiles per wave (gate_up: TN/2 gate + TN/2 up tiles).
// MT: 16-row activation tiles (rows per expert <= 16*MT).  PF: K steps in
// flight.  The steady-state loop has no data-dependent branch, so the
// compiler can wait for exactly the step it is about to use.
// One item: expert E, weight slice SL (COLS_W output columns), rows
// [R0, R0 + 16*MT) of the expert's segment, on this wave.
template <int MODE, bool GATEUP, int TN, int MT, int PF>
__device__ __forceinline__ void stream_item(const StreamArgs& p, const PermRef& pr, int e, int sl, int lane,
                                            int r0) {
    constexpr bool BLOCKQ = MODE == MOE_QUANT_BLOCK128_FP8;
    constexpr bool MX = MODE == MOE_QUANT_MXFP4;
    constexpr int COLS_W = GATEUP ? TN / 2 * 16 : TN * 16;     // output columns per wave
    const int row0 = pr.off[e] + r0;
    const int cnt = min(pr.off[e + 1] - row0, 16 * MT);        // padded rows of this chunk
    const int nl = pr.tok ? pr.live[e + 1] - pr.live[e] : 0;   // routed rows of the expert (LDS permutation)
    const int live = pr.tok ? pr.off[e] + nl - row0
                            : (p.counts ? p.offsets[e] + p.counts[e] - row0 : cnt);   // rows before the pads
    // token (gate_up) or row (down) of row r of this chunk; v: a routed row
    auto src_of = [&](int r, bool& v) {
        if (GATEUP && pr.tok) {
            v = r0 + r < nl;
            return v ? pr.tok[pr.live[e] + r0 + r] : 0;
        }
        return src_row(p, GATEUP, row0 + r, v);
    };
    const int c0 = sl * COLS_W;                                 // first output column of this wave
    const int r16 = lane & 15, kq = (lane >> 4) * 16;

    const uint8_t* wexp = p.w + static_cast<int64_t>(e) * p.w_expert_bytes;
    const int64_t wrow = MX ? p.K / 2 : static_cast<int64_t>(p.K) * (MODE == MOE_QUANT_NONE_BF16 ? 2 : 1);
    const uint8_t* bp[TN];
    int wn0[TN];                                                  // first weight row of each tile
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        wn0[t] = GATEUP ? (t < TN / 2 ? c0 + t * 16 : p.I + c0 + (t - TN / 2) * 16) : c0 + t * 16;
        // blocked weights: a tile's 16 rows x 128 bytes of one step are one
        // contiguous 2 KB block
        bp[t] = p.w_blocked ? wexp + static_cast<int64_t>(wn0[t] >> 4) * (wrow / 128) * 2048 + blocked_byte(r16, kq)
                            : wexp + (wn0[t] + r16) * wrow + kq;
    }
    // MXFP4: the scale row of the lane's weight row in each tile, and of its
    // activation row in each M tile (8 bytes per step)
    const int sld = p.K / 32;
    const uint8_t* wsp[MX ? TN : 1];
    const uint8_t* asp[MX ? MT : 1];
    if constexpr (MX) {
#pragma unroll
        for (int t = 0; t < TN; ++t) wsp[t] = p.w_mx + e * p.w_mx_expert + static_cast<int64_t>(wn0[t] + r16) * sld;
    }
    // operand rows: row r16 of each M tile; rows past the segment or on a pad
    // slot read a valid row and are zeroed by the epilogue's row mask
    const uint8_t* ap[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int r = m * 16 + r16;
        bool v = false;
        const int src = r < cnt ? src_of(r, v) : 0;
        const int64_t ar = v ? src : (GATEUP ? 0 : row0);
        if constexpr (MX) asp[m] = p.a_mx + ar * sld;
        ap[m] = p.a_blocked ? p.a + (ar >> 4) * (p.a_ld / 128) * 2048 + blocked_byte(static_cast<int>(ar & 15), kq)
                            : p.a + ar * p.a_ld + kq;
    }
    // accumulator rows: (lane / 16) * 4 + i of each tile
    int esrc[MT][4];
    float emask[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = m * 16 + (lane >> 4) * 4 + i;
            bool v = false;
            const int src = r < cnt ? src_of(r, v) : 0;
            esrc[m][i] = v ? src : (GATEUP ? 0 : row0);
            emask[m][i] = v && r < live ? 1.0f : 0.0f;
        }

    v4f acc[MT][TN];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[m][t] = v4f{0, 0, 0, 0};

    const int nk = static_cast<int>(wrow / 128);
    const int whi = p.w_blocked ? blocked_byte(0, 64) - blocked_byte(0, 0) : 64;   // second operand piece
    const int ahi = p.a_blocked ? blocked_byte(0, 64) - blocked_byte(0, 0) : 64;
    // Each item starts its K sweep at its own step (wrapping around), so the
    // waves spread over the byte offsets of the weight rows.  The K order is
    // fixed by the item (expert, slice): results stay deterministic.
    const int kbeg = (sl * 5 + e * 3) % nk;

    u32x8 bq[MX ? 1 : PF][TN], aqr[MX ? 1 : PF][MT];
    float asq[PF][MT][4];
    // MXFP4: the two 16-byte pieces of each operand as separate values (each
    // is a whole MFMA operand), and the step's scale dwords
    u32x4_s bq2[MX ? PF : 1][TN][2], aq2[MX ? PF : 1][MT][2];
    uint2 wsq[MX ? PF : 1][MX ? TN : 1], asx[MX ? PF : 1][MX ? MT : 1];
    auto fill = [&](int j, int s) {
        int ks = s + kbeg;
        ks = ks >= nk ? ks - nk : ks;
        const int64_t ko = static_cast<int64_t>(ks) * (p.a_blocked ? 2048 : 128);   // step offset in the rows
        const int64_t kw = static_cast<int64_t>(ks) * (p.w_blocked ? 2048 : 128);   // step offset in the weights
        if constexpr (MX) {
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                bq2[j][t][0] = *reinterpret_cast<const u32x4_s*>(bp[t] + kw);
                bq2[j][t][1] = *reinterpret_cast<const u32x4_s*>(bp[t] + kw + whi);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                aq2[j][m][0] = *reinterpret_cast<const u32x4_s*>(ap[m] + ko);
                aq2[j][m][1] = *reinterpret_cast<const u32x4_s*>(ap[m] + ko + ahi);
            }
#pragma unroll
            for (int t = 0; t < TN; ++t) wsq[j][t] = *reinterpret_cast<const uint2*>(wsp[t] + 8 * ks);
#pragma unroll
            for (int m = 0; m < MT; ++m) asx[j][m] = *reinterpret_cast<const uint2*>(asp[m] + 8 * ks);
        } else {
#pragma unroll
            for (int t = 0; t < TN; ++t) bq[j][t] = ld32(bp[t] + kw, whi);
#pragma unroll
            for (int m = 0; m < MT; ++m) aqr[j][m] = ld32(ap[m] + ko, ahi);
        }
        if constexpr (BLOCKQ) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) asq[j][m][i] = p.a_scale[static_cast<int64_t>(esrc[m][i]) * p.a_scale_ld + ks];
        }
    };
    auto compute = [&](int j, int s) {
        if constexpr (MX) {
            // every tile's first piece, then every tile's second: an
            // accumulator's two MFMAs of the step are MT*TN MFMAs apart
            const int sh = 8 * (lane >> 4);
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    mfma16_mx<0>(aq2[j][m][0], bq2[j][t][0], asx[j][m], wsq[j][t], sh, acc[m][t]);
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    mfma16_mx<1>(aq2[j][m][1], bq2[j][t][1], asx[j][m], wsq[j][t], sh, acc[m][t]);
        } else if constexpr (!BLOCKQ) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int t = 0; t < TN; ++t) mfma16<MODE>(aqr[j][m], bq[j][t], acc[m][t]);
        } else {
            int ks = s + kbeg;
            ks = ks >= nk ? ks - nk : ks;
            float wsc[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) wsc[t] = p.w_scale[e * p.ws_expert + (wn0[t] >> 7) * p.ws_ld + ks];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    v4f part = v4f{0, 0, 0, 0};
                    mfma16<MODE>(aqr[j][m], bq[j][t], part);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[m][t][i] += part[i] * (asq[j][m][i] * wsc[t]);
                }
        }
    };

    // prologue: PF fills, unconditional (a step index past the end reloads
    // the last step, never used) so the compiler knows exactly how many
    // loads are in flight when the steady loop starts
#pragma unroll
    for (int j = 0; j < PF; ++j) fill(j, j < nk ? j : nk - 1);
    int s0 = 0;
    // steady state: every refill targets a step < nk.  Scheduling barriers
    // keep "MFMAs of step s, then the loads of step s + PF" in program order
    // (hoisting the MFMAs above the loads would leave each step waiting on
    // loads issued just before it).
    for (; s0 + 2 * PF <= nk; s0 += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            compute(j, s0 + j);
            __builtin_amdgcn_sched_barrier(0);
            fill(j, s0 + j + PF);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // tail: the last PF .. 2PF-1 steps
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        if (s0 + j < nk) {
            compute(j, s0 + j);
            if (s0 + j + PF < nk) fill(j, s0 + j + PF);
        }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j)
        if (s0 + PF + j < nk) compute(j, s0 + PF + j);

    // epilogue: lane holds column (lane & 15) and rows (lane / 16) * 4 + i of each tile
    const int mtiles = cnt >> 4;
    const float* wsx = MODE == MOE_QUANT_PTPC_FP8 ? p.w_scale + e * p.ws_expert : nullptr;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m >= mtiles) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = m * 16 + (lane >> 4) * 4 + i;       // row within the expert segment
            float rs = emask[m][i];
            if constexpr (MODE == MOE_QUANT_PTPC_FP8) rs *= p.a_scale[esrc[m][i]];
            const int64_t orow = static_cast<int64_t>(row0 + r) * p.out_ld;
            if constexpr (GATEUP) {
#pragma unroll
                for (int t = 0; t < TN / 2; ++t) {
                    const int col = c0 + t * 16 + (lane & 15);
                    float g = acc[m][t][i] * rs, u = acc[m][t + TN / 2][i] * rs;
                    if constexpr (MODE == MOE_QUANT_PTPC_FP8) {
                        g *= wsx[col];
                        u *= wsx[p.I + col];
                    }
                    static_cast<uint16_t*>(p.out)[orow + col] = f32_to_bf16(silu_mul(g, u));
                }
            } else {
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    const int col = c0 + t * 16 + (lane & 15);
                    float v = acc[m][t][i] * rs;
                    if constexpr (MODE == MOE_QUANT_PTPC_FP8) v *= wsx[col];
                    if constexpr (MODE == MOE_QUANT_NONE_BF16) static_cast<float*>(p.out)[orow + col] = v;
                    else static_cast<uint16_t*>(p.out)[orow + col] = f32_to_bf16(v);
                }
            }
        }
    }
}

// Persistent: G workgroups of 4 waves.  Item i (active expert i / nslice,
// slice i % nslice) goes to workgroup i % G, wave (i / G) % 4, round
// i / (4G): consecutive items spread over workgroups first, so the per-CU
// item counts differ by at most one.
template <int MODE, bool GATEUP, int TN, int MT, int PF>
__global__ void __launch_bounds__(256) stream_gemm_kernel(const StreamArgs p) {
    __shared__ int s_act[MOE_MAX_EXPERTS];
    __shared__ int s_wcnt[4];
    // the in-kernel permutation (gate_up given routed ids)
    using PS = typename std::conditional<GATEUP, PermShared<kStreamPermMW>, int>::type;
    __shared__ PS s_perm;
    __shared__ int s_e[GATEUP ? 32 * kStreamPermMW * MOE_MAX_TOPK : 1];
    __shared__ int s_tok[GATEUP ? 32 * kStreamPermMW * (MOE_MAX_TOPK + 1) : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    PermRef pr{p.offsets, nullptr, nullptr};
    if constexpr (GATEUP) {
        if (p.ids) {
            perm_build<kStreamPermMW, 256>(p.ids, p.T, p.topk, p.E, p.n_shared, 16, p.max_rows, s_perm, s_e, s_tok,
                                           p.pout, blockIdx.x == 0);
            pr = PermRef{s_perm.off, s_perm.live, s_tok};
        }
    }
    // active experts in index order: thread t looks at experts t, t+256, ...
    int base = 0;
    for (int e0 = 0; e0 < p.n_exp; e0 += 256) {
        const int e = e0 + threadIdx.x;
        const bool act = e < p.n_exp && pr.off[e + 1] > pr.off[e];
        const uint64_t m = __ballot(act);
        if (lane == 0) s_wcnt[wave] = __popcll(m);
        __syncthreads();
        int before = base;
        for (int w = 0; w < wave; ++w) before += s_wcnt[w];
        if (act) s_act[before + __popcll(m & ((uint64_t{1} << lane) - 1))] = e;
        base += s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
        __syncthreads();
    }
    const int n_items = base * p.nslice;
    const int G = gridDim.x;
    for (int i = blockIdx.x + G * wave; i < n_items; i += 4 * G) {
        const int j = i / p.nslice, e = s_act[j], sl = i - j * p.nslice;
        const int rows = pr.off[e + 1] - pr.off[e];
        // experts with at most 16 (32) rows take the one-tile (two-tile) path:
        // fewer activation loads, registers and MFMAs; more rows than 16*MT
        // are handled in chunks.  Each path is branch-free inside.
        if (MT > 1 && rows <= 16) {
            stream_item<MODE, GATEUP, TN, 1, PF>(p, pr, e, sl, lane, 0);
        } else if (MT > 2 && rows <= 32) {
            stream_item<MODE, GATEUP, TN, 2, PF>(p, pr, e, sl, lane, 0);
        } else {
            for (int r0 = 0; r0 < rows; r0 += 16 * MT) stream_item<MODE, GATEUP, TN, MT, PF>(p, pr, e, sl, lane, r0);
        }
    }
}

// 16-row weight tiles per wave (gate/up: half gate, half up tiles) and K
// steps in flight per wave.  In the PTPC mode both GEMMs stream 4 tiles per
// wave (one wave per SIMD): Qwen3-235B decode step 165.9 -> 163.8 us with 4
// gate/up tiles instead of 2, then 162.9 -> 161.8 us with 4 down tiles.  The
// blockwise mode keeps 2 (its per-step scales would not fit the registers),
// and so does bf16 (4 tiles halve its waves; the 64-token bf16 layer went
// from 0.028 to 0.032 ms).  MXFP4 streams 4 tiles while a launch carries up
// to 32 rows per expert at a time (Qwen3-235B decode shape 120.3 -> 114.7
// us against 2 tiles) and 2 with 64 rows, where its scale dwords and
// two-piece operands would spill at 4.  One tile
// per wave for down spread its items more evenly over the waves but halved
// the bytes each wave keeps in flight, and measured slower (178 -> 196 us);
// so did splitting only the items of the last, partial round (177 ->
// 181 us): the waves share HBM bandwidth, and the few that run a last round
// get more of it.  3 or 6 steps in flight instead of 4 were slower (167.4,
// 167.3 against 165.9 us).
template <int MODE, bool GATEUP, int MT, bool WIDE>
constexpr int stream_tn() {
    return WIDE ? 8 : MODE == MOE_QUANT_PTPC_FP8 || (MODE == MOE_QUANT_MXFP4 && MT <= 2) ? 4 : 2;
}
// K steps in flight.  WIDE (the PTPC GEMMs of batches above 32 tokens that
// route at least 8 rows per expert on average) streams 8 tiles with 2 steps
// in flight: the same bytes in flight per wave as 4 tiles with 4, in items
// of twice the bytes and half as many, so each item's start latency is paid
// half as often.  Qwen3-30B-A3B-shaped layer (128 active experts, 16 rows
// each): down GEMM 49.2 -> 46.3 us, then gate/up 83.6 -> 80.2 us.  Decode
// batches with few active experts get too few items for the waves: the
// down GEMM at 32 / 64 tokens over 38 / 44 experts measured 156.9 -> 158.0
// and 186.7 -> 189.2 us, so they keep 4 tiles.
template <int MODE, bool GATEUP, int MT, bool WIDE>
constexpr int stream_pf() { return WIDE ? 2 : 4; }

// Workgroups of a kernel that fit on the device at once, per device (CACHE:
// one per kernel instantiation).
template <typename Kern>
static int resident_blocks(Kern kernel, int (&cache)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (n == 0) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, 0) != hipSuccess || occ <= 0) occ = 1;
        n = cus * occ;
        __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
    }
    return n;
}

template <int MODE, bool GATEUP, int MT, bool WIDE = false>
static int32_t stream_launch_mt(StreamArgs a, int ncols, hipStream_t s) {
    constexpr int TN = stream_tn<MODE, GATEUP, MT, WIDE>();
    constexpr int COLS_W = GATEUP ? TN / 2 * 16 : TN * 16;   // output columns per item
    a.nslice = ncols / COLS_W;
    auto kern = stream_gemm_kernel<MODE, GATEUP, TN, MT, stream_pf<MODE, GATEUP, MT, WIDE>()>;
    static int cache[64];
    // no more workgroups than items could need (E' experts x slices / 4 waves)
    const int wgs = min(resident_blocks(kern, cache),
                        static_cast<int>(ceil_div(static_cast<int64_t>(a.n_exp) * a.nslice, 4)));
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(max(wgs, 1))), dim3(256), 0, s, a);
    return moe_launch_status();
}

template <int MODE, bool GATEUP>
static int32_t stream_launch_mode(StreamArgs a, int Ep, int ncols, int T, bool wide, hipStream_t s) {
    a.n_exp = Ep;
    if (T <= 16) return stream_launch_mt<MODE, GATEUP, 1>(a, ncols, s);
    if (T <= 32) return stream_launch_mt<MODE, GATEUP, 2>(a, ncols, s);
    if constexpr (MODE == MOE_QUANT_PTPC_FP8)
        if (wide) return stream_launch_mt<MODE, GATEUP, 4, true>(a, ncols, s);
    return stream_launch_mt<MODE, GATEUP, 4>(a, ncols, s);
}

template <bool GATEUP>
static int32_t stream_launch(int quant, const StreamArgs& a, int Ep, int ncols, int T, hipStream_t s,
                             bool wide = false) {
    switch (quant) {
        case MOE_QUANT_NONE_BF16: return stream_launch_mode<MOE_QUANT_NONE_BF16, GATEUP>(a, Ep, ncols, T, wide, s);
        case MOE_QUANT_PTPC_FP8: return stream_launch_mode<MOE_QUANT_PTPC_FP8, GATEUP>(a, Ep, ncols, T, wide, s);
        case MOE_QUANT_BLOCK128_FP8: return stream_launch_mode<MOE_QUANT_BLOCK128_FP8, GATEUP>(a, Ep, ncols, T, wide, s);
        case MOE_QUANT_MXFP4: return stream_launch_mode<MOE_QUANT_MXFP4, GATEUP>(a, Ep, ncols, T, wide, s);
    }
    return MOE_ERR_UNSUPPORTED;
}


// The wide items (8 tiles, 2 steps in flight) for PTPC batches that route
// at least 8 rows per expert on average: most experts are active, so the
// items still fill the waves.
static bool stream_wide(const moe_layer_desc* L, int T) {
    return static_cast<int64_t>(T) * L->top_k >= 8LL * (L->E + L->n_shared);
}

// The gate/up arguments every variant shares.
static StreamArgs gateup_args(const moe_layer_desc* L, const void* a, const float* a_scale, int T, void* act) {
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    const bool mx = L->quant == MOE_QUANT_MXFP4;   // a_scale: the rows' E8M0 bytes
    StreamArgs g{};
    g.a = static_cast<const uint8_t*>(a);
    g.a_ld = mx ? L->D / 2 : static_cast<int64_t>(L->D) * elem;
    if (mx) {
        g.a_mx = reinterpret_cast<const uint8_t*>(a_scale);
        g.w_mx = reinterpret_cast<const uint8_t*>(L->w13_scale);
        g.w_mx_expert = 2LL * L->I * (L->D / 32);
    }
    g.a_scale = a_scale;
    g.a_scale_ld = L->D / 128;
    g.topk = L->top_k;
    g.TK = T * L->top_k;
    g.sentinel = T * (L->top_k + L->n_shared);
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
    return g;
}

int32_t stream_gateup_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T,
                             const int* sorted_ids, const int* offsets, const int* counts, void* act,
                             hipStream_t s) {
    StreamArgs g = gateup_args(L, a, a_scale, T, act);
    g.sorted_ids = sorted_ids;
    g.offsets = offsets;
    g.counts = counts;
    return stream_launch<true>(L->quant, g, L->E + L->n_shared, L->I, T, s, stream_wide(L, T));
}

// gate_up from the routed ids (T <= 256, k picks per token distinct): the
// kernel builds the permutation itself (workgroup 0 writes it to `pout`, for
// the launches that follow), so no permutation launch precedes it.
int32_t stream_gateup_fused_launch(const moe_layer_desc* L, const void* a, const float* a_scale, int T,
                                   const int* ids, int max_rows, const PermOut& pout, void* act, hipStream_t s) {
    StreamArgs g = gateup_args(L, a, a_scale, T, act);
    g.ids = ids;
    g.T = T;
    g.E = L->E;
    g.n_shared = L->n_shared;
    g.max_rows = max_rows;
    g.pout = pout;
    return stream_launch<true>(L->quant, g, L->E + L->n_shared, L->I, T, s, stream_wide(L, T));
}

bool stream_fused_perm_ok(int T) { return T >= 1 && T <= 32 * kStreamPermMW; }

int32_t stream_down_launch(const moe_layer_desc* L, const void* act, const float* act_scale, int T,
                           const int* offsets, const int* counts, void* out_perm, hipStream_t s, bool act_blocked) {
    const int elem = L->quant == MOE_QUANT_NONE_BF16 ? 2 : 1;
    const bool mx = L->quant == MOE_QUANT_MXFP4;   // act_scale: the rows' E8M0 bytes
    StreamArgs g{};
    g.a = static_cast<const uint8_t*>(act);
    g.a_ld = mx ? L->I / 2 : static_cast<int64_t>(L->I) * elem;
    g.a_blocked = act_blocked && elem == 1;
    if (mx) {
        g.a_mx = reinterpret_cast<const uint8_t*>(act_scale);
        g.w_mx = reinterpret_cast<const uint8_t*>(L->w2_scale);
        g.w_mx_expert = static_cast<int64_t>(L->D) * (L->I / 32);
    }
    g.a_scale = act_scale;
    g.a_scale_ld = L->I / 128;
    g.sorted_ids = nullptr;
    g.offsets = offsets;
    g.counts = counts;
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
    return stream_launch<false>(L->quant, g, L->E + L->n_shared, L->D, T, s, stream_wide(L, T));
}

}  // namespace moe

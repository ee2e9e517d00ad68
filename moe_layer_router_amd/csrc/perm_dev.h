// The expert permutation of routed ids built by one workgroup in LDS, for
// batches whose k picks per token are distinct experts (the library's own
// routing): every expert's routed rows are a mask of tokens, 32 per word
// (LDS atomicOr), and a row's rank in its expert's segment is the number of
// mask bits below its token -- the stable ascending order of flat indices
// of the general permutation (shared-expert rows: token order).  Counts,
// padded offsets, sorted ids, inverse map, pads, block -> expert map and the
// tail are written exactly as the general permutation writes them.
#pragma once
#include "common.h"

namespace moe {

// LDS of one build: MW mask words per expert (T <= 32 MW).
template <int MW>
struct PermShared {
    uint32_t mask[MW][MOE_MAX_EXPERTS];   // word w: tokens 32w .. 32w+31 routed to the expert
    int off[MOE_MAX_EXPERTS + 1];         // padded segment offsets (multiples of B)
    int live[MOE_MAX_EXPERTS + 1];        // offsets of the routed rows alone (no pads)
    int wsum[2][16];                      // per-wave totals of the two scans
};

// Global arrays of the permutation (written when `write`).
struct PermOut {
    int* counts;
    int* offsets;
    int* sorted;
    int* bexp;
    int* inv;
};

// NT threads (a multiple of 64, at most 1024) of the workgroup call it
// together.  s_e: T k ints of LDS (the expert of each pick, -1: no row);
// s_tok (may be NULL): T (k + ns) ints of LDS that receive, at
// live[e] + rank, the token of each routed row.  Ends with a barrier.
template <int MW, int NT>
__device__ __forceinline__ void perm_build(const int* __restrict__ ids, int T, int k, int E, int ns, int B,
                                           int max_rows, PermShared<MW>& S, int* s_e, int* s_tok,
                                           const PermOut& o, bool write) {
    static_assert(NT % 64 == 0 && NT <= 1024, "workgroup");
    constexpr int NWV = NT / 64;
    constexpr int XPT = (MOE_MAX_EXPERTS + NT - 1) / NT;    // experts per thread in the scans
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Ep = E + ns, TK = T * k, A = T * (k + ns);

    for (int e = tid; e < Ep; e += NT)
#pragma unroll
        for (int w = 0; w < MW; ++w) S.mask[w][e] = 0;
    __syncthreads();
    for (int f = tid; f < TK; f += NT) {
        const int id = ids[f], t = f / k;
        const int e = (id >= 0 && id < E) ? id : -1;         // no valid pick: no row
        s_e[f] = e;
        if (e >= 0) atomicOr(&S.mask[t >> 5][e], 1u << (t & 31));
    }
    __syncthreads();

    // counts, padded and live offsets: thread tid takes experts
    // XPT tid .. XPT tid + XPT - 1 (the shared expert holds every token)
    int cnt[XPT], pad_sum = 0, live_sum = 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = XPT * tid + i;
        int c = 0;
        if (e < E) {
#pragma unroll
            for (int w = 0; w < MW; ++w) c += __popc(S.mask[w][e]);
        } else if (e < Ep) {
            c = T;
        }
        cnt[i] = c;
        pad_sum += (c + B - 1) / B * B;
        live_sum += c;
    }
    const int pinc = wave_incl_scan_i(pad_sum, lane), linc = wave_incl_scan_i(live_sum, lane);
    if (lane == 63) {
        S.wsum[0][wave] = pinc;
        S.wsum[1][wave] = linc;
    }
    __syncthreads();
    int pp = pinc - pad_sum, lp = linc - live_sum;             // exclusive within the wave
#pragma unroll
    for (int w = 0; w < NWV; ++w)
        if (w < wave) {
            pp += S.wsum[0][w];
            lp += S.wsum[1][w];
        }
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = XPT * tid + i;
        if (e < Ep) {
            S.off[e] = pp;
            S.live[e] = lp;
            if (write) {
                o.counts[e] = cnt[i];
                o.offsets[e] = pp;
            }
        }
        pp += (cnt[i] + B - 1) / B * B;
        lp += cnt[i];
    }
    if (tid == NT - 1) {                                       // the totals (experts past Ep add nothing)
        S.off[Ep] = pp;
        S.live[Ep] = lp;
        if (write) o.offsets[Ep] = pp;
    }
    __syncthreads();

    // rows: rank of token t in expert e = tokens below t routed to e
    for (int f = tid; f < A; f += NT) {
        int e, t, rank;
        if (f < TK) {
            e = s_e[f];
            t = f / k;
            if (e < 0) {
                if (write) o.inv[f] = -1;
                continue;
            }
            rank = __popc(S.mask[t >> 5][e] & ((1u << (t & 31)) - 1u));
#pragma unroll
            for (int w = 0; w < MW; ++w)
                if (w < (t >> 5)) rank += __popc(S.mask[w][e]);
        } else {
            e = E;                                              // shared expert: token order
            t = f - TK;
            rank = t;
        }
        const int row = S.off[e] + rank;
        if (write) {
            o.sorted[row] = f;
            o.inv[f] = row;
        }
        if (s_tok) s_tok[S.live[e] + rank] = t;
    }
    if (write) {
        // pads and block map (one wave per expert), tail past the total
        for (int e = wave; e < Ep; e += NWV) {
            const int n = S.live[e + 1] - S.live[e];
            const int lo = S.off[e], hi = S.off[e + 1];
            for (int r = lo + n + lane; r < hi; r += 64) o.sorted[r] = A;
            for (int b = lo / B + lane; b < hi / B; b += 64) o.bexp[b] = e;
        }
        const int total = S.off[Ep];
        for (int b = total / B + tid; b < max_rows / B; b += NT) o.bexp[b] = -1;
        for (int r = total + tid; r < max_rows; r += NT) o.sorted[r] = A;
    }
    __syncthreads();
}

}  // namespace moe

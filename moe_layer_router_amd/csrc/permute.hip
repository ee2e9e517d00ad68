// Stable permutation of routed rows by expert with per-expert padding.
//
// The Qwen 3.5 TPU page gathers token rows into one contiguous buffer per
// expert (SparseCore permutation item) and runs the grouped GEMM over
// bounded per-expert slices with minimal padding (GMM V2 item).  Here the
// flat routed rows (t*k + j, then the shared-expert rows T*k + t) are cut into
// chunks of 256; three kernels do count -> scan -> scatter:
//   count:   per-chunk expert histogram (LDS), stored expert-major;
//   scan:    one block: per-expert exclusive prefix over chunks, padded
//            expert offsets, block -> expert map, sentinel fill;
//   scatter: rank of each row among the equal-expert rows before it in its
//            chunk (LDS scan), giving a stable, atomic-free order.
// Integer work only: every output is bit-exact and deterministic.
#include "common.h"

namespace moe {

constexpr int kChunk = 256;

__device__ __forceinline__ int expert_of(const int* __restrict__ ids, int f, int TK, int E) {
    if (f < TK) {
        const int e = ids[f];
        return (e >= 0 && e < E) ? e : -1;        // out-of-range ids get no row
    }
    return E;                                      // shared-expert row
}

__global__ void __launch_bounds__(kChunk) permute_count_kernel(const int* __restrict__ ids, int TK, int A, int E,
                                                               int Ep, int nchunks, int* __restrict__ chunk_cnt) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < Ep; e += kChunk) cnt[e] = 0;
    __syncthreads();
    const int f = blockIdx.x * kChunk + threadIdx.x;
    if (f < A) {
        const int e = expert_of(ids, f, TK, E);
        if (e >= 0) atomicAdd(&cnt[e], 1);        // integer counts: order-free
    }
    __syncthreads();
    for (int e = threadIdx.x; e < Ep; e += kChunk)
        chunk_cnt[static_cast<int64_t>(e) * nchunks + blockIdx.x] = cnt[e];
}

// One block of 1024 threads.  Latency-bound (a few KB of counts), so each
// wave keeps many loads in flight: it scans 4 experts at a time and loads
// 4 x 64 chunk counts of each before scanning.
__global__ void __launch_bounds__(1024) permute_scan_kernel(int* __restrict__ chunk_cnt, int Ep, int nchunks,
                                                            int block_m, int max_rows, int sentinel,
                                                            int* __restrict__ counts, int* __restrict__ offsets,
                                                            int* __restrict__ sorted_ids,
                                                            int* __restrict__ block_expert) {
    __shared__ int s_tot[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_wave[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    // per-expert exclusive prefix over chunks (in place) and total
    constexpr int EB = 4, CG = 4;
    for (int e0 = wave; e0 < Ep; e0 += nw * EB) {
        int carry[EB] = {0, 0, 0, 0};
        for (int c0 = 0; c0 < nchunks; c0 += 64 * CG) {
            int v[EB][CG];
#pragma unroll
            for (int i = 0; i < EB; ++i) {
                const int e = e0 + i * nw;
#pragma unroll
                for (int g = 0; g < CG; ++g) {
                    const int c = c0 + 64 * g + lane;
                    v[i][g] = (e < Ep && c < nchunks) ? chunk_cnt[static_cast<int64_t>(e) * nchunks + c] : 0;
                }
            }
#pragma unroll
            for (int i = 0; i < EB; ++i) {
                const int e = e0 + i * nw;
#pragma unroll
                for (int g = 0; g < CG; ++g) {
                    const int c = c0 + 64 * g + lane;
                    const int inc = wave_incl_scan_i(v[i][g], lane);
                    if (e < Ep && c < nchunks) chunk_cnt[static_cast<int64_t>(e) * nchunks + c] = carry[i] + inc - v[i][g];
                    carry[i] += __shfl(inc, 63, 64);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < EB; ++i)
            if (lane == 0 && e0 + i * nw < Ep) s_tot[e0 + i * nw] = carry[i];
    }
    __syncthreads();
    // padded sizes -> exclusive scan over experts (Ep <= 1024 = one per thread)
    const int e = threadIdx.x;
    const int c = e < Ep ? s_tot[e] : 0;
    const int padded = (c + block_m - 1) / block_m * block_m;
    int inc = wave_incl_scan_i(padded, lane);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const int v = lane < nw ? s_wave[lane] : 0;
        const int sc = wave_incl_scan_i(v, lane);
        if (lane < nw) s_wave[lane] = sc - v;          // exclusive wave bases
    }
    __syncthreads();
    inc += s_wave[wave];
    if (e < Ep) {
        s_off[e + 1] = inc;
        counts[e] = c;
        offsets[e + 1] = inc;
    }
    if (e == 0) { s_off[0] = 0; offsets[0] = 0; }
    __syncthreads();
    const int total = s_off[Ep];
    // one wave per expert: its blocks in the block -> expert map and the
    // sentinel in its pad rows
    for (int x = wave; x < Ep; x += nw) {
        const int lo = s_off[x], hi = s_off[x + 1];
        for (int b = lo / block_m + lane; b < hi / block_m; b += 64) block_expert[b] = x;
        for (int r = lo + s_tot[x] + lane; r < hi; r += 64) sorted_ids[r] = sentinel;
    }
    // past the total: no expert, sentinel rows
    const int nblocks = max_rows / block_m;
    for (int b = total / block_m + threadIdx.x; b < nblocks; b += blockDim.x) block_expert[b] = -1;
    for (int r = total + threadIdx.x; r < max_rows; r += blockDim.x) sorted_ids[r] = sentinel;
}

__global__ void __launch_bounds__(kChunk) permute_scatter_kernel(const int* __restrict__ ids, int TK, int A, int E,
                                                                 int nchunks, const int* __restrict__ chunk_base,
                                                                 const int* __restrict__ offsets,
                                                                 int* __restrict__ sorted_ids,
                                                                 int* __restrict__ inv_perm) {
    __shared__ int s_e[kChunk];
    const int f = blockIdx.x * kChunk + threadIdx.x;
    const int e = f < A ? expert_of(ids, f, TK, E) : -1;
    s_e[threadIdx.x] = e;
    __syncthreads();
    if (f >= A) return;
    if (e < 0) { inv_perm[f] = -1; return; }
    int rank = 0;
    for (int j = 0; j < static_cast<int>(threadIdx.x); ++j) rank += s_e[j] == e;
    const int row = offsets[e] + chunk_base[static_cast<int64_t>(e) * nchunks + blockIdx.x] + rank;
    sorted_ids[row] = f;
    inv_perm[f] = row;
}

size_t permute_scratch_bytes(int T, int k, int n_shared, int E) {
    const int64_t A = static_cast<int64_t>(T) * (k + n_shared);
    const int64_t nchunks = ceil_div(A, kChunk);
    return static_cast<size_t>(ceil_div(nchunks * (E + n_shared) * 4, 256) * 256);
}

int32_t permute_align_launch(const int* ids, int T, int k, int E, int n_shared, int block_m, int max_rows,
                             int* counts, int* offsets, int* sorted_ids, int* block_expert, int* inv_perm,
                             void* scratch, hipStream_t s) {
    const int Ep = E + n_shared;
    const int TK = T * k;
    const int A = T * (k + n_shared);
    const int nchunks = static_cast<int>(ceil_div(A, kChunk));
    int* chunk_cnt = static_cast<int*>(scratch);
    if (nchunks > 0)
        hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(kChunk), 0, s, ids, TK, A, E, Ep, nchunks,
                           chunk_cnt);
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, chunk_cnt, Ep, nchunks, block_m, max_rows,
                       A, counts, offsets, sorted_ids, block_expert);
    if (nchunks > 0)
        hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(kChunk), 0, s, ids, TK, A, E, nchunks,
                           chunk_cnt, offsets, sorted_ids, inv_perm);
    return moe_launch_status();
}

}  // namespace moe

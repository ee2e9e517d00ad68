// Stable permutation of routed rows by expert with per-expert padding.
//
// The Qwen 3.5 TPU page gathers token rows into one contiguous buffer per
// expert (SparseCore permutation item) and runs the grouped GEMM over
// bounded per-expert slices with minimal padding (GMM V2 item).  Here the
// flat routed rows (t*k + j, then the shared-expert rows T*k + t) are cut into
// chunks of 256; three kernels do count -> scan -> scatter:
//   count:   per-chunk expert histogram (LDS), stored expert-major;
//   scan:    one wave per expert: exclusive prefix over chunks, row count;
//   scatter: per chunk: padded expert offsets from the counts (every
//            workgroup computes them; the first publishes them), then the
//            rank of each row among the equal-expert rows before it in its
//            chunk (LDS scan), giving a stable, atomic-free order; the block
//            -> expert map and the sentinel fill are split over the chunks.
// No step runs in a single workgroup.
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

// Per-expert exclusive prefix over chunks, in place, and the expert's row
// count: one wave per expert (16 per workgroup), 64 chunk counts per load.
constexpr int kScanWaves = 16;
__global__ void __launch_bounds__(kScanWaves * 64) permute_scan_kernel(int* __restrict__ chunk_cnt, int Ep,
                                                                       int nchunks, int* __restrict__ counts) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * kScanWaves + (threadIdx.x >> 6);
    if (e >= Ep) return;
    int* row = chunk_cnt + static_cast<int64_t>(e) * nchunks;
    // all loads of the row first (latency-bound: a few KB)
    constexpr int CG = 4;
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64 * CG) {
        int v[CG];
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            const int c = c0 + 64 * g + lane;
            v[g] = c < nchunks ? row[c] : 0;
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) {
            const int c = c0 + 64 * g + lane;
            const int inc = wave_incl_scan_i(v[g], lane);
            if (c < nchunks) row[c] = carry + inc - v[g];
            carry += __shfl(inc, 63, 64);
        }
    }
    if (lane == 0) counts[e] = carry;
}

// Padded expert offsets from the counts, in LDS: 256 threads, Ep <= 1024
// (four consecutive experts per thread, then a workgroup scan).
__device__ __forceinline__ void padded_offsets(const int* __restrict__ counts, int Ep, int block_m, int* s_off,
                                               int* s_wave) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int pad[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        const int c = e < Ep ? counts[e] : 0;
        pad[i] = (c + block_m - 1) / block_m * block_m;
        sum += pad[i];
    }
    const int inc = wave_incl_scan_i(sum, lane);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
    int run = base + inc - sum;                       // exclusive prefix of this thread's first expert
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        if (e < Ep) s_off[e] = run;
        run += pad[i];
    }
    if (tid == 0) s_off[Ep] = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
}

// Each chunk's workgroup: the padded offsets (workgroup 0 also publishes
// them), then the rank of each row among the equal-expert rows before it in
// its chunk (LDS scan), giving a stable, atomic-free order; the block ->
// expert map, the sentinel in pad rows and the tail past the total are
// split over the workgroups.
__global__ void __launch_bounds__(kChunk) permute_scatter_kernel(const int* __restrict__ ids, int TK, int A, int E,
                                                                 int Ep, int nchunks, int block_m, int max_rows,
                                                                 const int* __restrict__ chunk_base,
                                                                 const int* __restrict__ counts,
                                                                 int* __restrict__ offsets,
                                                                 int* __restrict__ sorted_ids,
                                                                 int* __restrict__ block_expert,
                                                                 int* __restrict__ inv_perm) {
    __shared__ int s_e[kChunk];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_wave[kChunk / 64];
    static_assert(kChunk == 256 && MOE_MAX_EXPERTS <= 4 * kChunk, "one scan pass of four experts per thread");
    const int tid = threadIdx.x;
    const int f = blockIdx.x * kChunk + tid;
    const int e = f < A ? expert_of(ids, f, TK, E) : -1;
    s_e[tid] = e;
    padded_offsets(counts, Ep, block_m, s_off, s_wave);   // its barriers also publish s_e
    if (blockIdx.x == 0)
        for (int x = tid; x <= Ep; x += kChunk) offsets[x] = s_off[x];
    if (f < A) {
        if (e < 0) {
            inv_perm[f] = -1;
        } else {
            int rank = 0;
            for (int j = 0; j < tid; ++j) rank += s_e[j] == e;
            const int row = s_off[e] + chunk_base[static_cast<int64_t>(e) * nchunks + blockIdx.x] + rank;
            sorted_ids[row] = f;
            inv_perm[f] = row;
        }
    }
    // experts x = blockIdx.x, + nchunks, ...: one wave each for its blocks
    // and the sentinel in its pad rows
    const int lane = tid & 63, wave = tid >> 6;
    for (int x = blockIdx.x + nchunks * wave; x < Ep; x += nchunks * (kChunk / 64)) {
        const int lo = s_off[x], hi = s_off[x + 1];
        for (int b = lo / block_m + lane; b < hi / block_m; b += 64) block_expert[b] = x;
        for (int r = lo + counts[x] + lane; r < hi; r += 64) sorted_ids[r] = A;
    }
    // past the total: no expert, sentinel rows
    const int total = s_off[Ep];
    const int nblocks = max_rows / block_m;
    for (int b = total / block_m + blockIdx.x * kChunk + tid; b < nblocks; b += nchunks * kChunk) block_expert[b] = -1;
    for (int r = total + blockIdx.x * kChunk + tid; r < max_rows; r += nchunks * kChunk) sorted_ids[r] = A;
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
    if (nchunks == 0) return MOE_OK;
    hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(kChunk), 0, s, ids, TK, A, E, Ep, nchunks, chunk_cnt);
    hipLaunchKernelGGL(permute_scan_kernel, dim3(static_cast<unsigned>(ceil_div(Ep, kScanWaves))),
                       dim3(kScanWaves * 64), 0, s, chunk_cnt, Ep, nchunks, counts);
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(kChunk), 0, s, ids, TK, A, E, Ep, nchunks, block_m,
                       max_rows, chunk_cnt, counts, offsets, sorted_ids, block_expert, inv_perm);
    return moe_launch_status();
}

}  // namespace moe

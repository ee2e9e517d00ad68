// PTPC / blockwise FP8 and MXFP4 quantization.
//
// PTPC-FP8 (Qwen3 MI300X page, 2.1.1 and Figure 3) gives every activation row
// (token) its own dynamic scale and every weight output channel its own
// static scale; the MI355X MoRI page's blockwise FP8 uses one fp32 scale per
// 128 elements.  Per group: amax = max|x|, scale = amax/448,
// q = e4m3(x * (448/amax)), IEEE fp32 divisions and one fp32 multiply.
// MXFP4 (the MoRI page's A4W4 FusedMoE and its MXFP4 dispatch): blocks of
// 32 elements with a power-of-two E8M0 scale and E2M1 elements
// (mx_row_wave in quant_dev.h).
//
// HBM-bound: one wave per row reads 16 B per lane per step (1 KB coalesced
// per wave instruction), keeps the row in registers, reduces amax with
// cross-lane shuffles (16-lane segments for 1x128 groups), then writes 8 B of
// codes per lane.  No LDS, no block barrier.
#include "quant_dev.h"

namespace moe {

// Byte offset of code (row, k) of a [rows, K] code matrix: row-major, or in
// blocks of 16 rows x 128 bytes (blocked_byte; 8-byte pieces at k % 8 == 0
// never straddle a 16-byte piece).
__device__ __forceinline__ int64_t code_off(int64_t row, int k, int K, bool blocked) {
    if (!blocked) return row * K + k;
    return ((row >> 4) * (K >> 7) + (k >> 7)) * 2048 + blocked_byte(static_cast<int>(row & 15), k & 127);
}

// NV: vectors of 8 per lane (K = 512 * NV at most).  GROUP: 0 (row) or 128.
// Codes row-major, or (BLOCKED, rows a multiple of 16) in the blocked order.
template <int NV, int GROUP>
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                         const int* __restrict__ valid_rows, bool blocked,
                                                         const int* __restrict__ skip_ids, int skip_id,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    if (valid_rows && row >= *valid_rows) return;
    if (skip_ids && skip_ids[row] == skip_id) return;     // a row nothing reads (a pad of the permutation)
    const int nvec = K >> 3;
    const bf16x8* xr = reinterpret_cast<const bf16x8*>(x + row * K);
    bf16x8 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        if (c < nvec) v[i] = ld_once(xr + c);
    }
    auto put = [&](int c, uint2 v) { *reinterpret_cast<uint2*>(q + code_off(row, 8 * c, K, blocked)) = v; };
    if (GROUP == 0) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + 64 * i < nvec) m = fmaxf(m, amax8(v[i]));
        m = wave_max(m);
        float sc, inv;
        scale_pair(m, sc, inv);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = lane + 64 * i;
            if (c < nvec) put(c, quant8(v[i], inv));
        }
        if (lane == 0) scale[row] = sc;
    } else {
        // vector c covers elements 8c..8c+7; group g = c / 16 spans 16 lanes
        const int ngroups = K / GROUP;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = lane + 64 * i;
            float m = c < nvec ? amax8(v[i]) : 0.0f;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
            float sc, inv;
            scale_pair(m, sc, inv);
            if (c < nvec) {
                put(c, quant8(v[i], inv));
                if ((lane & 15) == 0) scale[row * ngroups + (c >> 4)] = sc;
            }
        }
    }
}

// Weight rows [M, K] (PTPC: one scale per row), one wave per row, codes in
// the requested layout.
template <int NV>
__global__ void __launch_bounds__(256) quant_wrows_kernel(const uint16_t* __restrict__ w, int64_t M, int K,
                                                          bool blocked, uint8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const int nvec = K >> 3;
    const bf16x8* wr = reinterpret_cast<const bf16x8*>(w + row * K);
    bf16x8 v[NV];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        if (c < nvec) {
            v[i] = wr[c];
            m = fmaxf(m, amax8(v[i]));
        }
    }
    m = wave_max(m);
    float sc, inv;
    scale_pair(m, sc, inv);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        if (c < nvec) *reinterpret_cast<uint2*>(q + code_off(row, 8 * c, K, blocked)) = quant8(v[i], inv);
    }
    if (lane == 0) scale[row] = sc;
}

// One 128x128 weight block per workgroup: 256 threads x 8 vectors of 8.
__global__ void __launch_bounds__(256) quant_wblock_kernel(const uint16_t* __restrict__ w, int N, int K, bool blocked,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float s_max[4];
    const int nbk = K / 128, nbn = N / 128;
    const int64_t blk = blockIdx.x;
    const int64_t mat = blk / (static_cast<int64_t>(nbn) * nbk);
    const int bn = static_cast<int>((blk / nbk) % nbn), bk = static_cast<int>(blk % nbk);
    const int64_t base = mat * N * K + static_cast<int64_t>(bn) * 128 * K + static_cast<int64_t>(bk) * 128;
    const int tid = threadIdx.x;
    bf16x8 v[8];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = (tid >> 4) + 16 * i, c = tid & 15;
        v[i] = *reinterpret_cast<const bf16x8*>(w + base + static_cast<int64_t>(r) * K + 8 * c);
        m = fmaxf(m, amax8(v[i]));
    }
    m = wave_max(m);
    if ((tid & 63) == 0) s_max[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    float sc, inv;
    scale_pair(m, sc, inv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = (tid >> 4) + 16 * i, c = tid & 15;
        const int64_t row = mat * N + static_cast<int64_t>(bn) * 128 + r;
        *reinterpret_cast<uint2*>(q + code_off(row, bk * 128 + 8 * c, K, blocked)) = quant8(v[i], inv);
    }
    if (tid == 0) scale[blk] = sc;
}

// MXFP4 rows [M, K] (activations, or weight rows with K the reduction
// dimension): E2M1 codes [M, K/2] bytes, row-major or (BLOCKED) in the
// blocked order of the byte matrix, and E8M0 scales [M, K/32]; one wave per
// row, one 16-byte vector of bf16 per lane at a time.
__global__ void __launch_bounds__(256) mx_rows_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                      const int* __restrict__ valid_rows, bool blocked,
                                                      const int* __restrict__ skip_ids, int skip_id,
                                                      uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    if (valid_rows && row >= *valid_rows) return;
    if (skip_ids && skip_ids[row] == skip_id) return;
    const int Kb = K >> 1;
    mx_row_wave(x + row * K, K, [&](int b) { return q + code_off(row, b, Kb, blocked); },
                scale + row * (K >> 5), lane);
}

int32_t quant_mx_rows_launch(const uint16_t* x, int64_t M, int K, const int* valid_rows, bool blocked,
                             const int* skip_ids, int skip_id, uint8_t* q, uint8_t* scale, hipStream_t s) {
    if (M == 0) return MOE_OK;
    hipLaunchKernelGGL(mx_rows_kernel, dim3(static_cast<unsigned>(ceil_div(M, 4))), dim3(256), 0, s, x, M, K,
                       valid_rows, blocked, skip_ids, skip_id, q, scale);
    return moe_launch_status();
}

template <int GROUP>
static void launch_rows(int nv, dim3 g, hipStream_t s, const uint16_t* x, int64_t M, int K, const int* valid,
                        bool blocked, const int* skip_ids, int skip_id, uint8_t* q, float* sc) {
    const dim3 b(256);
#define MOE_ROWS(NV) hipLaunchKernelGGL((quant_rows_kernel<NV, GROUP>), g, b, 0, s, x, M, K, valid, blocked, skip_ids, \
                                        skip_id, q, sc)
    if (nv <= 1) MOE_ROWS(1);
    else if (nv <= 2) MOE_ROWS(2);
    else if (nv <= 4) MOE_ROWS(4);
    else if (nv <= 8) MOE_ROWS(8);
    else if (nv <= 16) MOE_ROWS(16);
    else MOE_ROWS(32);
#undef MOE_ROWS
}

// skip_ids (may be NULL): rows whose skip_ids entry equals skip_id are left
// unwritten
int32_t quant_rows_launch(const uint16_t* x, int64_t M, int K, int group, const int* valid_rows, uint8_t* q,
                          float* scale, hipStream_t s, bool blocked, const int* skip_ids, int skip_id) {
    if (M == 0) return MOE_OK;
    const int nv = static_cast<int>(ceil_div(K / 8, 64));
    const dim3 g(static_cast<unsigned>(ceil_div(M, 4)));
    if (group == 0) launch_rows<0>(nv, g, s, x, M, K, valid_rows, blocked, skip_ids, skip_id, q, scale);
    else launch_rows<128>(nv, g, s, x, M, K, valid_rows, blocked, skip_ids, skip_id, q, scale);
    return moe_launch_status();
}

int32_t quant_wblock_launch(const uint16_t* w, int64_t n_mats, int N, int K, bool blocked, uint8_t* q, float* scale,
                            hipStream_t s) {
    const int64_t nblk = n_mats * (N / 128) * (K / 128);
    if (nblk == 0) return MOE_OK;
    hipLaunchKernelGGL(quant_wblock_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, w, N, K, blocked, q,
                       scale);
    return moe_launch_status();
}

int32_t quant_wrows_launch(const uint16_t* w, int64_t M, int K, bool blocked, uint8_t* q, float* scale,
                           hipStream_t s) {
    if (M == 0) return MOE_OK;
    const int nv = static_cast<int>(ceil_div(K / 8, 64));
    const dim3 g(static_cast<unsigned>(ceil_div(M, 4))), b(256);
    if (nv <= 4) hipLaunchKernelGGL((quant_wrows_kernel<4>), g, b, 0, s, w, M, K, blocked, q, scale);
    else if (nv <= 8) hipLaunchKernelGGL((quant_wrows_kernel<8>), g, b, 0, s, w, M, K, blocked, q, scale);
    else if (nv <= 16) hipLaunchKernelGGL((quant_wrows_kernel<16>), g, b, 0, s, w, M, K, blocked, q, scale);
    else hipLaunchKernelGGL((quant_wrows_kernel<32>), g, b, 0, s, w, M, K, blocked, q, scale);
    return moe_launch_status();
}

}  // namespace moe

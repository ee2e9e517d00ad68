// Unpermute + weighted combine.
//
// The Qwen 3.5 TPU page moves the token unpermutation and the local
// reduction to the SparseCore so that no padded intermediate is written back
// (SparseCore unpermutation item).  Here the token's k expert-output rows
// (plus the shared row) are gathered through the inverse permutation and
// reduced in registers, j = 0..k-1 then shared, fp32 accumulate, one bf16
// rounding -- each out_perm row is read once and y written once.
#include "quant_dev.h"

namespace moe {

struct alignas(16) f32x4 { float v[4]; };

// OUT_BF16: out_perm rows are bf16 (else fp32).  Workgroup (t, y) owns
// columns [2048 y, 2048 y + 2048) of token t, 8 per thread.  The row indices
// and weights come first (uniform per workgroup), then the token's
// k + n_shared rows are loaded a few at a time (the kernel is bound by
// memory latency and bandwidth, not arithmetic).  NR >= k + n_shared.
template <bool OUT_BF16, int NR>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ out_perm,
                                                      const int* __restrict__ inv_perm,
                                                      const float* __restrict__ topk_w, int T, int k,
                                                      int n_shared, int D, uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    const int c = blockIdx.y * 256 + threadIdx.x;       // 8-column group
    const int nr = k + n_shared;
    int r[NR];
    float w[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        r[j] = -1;
        w[j] = 1.0f;
        if (j < nr) {
            r[j] = inv_perm[j < k ? static_cast<int64_t>(t) * k + j : static_cast<int64_t>(T) * k + t];
            if (j < k) w[j] = topk_w[static_cast<int64_t>(t) * k + j];
        }
    }
    if (c >= (D >> 3)) return;
    // Rows are loaded BATCH at a time and summed in index order: j = 0 ..
    // k-1 weighted (fused multiply-add), then the shared row, the same order
    // whatever the batch.  Small batches keep few registers (52-60 VGPRs, 8
    // waves per SIMD): with every row of a 9-row token in flight at once (90
    // VGPRs, 5 waves) the Qwen3-235B-shaped prefill combine took ~10 us more,
    // and batches of 6 for the 12-row one (76 VGPRs, 6 waves) ~6 us more on
    // the 512-expert layer than batches of 3 and 4.
    constexpr int BATCH = NR <= 9 ? 3 : 4;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int b0 = 0; b0 < NR; b0 += BATCH) {
        float o[BATCH][8];
#pragma unroll
        for (int jj = 0; jj < BATCH; ++jj) {
            const int j = b0 + jj;
            if (j < NR && r[j] >= 0) {
                if (OUT_BF16) {
                    // each expert-output row is read once: non-temporal
                    const bf16x8 v = ld_once(reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(out_perm) +
                                                                             static_cast<int64_t>(r[j]) * D) + c);
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[jj][i] = bf16_to_f32(v.v[i]);
                } else {
                    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(out_perm) +
                                                                    static_cast<int64_t>(r[j]) * D) + 2 * c;
                    const f32x4 a = p[0], b = p[1];
#pragma unroll
                    for (int i = 0; i < 4; ++i) { o[jj][i] = a.v[i]; o[jj][4 + i] = b.v[i]; }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) o[jj][i] = 0.0f;
            }
        }
#pragma unroll
        for (int jj = 0; jj < BATCH; ++jj) {
            const int j = b0 + jj;
            if (j < NR && r[j] >= 0) {
                if (j < k) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[j], o[jj][i], acc[i]);
                } else if (j < nr) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += o[jj][i];
                }
            }
        }
    }
    bf16x8 out;
#pragma unroll
    for (int i = 0; i < 8; ++i) out.v[i] = f32_to_bf16(acc[i]);
    reinterpret_cast<bf16x8*>(y + static_cast<int64_t>(t) * D)[c] = out;
}

template <bool OUT_BF16>
static void combine_dispatch(dim3 grid, hipStream_t s, const void* out_perm, const int* inv_perm, const float* topk_w,
                             int T, int k, int n_shared, int D, uint16_t* y) {
    // the rows a token gathers set the registers (all its loads are in
    // flight at once) and so the waves per SIMD: 9 rows take 82 VGPRs (5
    // waves), 12 rows (top-10 + shared) 106 (4), 17 rows 146 (3)
    if (k + n_shared <= 9)
        hipLaunchKernelGGL((combine_kernel<OUT_BF16, 9>), grid, dim3(256), 0, s, out_perm, inv_perm, topk_w, T, k,
                           n_shared, D, y);
    else if (k + n_shared <= 12)
        hipLaunchKernelGGL((combine_kernel<OUT_BF16, 12>), grid, dim3(256), 0, s, out_perm, inv_perm, topk_w, T, k,
                           n_shared, D, y);
    else
        hipLaunchKernelGGL((combine_kernel<OUT_BF16, MOE_MAX_TOPK + 1>), grid, dim3(256), 0, s, out_perm, inv_perm,
                           topk_w, T, k, n_shared, D, y);
}

int32_t combine_launch(const void* out_perm, int out_dtype, const int* inv_perm, const float* topk_w, int T,
                       int k, int n_shared, int D, uint16_t* y, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(ceil_div(D / 8, 256)));
    if (out_dtype == 1) combine_dispatch<true>(grid, s, out_perm, inv_perm, topk_w, T, k, n_shared, D, y);
    else combine_dispatch<false>(grid, s, out_perm, inv_perm, topk_w, T, k, n_shared, D, y);
    return moe_launch_status();
}

}  // namespace moe

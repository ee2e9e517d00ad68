// Unpermute + weighted combine.
//
// The Qwen 3.5 TPU page moves the token unpermutation and the local
// reduction to the SparseCore so that no padded intermediate is written back
// (SparseCore unpermutation item).  Here one workgroup owns one token: it
// gathers the token's k expert-output rows (plus the shared row) through the
// inverse permutation and reduces them in registers, j = 0..k-1 then shared,
// fp32 accumulate, one bf16 rounding -- each out_perm row is read once and y
// written once.
#include "common.h"

namespace moe {

struct alignas(16) u16x8 { uint16_t v[8]; };
struct alignas(16) f32x4 { float v[4]; };

// OUT_BF16: out_perm rows are bf16 (else fp32).  Each thread owns 8 columns.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ out_perm,
                                                      const int* __restrict__ inv_perm,
                                                      const float* __restrict__ topk_w, int T, int k,
                                                      int n_shared, int D, uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    const int nvec = D >> 3;
    for (int c = threadIdx.x; c < nvec; c += blockDim.x) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int j = 0; j < k + n_shared; ++j) {
            const int f = j < k ? t * k + j : T * k + t;
            const int r = inv_perm[f];
            if (r < 0) continue;
            const float w = j < k ? topk_w[static_cast<int64_t>(t) * k + j] : 1.0f;
            float o[8];
            if (OUT_BF16) {
                const u16x8 v = reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(out_perm) +
                                                               static_cast<int64_t>(r) * D)[c];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = bf16_to_f32(v.v[i]);
            } else {
                const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(out_perm) +
                                                                static_cast<int64_t>(r) * D) + 2 * c;
                const f32x4 a = p[0], b = p[1];
#pragma unroll
                for (int i = 0; i < 4; ++i) { o[i] = a.v[i]; o[4 + i] = b.v[i]; }
            }
            if (j < k) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, o[i], acc[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += o[i];
            }
        }
        u16x8 out;
#pragma unroll
        for (int i = 0; i < 8; ++i) out.v[i] = f32_to_bf16(acc[i]);
        reinterpret_cast<u16x8*>(y + static_cast<int64_t>(t) * D)[c] = out;
    }
}

int32_t combine_launch(const void* out_perm, int out_dtype, const int* inv_perm, const float* topk_w, int T,
                       int k, int n_shared, int D, uint16_t* y, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const int nvec = D / 8;
    const int threads = nvec >= 256 ? 256 : ((nvec + 63) / 64) * 64;
    if (out_dtype == 1)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(threads), 0, s, out_perm, inv_perm, topk_w, T, k,
                           n_shared, D, y);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(threads), 0, s, out_perm, inv_perm, topk_w, T, k,
                           n_shared, D, y);
    return moe_launch_status();
}

}  // namespace moe

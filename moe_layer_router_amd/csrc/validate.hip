// Debug validation of a forward's inputs: counts of non-finite activations
// and logits and of routed ids outside [0, E).  The forward takes such
// inputs without complaint (an id outside [0, E) gets no row; Inf and NaN
// go through the arithmetic as IEEE values), so a caller that wants them
// flagged runs this first.  The kernel only counts: nothing traps, and the
// counts land in a caller buffer read after the stream synchronizes.
#include "common.h"

namespace moe {

__global__ void validate_zero_kernel(int* __restrict__ counts) {
    if (threadIdx.x < 3) counts[threadIdx.x] = 0;
}

// Grid-stride over the three arrays; one atomic per wave and counter.
__global__ void __launch_bounds__(256) validate_kernel(const uint16_t* __restrict__ x, int64_t nx,
                                                       const float* __restrict__ lg, int64_t nl,
                                                       const int* __restrict__ ids, int64_t ni, int E,
                                                       int* __restrict__ counts) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int bx = 0, bl = 0, bi = 0;
    for (int64_t i = first; i < nx; i += stride) bx += (x[i] & 0x7F80u) == 0x7F80u;              // bf16 exponent all ones
    for (int64_t i = first; i < nl; i += stride) bl += (__float_as_uint(lg[i]) & 0x7F800000u) == 0x7F800000u;
    for (int64_t i = first; i < ni; i += stride) bi += ids[i] < 0 || ids[i] >= E;
    bx = wave_sum_i(bx);
    bl = wave_sum_i(bl);
    bi = wave_sum_i(bi);
    if ((threadIdx.x & 63) == 0) {
        if (bx) atomicAdd(&counts[0], bx);
        if (bl) atomicAdd(&counts[1], bl);
        if (bi) atomicAdd(&counts[2], bi);
    }
}

}  // namespace moe

extern "C" int32_t moe_validate_inputs(const void* x_bf16, int32_t T, int32_t D, const float* logits, int32_t E,
                                       const int32_t* ids, int32_t k, int32_t* counts, void* stream) {
    using namespace moe;
    MOE_CHECK_ARG(counts != nullptr && T >= 0);
    MOE_CHECK_ARG(x_bf16 == nullptr || D > 0);
    MOE_CHECK_ARG((logits == nullptr && ids == nullptr) || E > 0);
    MOE_CHECK_ARG(ids == nullptr || k > 0);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nx = x_bf16 ? static_cast<int64_t>(T) * D : 0;
    const int64_t nl = logits ? static_cast<int64_t>(T) * E : 0;
    const int64_t ni = ids ? static_cast<int64_t>(T) * k : 0;
    hipLaunchKernelGGL(validate_zero_kernel, dim3(1), dim3(64), 0, s, counts);
    const int64_t n = nx > nl ? (nx > ni ? nx : ni) : (nl > ni ? nl : ni);
    if (n > 0) {
        const int64_t blocks = ceil_div(n, 256 * 8);
        hipLaunchKernelGGL(validate_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                           s, static_cast<const uint16_t*>(x_bf16), nx, logits, nl, ids, ni, E, counts);
    }
    return moe_launch_status();
}

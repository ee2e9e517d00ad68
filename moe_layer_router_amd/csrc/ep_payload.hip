// Expert-parallel payloads: MXFP4 dispatch and FP8-blockwise combine.
//
// The MI355X MoRI page ("Hybrid FP4/FP8 quantized all-to-all") sends each
// token to its experts as MXFP4 and brings the expert outputs back as FP8
// with one fp32 scale per 128 elements; at hidden size 7168 that cuts the
// round trip from 28,672 to 11,200 bytes per token.  These kernels build and
// read those payloads on one GPU (the exchange between GPUs is not part of
// this library).  Per token row of D elements (D a multiple of 128):
//   MXFP4 (OCP Microscaling v1.0, blocks of 32 elements): D/2 bytes of FP4
//     E2M1 codes, element 2i in the low nibble of byte i, then D/32 E8M0
//     scale bytes; the block exponent is floor(log2(amax)) - 2 (E2M1's
//     largest value is 1.5 * 2^2), clamped to E8M0's [-127, 127]; elements
//     are x / 2^e rounded to the nearest E2M1 value, ties to the even
//     mantissa, saturating at 6; an all-zero block has scale byte 0.
//   FP8: D e4m3fn codes of the 1x128 blockwise quantization (the same
//     arithmetic as the activation quantizer), then D/128 fp32 scales.
// HBM-bound: one wave per row, 16 bytes of bf16 per lane per vector, codes
// and scales written as 4-byte words (every payload row starts 4-byte
// aligned).
#include "quant_dev.h"

namespace moe {

// 16-byte vectors per lane loaded before any is used: the unpack kernels
// keep a 4096-element row in flight at once; the pack kernels go one vector
// at a time (their amax, shuffles and encoding then overlap other waves'
// loads; holding 8 vectors measured 18.8 -> 24.9 us for the FP8 pack of
// 8192 x 4096)
constexpr int kPackUnroll = 1, kUnpackUnroll = 8;

__global__ void __launch_bounds__(256) ep_pack_mxfp4_kernel(const uint16_t* __restrict__ x, int T, int D,
                                                            uint8_t* __restrict__ payload) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= T) return;
    const int nvec = D >> 3, P = D / 2 + D / 32;
    const bf16x8* xr = reinterpret_cast<const bf16x8*>(x + row * D);
    uint8_t* pr = payload + row * P;
    // vector c holds elements 8c .. 8c+7; a 32-element block is 4 lanes
    for (int c0 = 0; c0 < nvec; c0 += 64 * kPackUnroll) {
        bf16x8 v[kPackUnroll];
#pragma unroll
        for (int i = 0; i < kPackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            v[i] = c < nvec ? ld_once(xr + c) : bf16x8{};
        }
#pragma unroll
        for (int i = 0; i < kPackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            const bool valid = c < nvec;      // uniform over each 16-lane group (nvec % 16 == 0)
            float m = amax8(v[i]);
            m = fmaxf(m, __shfl_xor(m, 1, 64));
            m = fmaxf(m, __shfl_xor(m, 2, 64));
            const int e = mx_exponent(m);
            const uint32_t w = mx_codes8(v[i], exp2i(-e));   // x / 2^e, exact (a power of two)
            // the scale bytes of 4 consecutive blocks (lanes l, l+4, l+8, l+12)
            // go out as one word from lane l, l % 16 == 0
            const uint32_t sb = static_cast<uint32_t>(e + 127);
            const uint32_t s4 = __shfl_down(sb, 0, 64) | (__shfl_down(sb, 4, 64) << 8) |
                                (__shfl_down(sb, 8, 64) << 16) | (__shfl_down(sb, 12, 64) << 24);
            if (valid) {
                *reinterpret_cast<uint32_t*>(pr + 4 * c) = w;
                if ((lane & 15) == 0) *reinterpret_cast<uint32_t*>(pr + D / 2 + (c >> 2)) = s4;
            }
        }
    }
}

__global__ void __launch_bounds__(256) ep_unpack_mxfp4_kernel(const uint8_t* __restrict__ payload, int T, int D,
                                                              uint16_t* __restrict__ x) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= T) return;
    const int nvec = D >> 3, P = D / 2 + D / 32;
    const uint8_t* pr = payload + row * P;
    bf16x8* xr = reinterpret_cast<bf16x8*>(x + row * D);
    for (int c0 = 0; c0 < nvec; c0 += 64 * kUnpackUnroll) {
        uint32_t w[kUnpackUnroll], sb[kUnpackUnroll];
#pragma unroll
        for (int i = 0; i < kUnpackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            w[i] = c < nvec ? *reinterpret_cast<const uint32_t*>(pr + 4 * c) : 0u;
            sb[i] = c < nvec ? pr[D / 2 + (c >> 2)] : 127u;
        }
#pragma unroll
        for (int i = 0; i < kUnpackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            const float X = exp2i(static_cast<int>(sb[i]) - 127);
            bf16x8 o;
#pragma unroll
            for (int j = 0; j < 8; ++j) o.v[j] = f32_to_bf16(e2m1_value((w[i] >> (4 * j)) & 0xF) * X);   // exact
            if (c < nvec) xr[c] = o;
        }
    }
}

__global__ void __launch_bounds__(256) ep_pack_fp8_kernel(const uint16_t* __restrict__ x, int T, int D,
                                                          uint8_t* __restrict__ payload) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= T) return;
    const int nvec = D >> 3, P = D + D / 32;
    const bf16x8* xr = reinterpret_cast<const bf16x8*>(x + row * D);
    uint8_t* pr = payload + row * P;
    float* sr = reinterpret_cast<float*>(pr + D);
    // a 128-element group is 16 lanes
    for (int c0 = 0; c0 < nvec; c0 += 64 * kPackUnroll) {
        bf16x8 v[kPackUnroll];
#pragma unroll
        for (int i = 0; i < kPackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            v[i] = c < nvec ? ld_once(xr + c) : bf16x8{};
        }
#pragma unroll
        for (int i = 0; i < kPackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            const bool valid = c < nvec;      // uniform over each 16-lane group (nvec % 16 == 0)
            float m = amax8(v[i]);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
            float sc, inv;
            scale_pair(m, sc, inv);
            if (valid) {
                const uint2 q = quant8(v[i], inv);
                reinterpret_cast<uint32_t*>(pr + 8 * c)[0] = q.x;
                reinterpret_cast<uint32_t*>(pr + 8 * c)[1] = q.y;
                if ((lane & 15) == 0) sr[c >> 4] = sc;
            }
        }
    }
}

__global__ void __launch_bounds__(256) ep_unpack_fp8_kernel(const uint8_t* __restrict__ payload, int T, int D,
                                                            uint16_t* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= T) return;
    const int nvec = D >> 3, P = D + D / 32;
    const uint8_t* pr = payload + row * P;
    const float* sr = reinterpret_cast<const float*>(pr + D);
    bf16x8* yr = reinterpret_cast<bf16x8*>(y + row * D);
    for (int c0 = 0; c0 < nvec; c0 += 64 * kUnpackUnroll) {
        uint32_t lo[kUnpackUnroll], hi[kUnpackUnroll];
        float s[kUnpackUnroll];
#pragma unroll
        for (int i = 0; i < kUnpackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            const bool valid = c < nvec;
            lo[i] = valid ? reinterpret_cast<const uint32_t*>(pr + 8 * c)[0] : 0u;
            hi[i] = valid ? reinterpret_cast<const uint32_t*>(pr + 8 * c)[1] : 0u;
            s[i] = valid ? sr[c >> 4] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kUnpackUnroll; ++i) {
            const int c = c0 + 64 * i + lane;
            bf16x8 o;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t code = ((j < 4 ? lo[i] : hi[i]) >> (8 * (j & 3))) & 0xFF;
                o.v[j] = f32_to_bf16(e4m3_to_f32(code) * s[i]);     // one fp32 product, then bf16
            }
            if (c < nvec) yr[c] = o;
        }
    }
}

int64_t ep_payload_row_bytes(int D, int format) {
    if (format == MOE_PAYLOAD_MXFP4) return D / 2 + D / 32;
    if (format == MOE_PAYLOAD_FP8_BLOCK) return D + D / 32;
    return -1;
}

int32_t ep_pack_launch(const uint16_t* x, int T, int D, int format, uint8_t* payload, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const dim3 g(static_cast<unsigned>(ceil_div(T, 4))), b(256);
    if (format == MOE_PAYLOAD_MXFP4) hipLaunchKernelGGL(ep_pack_mxfp4_kernel, g, b, 0, s, x, T, D, payload);
    else hipLaunchKernelGGL(ep_pack_fp8_kernel, g, b, 0, s, x, T, D, payload);
    return moe_launch_status();
}

int32_t ep_unpack_launch(const uint8_t* payload, int T, int D, int format, uint16_t* x, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const dim3 g(static_cast<unsigned>(ceil_div(T, 4))), b(256);
    if (format == MOE_PAYLOAD_MXFP4) hipLaunchKernelGGL(ep_unpack_mxfp4_kernel, g, b, 0, s, payload, T, D, x);
    else hipLaunchKernelGGL(ep_unpack_fp8_kernel, g, b, 0, s, payload, T, D, x);
    return moe_launch_status();
}

}  // namespace moe

// Device helpers shared by the MoE kernels: number-format conversions, wave
// reductions and launch plumbing.  gfx950 only (wave64, CDNA4 MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_WAVE 64

namespace moe {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round-to-nearest-even fp32 -> bf16 (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// two fp32 -> bf16, round to nearest even, packed (a in the low half): one
// v_cvt_pk_bf16_f32; the same values as f32_to_bf16 for finite inputs
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// SwiGLU: silu(g) * u = g / (1 + e^-g) * u, with the hardware base-2
// exponential and reciprocal (each within about 1 ulp in fp32, far below the
// bf16 rounding that follows)
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f)) * u;
}

// ---------------------------------------------------------------- e4m3fn
// OCP e4m3fn: bias 7, 3 mantissa bits, subnormals m * 2^-9, max 448 (0x7E),
// 0x7F/0xFF NaN.  Value of a code (encoding uses the hardware converter
// after a +-448 clamp; see quant_dev.h).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float v = e == 0 ? static_cast<float>(m) * 0.001953125f
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
        int t = __shfl_up(v, o, MOE_WAVE);
        if (lane >= o) v += t;
    }
    return v;
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Blocked FP8 weights (MOE_WEIGHTS_BLOCKED): a [N, K] code matrix is stored
// as blocks of 16 rows x 128 bytes (one K step of the expert GEMMs), block
// (n / 16, b / 128) at ((n / 16) * (K / 128) + b / 128) * 2048.  Inside a
// block, each 128-byte line holds one 64-byte K half of two consecutive
// rows: byte (r, b) at line (r / 2) + 8 * (b / 64), 16-byte piece
// (r % 2) * 4 + (b % 64) / 16.  The prefill GEMM's copy of 8 rows x 128
// bytes and the decode GEMM's load of 16 rows x 4 pieces (one MFMA operand
// half) then both read 8 whole lines.
__host__ __device__ constexpr int blocked_byte(int r, int b) {
    return ((r >> 1) + 8 * (b >> 6)) * 128 + ((r & 1) * 4 + ((b >> 4) & 3)) * 16 + (b & 15);
}

}  // namespace moe

// ---------------------------------------------------------------- host side
#define MOE_CHECK_ARG(c)            \
    do {                            \
        if (!(c)) return MOE_ERR_INVALID_ARG; \
    } while (0)
#define MOE_CHECK_SUP(c)            \
    do {                            \
        if (!(c)) return MOE_ERR_UNSUPPORTED; \
    } while (0)

static inline int32_t moe_launch_status() {
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

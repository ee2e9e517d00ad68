// FP8 (OCP e4m3fn) row-quantization helpers shared by the quantization
// kernels and the fused small-batch front end: per group amax, scale =
// amax/448, codes e4m3(x * (448/amax)) with IEEE fp32 divisions.
#pragma once
#include "common.h"

namespace moe {

struct alignas(16) bf16x8 { uint16_t v[8]; };

// A 16-byte load of data read once (rows that are quantized or combined and
// not read again): marked non-temporal, so it does not displace reused data
// in the caches.
__device__ __forceinline__ bf16x8 ld_once(const bf16x8* p) {
    typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p)));
}

// Eight codes with the packed hardware conversion (v_cvt_pk_fp8_f32, round to
// nearest even, subnormals kept) after clamping to +-448, so that nothing
// reaches the NaN codes.  The GPU tests compare these codes with an encoder
// written from the format definition on every bf16 value at scale 1 and at
// a scale that is not a power of two, and on every rounding midpoint.
__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
}
__device__ __forceinline__ uint2 quant8(const bf16x8& x, float inv) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = bf16_to_f32(x.v[i]) * inv;
    return make_uint2(cvt4(f[0], f[1], f[2], f[3]), cvt4(f[4], f[5], f[6], f[7]));
}

__device__ __forceinline__ float amax8(const bf16x8& x) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(bf16_to_f32(x.v[i])));
    return m;
}

__device__ __forceinline__ void scale_pair(float amax, float& scale, float& inv) {
    if (amax == 0.0f) { scale = 1.0f; inv = 1.0f; }
    else { scale = amax / 448.0f; inv = 448.0f / amax; }
}

}  // namespace moe

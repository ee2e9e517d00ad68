// FP8 (OCP e4m3fn) row-quantization helpers shared by the quantization
// kernels and the fused small-batch front end: per group amax, scale =
// amax/448, codes e4m3(x * (448/amax)) with IEEE fp32 divisions.
#pragma once
#include "common.h"

#include <type_traits>

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

// Codes of the vectors c = c0 + lane + 64 i (i < 8, c < nvec) of one row,
// 8 elements each: GROUP 0 with the row's inverse scale; GROUP 128 forms each
// 1x128 group's scale from the 16 lanes that hold the group.
template <int GROUP>
__device__ __forceinline__ void quant_vecs(const bf16x8 (&v)[8], int c0, int nvec, float inv, uint2* __restrict__ qv,
                                           float* __restrict__ sr, int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = c0 + lane + 64 * i;
        if constexpr (GROUP == 0) {
            if (c < nvec) qv[c] = quant8(v[i], inv);
        } else {
            float m = amax8(v[i]);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
            float sc, gi;
            scale_pair(m, sc, gi);
            if (c < nvec) {
                qv[c] = quant8(v[i], gi);
                if ((lane & 15) == 0) sr[c >> 4] = sc;
            }
        }
    }
}

__device__ __forceinline__ float amax_vecs(const bf16x8 (&v)[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, amax8(v[i]));
    return m;
}

// One row of x into codes with the wave, in chunks of 4096 elements (8
// vectors of 8 per lane, all loads of a chunk in flight together).  GROUP 0
// (one scale per row): amax over the chunks, then codes (a single-chunk row
// stays in registers, longer rows are read again); GROUP 128: one pass,
// 16-lane groups.
template <int GROUP>
__device__ __forceinline__ void quant_row_wave(const uint16_t* __restrict__ xr, int K, uint8_t* __restrict__ qr,
                                               float* __restrict__ sr, int lane) {
    constexpr int CV = 8;
    const int nvec = K >> 3;
    const int nch = (nvec + 64 * CV - 1) / (64 * CV);
    const bf16x8* xv = reinterpret_cast<const bf16x8*>(xr);
    uint2* qv = reinterpret_cast<uint2*>(qr);
    bf16x8 v[CV];
    auto load = [&](int ch) {
#pragma unroll
        for (int i = 0; i < CV; ++i) {
            const int c = ch * 64 * CV + lane + 64 * i;
            v[i] = c < nvec ? xv[c] : bf16x8{};
        }
    };
    if constexpr (GROUP == 0) {
        float m = 0.0f;
        for (int ch = 0; ch < nch; ++ch) {
            load(ch);
            m = fmaxf(m, amax_vecs(v));
        }
        m = wave_max(m);
        float sc, inv;
        scale_pair(m, sc, inv);
        for (int ch = 0; ch < nch; ++ch) {
            if (nch > 1) load(ch);
            quant_vecs<0>(v, ch * 64 * CV, nvec, inv, qv, sr, lane);
        }
        if (lane == 0) sr[0] = sc;
    } else {
        for (int ch = 0; ch < nch; ++ch) {
            load(ch);
            quant_vecs<128>(v, ch * 64 * CV, nvec, 0.0f, qv, sr, lane);
        }
    }
}

// A row of at most 4096 elements already in registers (v[i] = vector
// lane + 64 i of the row, zero past its end): the same codes and scales as
// quant_row_wave.
template <int GROUP>
__device__ __forceinline__ void quant_row_regs(const bf16x8 (&v)[8], int K, uint8_t* __restrict__ qr,
                                               float* __restrict__ sr, int lane) {
    uint2* qv = reinterpret_cast<uint2*>(qr);
    float inv = 0.0f;
    if constexpr (GROUP == 0) {
        float sc;
        scale_pair(wave_max(amax_vecs(v)), sc, inv);
        if (lane == 0) sr[0] = sc;
    }
    quant_vecs<GROUP>(v, 0, K >> 3, inv, qv, sr, lane);
}

// value of an E2M1 code: exponent field 0 is 0 or 0.5, else (1 + m/2) * 2^(e-1)
__device__ __forceinline__ float e2m1_value(uint32_t c) {
    const uint32_t e = (c >> 1) & 3, m = c & 1;
    const float mag = e == 0 ? 0.5f * static_cast<float>(m) : __uint_as_float(((e + 126) << 23) | (m << 22));
    return (c & 8) ? -mag : mag;
}

// 2^k as fp32 for k in [-127, 127] (2^-127 is a subnormal)
__device__ __forceinline__ float exp2i(int k) {
    return k >= -126 ? __uint_as_float(static_cast<uint32_t>(k + 127) << 23) : __uint_as_float(0x00400000u);
}

// floor(log2(a)) for finite a > 0, from the exponent field (subnormals by
// the position of their leading mantissa bit)
__device__ __forceinline__ int floor_log2(float a) {
    const uint32_t b = __float_as_uint(a);
    const int ef = static_cast<int>((b >> 23) & 0xFF);
    return ef > 0 ? ef - 127 : (31 - __clz(b & 0x7FFFFF)) - 149;
}

// f(0) .. f(3) with compile-time indices (the conversion's byte selector
// must be a constant)
template <typename F>
__device__ __forceinline__ void static_for_pk(F&& f) {
    f(std::integral_constant<int, 0>{});
    f(std::integral_constant<int, 1>{});
    f(std::integral_constant<int, 2>{});
    f(std::integral_constant<int, 3>{});
}

// MXFP4 (OCP Microscaling v1.0) block exponent of a 32-element block with
// largest magnitude amax: floor(log2(amax)) - 2 (E2M1's largest value is
// 1.5 * 2^2), clamped to E8M0's [-127, 127]; an all-zero block gets -127.
__device__ __forceinline__ int mx_exponent(float amax) {
    return amax > 0.0f ? max(floor_log2(amax) - 2, -127) : -127;
}

// E2M1 codes of 8 elements scaled by inv (a power of two, so the scaling is
// exact), two per byte with element 2j in the low nibble of byte j, by the
// hardware conversion (v_cvt_scalef32_pk_fp4_f32 with scale 1: round to
// nearest, ties to the even mantissa, saturating to +-6, sign of zero
// kept), which matches the E2M1 encoder written from the format definition
// on every bf16 value (tested).
__device__ __forceinline__ uint32_t mx_codes8(const bf16x8& v, float inv) {
    uint32_t w = 0;
    static_for_pk([&](auto J) {
        constexpr int j = decltype(J)::value;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, bf16_to_f32(v.v[2 * j]) * inv,
                                                     bf16_to_f32(v.v[2 * j + 1]) * inv, 1.0f, j);
    });
    return w;
}

// One row of K bf16 values (K % 128 == 0) to MXFP4 with the wave: codes
// [K/2] bytes (4 bytes per lane per vector of 8, at code_byte(4c)), E8M0
// scale bytes [K/32] (four blocks per word, from every 16th lane).  Vector
// c covers elements 8c .. 8c+7; a 32-element block is 4 consecutive lanes.
template <typename CodeByte>
__device__ __forceinline__ void mx_row_wave(const uint16_t* __restrict__ xr, int K, CodeByte code_byte,
                                            uint8_t* __restrict__ sr, int lane) {
    const int nvec = K >> 3;
    const bf16x8* xv = reinterpret_cast<const bf16x8*>(xr);
    for (int c0 = 0; c0 < nvec; c0 += 64) {
        const int c = c0 + lane;
        const bool valid = c < nvec;          // uniform over each 16-lane group (nvec % 16 == 0)
        const bf16x8 v = valid ? ld_once(xv + c) : bf16x8{};
        float m = amax8(v);
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        const int e = mx_exponent(m);
        const uint32_t w = mx_codes8(v, exp2i(-e));
        const uint32_t sb = static_cast<uint32_t>(e + 127);
        const uint32_t s4 = __shfl_down(sb, 0, 64) | (__shfl_down(sb, 4, 64) << 8) |
                            (__shfl_down(sb, 8, 64) << 16) | (__shfl_down(sb, 12, 64) << 24);
        if (valid) {
            *reinterpret_cast<uint32_t*>(code_byte(4 * c)) = w;
            if ((lane & 15) == 0) *reinterpret_cast<uint32_t*>(sr + (c >> 2)) = s4;
        }
    }
}

// Token t's row of x [T, D] to the layer's activation format with the wave:
// GROUP 0 (PTPC: fp32 scale per row), 128 (fp32 scale per 1x128 group) or
// 32 (MXFP4: codes [T, D/2], E8M0 scale bytes [T, D/32] at xs).
template <int GROUP>
__device__ __forceinline__ void quant_x_row(const uint16_t* __restrict__ x, int D, int64_t t, uint8_t* xq, void* xs,
                                            int lane) {
    if constexpr (GROUP == 32) {
        uint8_t* qr = xq + t * (D / 2);
        mx_row_wave(x + t * D, D, [&](int b) { return qr + b; }, static_cast<uint8_t*>(xs) + t * (D / 32), lane);
    } else {
        quant_row_wave<GROUP>(x + t * D, D, xq + t * D, static_cast<float*>(xs) + t * (GROUP == 128 ? D / 128 : 1),
                              lane);
    }
}

}  // namespace moe

// fp8 K/V cache codes: OCP E4M3 "fn" (bias 7, max 448, S.1111.111 = NaN, no
// infinities) and E5M2 (bias 15, max 57344, IEEE-like infinities and NaNs),
// in plain integer arithmetic so that the result does not depend on a
// conversion instruction's mode bits.
#pragma once

#include "common.h"

namespace dflash {

enum { FP8_NONE = 0, FP8_E4M3 = 1, FP8_E5M2 = 2 };

// fp32 -> fp8 code: nearest value, ties to the even code, magnitudes past the
// largest finite value saturate to it; NaN -> 0x7F.
template <int FMT>
__device__ __forceinline__ uint32_t f32_to_fp8(float x) {
    constexpr int EB = FMT == FP8_E4M3 ? 4 : 5;
    constexpr int MB = FMT == FP8_E4M3 ? 3 : 2;
    constexpr int BIAS = (1 << (EB - 1)) - 1;
    constexpr uint32_t MAXC = FMT == FP8_E4M3 ? 0x7Eu : 0x7Bu;
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7Fu;
    const int e = (int)(a >> 23) - 127;
    if (e < 1 - BIAS) {
        // below the smallest normal: multiples of 2^(1 - BIAS - MB); the scaling
        // by a power of two is exact, rintf rounds to nearest even; 2^MB is the
        // smallest normal's code
        const float q = rintf(__uint_as_float(a) * (float)(1 << (BIAS - 1 + MB)));
        return sign | (uint32_t)q;
    }
    constexpr int SH = 23 - MB;
    const uint32_t mant = a & 0x7fffffu;
    uint32_t m = (mant + ((1u << (SH - 1)) - 1u) + ((mant >> SH) & 1u)) >> SH;
    int ef = e + BIAS;
    if (m == (1u << MB)) { m = 0; ++ef; }
    if (ef >= (1 << EB)) return sign | MAXC;
    const uint32_t code = ((uint32_t)ef << MB) | m;
    return sign | (code > MAXC ? MAXC : code);
}

// fp8 code -> bf16 bits (exact: every finite fp8 value is a bf16 value).
template <int FMT>
__device__ __forceinline__ uint32_t fp8_to_bf16_bits(uint32_t c) {
    constexpr int EB = FMT == FP8_E4M3 ? 4 : 5;
    constexpr int MB = FMT == FP8_E4M3 ? 3 : 2;
    constexpr int BIAS = (1 << (EB - 1)) - 1;
    const uint32_t sign = (c & 0x80u) << 8;
    const uint32_t e = (c >> MB) & ((1u << EB) - 1u);
    const uint32_t m = c & ((1u << MB) - 1u);
    if (e == 0) {
        if (m == 0) return sign;
        const int p = 31 - __builtin_clz(m);  // leading bit of the subnormal's mantissa
        const uint32_t exp = (uint32_t)(p + 1 - BIAS - MB + 127);
        return sign | (exp << 7) | ((m - (1u << p)) << (7 - p));
    }
    if (FMT == FP8_E4M3 && e == 15 && m == 7) return 0x7FC0u;
    if (FMT == FP8_E5M2 && e == 31) return sign | (m == 0 ? 0x7F80u : 0x7FC0u);
    return sign | ((e - BIAS + 127) << 7) | (m << (7 - MB));
}

// Eight fp32 values divided by a scale -> eight fp8 codes, little-endian in
// two words.
template <int FMT>
__device__ __forceinline__ u32x2 pack_fp8x8(const float (&v)[8], float scale) {
    u32x2 w = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e >> 2] |= f32_to_fp8<FMT>(v[e] / scale) << (8 * (e & 3));
    return w;
}

}  // namespace dflash

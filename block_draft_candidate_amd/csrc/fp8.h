// fp8 K/V cache codes: OCP E4M3 "fn" (bias 7, max 448, S.1111.111 = NaN, no
// infinities) and E5M2 (bias 15, max 57344, IEEE-like infinities and NaNs).
// The encoder is plain integer arithmetic, so its rounding and saturation do
// not depend on a conversion instruction's mode bits.  (Decoding uses the
// hardware conversions, which give these formats' values exactly.)
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

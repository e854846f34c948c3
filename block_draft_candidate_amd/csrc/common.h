// Shared device helpers of libdflash (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed pair of bf16 (lo, hi).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 16-byte chunk of 8 bf16 <-> 8 floats.
__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void stg16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

}  // namespace dflash

// Host-side helpers shared by the entry points.
#define DFLASH_ALIGNED16(p) ((reinterpret_cast<uintptr_t>(p) & 15u) == 0)

#define DFLASH_LAUNCH_CHECK()                                   \
    do {                                                        \
        if (hipGetLastError() != hipSuccess) return DFLASH_ERR_HIP; \
    } while (0)

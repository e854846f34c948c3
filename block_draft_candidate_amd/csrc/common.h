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
typedef __attribute__((ext_vector_type(16))) float f32x16;

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

// ---------------------------------------------------------------------------
// LDS-DMA tile loads (buffer_load_dwordx4 ... lds): 64-wide K slices of
// K-contiguous bf16 rows, 128 bytes per row in LDS, 16-byte chunks XOR-swizzled
// by row (chunk ^ row % 8) so that 16x16x32 / 32x32x16 fragment reads are
// bank-conflict free.
// ---------------------------------------------------------------------------
// Per-lane byte offsets of the LDS-DMA loads of one 64-wide K slice of the
// rows this wave loads: instructions q = wave * NI + j, each filling 1 KB = 8
// rows of 128 B.  Lane i of instruction q lands at LDS byte q*1024 + i*16,
// i.e. row 8q + i/8, physical chunk i%8; it therefore loads logical chunk
// (i%8) ^ (row%8), which realises the XOR swizzle the fragment reads expect.
template <int NI>
__device__ __forceinline__ void dma_offsets(int (&voff)[NI], int wave_s, int lane, int Hd) {
    const int r8 = lane >> 3;
    const int lc = (lane & 7) ^ r8;
#pragma unroll
    for (int j = 0; j < NI; ++j) voff[j] = (((wave_s * NI + j) * 8 + r8) * Hd + lc * 8) * 2;
}

// Issue them for the slice starting at column k0.  Rows past the tile and
// columns past Hd read as zero (offsets past the buffer range); branch-free, so
// the loads can be interleaved with MFMAs by the scheduler.
template <int NI>
__device__ __forceinline__ void dma_slice(__amdgpu_buffer_rsrc_t rsrc, uint16_t* lds_tile, const int* voff,
                                          int wave_s, int lane, int Hd, int k0) {
    const bool in = k0 + (((lane & 7) ^ (lane >> 3)) * 8) < Hd;
#pragma unroll
    for (int j = 0; j < NI; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(lds_tile + (wave_s * NI + j) * 512), 16,
            in ? voff[j] + k0 * 2 : (int)0x80000000, 0, 0, 0);
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

}  // namespace dflash

// Host-side helpers shared by the entry points.
#define DFLASH_ALIGNED16(p) ((reinterpret_cast<uintptr_t>(p) & 15u) == 0)

#define DFLASH_LAUNCH_CHECK()                                   \
    do {                                                        \
        if (hipGetLastError() != hipSuccess) return DFLASH_ERR_HIP; \
    } while (0)

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

// A 16-byte load of data read once (a weight stream): the nontemporal hint keeps
// it from being allocated in the caches on the way in, which lets a streaming
// read run markedly closer to the HBM peak than plain loads do.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void stg16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// LDS-DMA tile loads (buffer_load_dwordx4 ... lds): 64-wide K slices of
// K-contiguous bf16 rows, 128 bytes per row in LDS, 16-byte chunks XOR-swizzled
// by row: physical chunk = logical chunk ^ swz8(row).
//
// swz8 folds bits 2..4 of the row into bits 0..2: with chunk ^ (row % 8) alone,
// rows r and r + 8 of the 32 rows a 32x32x16 fragment read touches land on the
// same banks, and ds_read_b128 runs at about 55% of the rate it reaches for
// linear addresses (measured on gfx950); with swz8 it reaches that rate.  For a
// row inside an aligned 32-row block swz8 depends only on row % 32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 2)) & 7; }

// Per-lane byte offsets of the LDS-DMA loads of one 64-wide K slice of the
// rows this wave loads: instructions q = wave * NI + j, each filling 1 KB = 8
// rows of 128 B.  Lane i of instruction q lands at LDS byte q*1024 + i*16,
// i.e. row 8q + i/8, physical chunk i%8; it therefore loads logical chunk
// (i%8) ^ swz8(row).  The logical chunks (3 bits per j) go to lcpack for the
// K-tail check.
template <int NI>
__device__ __forceinline__ void dma_offsets(int (&voff)[NI], int& lcpack, int wave_s, int lane, int Hd) {
    static_assert(NI <= 10, "3 bits per instruction in lcpack");
    const int r8 = lane >> 3;
    lcpack = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int row = (wave_s * NI + j) * 8 + r8;
        const int lc = (lane & 7) ^ swz8(row);
        voff[j] = (row * Hd + lc * 8) * 2;
        lcpack |= lc << (3 * j);
    }
}

// One of those loads (instruction j of this wave) for the slice starting at
// column k0; see dma_slice.  AUX is the load's cache policy (2: nontemporal).
template <int NI, bool TAIL, int AUX = 0>
__device__ __forceinline__ void dma_one(__amdgpu_buffer_rsrc_t rsrc, uint16_t* lds_tile, const int* voff,
                                        int lcpack, int wave_s, int Hd, int k0, int j) {
    auto* dst = (__attribute__((address_space(3))) void*)(lds_tile + (wave_s * NI + j) * 512);
    if (TAIL) {
        const bool in = k0 + ((lcpack >> (3 * j)) & 7) * 8 < Hd;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, in ? voff[j] + k0 * 2 : (int)0x80000000, 0, 0, AUX);
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff[j], k0 * 2, 0, AUX);
    }
}

// Issue them for the slice starting at column k0.  Rows past the tile read as
// zero (offsets past the buffer range).  Without a K tail (Hd % 64 == 0) the
// column offset goes into the scalar offset and no vector work is needed; with
// one, chunks past Hd get an out-of-range offset.  Branch-free, so the loads
// can be interleaved with MFMAs by the scheduler.
template <int NI, bool TAIL, int AUX = 0>
__device__ __forceinline__ void dma_slice(__amdgpu_buffer_rsrc_t rsrc, uint16_t* lds_tile, const int* voff,
                                          int lcpack, int wave_s, int Hd, int k0) {
#pragma unroll
    for (int j = 0; j < NI; ++j) dma_one<NI, TAIL, AUX>(rsrc, lds_tile, voff, lcpack, wave_s, Hd, k0, j);
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// s_waitcnt immediate that waits for vmcnt <= n and lgkmcnt == 0.
constexpr int vm_lgkm0_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// Wait until at most `ahead` ring stages of NI loads each are still in flight
// (and lgkmcnt == 0); ahead is clamped to [0, MAXA].  The immediate must be a
// constant, hence the cases.
template <int MAXA, int NI>
__device__ __forceinline__ void wait_stages_ahead(int ahead) {
    if constexpr (MAXA <= 0) {
        __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
    } else {
        if (ahead >= MAXA) __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(MAXA * NI));
        else wait_stages_ahead<MAXA - 1, NI>(ahead);
    }
}

}  // namespace dflash

// Host-side helpers shared by the entry points.
#define DFLASH_ALIGNED16(p) ((reinterpret_cast<uintptr_t>(p) & 15u) == 0)

#define DFLASH_LAUNCH_CHECK()                                   \
    do {                                                        \
        if (hipGetLastError() != hipSuccess) return DFLASH_ERR_HIP; \
    } while (0)

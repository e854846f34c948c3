// One 256 x BN output tile of a bf16 GEMM C = A . B^T (A [rows, K], B [cols,
// K], both K-contiguous), fp32 accumulate, for the kernels whose epilogue
// needs whole rows of the tile in one workgroup (the context K/V precompute,
// the plain linear).  It is the LM head's operand pipeline:
//
//   * 256 threads, 4 waves in 2 x 2, one per SIMD; a wave computes a 128 x BN/2
//     block with v_mfma_f32_32x32x16_bf16 (4 x BN/64 blocks of 32 x 32);
//   * 64-wide K slices of both operands by LDS-DMA (buffer_load ... lds) into
//     a ring of five 32 KB LDS slots: slice k keeps its B half in slot 2k mod 5
//     and its A half in slot 2k+1 mod 5, so a B half is in flight for about two
//     slices; 16-byte chunks are XOR-swizzled by swz8(row);
//   * fragment reads in MFMA use order, interleaved with the DMA issue by
//     scheduling group barriers.
//
// Rows or columns past the operands' buffer ranges read as zero, and with TAIL
// the K columns past Hd do too.
#pragma once

#include "common.h"

namespace dflash {

constexpr int GT_BM = 256;
constexpr int GT_BK = 64;
constexpr int GT_THREADS = 256;
constexpr int GT_UNIT = GT_BM * GT_BK;          // elements of one operand's K slice
constexpr int GT_NSLOT = 5;
constexpr int GT_SP = 128 + 4;                  // pitch (floats) of a staged 128-column group
constexpr int GT_SMEM = GT_NSLOT * GT_UNIT;     // uint16 elements (160 KB)
static_assert(GT_BM * GT_SP * 2 <= GT_SMEM, "staging fits the ring");

__device__ __forceinline__ uint32_t gt_lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int BN, bool TAIL>
__device__ __forceinline__ void gemm_tile_mainloop(uint16_t* smem, __amdgpu_buffer_rsrc_t rsA,
                                                   __amdgpu_buffer_rsrc_t rsB, int Hd,
                                                   f32x16 (&acc)[4][BN / 64]) {
    constexpr int WN = BN / 2;               // columns per wave
    constexpr int NB = WN / 32;              // 32-column MFMA blocks per wave
    constexpr int MB = 4;                    // 32-row MFMA blocks per wave (128 rows)
    constexpr int NIA = GT_BM / 8 / 4;       // LDS-DMA instructions per wave per slice (A)
    constexpr int NIB = BN / 8 / 4;          // (B)
    constexpr int UNIT = GT_UNIT;
    constexpr int NSLOT = GT_NSLOT;
    static_assert(BN == 128 || BN == 192 || BN == 256, "tile width");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave >> 1, wn = wave & 1;
    const int nK = (Hd + GT_BK - 1) / GT_BK;

    const int fr = lane & 31;
    const int a_row0 = (wm * 128 + fr) * GT_BK;
    const int b_row0 = (wn * WN + fr) * GT_BK;
    int voffA[NIA], voffB[NIB], lcA, lcB;
    dma_offsets<NIA>(voffA, lcA, wave_s, lane, Hd);
    dma_offsets<NIB>(voffB, lcB, wave_s, lane, Hd);

#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Fragment qf of one 16-wide K step (A0, B0..B{NB-1}, A1..A{MB-1}: the order
    // the MFMAs consume them) of the slice whose halves sit in slots sa / sb.
    constexpr int NFR = MB + NB;
    auto read_frag = [&](int sa, int sb, int k16, int qf, bf16x8 (&fa)[MB], bf16x8 (&fb)[NB]) {
        const int chs = ((2 * k16 + (lane >> 5)) ^ swz8(fr)) << 3;
        if (qf >= 1 && qf <= NB)
            fb[qf - 1] = as_bf16x8(*reinterpret_cast<const u32x4*>(smem + sb * UNIT + b_row0 + (qf - 1) * 32 * GT_BK + chs));
        else {
            const int i = qf == 0 ? 0 : qf - NB;
            fa[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(smem + sa * UNIT + a_row0 + i * 32 * GT_BK + chs));
        }
    };
    auto mfmas = [&](const bf16x8 (&fa)[MB], const bf16x8 (&fb)[NB]) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // One K step: its MFMAs, with the next step's fragment reads and (dma = 1 /
    // 2) the LDS-DMA loads of an A / B half interleaved by group barriers.
    constexpr int MPK = MB * NB;
    auto kstep = [&](const bf16x8 (&fa)[MB], const bf16x8 (&fb)[NB], int ra, int rb, int rk16,
                     bf16x8 (&na)[MB], bf16x8 (&nb)[NB], int dma, int dkt, int dslot) {
#pragma unroll
        for (int qq = 0; qq < (NFR > NIA ? NFR : NIA); ++qq) {
            if (qq < NFR && rk16 >= 0) read_frag(ra, rb, rk16, qq, na, nb);
            if (dma == 1 && qq < NIA)
                dma_one<NIA, TAIL>(rsA, smem + dslot * UNIT, voffA, lcA, wave_s, Hd, dkt * GT_BK, qq);
            if (dma == 2 && qq < NIB)
                dma_one<NIB, TAIL>(rsB, smem + dslot * UNIT, voffB, lcB, wave_s, Hd, dkt * GT_BK, qq);
        }
        mfmas(fa, fb);
#pragma unroll
        for (int qq = 0; qq < MPK; ++qq) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (qq < NFR && rk16 >= 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if ((dma == 1 && qq < NIA) || (dma == 2 && qq < NIB)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };

    // The barrier at the end of slice k frees both of its slots: the A half of
    // slice k+2 goes into one right after it, the B half of slice k+3 into the
    // other during the first K step of slice k+1.
    bf16x8 fa0[MB], fb0[NB], fa1[MB], fb1[NB];
    dma_slice<NIB, TAIL>(rsB, smem + 0 * UNIT, voffB, lcB, wave_s, Hd, 0);
    dma_slice<NIA, TAIL>(rsA, smem + 1 * UNIT, voffA, lcA, wave_s, Hd, 0);
    dma_slice<NIB, TAIL>(rsB, smem + 2 * UNIT, voffB, lcB, wave_s, Hd, GT_BK);  // past K: zeros, unused
    dma_slice<NIA, TAIL>(rsA, smem + 3 * UNIT, voffA, lcA, wave_s, Hd, GT_BK);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NIB + NIA));  // slice 0 landed
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    int sb = 0, sa = 1;
#pragma unroll
    for (int qq = 0; qq < NFR; ++qq) read_frag(sa, sb, 0, qq, fa0, fb0);
    for (int kt = 0; kt + 1 < nK; ++kt) {
        const int sn = sb == 0 ? NSLOT - 1 : sb - 1;  // slot of the B half of slice kt+2
        kstep(fa0, fb0, sa, sb, 1, fa1, fb1, 2, kt + 2, sn);
        kstep(fa1, fb1, sa, sb, 2, fa0, fb0, 0, 0, 0);
        kstep(fa0, fb0, sa, sb, 3, fa1, fb1, 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(NIB));  // slice kt+1 landed
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        const int sa2 = sb;
        sb = sb + 2 >= NSLOT ? sb + 2 - NSLOT : sb + 2;
        sa = sa + 2 >= NSLOT ? sa + 2 - NSLOT : sa + 2;
        kstep(fa1, fb1, sa, sb, 0, fa0, fb0, 1, kt + 2, sa2);
    }
    kstep(fa0, fb0, sa, sb, 1, fa1, fb1, 0, 0, 0);
    kstep(fa1, fb1, sa, sb, 2, fa0, fb0, 0, 0, 0);
    kstep(fa0, fb0, sa, sb, 3, fa1, fb1, 0, 0, 0);
    kstep(fa1, fb1, sa, sb, -1, fa0, fb0, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Column groups of a staged pass: 128 columns, or (BN = 192) one wave
// column's 96.
template <int BN>
constexpr int gemm_tile_group() { return BN % 128 == 0 ? 128 : BN / 2; }

// Stage the tile's column group `pass` (columns GW * pass .., GW =
// gemm_tile_group<BN>()) row-major into `stage` (pitch GT_SP floats) from the
// waves that hold it, then wait for the whole workgroup.  In the 32x32 MFMA
// layout lane l holds column l % 32 and rows 8b + 4(l / 32) + e, e = 0..3; the
// writes go straight from the accumulator registers.
template <int BN>
__device__ __forceinline__ void gemm_tile_stage(float* stage, const f32x16 (&acc)[4][BN / 64], int pass) {
    constexpr int WN = BN / 2, NB = WN / 32, MB = 4;
    constexpr int GW = gemm_tile_group<BN>();
    static_assert(GW + 4 <= GT_SP, "a group fits the staging pitch");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31;
    if ((wn * WN) / GW == pass) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int col = (wn * WN) % GW + j * 32 + fr;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t dst = gt_lds_offset(stage + (wm * 128 + i * 32 + 8 * b + 4 * (lane >> 5)) * GT_SP + col);
                    asm volatile("ds_write_b32 %0, %1" ::"v"(dst), "a"(acc[i][j][4 * b]) : "memory");
                    asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(dst), "a"(acc[i][j][4 * b + 1]),
                                 "i"(GT_SP * 4) : "memory");
                    asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(dst), "a"(acc[i][j][4 * b + 2]),
                                 "i"(GT_SP * 8) : "memory");
                    asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(dst), "a"(acc[i][j][4 * b + 3]),
                                 "i"(GT_SP * 12) : "memory");
                }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staging writes done
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// End of a staged pass: every row read of `stage` is done before the next
// pass overwrites it.
__device__ __forceinline__ void gemm_tile_pass_done() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Tile width for a launch of 256 x BN tiles over rows x cols outputs, one tile
// per CU at a time: 256, 192 (only where the epilogue takes 96-column groups,
// allow192) or 128, whichever needs the fewest width-weighted rounds of the
// device's compute units (ties: the wider).
static inline int gemm_tile_width(int64_t rows, int64_t cols, bool allow192 = false) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ncu = v;
    }
    const int64_t nM = (rows + GT_BM - 1) / GT_BM;
    auto cost = [&](int64_t bn) { return ((nM * ((cols + bn - 1) / bn) + ncu - 1) / ncu) * bn; };
    int best = 256;
    if (allow192 && cost(192) < cost(best)) best = 192;
    if (cost(128) < cost(best)) best = 128;
    return best;
}

// Tile q of the launch: workgroup ids go to the 8 XCDs round-robin, and XCD x
// takes tiles [x * per, (x + 1) * per) (row tiles fastest), so its workgroups
// share B tiles and A slices in its L2.  Returns false past the last tile.
__device__ __forceinline__ bool gemm_tile_index(int ntiles, int nM, int& m_tile, int& n_tile) {
    const int per = gridDim.x >> 3;
    const int q = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (q >= ntiles) return false;
    m_tile = q % nM;
    n_tile = q / nM;
    return true;
}

}  // namespace dflash

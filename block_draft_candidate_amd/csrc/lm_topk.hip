// LM-head top-k of the DFlash2 drafter's candidate head
// (DFlash2BeamForCausalLM.compute_candidates through its LogitsProcessor:
// scale = output_multiplier, soft cap = final_logit_softcapping).
//
// One pass over the LM-head weight W [V, Hd] computes logit tiles with bf16
// MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate) and selects top-k in the
// tile epilogue; the [T, V] logits are never written to HBM.
//
//   * A workgroup (256 threads, 4 waves in 2 x 2, one per SIMD) owns a 256-row
//     slice of H and a contiguous run of BN-column tiles of W (its "group").
//     Each wave computes a 128 x BN/2 block of a 256 x BN tile.  With 64 rows
//     or fewer the row tile is 64 (32 x BN/2 per wave): the call is then a
//     skinny, bandwidth-bound product and the smaller tile saves 3/4 of the
//     MFMA work.  The K loop
//     streams 64-wide slices of H and W with LDS-DMA into a ring of five LDS
//     slots, so the W half of a slice is in flight for two slices.
//   * Epilogue: the tile is staged through LDS in two column halves; thread t
//     scans row t and keeps that row's running top-k of the group in registers
//     as packed words (ordered bf16 key << 16 | 0xFFFF - column-in-group), so
//     one unsigned compare orders (key desc, id asc).  A raw-accumulator
//     threshold derived from the current k-th key skips the scale/softcap work
//     for almost every column.
//   * Row slices and groups are blocked per XCD (workgroup ids go to XCDs
//     round-robin), so each XCD's L2 serves W tiles to several row slices and
//     H slices to several groups.
//   * Up to 32 rows (k <= 16 above 16 rows) with Hd / 256 a power of two up to
//     16, lm_topk_stream replaces the tiles: the head is then a stream over W.
//   * A merge kernel picks the k best of the groups' partial lists per row:
//     16 lanes per row up to 16 groups, a workgroup per row up to 256 groups
//     (beyond that, after launches that merge blocks of 16 lists).
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace dflash {

constexpr int LM_BM = 256;

// Byte offset in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
constexpr int LM_BK = 64;
constexpr int LM_THREADS = 256;

// bf16 bits -> 16-bit code whose unsigned order is the value order (-0 == +0).
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
    if (b == 0x8000u) b = 0;
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}
__device__ __forceinline__ uint32_t unorder_key(uint32_t o) {
    return (o & 0x8000u) ? (o & 0x7fffu) : (~o & 0xffffu);
}

// tanh in fp32 for the soft cap, within a few ulp: the odd Taylor series of
// tanh through y^15 below |y| = 0.55 (truncation under half an ulp there), and
// 1 - 2 / (e^{2|y|} + 1) above, where tanh >= 0.5 keeps the subtraction exact
// enough (hardware exp2 and reciprocal, about 1 ulp each).
// Both forms are evaluated and one is selected (no divergent branch: this runs
// once per candidate inside the wave's candidate rounds).
__device__ __forceinline__ float cap_tanh(float y) {
    const float a = fabsf(y);
    const float z = a * a;
    float q = -929569.f / 638512875.f;
    q = fmaf(q, z, 21844.f / 6081075.f);
    q = fmaf(q, z, -1382.f / 155925.f);
    q = fmaf(q, z, 62.f / 2835.f);
    q = fmaf(q, z, -17.f / 315.f);
    q = fmaf(q, z, 2.f / 15.f);
    q = fmaf(q, z, -1.f / 3.f);
    const float tp = fmaf(a * z, q, a);
    const float e = __builtin_amdgcn_exp2f(a * 2.8853900817779268f);  // e^{2a}; inf for large a
    const float te = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
    return copysignf(a < 0.55f ? tp : te, y);
}

// fp32 -> bf16 bits, round to nearest even; a NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_key_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : rne;
}

// The top-k key of one accumulator: bf16(c * tanh(s * acc / c)), or bf16(s * acc)
// without a cap (c = 0; c is uniform) ...
__device__ __forceinline__ uint32_t logit_key_bits(float acc, float s, float c, float inv_c) {
    float x = s * acc;
    if (c > 0.f) x = c * cap_tanh(x * inv_c);
    return bf16_key_bits(x);
}
// ... and the same with the cap setting known at compile time.
template <bool CAP>
__device__ __forceinline__ uint32_t logit_key_bits_as(float acc, float s, float c, float inv_c) {
    float x = s * acc;
    if constexpr (CAP) x = c * cap_tanh(x * inv_c);
    return bf16_key_bits(x);
}

// atanh for |z| < 0.9 in fp32, within about 1e-6 relative: the odd series
// through z^13 below |z| = 0.25 (the first dropped term is under 3e-10 of the
// sum), above it half the natural log of (1 + |z|) / (1 - |z|), a ratio of at
// least 5/3 whose hardware log2 and reciprocal err by about an ulp each.  Both
// forms are evaluated and one is selected.
__device__ __forceinline__ float bound_atanh(float z) {
    const float a = fabsf(z);
    const float q = a * a;
    float p = 1.f / 13.f;
    p = fmaf(p, q, 1.f / 11.f);
    p = fmaf(p, q, 1.f / 9.f);
    p = fmaf(p, q, 1.f / 7.f);
    p = fmaf(p, q, 1.f / 5.f);
    p = fmaf(p, q, 1.f / 3.f);
    const float ts = fmaf(a * q, p, a);
    const float tl = 0.34657359027997264f * __builtin_amdgcn_logf((1.f + a) * __builtin_amdgcn_rcpf(1.f - a));
    return copysignf(a < 0.25f ? ts : tl, z);
}

// A raw-accumulator bound below which a logit's key is certainly smaller than
// the key `okey`: a logit that rounds to the key or above lies above the bf16
// value one step below it, which is mapped back through the cap and the scale
// (products with the reciprocals 1 / c and 1 / s) with a relative margin of
// 2^-12 at each step, far above the few-ulp error of those products, of the
// atanh above and of the kernel's tanh.  Near saturation of the cap
// (|x| > 0.9 c) no bound is used.
__device__ __forceinline__ float acc_lower_bound(uint32_t okey, float inv_s, float c, float inv_c) {
    if (okey < 0x0081u) return -INFINITY;  // the step below is -inf: nothing to bound
    const float xlo = bf16_bits_to_f32(unorder_key(okey - 1));
    if (!(xlo > -INFINITY)) return -INFINITY;
    float y = xlo;
    if (c > 0.f) {
        const float z = xlo * inv_c;
        if (!(fabsf(z) < 0.9f)) return -INFINITY;
        y = c * bound_atanh(z);
    }
    y -= fabsf(y) * 0x1p-12f + 1e-30f;
    float a = y * inv_s;
    a -= fabsf(a) * 0x1p-12f + 1e-30f;
    return a == a ? a : -INFINITY;  // (an overflow to +inf leaves inf - inf)
}

// Insert p into the descending list L (the smallest falls off).  A no-op when
// p <= L[n-1].  With L[j-1] >= L[j], the new L[j] = max(L[j], min(L[j-1], p))
// is the median of the three: one v_med3_u32 per entry.
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t d;
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
template <int N>
__device__ __forceinline__ void list_insert(uint32_t (&L)[N], uint32_t p) {
#pragma unroll
    for (int j = N - 1; j > 0; --j) L[j] = med3_u32(L[j], L[j - 1], p);
    L[0] = max(L[0], p);
}

// Position of the lowest set bit, ~0u for zero (v_ffbl_b32 as such: written
// as a select around a count of trailing zeros it is not always folded).
__device__ __forceinline__ uint32_t ffbl(uint32_t x) {
    uint32_t r;
    asm("v_ffbl_b32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// m &= m - 1 over MW 32-bit words read as one number, word 0 least
// significant: clears its lowest set bit (a subtract-with-borrow chain).
template <int MW>
__device__ __forceinline__ void clear_lowest_bit(uint32_t (&m)[MW]) {
    if constexpr (MW == 4) {
        unsigned __int128 x = ((unsigned __int128)(((uint64_t)m[3] << 32) | m[2]) << 64) | (((uint64_t)m[1] << 32) | m[0]);
        x &= x - 1;
        m[0] = (uint32_t)x;
        m[1] = (uint32_t)(x >> 32);
        m[2] = (uint32_t)(x >> 64);
        m[3] = (uint32_t)(x >> 96);
    } else if constexpr (MW == 2) {
        uint64_t x = ((uint64_t)m[1] << 32) | m[0];
        x &= x - 1;
        m[0] = (uint32_t)x;
        m[1] = (uint32_t)(x >> 32);
    } else {
        static_assert(MW == 1, "mask of 1, 2 or 4 words");
        m[0] &= m[0] - 1u;
    }
}

// Bitonic sort of N (a power of two) values in registers, descending if DESC.
template <int N, bool DESC>
__device__ __forceinline__ void bitonic_sort(float (&a)[N]) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    // blocks of `size` alternate direction; the last stage (size N) is one block
                    const bool asc = ((i & size) == 0) != DESC;
                    const float lo = fminf(a[i], a[j]), hi = fmaxf(a[i], a[j]);
                    a[i] = asc ? lo : hi;
                    a[j] = asc ? hi : lo;
                }
            }
}

template <int BM, int BN, int KCAP, bool TAIL, bool WNT>
__global__ __launch_bounds__(LM_THREADS, 1) void lm_topk_tiles(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ W, int T, int V, int Hd,
    int nM, int nN, int G, int xmx, float s, float c, float inv_c,
    uint64_t* __restrict__ part, const uint16_t* __restrict__ Wp, int R, float* __restrict__ hp) {
    constexpr int WN = BN / 2;               // columns per wave
    constexpr int NB = WN / 32;              // 32-column MFMA blocks per wave
    constexpr int MB = BM / 64;              // 32-row MFMA blocks per wave (BM / 2 rows)
    constexpr int NIA = BM / 8 / 4;          // LDS-DMA instructions per wave per slice (A)
    constexpr int NIB = BN / 8 / 4;          // (B)
    constexpr int UNIT = (BM > BN ? BM : BN) * LM_BK;  // elements of one operand's K slice
    constexpr int NSLOT = 5;                 // LDS ring of operand slices (2.5 K slices)
    constexpr int QCOLS = WN;                // epilogue pass width: one wave's columns
    constexpr int MW = QCOLS / 32;           // 32-bit words of a pass's candidate mask
    constexpr int SP = QCOLS + 4;            // row pitch (floats) of the epilogue staging
    constexpr int SMEM = (NSLOT * UNIT > BM * SP * 2) ? NSLOT * UNIT : BM * SP * 2;
    static_assert(BM == 256 || BM == 64, "row tile");
    // WNT: the weight's LDS-DMA loads carry the nontemporal hint.  It is set when
    // one row tile covers every row, so that each W tile is read by one
    // workgroup only; the hint then lets the weight stream run closer to the HBM
    // peak.  With several row tiles the workgroups of an XCD share W tiles
    // through L2, and the hint would cost those hits.
    constexpr int WAUX = WNT ? 2 : 0;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM];
    float* stage = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave >> 1, wn = wave & 1;

    // Workgroup ids go to the 8 XCDs round-robin.  With xmx > 0 the (group,
    // row-tile) grid is cut into 8 blocks of (per / xmx) groups x xmx row tiles,
    // one per XCD, so each XCD's L2 serves W tiles to xmx row tiles and H slices
    // to per / xmx groups.
    int m_tile, g;
    if (xmx > 0) {
        const int per = gridDim.x >> 3;
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        const int gx = per / xmx, bms = nM / xmx;
        g = (x / bms) * gx + j / xmx;
        m_tile = (x % bms) * xmx + j % xmx;
    } else {
        m_tile = blockIdx.x % nM;
        g = blockIdx.x / nM;
    }
    const int n_begin = (int)((int64_t)g * nN / G);
    const int n_end = (int)((int64_t)(g + 1) * nN / G);
    const int m0 = m_tile * BM;
    const int gcol0 = n_begin * BN;
    const int my_row = m0 + tid;
    // thread t owns row t of the tile (rows past BM: none); evaluated where used
    auto row_ok = [&]() { return (BM >= LM_THREADS || tid < BM) && my_row < T; };

    uint32_t list[KCAP];
#pragma unroll
    for (int j = 0; j < KCAP; ++j) list[j] = 0u;
    float thr = -INFINITY;
    const float inv_s = 1.0f / s;  // (s > 0: checked on the host)

    const int nK = (Hd + LM_BK - 1) / LM_BK;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(H + (int64_t)m0 * Hd), (short)0, min(BM, T - m0) * Hd * 2, 0x00020000);

    // Per-lane LDS element offsets of the 32 x 16 fragments: row = lane % 32 of
    // each 32-row block, 16-byte chunk (2 * k16 + lane / 32) ^ swz8(row).
    const int fr = lane & 31;
    const int a_row0 = (wm * (BM / 2) + fr) * LM_BK;
    const int b_row0 = (wn * WN + fr) * LM_BK;

    // The rank projection, when hp is given: W_proj's R rows are appended to the
    // vocabulary's columns, and the epilogue stores the staged raw fp32 sums of
    // those columns to hp instead of selecting from them.
    //  - merged: the last vocabulary tile has room for them (V % BN > 0 is a
    //    multiple of a wave's BN / 4 DMA rows, R <= BN - V % BN, R % 4 == 0);
    //    there the waves past the vocabulary rows load W_proj's rows instead, so
    //    the projection costs no MFMA work (those columns were zeros anyway);
    //  - else group 0 (which has the fewest tiles) runs ceil(R / BN) extra
    //    tiles of W_proj after its own.  (Run first, they would put group 0 a
    //    tile behind the groups that share its H slices in L2 for the whole
    //    kernel: +17% fetched bytes.)
    const int vtail = V % BN;
    const bool merged = hp != nullptr && vtail > 0 && vtail % (BN / 4) == 0 && R <= BN - vtail && R % 4 == 0;
    const int nproj = (hp != nullptr && !merged && g == 0) ? (R + BN - 1) / BN : 0;
    for (int nt = n_begin; nt < n_end + nproj; ++nt) {
        const bool proj = nt >= n_end;
        const bool mixed = merged && nt == nN - 1;
        const int n0 = (proj ? nt - n_end : nt) * BN;
        // B operand of this wave: vocabulary rows, or (projection tiles, and the
        // waves past the vocabulary rows of the mixed tile) W_proj's rows, with
        // the rsrc based so that tile row vtail + i is W_proj row i
        const bool wproj = proj || (mixed && wave_s * (BN / 4) >= vtail);
        const uint64_t bbase = proj ? (uint64_t)(uintptr_t)(Wp + (int64_t)n0 * Hd)
                               : mixed && wproj ? (uint64_t)(uintptr_t)Wp - (uint64_t)vtail * (uint64_t)Hd * 2u
                                                : (uint64_t)(uintptr_t)(W + (int64_t)n0 * Hd);
        const int brows = proj ? min(BN, R - n0) : mixed && wproj ? vtail + R : min(BN, V - n0);
        const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(uintptr_t)bbase, (short)0, brows * Hd * 2, 0x00020000);
        // LDS-DMA lane offsets, recomputed per tile (from opaque copies of Hd
        // and the lane, so that they are not hoisted): kept live across the
        // epilogue they get spilled, and each reload waits for every load in
        // flight.
        int hd_t = Hd, lane_t = lane;
        asm volatile("" : "+s"(hd_t), "+v"(lane_t));
        int voffA[NIA], voffB[NIB], lcA, lcB;
        dma_offsets<NIA>(voffA, lcA, wave_s, lane_t, hd_t);
        dma_offsets<NIB>(voffB, lcB, wave_s, lane_t, hd_t);
        f32x16 acc[MB][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        // Column offset of K slice sl.  With one row tile (WNT) the workgroups
        // start at different slices (slice sl is read as (sl + krot) mod nK):
        // in lockstep every workgroup would read its W rows, 8 KB apart, at
        // one column offset, and such requests crowd a few memory channels.
        // (Slices past nK stay past it: the prologue's spare slice reads zeros.)
        const int krot = WNT ? (int)((blockIdx.x >> 3) % (unsigned)nK) : 0;
        auto kof = [&](int sl) { return (sl < nK ? (sl + krot >= nK ? sl + krot - nK : sl + krot) : sl) * LM_BK; };
        // Fragment q (in the order the MFMAs below consume them: A0, B0..B{NB-1},
        // A1..A{MB-1}) of one 16-wide K step (k16 = 0..3) of the slice whose A
        // and B halves sit in ring slots sa and sb.
        constexpr int NFR = MB + NB;
        auto read_frag = [&](int sa, int sb, int k16, int q, bf16x8 (&fa)[MB], bf16x8 (&fb)[NB]) {
            const int chs = ((2 * k16 + (lane >> 5)) ^ swz8(fr)) << 3;  // swz8(row) == swz8(row % 32)
            if (q >= 1 && q <= NB)
                fb[q - 1] = as_bf16x8(*reinterpret_cast<const u32x4*>(smem + sb * UNIT + b_row0 + (q - 1) * 32 * LM_BK + chs));
            else {
                const int i = q == 0 ? 0 : q - NB;
                fa[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(smem + sa * UNIT + a_row0 + i * 32 * LM_BK + chs));
            }
        };
        auto mfmas = [&](const bf16x8 (&fa)[MB], const bf16x8 (&fb)[NB]) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        };
        // One K step: its MFMAs, with the next step's fragment reads and (for
        // DMA = 1 / 2) the LDS-DMA loads of an A / B half written between them
        // in program order.  The order matters: the compiler cannot tell the
        // DMA's LDS writes from the reads apart, so it keeps them as written,
        // and the group barriers then spread both between the MFMAs (reads
        // first, one per MFMA).
        constexpr int MPK = MB * NB;  // MFMAs per K step
        // fragment reads and DMA loads per K step: every one of each kind
        constexpr int NQ = NFR > NIA ? (NFR > NIB ? NFR : NIB) : (NIA > NIB ? NIA : NIB);
        auto kstep = [&](const bf16x8 (&fa)[MB], const bf16x8 (&fb)[NB], int ra, int rb, int rk16,
                         bf16x8 (&na)[MB], bf16x8 (&nb)[NB], int dma, int dkt, int dslot) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (q < NFR && rk16 >= 0) read_frag(ra, rb, rk16, q, na, nb);
                if (dma == 1 && q < NIA)
                    dma_one<NIA, TAIL>(rsA, smem + dslot * UNIT, voffA, lcA, wave_s, hd_t, kof(dkt), q);
                if (dma == 2 && q < NIB)
                    dma_one<NIB, TAIL, WAUX>(rsB, smem + dslot * UNIT, voffB, lcB, wave_s, hd_t, kof(dkt), q);
            }
            mfmas(fa, fb);
#pragma unroll
            for (int q = 0; q < (MPK > NQ ? MPK : NQ); ++q) {
                if (q < MPK) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < NFR && rk16 >= 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if ((dma == 1 && q < NIA) || (dma == 2 && q < NIB)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        };

        // Software pipeline over 64-wide K slices, one barrier per slice, with
        // the operand halves of the slices in a ring of five LDS slots: slice k
        // keeps its B half in slot 2k mod 5 and its A half in slot 2k+1 mod 5.
        // The barrier at the end of slice k frees its two slots: the A half of
        // slice k+2 is loaded into one right after it, the B half of slice k+3
        // into the other during the first K step of slice k+1.  So a B half
        // (the weight, streamed from HBM) is in flight for about two slices and
        // an A half (the hidden states, L2/MALL resident) for one.  The wait
        // before each barrier lets exactly the newest B half stay in flight.
        bf16x8 fa0[MB], fb0[NB], fa1[MB], fb1[NB];
        dma_slice<NIB, TAIL, WAUX>(rsB, smem + 0 * UNIT, voffB, lcB, wave_s, hd_t, kof(0));
        dma_slice<NIA, TAIL>(rsA, smem + 1 * UNIT, voffA, lcA, wave_s, hd_t, kof(0));
        dma_slice<NIB, TAIL, WAUX>(rsB, smem + 2 * UNIT, voffB, lcB, wave_s, hd_t, kof(1));  // past K: zeros, unused
        dma_slice<NIA, TAIL>(rsA, smem + 3 * UNIT, voffA, lcA, wave_s, hd_t, kof(1));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NIB + NIA));  // slice 0 landed
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        int sb = 0, sa = 1;  // ring slots of the current slice
#pragma unroll
        for (int q = 0; q < NFR; ++q) read_frag(sa, sb, 0, q, fa0, fb0);
        for (int kt = 0; kt + 1 < nK; ++kt) {
            const int sn = sb == 0 ? NSLOT - 1 : sb - 1;  // slot of the B half of slice kt+2
            kstep(fa0, fb0, sa, sb, 1, fa1, fb1, 2, kt + 2, sn);
            kstep(fa1, fb1, sa, sb, 2, fa0, fb0, 0, 0, 0);
            kstep(fa0, fb0, sa, sb, 3, fa1, fb1, 0, 0, 0);
            // slice kt+1 landed (only the B half of slice kt+2 may still be in flight)
            __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(NIB));
            __builtin_amdgcn_s_barrier();
            compiler_fence();
            const int sa2 = sb;  // the A half of slice kt+2 goes into the B slot of slice kt
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


        // Epilogue, two passes: the columns of wave wn = pass are staged
        // row-major with a row pitch of QCOLS + 4 floats (the 32-lane halves of
        // a 4-byte write cover 32 consecutive columns of one row; 16-byte reads
        // of 8 consecutive rows hit distinct banks), then thread t scans row t.
        // In the 32x32 MFMA layout lane l holds column l % 32 and rows
        // 8b + 4(l / 32) + e, e = 0..3.
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wn == pass) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int col = j * 32 + fr;
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            // 4-byte writes straight from the accumulator AGPRs: element
                            // access from C++ makes the allocator move the accumulators
                            // to VGPRs and spill.  (lgkmcnt is waited for explicitly
                            // before the barrier below.)
                            const uint32_t dst = lds_offset(
                                stage + (wm * (BM / 2) + i * 32 + 8 * b + 4 * (lane >> 5)) * SP + col);
                            asm volatile("ds_write_b32 %0, %1" ::"v"(dst), "a"(acc[i][j][4 * b]) : "memory");
                            asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(dst), "a"(acc[i][j][4 * b + 1]),
                                         "i"(SP * 4) : "memory");
                            asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(dst), "a"(acc[i][j][4 * b + 2]),
                                         "i"(SP * 8) : "memory");
                            asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(dst), "a"(acc[i][j][4 * b + 3]),
                                         "i"(SP * 12) : "memory");
                        }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staging writes done
            __builtin_amdgcn_s_barrier();
            compiler_fence();
            if (row_ok() && proj) {
                // a projection tile: the row's raw fp32 sums (no scale, cap or
                // selection) go to hp; columns past R were read as zero
                const int cbase = n0 + pass * QCOLS;
                const int ncols = min(QCOLS, R - cbase);
                const float* rowp = stage + tid * SP;
                // (the address from an opaque copy of the row: hoisted out of the
                // tile loop it would be spilled, and its reload waits for every
                // load in flight)
                int row_t = my_row;
                asm volatile("" : "+v"(row_t));
                float* dstp = hp + (int64_t)row_t * R + cbase;
                if ((R & 3) == 0) {
                    for (int cc = 0; cc < ncols; cc += 4)
                        *reinterpret_cast<f32x4*>(dstp + cc) = *reinterpret_cast<const f32x4*>(rowp + cc);
                } else {
                    for (int cc = 0; cc < ncols; ++cc) dstp[cc] = rowp[cc];
                }
            } else if (row_ok()) {
                const int cbase = n0 + pass * QCOLS;
                const int ncols = min(QCOLS, V - cbase);
                const float* rowp = stage + tid * SP;
                auto at = [&](int cc) { return rowp[cc]; };
                // 0) a row's first pass (empty list): start from a value that at
                //    least KCAP of the pass's columns reach, so a key below it is
                //    out.  With room for 2 KCAP groups of 4 or more columns it is
                //    the KCAP-th largest of their maxima: one group set sorted
                //    descending, the other ascending, the pairwise maxima are the
                //    top KCAP of the 2 KCAP (a bitonic split), and their minimum
                //    is the KCAP-th largest.  Else it is the smallest of KCAP
                //    group maxima.  (The first takes about a third of the
                //    candidates of the second on random rows.)
                constexpr int GS = QCOLS / KCAP;        // columns per group
                constexpr int GS2 = QCOLS / (2 * KCAP);  // (with 2 KCAP groups)
                if (GS >= 4 && thr == -INFINITY && ncols == QCOLS) {
                    float mn = INFINITY;
                    if constexpr (GS2 >= 4) {
                        float ga[KCAP], gb[KCAP];
#pragma unroll
                        for (int gq = 0; gq < 2 * KCAP; ++gq) {
                            float mx = -INFINITY;
#pragma unroll
                            for (int q = 0; q < GS2 / 4; ++q) {
                                const f32x4 x = *reinterpret_cast<const f32x4*>(rowp + gq * GS2 + 4 * q);
                                mx = fmaxf(mx, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
                            }
                            if (gq < KCAP) ga[gq] = mx;
                            else gb[gq - KCAP] = mx;
                        }
                        bitonic_sort<KCAP, true>(ga);
                        bitonic_sort<KCAP, false>(gb);
#pragma unroll
                        for (int i = 0; i < KCAP; ++i) mn = fminf(mn, fmaxf(ga[i], gb[i]));
                    } else {
#pragma unroll
                        for (int gq = 0; gq < KCAP; ++gq) {
                            float mx = -INFINITY;
#pragma unroll
                            for (int q = 0; q < GS / 4; ++q) {
                                const f32x4 x = *reinterpret_cast<const f32x4*>(rowp + gq * GS + 4 * q);
                                mx = fmaxf(mx, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
                            }
                            mn = fminf(mn, mx);
                        }
                    }
                    if (mn > -INFINITY && mn < INFINITY)
                        thr = acc_lower_bound(order_key(logit_key_bits(mn, s, c, inv_c)), inv_s, c, inv_c);
                }
                // 1) mask of this row's columns whose raw accumulator reaches the
                //    threshold (16-byte reads, no divergence)
                // Bit 31 - j of word w is column 32w + j: each compare's result is
                // shifted in through the carry (v_cmp + v_addc, two VALU per
                // column), so the word is built most significant bit first.
                uint32_t m[MW];
#pragma unroll
                for (int w = 0; w < MW; ++w) {
                    f32x4 v4[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) v4[q] = *reinterpret_cast<const f32x4*>(rowp + 32 * w + 4 * q);
                    uint32_t mw = 0u;
#pragma unroll
                    for (int q = 0; q < 8; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            asm volatile("v_cmp_ge_f32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
                                         : "+v"(mw) : "v"(v4[q][e]), "v"(thr) : "vcc");
                    // columns past V (the last tile of the vocabulary) never count
                    const int valid = min(max(ncols - 32 * w, 0), 32);
                    if (valid < 32) mw &= valid == 0 ? 0u : ~((1u << (32 - valid)) - 1u);
                    m[w] = mw;
                }
                // 2) candidates, one per lane per round, the LDS read of the next
                //    one issued ahead; the threshold is raised once per pass,
                //    after the rounds.  The list is kept under a strict total
                //    order, so the order of the inserts does not change it.
                // pop: the lowest set bit of the mask read as one MW-word number
                // (word 0 least significant), found as the smallest of the
                // words' lowest set bits offset by 32 w (a zero word gives ~0u,
                // which the OR keeps), and cleared by m &= m - 1 over all words
                // (a borrow chain, no branch).  Bit b of word w is column
                // 32 w + 31 - b, i.e. position ^ 31; none left gives -32.
                auto pop = [&]() {
                    uint32_t pos = ~0u;
#pragma unroll
                    for (int w = 0; w < MW; ++w) pos = min(pos, ffbl(m[w]) | (uint32_t)(32 * w));
                    clear_lowest_bit<MW>(m);
                    return (int)(pos ^ 31u);
                };
                bool changed = false;
                // (the threshold does not move inside a pass, so every masked
                // candidate is evaluated; the insert is a no-op for a key below
                // the list, and the round body has no branch.)  Up to 16
                // entries the loop is compiled once per cap setting, which is
                // uniform; with longer lists that costs spilled registers, and
                // the cap stays a uniform branch inside the key function.
                auto rounds = [&](auto cap) {
                    int cc = pop();
                    float v = at(cc < 0 ? 0 : cc);
                    while (cc >= 0) {
                        const int cn = pop();
                        const float vn = at(cn < 0 ? 0 : cn);
                        const uint32_t kb = logit_key_bits_as<decltype(cap)::value>(v, s, c, inv_c);
                        const uint32_t p = (order_key(kb) << 16) | (0xffffu - (uint32_t)(cbase + cc - gcol0));
                        changed |= p > list[KCAP - 1];
                        list_insert(list, p);
                        cc = cn;
                        v = vn;
                    }
                };
                if constexpr (KCAP > 16) {
                    int cc = pop();
                    float v = at(cc < 0 ? 0 : cc);
                    while (cc >= 0) {
                        const int cn = pop();
                        const float vn = at(cn < 0 ? 0 : cn);
                        const uint32_t kb = logit_key_bits(v, s, c, inv_c);
                        const uint32_t p = (order_key(kb) << 16) | (0xffffu - (uint32_t)(cbase + cc - gcol0));
                        changed |= p > list[KCAP - 1];
                        list_insert(list, p);
                        cc = cn;
                        v = vn;
                    }
                } else if (c > 0.f) {
                    rounds(std::integral_constant<bool, true>{});
                } else {
                    rounds(std::integral_constant<bool, false>{});
                }
                if (changed && list[KCAP - 1] != 0u) thr = acc_lower_bound(list[KCAP - 1] >> 16, inv_s, c, inv_c);
            }
            if (row_ok() && mixed) {
                // the mixed tile's projection columns V .. V + R - 1 (R % 4 == 0,
                // V % 4 == 0: 16-byte aligned)
                const int cbase = n0 + pass * QCOLS;
                const int c0 = max(0, V - cbase), c1 = min(QCOLS, V + R - cbase);
                const float* rowp = stage + tid * SP;
                int row_t = my_row;
                asm volatile("" : "+v"(row_t));
                float* dstp = hp + (int64_t)row_t * R + (cbase - V);
                for (int cc = c0; cc < c1; cc += 4)
                    *reinterpret_cast<f32x4*>(dstp + cc) = *reinterpret_cast<const f32x4*>(rowp + cc);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): row reads done before the next pass writes
            __builtin_amdgcn_s_barrier();
            compiler_fence();
        }
    }

    if (row_ok()) {
        uint64_t* dst = part + ((int64_t)my_row * G + g) * KCAP;
#pragma unroll
        for (int j = 0; j < KCAP; ++j) {
            const uint32_t p = list[j];
            uint64_t e = 0;
            if (p != 0u) {
                const uint32_t id = (uint32_t)gcol0 + (0xffffu - (p & 0xffffu));
                e = ((uint64_t)(p >> 16) << 32) | (uint64_t)(~id);
            }
            dst[j] = e;
        }
    }
}

// Merge for G <= 16 groups: 16 lanes per row (four rows per wave), lane g
// holding group g's sorted list in registers.  Each round takes the largest
// head over the 16 lanes (DPP row rotations, no LDS round trip) and the lane
// that owns it (entries are distinct; 0 = empty) drops it.
template <int SH>
__device__ __forceinline__ uint64_t max_ror(uint64_t x) {
    constexpr int ctrl = 0x120 + SH;  // DPP row_ror:SH (rotate within each 16-lane row)
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, ctrl, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), ctrl, 0xF, 0xF, false);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    return y > x ? y : x;
}
__device__ __forceinline__ uint64_t row16_max(uint64_t x) {
    return max_ror<8>(max_ror<4>(max_ror<2>(max_ror<1>(x))));
}

template <int KCAP>
__global__ __launch_bounds__(256) void lm_topk_merge16(const uint64_t* __restrict__ part, int T, int G, int k,
                                                       int32_t* __restrict__ ids, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const int g = lane & 15;
    uint64_t L[KCAP];
    if (row < T && g < G) {
        const u32x4* src = reinterpret_cast<const u32x4*>(part + ((int64_t)row * G + g) * KCAP);
#pragma unroll
        for (int j = 0; j < KCAP / 2; ++j) {
            const u32x4 v = src[j];
            L[2 * j] = ((uint64_t)v[1] << 32) | v[0];
            L[2 * j + 1] = ((uint64_t)v[3] << 32) | v[2];
        }
    } else {
#pragma unroll
        for (int j = 0; j < KCAP; ++j) L[j] = 0;
    }
    for (int r = 0; r < k; ++r) {
        const uint64_t best = row16_max(L[0]);
        if (best != 0 && L[0] == best) {
#pragma unroll
            for (int j = 0; j < KCAP - 1; ++j) L[j] = L[j + 1];
            L[KCAP - 1] = 0;
        }
        if (g == 0 && row < T) {
            const uint32_t okey = (uint32_t)(best >> 32);
            ids[(int64_t)row * k + r] = (int32_t)(~(uint32_t)best);
            logits[(int64_t)row * k + r] = best ? bf16_bits_to_f32(unorder_key(okey)) : -INFINITY;
        }
    }
}

// One level of the merge for G > 16 groups: the same 16-lane rounds over
// blocks of 16 groups, a "virtual row" per (row, block), writing the block's
// KCAP best entries as one partial list: [T, G, KCAP] -> [T, ceil(G/16), KCAP].
// Any strict total order keeps the global top k inside the union of the
// blocks' top-KCAP lists, so levels compose until G <= 16.
template <int KCAP>
__global__ __launch_bounds__(256) void lm_topk_merge16_level(const uint64_t* __restrict__ part, int T, int G,
                                                             int G2, uint64_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t vrow = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const int64_t row = vrow / G2;
    const int blk = (int)(vrow - row * G2);
    const int g = blk * 16 + (lane & 15);
    uint64_t L[KCAP];
    if (row < T && g < G) {
        const u32x4* src = reinterpret_cast<const u32x4*>(part + (row * G + g) * KCAP);
#pragma unroll
        for (int j = 0; j < KCAP / 2; ++j) {
            const u32x4 v = src[j];
            L[2 * j] = ((uint64_t)v[1] << 32) | v[0];
            L[2 * j + 1] = ((uint64_t)v[3] << 32) | v[2];
        }
    } else {
#pragma unroll
        for (int j = 0; j < KCAP; ++j) L[j] = 0;
    }
    for (int r = 0; r < KCAP; ++r) {
        const uint64_t best = row16_max(L[0]);
        if (best != 0 && L[0] == best) {
#pragma unroll
            for (int j = 0; j < KCAP - 1; ++j) L[j] = L[j + 1];
            L[KCAP - 1] = 0;
        }
        if ((lane & 15) == 0 && row < T) out[(row * G2 + blk) * KCAP + r] = best;
    }
}

// The whole merge for 16 < G <= 256 groups and k <= 16 in one launch, one
// workgroup per row, by ranking instead of rounds:
//  1. The row's top k lies in the lists of the k largest heads (a list whose
//     head is below the k-th largest head has every entry below k distinct
//     entries).  Thread t loads list t whole and ranks its head against all
//     heads (ties of the 16-bit key go to the lower list index, which holds
//     the lower token ids: groups own increasing column ranges); the k best
//     lists go to LDS in head order, so no second load from memory is needed.
//  2. Thread 16 s + j holds entry j of kept list s.  Its rank in the union of
//     the kept lists is the number of their entries above it (all distinct):
//     in each sorted list that count comes from a binary search (in its own
//     list it is j), and a rank below k is its output slot.
template <int KCAP>
__global__ __launch_bounds__(256) void lm_topk_merge_rank(const uint64_t* __restrict__ part, int T, int G, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ logits) {
    static_assert(KCAP <= 16, "16 kept lists of at most 16 entries");
    __shared__ __attribute__((aligned(16))) uint32_t heads[256];
    __shared__ __attribute__((aligned(16))) uint64_t ent[16][16];
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    uint64_t L[KCAP];
    if (tid < G) {
        const u32x4* src = reinterpret_cast<const u32x4*>(part + ((int64_t)row * G + tid) * KCAP);
#pragma unroll
        for (int j = 0; j < KCAP / 2; ++j) {
            const u32x4 v = src[j];
            L[2 * j] = ((uint64_t)v[1] << 32) | v[0];
            L[2 * j + 1] = ((uint64_t)v[3] << 32) | v[2];
        }
    } else {
#pragma unroll
        for (int j = 0; j < KCAP; ++j) L[j] = 0;
    }
    // (key + 1, list index reversed): nonzero for a non-empty list
    const uint32_t hk = L[0] ? ((uint32_t)((L[0] >> 32) + 1) << 8) | (uint32_t)(255 - tid) : 0u;
    heads[tid] = hk;
    ent[tid >> 4][tid & 15] = 0;  // slots of lists not kept (and past KCAP) stay empty
    __syncthreads();
    int rank = 0;
#pragma unroll 8
    for (int u = 0; u < 64; ++u) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(heads + 4 * u);
        rank += (q[0] > hk) + (q[1] > hk) + (q[2] > hk) + (q[3] > hk);
    }
    if (hk && rank < k) {
        // entries at list position k or later have k entries above them
#pragma unroll
        for (int j = 0; j < KCAP; ++j) ent[rank][j] = j < k ? L[j] : 0;
    }
    __syncthreads();
    const int s = tid >> 4, j = tid & 15;
    const uint64_t e = ent[s][j];
    const int nz = __syncthreads_count(e != 0);
    // count of entries above e in each descending list of 16: steps of 8, 4, 2,
    // 1 leave it exact except that 15 may still be 16
    int r = 0;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
        const uint64_t* a = ent[s2];
        int c = a[7] > e ? 8 : 0;
        c += a[c + 3] > e ? 4 : 0;
        c += a[c + 1] > e ? 2 : 0;
        c += a[c] > e ? 1 : 0;
        c += (c == 15 && a[15] > e) ? 1 : 0;
        r += c;
    }
    if (e != 0 && r < k) {
        ids[(int64_t)row * k + r] = (int32_t)(~(uint32_t)e);
        logits[(int64_t)row * k + r] = bf16_bits_to_f32(unorder_key((uint32_t)(e >> 32)));
    }
    if (tid >= nz && tid < k) {  // fewer than k entries in all: the rest is empty
        ids[(int64_t)row * k + tid] = -1;
        logits[(int64_t)row * k + tid] = -INFINITY;
    }
}

// The whole merge for 16 < G <= 256 groups in one launch: one workgroup per
// row.  Its 16 lane groups (16 lanes each, one DPP row) first take the k best
// of 16 lists each, as lm_topk_merge16_level does, into LDS; then the first
// lane group merges those (at most 16) lists as lm_topk_merge16 does.  Only k
// entries per block are needed: the union of the blocks' top-k lists holds the
// row's top k.
template <int KCAP>
__global__ __launch_bounds__(256) void lm_topk_merge256(const uint64_t* __restrict__ part, int T, int G, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ logits) {
    __shared__ uint64_t blk[16][KCAP];
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int b = tid >> 4, g = tid & 15;
    const int gi = b * 16 + g;
    uint64_t L[KCAP];
    if (gi < G) {
        const u32x4* src = reinterpret_cast<const u32x4*>(part + ((int64_t)row * G + gi) * KCAP);
#pragma unroll
        for (int j = 0; j < KCAP / 2; ++j) {
            const u32x4 v = src[j];
            L[2 * j] = ((uint64_t)v[1] << 32) | v[0];
            L[2 * j + 1] = ((uint64_t)v[3] << 32) | v[2];
        }
    } else {
#pragma unroll
        for (int j = 0; j < KCAP; ++j) L[j] = 0;
    }
    for (int r = 0; r < k; ++r) {
        const uint64_t best = row16_max(L[0]);
        if (best != 0 && L[0] == best) {
#pragma unroll
            for (int j = 0; j < KCAP - 1; ++j) L[j] = L[j + 1];
            L[KCAP - 1] = 0;
        }
        if (g == 0) blk[b][r] = best;
    }
    __syncthreads();
    if (tid >= 16) return;
    // lane g of the first lane group: block g's list (k entries, zeros past it)
#pragma unroll
    for (int j = 0; j < KCAP; ++j) L[j] = j < k ? blk[g][j] : 0;
    for (int r = 0; r < k; ++r) {
        const uint64_t best = row16_max(L[0]);
        if (best != 0 && L[0] == best) {
#pragma unroll
            for (int j = 0; j < KCAP - 1; ++j) L[j] = L[j + 1];
            L[KCAP - 1] = 0;
        }
        if (g == 0) {
            const uint32_t okey = (uint32_t)(best >> 32);
            ids[(int64_t)row * k + r] = (int32_t)(~(uint32_t)best);
            logits[(int64_t)row * k + r] = best ? bf16_bits_to_f32(unorder_key(okey)) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// lm_topk_stream: the LM head for at most 32 rows, where the contraction is a
// stream over W with little arithmetic per byte (16 rows: 16 flop per W byte).
//
// Workgroup g (512 threads, one per CU) owns a contiguous run of 16-row
// vocabulary tiles, and its 8 waves split the hidden dimension: wave w owns
// columns [w KW, (w + 1) KW), KW = Hd / 8 = 32 NL.  Per tile a wave reads its
// 16 x KW slice of W as NL nontemporal loads of 1 KB of row-contiguous bytes
// (rows read in whole runs: with an MFMA operand layout each load instruction
// would touch 16 rows at one offset, and that pattern streams ~13% slower),
// writes it to its own LDS region (16-byte chunks XOR-swizzled by row) and
// reads it back as v_mfma_f32_16x16x32_bf16 A fragments, vocabulary rows as M;
// its hidden-row fragments (B, hidden rows as N; NBH blocks of 16 rows) sit in
// registers for the whole stream.  The next tile's loads are issued as soon as
// the slice is in LDS.  The 8 waves' 16 x 16 partial sums (per hidden block)
// meet in LDS (one barrier per tile) and waves 0 .. 4 NBH - 1 add them in wave
// order: thread (w, lane) takes vocabulary row 4 (lane / 16) + w % 4 of hidden
// row 16 (w / 4) + lane % 16, keys it (scale, cap, bf16) and keeps its own
// sorted list of the best KCAP keys.  At the end the 16 lists of each hidden
// row are merged in LDS into the group's partial list, the tile kernel's
// format, and the merge kernels finish as for the tile kernel.
// ---------------------------------------------------------------------------
constexpr int ST_THREADS = 512;
constexpr int ST_WAVES = ST_THREADS / 64;
constexpr int ST_MAXHD = 4096;  // NL <= 16: 64 VGPRs of hidden-row fragments per block, 16 KB of LDS per wave

// Swizzle of the 16-byte chunks of a row's slice (CPR chunks): chunk c of row r
// is stored at c ^ st_swz(r), so the 16 rows of a fragment read hit distinct banks.
template <int CPR>
__device__ __forceinline__ int st_swz(int r) { return r & (CPR < 16 ? CPR - 1 : 15); }

template <int KCAP, int NL, int NBH>
__global__ __launch_bounds__(ST_THREADS) void lm_topk_stream(const uint16_t* __restrict__ H,
                                                             const uint16_t* __restrict__ W, int T, int V, int Hd,
                                                             int ntiles, int G, float s, float c, float inv_c,
                                                             uint64_t* __restrict__ part) {
    static_assert(NBH == 1 || NBH == 2, "16 or 32 hidden rows");
    constexpr int KW = 32 * NL;         // hidden columns per wave
    constexpr int RB = 2 * KW;          // bytes of one row's slice (a power of two)
    constexpr int CPR = RB / 16;        // 16-byte chunks per row slice
    constexpr int WT_BYTES = 16 * RB;   // a wave's slice of one tile: NL KB
    constexpr int NE = 4 * NBH;         // partial sums per lane per tile
    constexpr int P_FLOATS = ST_WAVES * NE * 64;  // one tile's partial sums
    constexpr int STREAM_BYTES = ST_WAVES * WT_BYTES + 2 * P_FLOATS * 4;
    constexpr int LIST_BYTES = 16 * NBH * 16 * KCAP * 4;
    constexpr int LDS_BYTES = STREAM_BYTES > LIST_BYTES ? STREAM_BYTES : LIST_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = blockIdx.x;
    const int t0 = (int)((int64_t)grp * ntiles / G), t1 = (int)((int64_t)(grp + 1) * ntiles / G);
    const int v0 = t0 * 16;  // the group's first vocabulary row: ids are v0 + column
    const int j = lane & 15, q = lane >> 4;
    const int k0 = wave * KW;
    uint8_t* wt = lds + wave * WT_BYTES;
    float* P = reinterpret_cast<float*>(lds + ST_WAVES * WT_BYTES);  // [2][wave][e][lane]

    // this wave's hidden-row fragments: lane (j, q) of block b holds row 16 b + j,
    // columns k0 + 32 s + 8 q .. + 8 of K step s (rows >= T are zero)
    u32x4 hf[NBH][NL];
#pragma unroll
    for (int hb = 0; hb < NBH; ++hb)
#pragma unroll
        for (int st = 0; st < NL; ++st)
            hf[hb][st] = 16 * hb + j < T ? ldg16(H + (int64_t)(16 * hb + j) * Hd + k0 + 32 * st + 8 * q)
                                         : u32x4{0u, 0u, 0u, 0u};

    // load i of a tile slice: bytes [1024 i + 16 lane, + 16) of the wave's
    // row-major 16 x RB slice, i.e. row (1024 i + 16 lane) / RB; rows past the
    // vocabulary reload the last row (never keyed)
    auto wptr = [&](int t, int i) {
        const int byte = 1024 * i + 16 * lane;
        const int r = byte / RB, col = (byte % RB) / 2;
        const int v = min(t * 16 + r, V - 1);
        return W + (int64_t)v * Hd + k0 + col;
    };
    auto lds_slot = [&](int i, int ln) {
        const int byte = 1024 * i + 16 * ln;
        const int r = byte / RB, cc = (byte % RB) / 16;
        return wt + r * RB + 16 * (cc ^ st_swz<CPR>(r));
    };

    const int nt = t1 - t0;
    u32x4 buf[NL];
    if (nt > 0) {
#pragma unroll
        for (int i = 0; i < NL; ++i) buf[i] = ldg16_stream(wptr(t0, i));
    }
    uint32_t L[KCAP];
#pragma unroll
    for (int e = 0; e < KCAP; ++e) L[e] = 0u;
    // the keying thread's output: hidden row 16 (wave / 4) + j, vocabulary row
    // 4 q + wave % 4 of each tile (waves 0 .. 4 NBH - 1)
    const bool keyer = wave < 4 * NBH;
    const int krow = 16 * (wave >> 2) + j, kvr = 4 * q + (wave & 3);

    for (int tt = 0; tt < nt; ++tt) {
        const int t = t0 + tt;
        // LDS addresses from an opaque copy of the lane, so that they are
        // recomputed per tile: hoisted out of the loop they hold ~30 registers,
        // and with 32 hidden rows the kernel then spills inside the loop, where
        // each reload waits for the next tile's loads in flight
        int lane_t = lane;
        asm volatile("" : "+v"(lane_t));
        const int jt = lane_t & 15, qt = lane_t >> 4;
        // the tile's slice -> this wave's LDS region, then the next tile's loads
        // into the same registers
#pragma unroll
        for (int i = 0; i < NL; ++i) *reinterpret_cast<u32x4*>(lds_slot(i, lane_t)) = buf[i];
        if (tt + 1 < nt) {
#pragma unroll
            for (int i = 0; i < NL; ++i) buf[i] = ldg16_stream(wptr(t + 1, i));
        }
        f32x4 acc[NBH];
#pragma unroll
        for (int hb = 0; hb < NBH; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NL; ++st) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(wt + jt * RB + 16 * ((4 * st + qt) ^ st_swz<CPR>(jt)));
#pragma unroll
            for (int hb = 0; hb < NBH; ++hb)
                acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(hf[hb][st]), acc[hb], 0, 0, 0);
        }
        // partial sums -> LDS (double-buffered by tile), one barrier, and the
        // keying waves add them in wave order: lane l of block b's MFMA output
        // holds vocabulary rows 4 (l / 16) + e of hidden row 16 b + l % 16
        float* Pb = P + (tt & 1) * P_FLOATS;
#pragma unroll
        for (int hb = 0; hb < NBH; ++hb)
#pragma unroll
            for (int e = 0; e < 4; ++e) Pb[(wave * NE + 4 * hb + e) * 64 + lane_t] = acc[hb][e];
        __syncthreads();
        if (keyer) {
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < ST_WAVES; ++w) x += Pb[(w * NE + wave) * 64 + lane_t];
            const int v = t * 16 + kvr;
            if (krow < T && v < V) {
                const uint32_t p = (order_key(logit_key_bits(x, s, c, inv_c)) << 16) | (0xffffu - (uint32_t)(v - v0));
                if (p > L[KCAP - 1]) list_insert<KCAP>(L, p);
            }
        }
    }

    // the 16 lists of each hidden row -> LDS (over the stream's buffers), then a
    // 16-lane merge per row: wave w < 4 NBH takes rows 4w .. 4w + 3
    __syncthreads();
    uint32_t* lists = reinterpret_cast<uint32_t*>(lds);
    if (keyer) {
        uint32_t* dst = lists + (krow * 16 + kvr) * KCAP;
#pragma unroll
        for (int e = 0; e < KCAP; ++e) dst[e] = L[e];
    }
    __syncthreads();
    if (!keyer) return;
    const int row = wave * 4 + q;
    {
        const uint32_t* src = lists + (row * 16 + j) * KCAP;
#pragma unroll
        for (int e = 0; e < KCAP; ++e) L[e] = src[e];
    }
    if (row >= T) return;
    uint64_t* out = part + ((int64_t)row * G + grp) * KCAP;
    for (int r = 0; r < KCAP; ++r) {
        uint32_t best = L[0];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) best = max(best, (uint32_t)__shfl_xor((int)best, off, 16));
        if (best != 0u && L[0] == best) {  // keys of one group differ in the column bits: one owner
#pragma unroll
            for (int e = 0; e < KCAP - 1; ++e) L[e] = L[e + 1];
            L[KCAP - 1] = 0u;
        }
        if (j == 0) {
            uint64_t e = 0;
            if (best != 0u) {
                const uint32_t id = (uint32_t)v0 + (0xffffu - (best & 0xffffu));
                e = ((uint64_t)(best >> 16) << 32) | (uint64_t)(~id);
            }
            out[r] = e;
        }
    }
}

struct LmPlan {
    int BM, BN, KCAP, nM, nN, G, xmx;
    int64_t nwg;
    size_t ws;
    int stream_nl;  // > 0: lm_topk_stream with this many 1 KB loads per wave per tile (Hd / 256)
    int stream_nbh;  // its 16-row blocks of hidden rows (1 or 2)
};

// allow_stream: the streaming kernel may be used (not with the rank projection
// riding along, which the tile kernel carries).
static bool lm_plan(int64_t T, int64_t V, int64_t Hd, int k, LmPlan& p, bool allow_stream = true) {
    p.KCAP = k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : k <= 32 ? 32 : 64;
    p.stream_nl = 0;
    if (allow_stream && T <= 32 && Hd <= ST_MAXHD && Hd % 256 == 0 && ((Hd / 256) & (Hd / 256 - 1)) == 0 &&
        (T <= 16 || p.KCAP <= 16)) {
        // up to 32 rows: one workgroup per CU streams a run of 16-row vocabulary
        // tiles, its 8 waves splitting the hidden dimension (above 16 rows with
        // KCAP <= 16: the hidden-row fragments of 32 rows and longer lists would
        // not fit the registers together)
        p.stream_nl = (int)(Hd / 256);
        p.stream_nbh = T > 16 ? 2 : 1;
        const int64_t ntiles = (V + 15) / 16;
        int64_t G = ntiles < 256 ? ntiles : 256;
        while (((ntiles + G - 1) / G) * 16 > 65536) ++G;
        p.BM = 16;
        p.BN = 16;
        p.nM = 1;
        p.nN = (int)ntiles;
        p.G = (int)G;
        p.nwg = G;
        p.xmx = 0;
        const size_t lists = (size_t)T * (size_t)p.G * (size_t)p.KCAP * sizeof(uint64_t);
        const size_t level = p.G > 16 ? (size_t)T * (size_t)((p.G + 15) / 16) * (size_t)p.KCAP * sizeof(uint64_t) : 0;
        p.ws = lists + 2 * level;
        return true;
    }
    // Up to 64 rows the contraction is far from dense: 64-row tiles do a quarter
    // of a 256-row tile's MFMA work for the same weight stream, and 128-column
    // tiles spread the vocabulary over more workgroups.
    p.BM = T <= 64 ? 64 : LM_BM;
    p.nM = (int)((T + p.BM - 1) / p.BM);
    const int target = 256;  // one workgroup per CU (the tile kernel fills a CU's LDS)
    auto groups = [&](int BN) {
        const int64_t nN = (V + BN - 1) / BN;
        int64_t G = (target + p.nM - 1) / p.nM;
        if (G > nN) G = nN;
        if (G < 1) G = 1;
        // a group's columns must fit the 16-bit column field of the packed word
        while (((nN + G - 1) / G) * BN > 65536) ++G;
        p.BN = BN;
        p.nN = (int)nN;
        p.G = (int)G;
    };
    groups(256);
    if (p.BM == 64 || (int64_t)p.nM * p.G < target) groups(128);
    p.nwg = (int64_t)p.nM * p.G;
    if (p.nwg > (int64_t)1 << 30) return false;
    // XCD blocks: xmx row tiles x (per / xmx) groups per XCD, xmx the divisor of
    // gcd(nM, per) closest to sqrt(2 * per)
    p.xmx = 0;
    if (p.nwg % 8 == 0) {
        const int per = (int)(p.nwg / 8);
        int best = 0;
        double bestd = 1e30;
        for (int d = 1; d <= per && d <= p.nM; ++d) {
            if (per % d || p.nM % d || p.G % (per / d)) continue;
            const double dist = fabs(log((double)d / sqrt(2.0 * per)));
            if (dist < bestd) { bestd = dist; best = d; }
        }
        if (best > 0 && (p.G / (per / best)) * (p.nM / best) == 8) p.xmx = best;
    }
    // partial lists, plus two ping-pong buffers for the merge levels of G > 16
    const size_t lists = (size_t)T * (size_t)p.G * (size_t)p.KCAP * sizeof(uint64_t);
    const size_t level = p.G > 16 ? (size_t)T * (size_t)((p.G + 15) / 16) * (size_t)p.KCAP * sizeof(uint64_t) : 0;
    p.ws = lists + 2 * level;
    return true;
}

// The rank projection rides along when Wp / hp are given (R rows of Wp, hp
// [T, R] fp32); else Wp = hp = NULL, R = 0.
struct LmProj {
    const uint16_t* Wp;
    int R;
    float* hp;
};

template <int BM, int BN, int KCAP>
static void launch_tiles(const LmPlan& p, const uint16_t* H, const uint16_t* W, int T, int V, int Hd,
                         float s, float c, uint64_t* part, const LmProj& pj, hipStream_t st) {
    const float inv_c = c > 0.f ? 1.0f / c : 0.f;
    if (Hd % LM_BK == 0 && p.nM == 1)
        hipLaunchKernelGGL((lm_topk_tiles<BM, BN, KCAP, false, true>), dim3((unsigned)p.nwg), dim3(LM_THREADS), 0, st,
                           H, W, T, V, Hd, p.nM, p.nN, p.G, p.xmx, s, c, inv_c, part, pj.Wp, pj.R, pj.hp);
    else if (Hd % LM_BK == 0)
        hipLaunchKernelGGL((lm_topk_tiles<BM, BN, KCAP, false, false>), dim3((unsigned)p.nwg), dim3(LM_THREADS), 0,
                           st, H, W, T, V, Hd, p.nM, p.nN, p.G, p.xmx, s, c, inv_c, part, pj.Wp, pj.R, pj.hp);
    else
        hipLaunchKernelGGL((lm_topk_tiles<BM, BN, KCAP, true, false>), dim3((unsigned)p.nwg), dim3(LM_THREADS), 0, st,
                           H, W, T, V, Hd, p.nM, p.nN, p.G, p.xmx, s, c, inv_c, part, pj.Wp, pj.R, pj.hp);
}

template <int KCAP>
static void launch_all(const LmPlan& p, const uint16_t* H, const uint16_t* W, int T, int V, int Hd, int k,
                       float s, float c, uint64_t* part, int32_t* ids, float* logits, const LmProj& pj,
                       hipStream_t st) {
    if (p.stream_nl > 0) {
        const float inv_c = c > 0.f ? 1.0f / c : 0.f;
        const dim3 grid((unsigned)p.nwg), block(ST_THREADS);
        switch (p.stream_nl) {
#define ST_CASE(n)                                                                                             \
    case n:                                                                                                    \
        if (p.stream_nbh == 1)                                                                                 \
            hipLaunchKernelGGL((lm_topk_stream<KCAP, n, 1>), grid, block, 0, st, H, W, T, V, Hd, p.nN, p.G, s, \
                               c, inv_c, part);                                                                \
        else if constexpr (KCAP <= 16)                                                                         \
            hipLaunchKernelGGL((lm_topk_stream<KCAP, n, 2>), grid, block, 0, st, H, W, T, V, Hd, p.nN, p.G, s, \
                               c, inv_c, part);                                                                \
        break;
            ST_CASE(1) ST_CASE(2) ST_CASE(4) ST_CASE(8) ST_CASE(16)
#undef ST_CASE
            default: break;
        }
    } else if (p.BM == 64)
        launch_tiles<64, 128, KCAP>(p, H, W, T, V, Hd, s, c, part, pj, st);
    else if (p.BN == 256)
        launch_tiles<LM_BM, 256, KCAP>(p, H, W, T, V, Hd, s, c, part, pj, st);
    else
        launch_tiles<LM_BM, 128, KCAP>(p, H, W, T, V, Hd, s, c, part, pj, st);
    const uint64_t* cur = part;
    int G = p.G;
    if (G > 256) {
        // levels of 16 -> 1 until 256 or fewer lists per row remain
        uint64_t* buf[2];
        buf[0] = part + (size_t)T * (size_t)p.G * KCAP;
        buf[1] = buf[0] + (size_t)T * (size_t)((p.G + 15) / 16) * KCAP;
        for (int lv = 0; G > 256; ++lv) {
            const int G2 = (G + 15) / 16;
            const int64_t vrows = (int64_t)T * G2;
            hipLaunchKernelGGL((lm_topk_merge16_level<KCAP>), dim3((unsigned)((vrows + 15) / 16)), dim3(256), 0, st,
                               cur, T, G, G2, buf[lv & 1]);
            cur = buf[lv & 1];
            G = G2;
        }
    }
    if (G > 16) {
        if constexpr (KCAP <= 16)
            hipLaunchKernelGGL((lm_topk_merge_rank<KCAP>), dim3((unsigned)T), dim3(256), 0, st, cur, T, G, k, ids,
                               logits);
        else
            hipLaunchKernelGGL((lm_topk_merge256<KCAP>), dim3((unsigned)T), dim3(256), 0, st, cur, T, G, k, ids,
                               logits);
    } else
        hipLaunchKernelGGL((lm_topk_merge16<KCAP>), dim3((T + 15) / 16), dim3(256), 0, st, cur, T, G, k, ids,
                           logits);
}

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_lm_topk_workspace_size(int64_t T, int64_t V, int64_t Hd, int32_t k) {
    LmPlan p, q;
    if (T < 1 || V < 1 || Hd < 1 || k < 1 || k > 64 || !lm_plan(T, V, Hd, k, p) || !lm_plan(T, V, Hd, k, q, false))
        return 0;
    // enough for either kernel (dflash_lm_topk_proj never takes the streaming one)
    return p.ws > q.ws ? p.ws : q.ws;
}

// Host checks of the arguments every LM-head call shares (no HIP call); fills
// the launch plan.
static int lm_topk_validate(const uint16_t* H, const uint16_t* W, int64_t T, int64_t V, int64_t Hd, int32_t k,
                            float output_multiplier, float softcap, int32_t* ids, float* logits, LmPlan& p,
                            bool allow_stream) {
    if (!H || !W || !ids || !logits) return DFLASH_ERR_INVALID_ARG;
    if (!DFLASH_ALIGNED16(H) || !DFLASH_ALIGNED16(W)) return DFLASH_ERR_INVALID_ARG;
    if (T < 1 || V < 1 || Hd < 1 || k < 1 || k > V) return DFLASH_ERR_INVALID_ARG;
    if (!(output_multiplier > 0.f) || !(output_multiplier < INFINITY)) return DFLASH_ERR_INVALID_ARG;
    if (softcap != softcap || softcap == INFINITY) return DFLASH_ERR_INVALID_ARG;
    if (k > 64 || Hd % 8 != 0) return DFLASH_ERR_UNSUPPORTED;
    if (T > INT32_MAX || V > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    // tile buffer ranges and lane offsets (up to 256 rows of Hd bf16) are int32 byte counts
    if ((int64_t)256 * Hd * 2 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (!lm_plan(T, V, Hd, k, p, allow_stream)) return DFLASH_ERR_UNSUPPORTED;
    return DFLASH_OK;
}

static int lm_topk_launch(const LmPlan& p, const uint16_t* H, const uint16_t* W, int64_t T, int64_t V, int64_t Hd,
                          int32_t k, float output_multiplier, float softcap, int32_t* ids, float* logits, void* ws,
                          const LmProj& pj, void* stream) {
    const float c = softcap > 0.f ? softcap : 0.f;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint64_t* part = reinterpret_cast<uint64_t*>(ws);
    const int Ti = (int)T, Vi = (int)V, Hi = (int)Hd;
    switch (p.KCAP) {
        case 4: launch_all<4>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, pj, st); break;
        case 8: launch_all<8>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, pj, st); break;
        case 16: launch_all<16>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, pj, st); break;
        case 32: launch_all<32>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, pj, st); break;
        default: launch_all<64>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, pj, st); break;
    }
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

static int lm_topk_common(const uint16_t* H, const uint16_t* W, int64_t T, int64_t V, int64_t Hd, int32_t k,
                          float output_multiplier, float softcap, int32_t* ids, float* logits, void* ws,
                          size_t ws_bytes, const LmProj& pj, void* stream) {
    if (!ws || !DFLASH_ALIGNED16(ws)) return DFLASH_ERR_INVALID_ARG;
    LmPlan p;
    const int st = lm_topk_validate(H, W, T, V, Hd, k, output_multiplier, softcap, ids, logits, p, pj.Wp == nullptr);
    if (st != DFLASH_OK) return st;
    // the documented size (enough for either kernel), not just this call's plan
    if (ws_bytes < dflash_lm_topk_workspace_size(T, V, Hd, k)) return DFLASH_ERR_WORKSPACE;
    return lm_topk_launch(p, H, W, T, V, Hd, k, output_multiplier, softcap, ids, logits, ws, pj, stream);
}

extern "C" int dflash_lm_topk(const uint16_t* H, const uint16_t* W, int64_t T, int64_t V, int64_t Hd,
                              int32_t k, float output_multiplier, float softcap, int32_t* ids,
                              float* logits, void* ws, size_t ws_bytes, void* stream) {
    return lm_topk_common(H, W, T, V, Hd, k, output_multiplier, softcap, ids, logits, ws, ws_bytes,
                          LmProj{nullptr, 0, nullptr}, stream);
}

extern "C" int dflash_lm_topk_proj(const uint16_t* H, const uint16_t* W, int64_t T, int64_t V, int64_t Hd,
                                   int32_t k, float output_multiplier, float softcap, const uint16_t* W_proj,
                                   int32_t R, int32_t* ids, float* logits, float* hp, void* ws, size_t ws_bytes,
                                   void* stream) {
    if (!W_proj || !hp || !DFLASH_ALIGNED16(W_proj) || !DFLASH_ALIGNED16(hp)) return DFLASH_ERR_INVALID_ARG;
    if (R < 1) return DFLASH_ERR_INVALID_ARG;
    if (R > 4096 || (int64_t)R * Hd * 2 > INT32_MAX || T * (int64_t)R * 4 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    return lm_topk_common(H, W, T, V, Hd, k, output_multiplier, softcap, ids, logits, ws, ws_bytes,
                          LmProj{W_proj, R, hp}, stream);
}

// ---------------------------------------------------------------------------
// dflash_lm_topk_noalloc: the same kernels with their partial lists in a
// library-owned device array instead of a caller workspace, for callers that
// cannot allocate.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a
// host-side stand-in, never a device address; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current (on the
// entry point's first call there) and kept in lm_scratch_ptr.  Every call on a
// GPU shares that GPU's array and it keeps the last call's contents; nothing in
// it has to start at zero (each workgroup writes every entry of its lists before
// the merge reads them).  Calls that overlap on one GPU race on the array.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[DFLASH_LM_TOPK_SCRATCH_BYTES];

namespace {
constexpr int LM_SCRATCH_MAX_DEVICES = 64;
std::atomic<void*> lm_scratch_ptr[LM_SCRATCH_MAX_DEVICES];
std::mutex lm_scratch_mu;

// Device address of `scratch` on the current device.
int lm_scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= LM_SCRATCH_MAX_DEVICES) return DFLASH_ERR_HIP;
    void* ptr = lm_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(lm_scratch_mu);
        ptr = lm_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DFLASH_ERR_HIP;
            lm_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return DFLASH_OK;
}
}  // namespace

extern "C" int dflash_lm_topk_noalloc(const uint16_t* H, const uint16_t* W, int64_t T, int64_t V, int64_t Hd,
                                      int32_t k, float output_multiplier, float softcap, int32_t* ids,
                                      float* logits, void* stream) {
    LmPlan p;
    int st = lm_topk_validate(H, W, T, V, Hd, k, output_multiplier, softcap, ids, logits, p, true);
    if (st != DFLASH_OK) return st;
    if (dflash_lm_topk_workspace_size(T, V, Hd, k) > DFLASH_LM_TOPK_SCRATCH_BYTES) return DFLASH_ERR_SCRATCH;
    void* ws = nullptr;
    st = lm_scratch_address(&ws);
    if (st != DFLASH_OK) return st;
    return lm_topk_launch(p, H, W, T, V, Hd, k, output_multiplier, softcap, ids, logits, ws,
                          LmProj{nullptr, 0, nullptr}, stream);
}

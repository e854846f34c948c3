// Candidate-selector edge scores of the DFlash2 drafter
// (DFlash2BeamCandidateSelector: score = the candidate's own logit +
// <predecessor[q] * h_p, successor[c]>, h_p = the hidden state projected to the
// codebook rank, the first position's predecessor = the anchor token).
//
// Two kernels:
//   1. edges_projection: h_p = H . W_proj^T, a skinny bf16 MFMA GEMM
//      [T, Hd] x [R, Hd]^T.  The Hd axis is split into KS slices so that enough
//      workgroups stream H; each slice writes fp32 partial sums to the caller's
//      workspace (no atomics: the edge kernel adds them in slice order).  A deep
//      LDS-DMA ring keeps enough bytes in flight per CU.
//   2. edges_bilinear: one wave per (request, step), independent of the other
//      waves of its workgroup.  It issues all of its loads up front (ids, h_p
//      partials, unary logits), then loads its 16 * KB candidate (successor)
//      codebook rows straight into registers in the MFMA B layout and moves its
//      predecessor rows into LDS (global_load_lds, 16 bytes per lane), so the
//      wave waits on two memory latencies only: the ids, then the rows they
//      name.  a = P[pred] * h_p is formed in fp32 and split into three bf16 parts
//      whose products with the bf16 successor rows are exact, so the k x k block
//      comes out of bf16 MFMA with fp32 products and fp32 accumulation.
#include <atomic>

#include "common.h"

namespace dflash {

constexpr int PJ_ROWS = 64;     // rows of H per workgroup (4 waves x 16)
constexpr int PJ_BK = 64;       // Hd columns per ring stage: 128-byte LDS rows
constexpr int PJ_THREADS = 256;
constexpr int PJ_LDS = 128 * 1024;  // ring budget

// LDS-DMA of rows [0, 8 NQ) x columns [k0, k0 + 64) of a K-contiguous bf16 matrix
// (buffer rsrc based at row 0, row pitch ld) into an LDS tile of 128-byte rows,
// 16-byte chunks XOR-swizzled by row % 8.  Instruction q fills rows 8q .. 8q + 7;
// wave w issues q = w, w + 4, ...  Rows past the rsrc range and columns >= kend
// read as zero (kend % 8 == 0, so a chunk is all in or all out).
template <int NQ>
__device__ __forceinline__ void pj_dma(__amdgpu_buffer_rsrc_t rsrc, uint16_t* lds_tile, int wave_s, int lane,
                                       int ld, int k0, int kend) {
    const int r8 = lane >> 3;
    const int lc = (lane & 7) ^ r8;
    const int gk = k0 + lc * 8;
#pragma unroll
    for (int q0 = 0; q0 < NQ; q0 += 4) {
        const int q = q0 + wave_s;
        if (NQ % 4 == 0 || q < NQ) {
            const int voff = gk < kend ? ((q * 8 + r8) * ld + gk) * 2 : (int)0x80000000;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(lds_tile + q * 512), 16, voff, 0, 0, 0);
        }
    }
}

// part[ks][t][i] = sum over the ks-th Hd slice of H[t, j] * Wp[i, j]: a workgroup
// owns 64 rows x all R ranks x one slice, bf16 MFMA 16x16x32 (wave w: rows
// 16w .., every rank), three ring stages (deeper rings measured no faster on
// MI355X: 13.6 us with 3 stages, 13.8 with 4, 14.7 with 6 at 4096 x 4096 x 128).
template <int RB>  // R / 16
__global__ __launch_bounds__(PJ_THREADS) void edges_projection(const uint16_t* __restrict__ H,
                                                               const uint16_t* __restrict__ Wp, int T,
                                                               int Hd, int kslice,
                                                               float* __restrict__ part) {
    constexpr int R = RB * 16;
    constexpr int NQA = PJ_ROWS / 8;
    constexpr int NQB = R / 8;
    constexpr int STAGE = (PJ_ROWS + R) * PJ_BK;                     // elements
    constexpr int NST = PJ_LDS / (STAGE * 2) < 3 ? PJ_LDS / (STAGE * 2) : 3;
    static_assert(NST >= 2, "two ring stages fit");
    // DMA instructions every wave issues per stage, rounded down: a wave that
    // issues one more waits for one more completion than needed, which is safe
    constexpr int PER_WAVE = NQA / 4 + NQB / 4;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NST * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int row0 = blockIdx.x * PJ_ROWS;
    const int ks = blockIdx.y;
    const int kbeg = ks * kslice;
    const int kend = min(Hd, kbeg + kslice);
    const int nS = kend > kbeg ? (kend - kbeg + PJ_BK - 1) / PJ_BK : 0;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(H + (int64_t)row0 * Hd), (short)0, min(PJ_ROWS, T - row0) * Hd * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc((void*)Wp, (short)0, R * Hd * 2, 0x00020000);

    f32x4 acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int sl = 0; sl < NST - 1 && sl < nS; ++sl) {
        pj_dma<NQA>(rsA, smem + sl * STAGE, wave_s, lane, Hd, kbeg + sl * PJ_BK, kend);
        pj_dma<NQB>(rsB, smem + sl * STAGE + PJ_ROWS * PJ_BK, wave_s, lane, Hd, kbeg + sl * PJ_BK, kend);
    }
    for (int kt = 0; kt < nS; ++kt) {
        // slice kt has landed (and this wave's reads of slice kt - 1 are done) once
        // at most the later slices' loads are in flight; after the barrier, every
        // wave's have
        compiler_fence();
        wait_stages_ahead<NST - 2, PER_WAVE>(nS - 1 - kt);
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        const int sn = kt + NST - 1;  // refill the slot read in iteration kt - 1
        if (sn < nS) {
            uint16_t* base = smem + (sn % NST) * STAGE;
            pj_dma<NQA>(rsA, base, wave_s, lane, Hd, kbeg + sn * PJ_BK, kend);
            pj_dma<NQB>(rsB, base + PJ_ROWS * PJ_BK, wave_s, lane, Hd, kbeg + sn * PJ_BK, kend);
        }
        const uint16_t* a_base = smem + (kt % NST) * STAGE;
        const uint16_t* b_base = a_base + PJ_ROWS * PJ_BK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int chs = ((kk * 4 + (lane >> 4)) ^ (lane & 7)) << 3;  // row % 8 == lane % 8
            const bf16x8 af =
                as_bf16x8(*reinterpret_cast<const u32x4*>(a_base + (wave * 16 + (lane & 15)) * PJ_BK + chs));
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                const bf16x8 bfr =
                    as_bf16x8(*reinterpret_cast<const u32x4*>(b_base + (j * 16 + (lane & 15)) * PJ_BK + chs));
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[j], 0, 0, 0);
            }
        }
    }
    float* dst = part + (int64_t)ks * T * R;
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = row0 + wave * 16 + 4 * (lane >> 4) + e;
            if (t < T) dst[(int64_t)t * R + j * 16 + (lane & 15)] = acc[j][e];
        }
}

// Per-wave LDS tile: NR = 16 * KB gathered predecessor-codebook rows, packed at
// 2R bytes, NJ LDS-DMA instructions of 1 KB (the last one padded), then the KS
// projection partials of the wave's row (fp32 [KS, R], NH instructions) and its
// unary logits (fp32 [k <= 64]).  The successor rows go straight to registers.
template <int KB, int R, int KS>
struct EdgeTile {
    static constexpr int NR = 16 * KB;
    static constexpr int CPR = R / 8;                      // 16-byte chunks per row
    static constexpr int NJ = (NR * CPR + 63) / 64;
    static constexpr int TILE = NJ * 512;                  // elements per codebook
    static constexpr int NH = (KS * R / 4 + 63) / 64;      // LDS-DMA instructions for the partials
    static constexpr int WAVE_ELEMS = TILE + NH * 512 + 128;   // + 64 fp32 unary logits
    static constexpr int WAVE_BYTES = WAVE_ELEMS * 2;
};

// a = hi + mid + lo exactly, each part a bf16 (truncating splits: every remainder
// is exact in fp32, and the last one has at most 8 significant bits).  With b a
// bf16, hi * b, mid * b and lo * b are exact in fp32, so three bf16 MFMAs give
// the fp32 product a * b, with fp32 accumulation.
template <int N>
__device__ __forceinline__ void split3_bf16(const float (&a)[N], uint32_t (&hi)[N / 2], uint32_t (&mid)[N / 2],
                                            uint32_t (&lo)[N / 2]) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const uint32_t x0 = __float_as_uint(a[2 * i]), x1 = __float_as_uint(a[2 * i + 1]);
        const float r0 = a[2 * i] - __uint_as_float(x0 & 0xffff0000u);
        const float r1 = a[2 * i + 1] - __uint_as_float(x1 & 0xffff0000u);
        const uint32_t y0 = __float_as_uint(r0), y1 = __float_as_uint(r1);
        const float s0 = r0 - __uint_as_float(y0 & 0xffff0000u);
        const float s1 = r1 - __uint_as_float(y1 & 0xffff0000u);
        // v_perm_b32 selector 0x07060302: the high halves of (second, first) -> (hi16, lo16)
        hi[i] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
        mid[i] = __builtin_amdgcn_perm(y1, y0, 0x07060302u);
        lo[i] = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), 0x07060302u);
    }
}

typedef __attribute__((ext_vector_type(4))) short i16x4;

// One wave per row t = r * S + p, WAVES waves per workgroup, each with its own LDS
// tile and no synchronisation with the others.
//
// The wave's predecessor rows (row = 16b + lane % 16 <-> predecessor q) and
// candidate rows are gathered with LDS-DMA: instruction j moves the 16-byte chunks
// f = 64j + lane of the tile (row f / CPR, slot f % CPR), and a row keeps logical
// chunk c in slot (c + row) % CPR, so the 16 lanes that read one logical chunk of
// 16 rows hit different slots.  Then lane l takes predecessor row q = l % 16 (MFMA
// row) and candidate row c = l % 16 (MFMA column); lane group g = l / 16 holds
// ranks 8g .. 8g + 7 of every 32-rank chunk (bf16 MFMA 16x16x32), or 4g .. 4g + 3
// of a last 16-rank chunk (16x16x16).  a = P[pred] * h_p is formed in fp32 and
// split into three bf16 parts (split3_bf16), so the k x k block accumulates exact
// fp32 products in fp32.
template <int KB, int R, int KS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void edges_bilinear(
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Sc, const int32_t* __restrict__ ids,
    const float* __restrict__ U, const float* __restrict__ part, const int32_t* __restrict__ anchor, int T,
    int St, int k, int V, float* __restrict__ E) {
    using TL = EdgeTile<KB, R, KS>;
    constexpr int CPR = TL::CPR, NR = TL::NR;
    constexpr int NC = R / 32;             // 32-rank chunks
    constexpr bool HALF = (R % 32) != 0;   // and a last 16-rank chunk
    extern __shared__ __attribute__((aligned(16))) uint16_t smem_e[];

    const int lane = threadIdx.x & 63;
    const int wave_s = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int t = blockIdx.x * WAVES + wave_s;
    const bool live = t < T;
    const int tt = live ? t : T - 1;  // dead waves mirror the last row and store nothing
    const int r = tt / St, p = tt - r * St;
    const int g = lane >> 4, li = lane & 15;
    uint16_t* sP = smem_e + wave_s * TL::WAVE_ELEMS;
    float* sH = reinterpret_cast<float*>(sP + TL::TILE);
    float* sU = sH + TL::NH * 256;

    // ids of the predecessor rows (q) and candidate rows (c) this lane stands for;
    // the loads are unconditional (index clamped to k - 1, lanes q >= k dropped
    // afterwards) so that nothing waits for them before the next loads are issued
    int pred[KB], cid[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const int q = min(b * 16 + li, k - 1);
        pred[b] = (p == 0) ? anchor[r] : ids[(int64_t)max(tt - 1, 0) * k + q];
        cid[b] = ids[(int64_t)tt * k + q];
    }
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const bool in = b * 16 + li < k;
        pred[b] = in ? min(max(pred[b], 0), V - 1) : 0;
        cid[b] = in ? min(max(cid[b], 0), V - 1) : 0;
    }

    // the successor rows, in the MFMA B layout: lane (g, li) holds ranks
    // 32 ic + 8 g .. + 7 of candidate row 16 b + li (and ranks 32 NC + 4 g .. + 3
    // of a last 16-rank chunk), which is its own cid[b]
    u32x4 sv[KB][NC > 0 ? NC : 1];
    u32x2 sh[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const uint16_t* srow = Sc + (int64_t)cid[b] * R;
#pragma unroll
        for (int ic = 0; ic < NC; ++ic) sv[b][ic] = *reinterpret_cast<const u32x4*>(srow + ic * 32 + g * 8);
        if constexpr (HALF) sh[b] = *reinterpret_cast<const u32x2*>(srow + NC * 32 + g * 4);
    }

    // predecessor gathers; chunks past the tile (f >= NR * CPR) reload row 0 into
    // the padding
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j) {
        const int f = j * 64 + lane;
        const int row = f < NR * CPR ? f / CPR : 0;
        const int slot = f - (f / CPR) * CPR;
        const int lc = (slot + CPR - row % CPR) % CPR;
        int pid = 0;
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const int x = __shfl(pred[b], row & 15);
            if ((row >> 4) == b) pid = x;
        }
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(P + (int64_t)pid * R + lc * 8),
            (__attribute__((address_space(3))) void*)(sP + j * 512), 16, 0, 0);
    }
    // the row's KS projection partials and unary logits, straight to LDS as well
    // (partials: flat float4 f = 64 j + lane is partial f / (R / 4), ranks
    // 4 (f % (R / 4)) ..; lanes past the end reload the last one into the
    // padding).  Issued after the gathers: a DS instruction after an LDS-DMA load
    // waits for that load.
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(U + (int64_t)tt * k + min(lane, k - 1)),
        (__attribute__((address_space(3))) void*)sU, 4, 0, 0);
#pragma unroll
    for (int j = 0; j < TL::NH; ++j) {
        const int f = min(j * 64 + lane, KS * R / 4 - 1);
        const int q = f / (R / 4);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(part + ((int64_t)q * T + tt) * R + (f - q * (R / 4)) * 4),
            (__attribute__((address_space(3))) void*)(sH + j * 256), 16, 0, 0);
    }
    // the rows and partials are in LDS once this wave's loads have returned
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
    compiler_fence();
    // h_p[i] = the partials added in slice order
    auto hsum4 = [&](int i) {
        f32x4 x = *reinterpret_cast<const f32x4*>(sH + i);
#pragma unroll
        for (int q = 1; q < KS; ++q) x += *reinterpret_cast<const f32x4*>(sH + q * R + i);
        return x;
    };

    // Rows q >= k (a) and columns c >= k (b) hold the row of id 0; they only reach
    // outputs that are not stored.
    f32x4 acc[KB][KB];
#pragma unroll
    for (int a = 0; a < KB; ++a)
#pragma unroll
        for (int b = 0; b < KB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int ic = 0; ic < NC; ++ic) {
        const int lcq = ic * 4 + g;  // logical 16-byte chunk of this lane group
        uint32_t ahi[KB][4], amid[KB][4], alo[KB][4];
        u32x4 bv[KB];
        const f32x4 h0 = hsum4(ic * 32 + g * 8), h1 = hsum4(ic * 32 + g * 8 + 4);
        const float h[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
        for (int bq = 0; bq < KB; ++bq) {
            const int row = bq * 16 + li;
            const int off = row * R + ((lcq + row) % CPR) * 8;
            float a[8];
            unpack8(*reinterpret_cast<const u32x4*>(sP + off), a);
            bv[bq] = sv[bq][ic];
#pragma unroll
            for (int v = 0; v < 8; ++v) a[v] *= h[v];
            split3_bf16<8>(a, ahi[bq], amid[bq], alo[bq]);
        }
#pragma unroll
        for (int bq = 0; bq < KB; ++bq)
#pragma unroll
            for (int bc = 0; bc < KB; ++bc) {
                const bf16x8 bb = as_bf16x8(bv[bc]);
                acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(u32x4{alo[bq][0], alo[bq][1], alo[bq][2], alo[bq][3]}), bb, acc[bq][bc], 0, 0, 0);
                acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(u32x4{amid[bq][0], amid[bq][1], amid[bq][2], amid[bq][3]}), bb, acc[bq][bc], 0, 0, 0);
                acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(u32x4{ahi[bq][0], ahi[bq][1], ahi[bq][2], ahi[bq][3]}), bb, acc[bq][bc], 0, 0, 0);
            }
    }
    if constexpr (HALF) {
        const int lcq = NC * 4 + (g >> 1), sub = (g & 1) * 4;
        const f32x4 hh = hsum4(NC * 32 + g * 4);
        uint32_t ahi[KB][2], amid[KB][2], alo[KB][2];
        u32x2 bv[KB];
#pragma unroll
        for (int bq = 0; bq < KB; ++bq) {
            const int row = bq * 16 + li;
            const int off = row * R + ((lcq + row) % CPR) * 8 + sub;
            const u32x2 x = *reinterpret_cast<const u32x2*>(sP + off);
            bv[bq] = sh[bq];
            float a[4] = {__uint_as_float(x[0] << 16) * hh[0], __uint_as_float(x[0] & 0xffff0000u) * hh[1],
                          __uint_as_float(x[1] << 16) * hh[2], __uint_as_float(x[1] & 0xffff0000u) * hh[3]};
            split3_bf16<4>(a, ahi[bq], amid[bq], alo[bq]);
        }
#pragma unroll
        for (int bq = 0; bq < KB; ++bq)
#pragma unroll
            for (int bc = 0; bc < KB; ++bc) {
                const i16x4 bb = __builtin_bit_cast(i16x4, bv[bc]);
                acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(i16x4, u32x2{alo[bq][0], alo[bq][1]}), bb, acc[bq][bc], 0, 0, 0);
                acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(i16x4, u32x2{amid[bq][0], amid[bq][1]}), bb, acc[bq][bc], 0, 0, 0);
                acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(i16x4, u32x2{ahi[bq][0], ahi[bq][1]}), bb, acc[bq][bc], 0, 0, 0);
            }
    }

    if (!live) return;
#pragma unroll
    for (int bc = 0; bc < KB; ++bc) {
        const int c = bc * 16 + li;
        if (c >= k) continue;
        const float u = sU[c];
#pragma unroll
        for (int bq = 0; bq < KB; ++bq)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = bq * 16 + 4 * g + e;
                if (q < k) E[((int64_t)t * k + q) * k + c] = u + acc[bq][bc][e];
            }
    }
}

struct EdgePlan {
    int KS, kslice;
    size_t ws;
};

// KS (a power of two <= 8): enough workgroups to fill the chip, at least one
// 64-wide column block per slice.
static EdgePlan edge_plan(int64_t T, int R, int64_t Hd) {
    EdgePlan p;
    const int64_t row_blocks = (T + PJ_ROWS - 1) / PJ_ROWS;
    const int64_t max_ks = (Hd + PJ_BK - 1) / PJ_BK;
    int ks = 1;
    while (ks < 8 && row_blocks * ks < 256 && 2 * ks <= max_ks) ks *= 2;
    int64_t kslice = (Hd + ks - 1) / ks;
    kslice = (kslice + PJ_BK - 1) / PJ_BK * PJ_BK;
    p.KS = ks;
    p.kslice = (int)kslice;
    p.ws = (size_t)ks * (size_t)T * (size_t)R * sizeof(float);
    return p;
}

template <int KB, int R, int KS>
static void launch_bilinear_r(const uint16_t* P, const uint16_t* Sc, const int32_t* ids, const float* U,
                              const float* part, const int32_t* anchor, int T, int St, int k, int V, float* E,
                              hipStream_t st) {
    constexpr int wave_bytes = EdgeTile<KB, R, KS>::WAVE_BYTES;
    constexpr int WAVES = wave_bytes * 4 <= 64 * 1024 ? 4 : wave_bytes * 2 <= 64 * 1024 ? 2 : 1;
    static_assert(wave_bytes * WAVES <= 160 * 1024, "tile fits in LDS");
    if (wave_bytes * WAVES > 64 * 1024) {
        // the attribute is set once per device (bit d of `done`), not on every launch
        static std::atomic<uint64_t> done{0};
        int dev = 0;
        (void)hipGetDevice(&dev);
        const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
        if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(&edges_bilinear<KB, R, KS, WAVES>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, wave_bytes * WAVES) == hipSuccess)
                done.fetch_or(bit, std::memory_order_release);
        }
    }
    hipLaunchKernelGGL((edges_bilinear<KB, R, KS, WAVES>), dim3((T + WAVES - 1) / WAVES), dim3(64 * WAVES),
                       wave_bytes * WAVES, st, P, Sc, ids, U, part, anchor, T, St, k, V, E);
}

template <int KB, int KS>
static bool launch_bilinear_ks(const uint16_t* P, const uint16_t* Sc, const int32_t* ids, const float* U,
                               const float* part, const int32_t* anchor, int T, int St, int k, int V, int R,
                               float* E, hipStream_t st) {
    switch (R) {
#define BL_CASE(n) \
    case n: launch_bilinear_r<KB, n, KS>(P, Sc, ids, U, part, anchor, T, St, k, V, E, st); return true;
        BL_CASE(16) BL_CASE(32) BL_CASE(48) BL_CASE(64) BL_CASE(80) BL_CASE(96) BL_CASE(112) BL_CASE(128)
        BL_CASE(144) BL_CASE(160) BL_CASE(176) BL_CASE(192) BL_CASE(208) BL_CASE(224) BL_CASE(240) BL_CASE(256)
#undef BL_CASE
        default: return false;
    }
}

template <int KB>
static bool launch_bilinear(const uint16_t* P, const uint16_t* Sc, const int32_t* ids, const float* U,
                            const float* part, int KS, const int32_t* anchor, int T, int St, int k, int V, int R,
                            float* E, hipStream_t st) {
    switch (KS) {
        case 1: return launch_bilinear_ks<KB, 1>(P, Sc, ids, U, part, anchor, T, St, k, V, R, E, st);
        case 2: return launch_bilinear_ks<KB, 2>(P, Sc, ids, U, part, anchor, T, St, k, V, R, E, st);
        case 4: return launch_bilinear_ks<KB, 4>(P, Sc, ids, U, part, anchor, T, St, k, V, R, E, st);
        case 8: return launch_bilinear_ks<KB, 8>(P, Sc, ids, U, part, anchor, T, St, k, V, R, E, st);
        default: return false;
    }
}

template <int RB>
static void launch_projection(const uint16_t* H, const uint16_t* Wp, int T, int Hd, const EdgePlan& p,
                              float* part, hipStream_t st) {
    dim3 grid((T + PJ_ROWS - 1) / PJ_ROWS, p.KS);
    hipLaunchKernelGGL((edges_projection<RB>), grid, dim3(PJ_THREADS), 0, st, H, Wp, T, Hd, p.kslice, part);
}

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_candidate_edges_workspace_size(int64_t T, int32_t R, int64_t Hd) {
    if (T < 1 || R < 16 || Hd < 1) return 0;
    return edge_plan(T, R, Hd).ws;
}

extern "C" int dflash_candidate_edges(const uint16_t* pred_cb, const uint16_t* succ_cb, const int32_t* cand_ids,
                                      const float* unary, const uint16_t* H, const uint16_t* W_proj,
                                      const int32_t* anchor, int64_t Rq, int32_t S, int32_t k, int64_t V,
                                      int32_t R, int64_t Hd, float* edges, void* ws, size_t ws_bytes,
                                      void* stream) {
    const void* ptrs[] = {pred_cb, succ_cb, cand_ids, unary, H, W_proj, anchor, edges, ws};
    for (const void* q : ptrs)
        if (!q || !DFLASH_ALIGNED16(q)) return DFLASH_ERR_INVALID_ARG;
    if (Rq < 1 || S < 1 || V < 1 || Hd < 1 || k < 1 || k > V || R < 1) return DFLASH_ERR_INVALID_ARG;
    if (k > 64 || R % 16 != 0 || R > 256 || Hd % 8 != 0) return DFLASH_ERR_UNSUPPORTED;
    const int64_t T = Rq * (int64_t)S;
    if (T > INT32_MAX / 64 || V > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    // buffer ranges and lane offsets of the projection (up to 256 rows of Hd bf16) are int32 byte counts
    if ((int64_t)256 * Hd * 2 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    const EdgePlan p = edge_plan(T, R, Hd);
    if (ws_bytes < p.ws) return DFLASH_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    float* part = reinterpret_cast<float*>(ws);
    const int Ti = (int)T, Hi = (int)Hd;
    switch (R / 16) {
#define PJ_CASE(n) \
    case n: launch_projection<n>(H, W_proj, Ti, Hi, p, part, st); break;
        PJ_CASE(1) PJ_CASE(2) PJ_CASE(3) PJ_CASE(4) PJ_CASE(5) PJ_CASE(6) PJ_CASE(7) PJ_CASE(8)
        PJ_CASE(9) PJ_CASE(10) PJ_CASE(11) PJ_CASE(12) PJ_CASE(13) PJ_CASE(14) PJ_CASE(15) PJ_CASE(16)
#undef PJ_CASE
        default: return DFLASH_ERR_UNSUPPORTED;
    }
    DFLASH_LAUNCH_CHECK();
    const int KB = (k + 15) / 16;
    bool ok;
    if (KB == 1)
        ok = launch_bilinear<1>(pred_cb, succ_cb, cand_ids, unary, part, p.KS, anchor, Ti, S, k, (int)V, R, edges, st);
    else if (KB == 2)
        ok = launch_bilinear<2>(pred_cb, succ_cb, cand_ids, unary, part, p.KS, anchor, Ti, S, k, (int)V, R, edges, st);
    else
        ok = launch_bilinear<4>(pred_cb, succ_cb, cand_ids, unary, part, p.KS, anchor, Ti, S, k, (int)V, R, edges, st);
    if (!ok) return DFLASH_ERR_UNSUPPORTED;
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

extern "C" int dflash_candidate_edges_hp(const uint16_t* pred_cb, const uint16_t* succ_cb,
                                         const int32_t* cand_ids, const float* unary, const float* hp,
                                         const int32_t* anchor, int64_t Rq, int32_t S, int32_t k, int64_t V,
                                         int32_t R, float* edges, void* stream) {
    const void* ptrs[] = {pred_cb, succ_cb, cand_ids, unary, hp, anchor, edges};
    for (const void* q : ptrs)
        if (!q || !DFLASH_ALIGNED16(q)) return DFLASH_ERR_INVALID_ARG;
    if (Rq < 1 || S < 1 || V < 1 || k < 1 || k > V || R < 1) return DFLASH_ERR_INVALID_ARG;
    if (k > 64 || R % 16 != 0 || R > 256) return DFLASH_ERR_UNSUPPORTED;
    const int64_t T = Rq * (int64_t)S;
    if (T > INT32_MAX / 64 || V > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int Ti = (int)T;
    const int KB = (k + 15) / 16;
    bool ok;
    // h_p given: the bilinear stage alone, on one "partial"
    if (KB == 1)
        ok = launch_bilinear<1>(pred_cb, succ_cb, cand_ids, unary, hp, 1, anchor, Ti, S, k, (int)V, R, edges, st);
    else if (KB == 2)
        ok = launch_bilinear<2>(pred_cb, succ_cb, cand_ids, unary, hp, 1, anchor, Ti, S, k, (int)V, R, edges, st);
    else
        ok = launch_bilinear<4>(pred_cb, succ_cb, cand_ids, unary, hp, 1, anchor, Ti, S, k, (int)V, R, edges, st);
    if (!ok) return DFLASH_ERR_UNSUPPORTED;
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

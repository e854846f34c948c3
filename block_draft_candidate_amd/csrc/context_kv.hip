// Context K/V precompute of the DFlash2 drafter for every draft layer at once
// (DFlash2BeamModel.build_context_kv_weights / precompute_and_store_context_kv
// and the store_context_kv op it calls): hidden_norm RMSNorm of the context
// states, one linear against the stacked K/V rows of every layer's qkv_proj,
// then per layer the K-norm and NeoX RoPE of K and the slot-mapped write of K
// and V into that layer's paged cache.
//
//   * ctx_hidden_norm: one workgroup per context row; the row's sum of squares
//     is reduced across the workgroup, the normed row is written once as bf16
//     (the norm's output dtype) into the workspace.
//   * ctx_kv_tiles: the stacked linear as a bf16 MFMA GEMM (32x32x16, fp32
//     accumulate) over 256 x 256 or 256 x 128 output tiles, with the same
//     operand pipeline as the LM head's tile kernel (64-wide K slices by LDS-DMA
//     into a five-slot LDS ring, XOR-swizzled 16-byte chunks).  A tile's columns
//     are whole heads (head_dim 128) of one layer's K or V, so the epilogue
//     needs no data from other tiles: a head's columns are staged row-major in
//     LDS, thread t takes row t, rounds the fp32
//     sums to bf16 (the linear's output), and for a K head applies the layer's
//     RMSNorm over the 128 values and the NeoX rotation at the token's position
//     before one more bf16 rounding; V is stored as rounded.  The row then goes
//     straight to cache[slot / bs, h, slot % bs, 0:D] (K) or [D:2D] (V) of its
//     layer; the [num_ctx, L, 2, Hkv, D] intermediate is never written to HBM
//     unless the caller asks for it.
//   * Tiles are dealt to XCDs in contiguous runs (row tiles fastest), so the
//     workgroups of an XCD share weight tiles and context slices in its L2.
#include "common.h"

namespace dflash {

constexpr int CKV_BM = 256;
constexpr int CKV_BK = 64;
constexpr int CKV_THREADS = 256;
constexpr int CKV_D = 128;
constexpr int CKV_MAX_LAYERS = 64;

// Per-layer cache base pointers, passed by value (512 bytes of kernel
// arguments): no device-side pointer table to build or keep in sync.
struct CtxCaches {
    uint16_t* p[CKV_MAX_LAYERS];
};

__device__ __forceinline__ uint32_t ckv_lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---------------------------------------------------------------------------
// hidden_norm: normed[t, :] = bf16(x[t, :] * (mean(x[t, :]^2) + eps)^-1/2 * w)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ctx_hidden_norm_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w, int Hd, float eps,
                                                              uint16_t* __restrict__ out) {
    __shared__ float red[4];
    const int64_t t = blockIdx.x;
    const uint16_t* row = x + t * Hd;
    const int nch = Hd >> 3;  // 16-byte chunks
    float ss = 0.f;
    for (int c = threadIdx.x; c < nch; c += 256) {
        float v[8];
        unpack8(ldg16(row + c * 8), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    const float rinv = 1.0f / sqrtf(ss / (float)Hd + eps);
    uint16_t* orow = out + t * Hd;
    for (int c = threadIdx.x; c < nch; c += 256) {
        float v[8], wv[8];
        unpack8(ldg16(row + c * 8), v);
        unpack8(ldg16(w + c * 8), wv);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16x2(v[2 * e] * rinv * wv[2 * e], v[2 * e + 1] * rinv * wv[2 * e + 1]);
        stg16(orow + c * 8, o);
    }
}

// ---------------------------------------------------------------------------
// The stacked K/V linear with the K-norm / RoPE / cache-write epilogue.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_round(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }

template <int BN, bool TAIL>
__global__ __launch_bounds__(CKV_THREADS, 1) void ctx_kv_tiles(
    const uint16_t* __restrict__ A /*normed [n, Hd]*/, const uint16_t* __restrict__ W /*[N, Hd]*/, int n, int Hd,
    int N, int nM, int ntiles, int Hkv, const uint16_t* __restrict__ k_w /*[L, D]*/, float eps,
    const int64_t* __restrict__ positions, const float* __restrict__ cos_sin, int64_t max_pos,
    const int64_t* __restrict__ slots, CtxCaches caches, int64_t num_blocks, int block_size,
    uint16_t* __restrict__ kv_out) {
    constexpr int WN = BN / 2;               // columns per wave
    constexpr int NB = WN / 32;              // 32-column MFMA blocks per wave
    constexpr int MB = 4;                    // 32-row MFMA blocks per wave (128 rows)
    constexpr int NIA = CKV_BM / 8 / 4;      // LDS-DMA instructions per wave per slice (A)
    constexpr int NIB = BN / 8 / 4;          // (B)
    constexpr int UNIT = CKV_BM * CKV_BK;    // elements of one operand's K slice
    constexpr int NSLOT = 5;                 // LDS ring of operand slices (2.5 K slices)
    constexpr int SP = CKV_D + 4;            // row pitch (floats) of the epilogue staging (one head)
    constexpr int SMEM = (NSLOT * UNIT > CKV_BM * SP * 2) ? NSLOT * UNIT : CKV_BM * SP * 2;
    constexpr int NPASS = BN / CKV_D;        // heads per tile = epilogue passes
    static_assert(BN % CKV_D == 0 && (WN % CKV_D == 0 || CKV_D % WN == 0), "heads align with wave columns");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM];
    float* stage = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave >> 1, wn = wave & 1;

    // Workgroup ids go to the 8 XCDs round-robin; XCD x takes tiles
    // [x * per, (x + 1) * per) in (column tile, row tile) order.
    const int per = gridDim.x >> 3;
    const int q = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (q >= ntiles) return;
    const int m_tile = q % nM, n_tile = q / nM;
    const int m0 = m_tile * CKV_BM;
    const int n0 = n_tile * BN;
    const int my_row = m0 + tid;

    const int nK = (Hd + CKV_BK - 1) / CKV_BK;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + (int64_t)m0 * Hd), (short)0, min(CKV_BM, n - m0) * Hd * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (int64_t)n0 * Hd), (short)0, BN * Hd * 2, 0x00020000);

    const int fr = lane & 31;
    const int a_row0 = (wm * 128 + fr) * CKV_BK;
    const int b_row0 = (wn * WN + fr) * CKV_BK;
    int voffA[NIA], voffB[NIB], lcA, lcB;
    dma_offsets<NIA>(voffA, lcA, wave_s, lane, Hd);
    dma_offsets<NIB>(voffB, lcB, wave_s, lane, Hd);

    f32x16 acc[MB][NB];
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
            fb[qf - 1] = as_bf16x8(*reinterpret_cast<const u32x4*>(smem + sb * UNIT + b_row0 + (qf - 1) * 32 * CKV_BK + chs));
        else {
            const int i = qf == 0 ? 0 : qf - NB;
            fa[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(smem + sa * UNIT + a_row0 + i * 32 * CKV_BK + chs));
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
                dma_one<NIA, TAIL>(rsA, smem + dslot * UNIT, voffA, lcA, wave_s, Hd, dkt * CKV_BK, qq);
            if (dma == 2 && qq < NIB)
                dma_one<NIB, TAIL>(rsB, smem + dslot * UNIT, voffB, lcB, wave_s, Hd, dkt * CKV_BK, qq);
        }
        mfmas(fa, fb);
#pragma unroll
        for (int qq = 0; qq < MPK; ++qq) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (qq < NFR && rk16 >= 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if ((dma == 1 && qq < NIA) || (dma == 2 && qq < NIB)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };

    // Slice k keeps its B half in ring slot 2k mod 5 and its A half in 2k+1 mod
    // 5; the barrier at the end of slice k frees both, the A half of slice k+2
    // goes into one right after it and the B half of slice k+3 into the other
    // during the first K step of slice k+1 (B in flight for about two slices).
    bf16x8 fa0[MB], fb0[NB], fa1[MB], fb1[NB];
    dma_slice<NIB, TAIL>(rsB, smem + 0 * UNIT, voffB, lcB, wave_s, Hd, 0);
    dma_slice<NIA, TAIL>(rsA, smem + 1 * UNIT, voffA, lcA, wave_s, Hd, 0);
    dma_slice<NIB, TAIL>(rsB, smem + 2 * UNIT, voffB, lcB, wave_s, Hd, CKV_BK);  // past K: zeros, unused
    dma_slice<NIA, TAIL>(rsA, smem + 3 * UNIT, voffA, lcA, wave_s, Hd, CKV_BK);
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

    // Per-row data of the epilogue: the token's RoPE row and its cache row.
    int64_t pos = 0, cache_row = -1;  // element offset of [blk, 0, off, 0]
    if (my_row < n) {
        pos = positions[my_row];
        pos = pos < 0 ? 0 : (pos >= max_pos ? max_pos - 1 : pos);
        if (slots != nullptr) {
            const int64_t s = slots[my_row];
            if (s >= 0 && s < num_blocks * block_size) {
                const int64_t blk = s / block_size, off = s - blk * block_size;
                cache_row = (blk * Hkv * block_size + off) * (2 * CKV_D);
            }
        }
    }
    const int64_t head_stride = (int64_t)block_size * 2 * CKV_D;

    // One pass per head of the tile: the waves holding the head's columns
    // stage them row-major (pitch D + 4 floats), then thread t finishes row t.
    // In the 32x32 MFMA layout lane l holds column l % 32 and rows
    // 8b + 4(l / 32) + e, e = 0..3.
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        if ((wn * WN) / CKV_D == pass) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int col = (wn * WN) % CKV_D + j * 32 + fr;
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // 4-byte writes straight from the accumulator registers
                        const uint32_t dst =
                            ckv_lds_offset(stage + (wm * 128 + i * 32 + 8 * b + 4 * (lane >> 5)) * SP + col);
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
        if (my_row < n) {
            // head (layer l, K or V, kv head h) of these 128 columns
            const int gh = n0 / CKV_D + pass;
            const int l = gh / (2 * Hkv);
            const int r = gh - l * 2 * Hkv;
            const bool is_v = r >= Hkv;
            const int h = is_v ? r - Hkv : r;
            const float* rowp = stage + tid * SP;
            uint16_t* kvo = kv_out != nullptr ? kv_out + (int64_t)my_row * N + gh * CKV_D : nullptr;
            uint16_t* dst = cache_row >= 0 ? caches.p[l] + cache_row + h * head_stride + (is_v ? CKV_D : 0) : nullptr;
            if (is_v) {
#pragma unroll 4
                for (int c = 0; c < CKV_D / 8; ++c) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(rowp + 8 * c);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(rowp + 8 * c + 4);
                    const u32x4 o = {pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                                     pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
                    if (kvo) stg16(kvo + 8 * c, o);
                    if (dst) stg16(dst + 8 * c, o);
                }
            } else {
                // the linear's bf16 output, then the layer's K RMSNorm over the head
                float ss = 0.f;
#pragma unroll 8
                for (int c = 0; c < CKV_D / 4; ++c) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(rowp + 4 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = bf16_round(x[e]);
                        ss += v * v;
                    }
                }
                const float rinv = 1.0f / sqrtf(ss * (1.0f / CKV_D) + eps);
                const uint16_t* wl = k_w + l * CKV_D;
                const float* cs = cos_sin + pos * CKV_D;
                // NeoX pairs (i, i + 64): columns 8c.. and 64 + 8c.. together
#pragma unroll 2
                for (int c = 0; c < CKV_D / 16; ++c) {
                    float x1[8], x2[8], w1[8], w2[8];
#pragma unroll
                    for (int hq = 0; hq < 2; ++hq) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(rowp + 8 * c + 4 * hq);
                        const f32x4 b = *reinterpret_cast<const f32x4*>(rowp + CKV_D / 2 + 8 * c + 4 * hq);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x1[4 * hq + e] = bf16_round(a[e]);
                            x2[4 * hq + e] = bf16_round(b[e]);
                        }
                    }
                    unpack8(ldg16(wl + 8 * c), w1);
                    unpack8(ldg16(wl + CKV_D / 2 + 8 * c), w2);
                    const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + 8 * c);
                    const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 8 * c + 4);
                    const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + CKV_D / 2 + 8 * c);
                    const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + CKV_D / 2 + 8 * c + 4);
                    const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                    const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                    float o1[8], o2[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float y1 = x1[e] * rinv * w1[e];
                        const float y2 = x2[e] * rinv * w2[e];
                        o1[e] = y1 * cv[e] - y2 * sv[e];
                        o2[e] = y2 * cv[e] + y1 * sv[e];
                    }
                    if (kvo) {
                        stg16(kvo + 8 * c, u32x4{pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3]),
                                                 pack_bf16x2(x1[4], x1[5]), pack_bf16x2(x1[6], x1[7])});
                        stg16(kvo + CKV_D / 2 + 8 * c,
                              u32x4{pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3]),
                                    pack_bf16x2(x2[4], x2[5]), pack_bf16x2(x2[6], x2[7])});
                    }
                    if (dst) {
                        stg16(dst + 8 * c, u32x4{pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3]),
                                                 pack_bf16x2(o1[4], o1[5]), pack_bf16x2(o1[6], o1[7])});
                        stg16(dst + CKV_D / 2 + 8 * c,
                              u32x4{pack_bf16x2(o2[0], o2[1]), pack_bf16x2(o2[2], o2[3]),
                                    pack_bf16x2(o2[4], o2[5]), pack_bf16x2(o2[6], o2[7])});
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): row reads done before the next pass writes
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    }
}

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_context_kv_workspace_size(int64_t num_ctx, int64_t Hd) {
    if (num_ctx < 1 || Hd < 1) return 0;
    return (size_t)num_ctx * (size_t)Hd * 2u;
}

extern "C" int dflash_context_kv(const uint16_t* ctx_states, const uint16_t* hidden_norm_w, float hidden_eps,
                                 const uint16_t* W_kv, int64_t num_ctx, int64_t Hd, int32_t L, int32_t Hkv,
                                 int32_t D, const uint16_t* k_norm_w, float k_eps, const int64_t* positions,
                                 const float* cos_sin, int64_t max_pos, const int64_t* slots,
                                 uint16_t* const* caches, int64_t num_blocks, int32_t block_size,
                                 uint16_t* kv_out, void* ws, size_t ws_bytes, void* stream) {
    const void* req[] = {ctx_states, hidden_norm_w, W_kv, k_norm_w, positions, cos_sin, ws};
    for (const void* p : req)
        if (!p || !DFLASH_ALIGNED16(p)) return DFLASH_ERR_INVALID_ARG;
    if ((slots == nullptr) != (caches == nullptr)) return DFLASH_ERR_INVALID_ARG;
    if (kv_out && !DFLASH_ALIGNED16(kv_out)) return DFLASH_ERR_INVALID_ARG;
    if (num_ctx < 1 || Hd < 1 || L < 1 || Hkv < 1 || max_pos < 1) return DFLASH_ERR_INVALID_ARG;
    if (!(hidden_eps >= 0.f) || !(k_eps >= 0.f)) return DFLASH_ERR_INVALID_ARG;
    CtxCaches cp{};
    if (caches) {
        if (num_blocks < 1 || block_size < 1 || L > CKV_MAX_LAYERS) return L > CKV_MAX_LAYERS ? DFLASH_ERR_UNSUPPORTED
                                                                                             : DFLASH_ERR_INVALID_ARG;
        for (int l = 0; l < L; ++l) {
            if (!caches[l] || !DFLASH_ALIGNED16(caches[l])) return DFLASH_ERR_INVALID_ARG;
            cp.p[l] = caches[l];
        }
    }
    if (D != CKV_D || Hd % 8 != 0 || L > CKV_MAX_LAYERS) return DFLASH_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)L * 2 * Hkv * D;
    if (num_ctx > INT32_MAX || N > INT32_MAX || Hd > (int64_t)1 << 20) return DFLASH_ERR_UNSUPPORTED;
    if ((int64_t)256 * Hd * 2 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    if (ws_bytes < dflash_context_kv_workspace_size(num_ctx, Hd)) return DFLASH_ERR_WORKSPACE;
    // Tile width: 256 columns (two heads) or 128 (one head), whichever needs
    // fewer tile-rounds of the device's compute units, weighting a round by
    // the tile's width (one 256 x BN tile per CU at a time).
    const int nM = (int)((num_ctx + CKV_BM - 1) / CKV_BM);
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ncu = v;
    }
    auto cost = [&](int64_t bn) { return ((nM * (N / bn) + ncu - 1) / ncu) * bn; };
    const int BN = cost(128) < cost(256) ? 128 : 256;
    const int64_t ntiles = (int64_t)nM * (N / BN);
    if (ntiles > (int64_t)1 << 28) return DFLASH_ERR_UNSUPPORTED;
    const int per = (int)((ntiles + 7) / 8);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint16_t* normed = reinterpret_cast<uint16_t*>(ws);
    hipLaunchKernelGGL(ctx_hidden_norm_kernel, dim3((unsigned)num_ctx), dim3(256), 0, st, ctx_states, hidden_norm_w,
                       (int)Hd, hidden_eps, normed);
    const dim3 grid((unsigned)(8 * per));
#define CKV_LAUNCH(BNV, TL)                                                                                         \
    hipLaunchKernelGGL((ctx_kv_tiles<BNV, TL>), grid, dim3(CKV_THREADS), 0, st, normed, W_kv, (int)num_ctx, (int)Hd, \
                       (int)N, nM, (int)ntiles, (int)Hkv, k_norm_w, k_eps, positions, cos_sin, max_pos, slots, cp,    \
                       num_blocks, (int)block_size, kv_out)
    const bool tail = Hd % CKV_BK != 0;
    if (BN == 256) {
        if (tail) CKV_LAUNCH(256, true);
        else CKV_LAUNCH(256, false);
    } else {
        if (tail) CKV_LAUNCH(128, true);
        else CKV_LAUNCH(128, false);
    }
#undef CKV_LAUNCH
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

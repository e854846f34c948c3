// Context K/V precompute of the DFlash2 drafter for every draft layer at once
// (DFlash2BeamModel.build_context_kv_weights / precompute_and_store_context_kv
// and the store_context_kv op it calls): hidden_norm RMSNorm of the context
// states, one linear against the stacked K/V rows of every layer's qkv_proj,
// then per layer the K-norm and NeoX RoPE of K and the slot-mapped write of K
// and V into that layer's paged cache.
//
//   * ctx_hidden_norm: one workgroup per context row, the row held in
//     registers; the sum of squares is reduced across the workgroup and the
//     normed row written once as bf16 (the norm's output dtype) into the
//     workspace.
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
#include "fp8.h"
#include "gemm_tile.h"

namespace dflash {

constexpr int CKV_D = 128;
constexpr int CKV_MAX_LAYERS = 64;

// Per-layer cache base pointers, passed by value (512 bytes of kernel
// arguments): no device-side pointer table to build or keep in sync.
struct CtxCaches {
    uint16_t* p[CKV_MAX_LAYERS];
};

// ---------------------------------------------------------------------------
// hidden_norm: normed[t, :] = bf16(x[t, :] * (mean(x[t, :]^2) + eps)^-1/2 * w)
// One workgroup per row.  With CPT > 0 a thread holds its (up to CPT) 16-byte
// chunks of the row in registers between the reduction and the output, all
// loads issued up front; CPT = 0 is the general loop (rows past 8192).
// ---------------------------------------------------------------------------
template <int CPT>
__global__ __launch_bounds__(256) void ctx_hidden_norm_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w, int Hd, float eps,
                                                              uint16_t* __restrict__ out) {
    __shared__ float red[4];
    const int64_t t = blockIdx.x;
    const uint16_t* row = x + t * Hd;
    uint16_t* orow = out + t * Hd;
    const int nch = Hd >> 3;  // 16-byte chunks
    float ss = 0.f;
    u32x4 xv[CPT > 0 ? CPT : 1];
    if (CPT > 0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = threadIdx.x + 256 * i;
            xv[i] = c < nch ? ldg16(row + c * 8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            float v[8];
            unpack8(xv[i], v);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        }
    } else {
        for (int c = threadIdx.x; c < nch; c += 256) {
            float v[8];
            unpack8(ldg16(row + c * 8), v);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    const float rinv = 1.0f / sqrtf(ss / (float)Hd + eps);
    auto put = [&](int c, const u32x4 raw) {
        float v[8], wv[8];
        unpack8(raw, v);
        unpack8(ldg16(w + c * 8), wv);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack_bf16x2(v[2 * e] * rinv * wv[2 * e], v[2 * e + 1] * rinv * wv[2 * e + 1]);
        stg16(orow + c * 8, o);
    };
    if (CPT > 0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = threadIdx.x + 256 * i;
            if (c < nch) put(c, xv[i]);
        }
    } else {
        for (int c = threadIdx.x; c < nch; c += 256) put(c, ldg16(row + c * 8));
    }
}

// ---------------------------------------------------------------------------
// The stacked K/V linear with the K-norm / RoPE / cache-write epilogue.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_round(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }

// 8 / 4 consecutive entries of the RoPE table (fp32 or bf16) from element idx
__device__ __forceinline__ void rope_table8(const void* t, bool bf, int64_t idx, float (&v)[8]) {
    if (bf) {
        unpack8(ldg16(reinterpret_cast<const uint16_t*>(t) + idx), v);
    } else {
        const float* f = reinterpret_cast<const float*>(t) + idx;
        const f32x4 a = *reinterpret_cast<const f32x4*>(f);
        const f32x4 b = *reinterpret_cast<const f32x4*>(f + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
    }
}
__device__ __forceinline__ void rope_table4(const void* t, bool bf, int64_t idx, float (&v)[4]) {
    if (bf) {
        const u32x2 a = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(t) + idx);
        v[0] = __uint_as_float(a[0] << 16); v[1] = __uint_as_float(a[0] & 0xffff0000u);
        v[2] = __uint_as_float(a[1] << 16); v[3] = __uint_as_float(a[1] & 0xffff0000u);
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(t) + idx);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a[e];
    }
}

template <int BN, bool TAIL>
__global__ __launch_bounds__(GT_THREADS, 1) void ctx_kv_tiles(
    const uint16_t* __restrict__ A /*normed [n, Hd]*/, const uint16_t* __restrict__ W /*[N, Hd]*/, int n, int Hd,
    int N, int nM, int ntiles, int Hkv, const uint16_t* __restrict__ k_w /*[L, D]*/, float eps,
    const int64_t* __restrict__ positions, const void* __restrict__ cos_sin, int rot, bool neox, bool tab_bf16,
    int64_t max_pos, const int64_t* __restrict__ slots, CtxCaches caches, int64_t num_blocks, int block_size,
    uint16_t* __restrict__ kv_out, int fp8, const float* __restrict__ kv_scales) {
    constexpr int SP = GT_SP;                // row pitch (floats) of the epilogue staging (one head)
    constexpr int NPASS = BN / CKV_D;        // heads per tile = epilogue passes
    static_assert(BN % CKV_D == 0, "tiles hold whole heads");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[GT_SMEM];
    float* stage = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x;
    int m_tile, n_tile;
    if (!gemm_tile_index(ntiles, nM, m_tile, n_tile)) return;
    const int m0 = m_tile * GT_BM;
    const int n0 = n_tile * BN;
    const int my_row = m0 + tid;

    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + (int64_t)m0 * Hd), (short)0, min(GT_BM, n - m0) * Hd * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (int64_t)n0 * Hd), (short)0, BN * Hd * 2, 0x00020000);
    f32x16 acc[4][BN / 64];
    gemm_tile_mainloop<BN, TAIL>(smem, rsA, rsB, Hd, acc);

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

    // One pass per head of the tile: the head's 128 columns are staged
    // row-major, then thread t finishes row t.
    for (int pass = 0; pass < NPASS; ++pass) {
        gemm_tile_stage<BN>(stage, acc, pass);
        if (my_row < n) {
            // head (layer l, K or V, kv head h) of these 128 columns
            const int gh = n0 / CKV_D + pass;
            const int l = gh / (2 * Hkv);
            const int r = gh - l * 2 * Hkv;
            const bool is_v = r >= Hkv;
            const int h = is_v ? r - Hkv : r;
            const float* rowp = stage + tid * SP;
            uint16_t* kvo = kv_out != nullptr ? kv_out + (int64_t)my_row * N + gh * CKV_D : nullptr;
            // the row's place in the layer's cache: bf16 elements, or fp8 bytes
            // (the same element offsets) when the cache is fp8
            uint16_t* dst = nullptr;
            uint8_t* dst8 = nullptr;
            if (cache_row >= 0) {
                const int64_t off = cache_row + h * head_stride + (is_v ? CKV_D : 0);
                if (fp8 == FP8_NONE) dst = caches.p[l] + off;
                else dst8 = reinterpret_cast<uint8_t*>(caches.p[l]) + off;
            }
            const float qscale = fp8 == FP8_NONE ? 1.f : kv_scales[2 * l + (is_v ? 1 : 0)];
            // 8 values (already bf16 numbers) at column col of the fp8 row
            auto put8_fp8 = [&](int col, const float (&o)[8]) {
                float ob[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) ob[e] = bf16_round(o[e]);
                const u32x2 w = fp8 == FP8_E4M3 ? pack_fp8x8<FP8_E4M3>(ob, qscale) : pack_fp8x8<FP8_E5M2>(ob, qscale);
                *reinterpret_cast<u32x2*>(dst8 + col) = w;
            };
            if (is_v) {
#pragma unroll 4
                for (int c = 0; c < CKV_D / 8; ++c) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(rowp + 8 * c);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(rowp + 8 * c + 4);
                    const u32x4 o = {pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                                     pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
                    if (kvo) stg16(kvo + 8 * c, o);
                    if (dst) stg16(dst + 8 * c, o);
                    if (dst8) {
                        const float ov[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                        put8_fp8(8 * c, ov);
                    }
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
                if (kvo) {  // the row before the norm
#pragma unroll 4
                    for (int c = 0; c < CKV_D / 8; ++c) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(rowp + 8 * c);
                        const f32x4 b = *reinterpret_cast<const f32x4*>(rowp + 8 * c + 4);
                        stg16(kvo + 8 * c, u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                 pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
                    }
                }
                // normed values of columns col .. col + 7
                auto normed8 = [&](int col, float (&y)[8]) {
                    float w[8];
                    unpack8(ldg16(wl + col), w);
#pragma unroll
                    for (int hq = 0; hq < 2; ++hq) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(rowp + col + 4 * hq);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[4 * hq + e] = bf16_round(a[e]) * rinv * w[4 * hq + e];
                    }
                };
                auto put8 = [&](int col, const float (&o)[8]) {
                    if (dst)
                        stg16(dst + col, u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                               pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])});
                    if (dst8) put8_fp8(col, o);
                };
                const int half = rot >> 1;
                const int64_t trow = pos * rot;  // the position's table row: cos(0 .. half), sin(0 .. half)
                if (neox) {
                    // pairs (i, i + rot/2): columns 8c.. and rot/2 + 8c.. together
                    for (int c = 0; c < half / 8; ++c) {
                        float y1[8], y2[8], cv[8], sv[8], o1[8], o2[8];
                        normed8(8 * c, y1);
                        normed8(half + 8 * c, y2);
                        rope_table8(cos_sin, tab_bf16, trow + 8 * c, cv);
                        rope_table8(cos_sin, tab_bf16, trow + half + 8 * c, sv);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            o1[e] = y1[e] * cv[e] - y2[e] * sv[e];
                            o2[e] = y2[e] * cv[e] + y1[e] * sv[e];
                        }
                        put8(8 * c, o1);
                        put8(half + 8 * c, o2);
                    }
                } else {
                    // pairs (2i, 2i + 1): columns 8c.. hold pairs 4c .. 4c + 3
                    for (int c = 0; c < rot / 8; ++c) {
                        float y[8], c4[4], s4[4], o[8];
                        normed8(8 * c, y);
                        rope_table4(cos_sin, tab_bf16, trow + 4 * c, c4);
                        rope_table4(cos_sin, tab_bf16, trow + half + 4 * c, s4);
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            o[2 * m] = y[2 * m] * c4[m] - y[2 * m + 1] * s4[m];
                            o[2 * m + 1] = y[2 * m + 1] * c4[m] + y[2 * m] * s4[m];
                        }
                        put8(8 * c, o);
                    }
                }
                // columns past the rotary dim: the norm alone
                for (int c = rot / 8; c < CKV_D / 8; ++c) {
                    float y[8];
                    normed8(8 * c, y);
                    put8(8 * c, y);
                }
            }
        }
        gemm_tile_pass_done();
    }
}

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_context_kv_workspace_size(int64_t num_ctx, int64_t Hd) {
    if (num_ctx < 1 || Hd < 1) return 0;
    return (size_t)num_ctx * (size_t)Hd * 2u;
}

extern "C" int dflash_context_kv_ex(const uint16_t* ctx_states, const uint16_t* hidden_norm_w, float hidden_eps,
                                    const uint16_t* W_kv, int64_t num_ctx, int64_t Hd, int32_t L, int32_t Hkv,
                                    int32_t D, const uint16_t* k_norm_w, float k_eps, const int64_t* positions,
                                    const void* cos_sin, int64_t max_pos, int32_t rotary_dim, int32_t is_neox,
                                    int32_t table_bf16, const int64_t* slots, uint16_t* const* caches,
                                    int64_t num_blocks, int32_t block_size, int32_t cache_fp8,
                                    const float* kv_scales, uint16_t* kv_out, void* ws, size_t ws_bytes,
                                    void* stream) {
    const void* req[] = {ctx_states, hidden_norm_w, W_kv, k_norm_w, positions, cos_sin, ws};
    for (const void* p : req)
        if (!p || !DFLASH_ALIGNED16(p)) return DFLASH_ERR_INVALID_ARG;
    if ((slots == nullptr) != (caches == nullptr)) return DFLASH_ERR_INVALID_ARG;
    if (kv_out && !DFLASH_ALIGNED16(kv_out)) return DFLASH_ERR_INVALID_ARG;
    if (num_ctx < 1 || Hd < 1 || L < 1 || Hkv < 1 || max_pos < 1) return DFLASH_ERR_INVALID_ARG;
    if (!(hidden_eps >= 0.f) || !(k_eps >= 0.f)) return DFLASH_ERR_INVALID_ARG;
    if ((table_bf16 != 0 && table_bf16 != 1) || (is_neox != 0 && is_neox != 1)) return DFLASH_ERR_INVALID_ARG;
    if (rotary_dim < 2 || rotary_dim > D || (rotary_dim & 1)) return DFLASH_ERR_INVALID_ARG;
    if (rotary_dim % (is_neox ? 16 : 8) != 0) return DFLASH_ERR_UNSUPPORTED;
    if (cache_fp8 < FP8_NONE || cache_fp8 > FP8_E5M2) return DFLASH_ERR_INVALID_ARG;
    if (cache_fp8 != FP8_NONE && (!caches || !kv_scales || !DFLASH_ALIGNED16(kv_scales))) return DFLASH_ERR_INVALID_ARG;
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
    // fewer tile-rounds of the device's compute units.
    const int nM = (int)((num_ctx + GT_BM - 1) / GT_BM);
    const int BN = gemm_tile_width(num_ctx, N);
    const int64_t ntiles = (int64_t)nM * (N / BN);
    if (ntiles > (int64_t)1 << 28) return DFLASH_ERR_UNSUPPORTED;
    const int per = (int)((ntiles + 7) / 8);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint16_t* normed = reinterpret_cast<uint16_t*>(ws);
    {
        const int nch = (int)(Hd / 8);
        const dim3 g((unsigned)num_ctx), b(256);
        if (nch <= 256)
            hipLaunchKernelGGL(ctx_hidden_norm_kernel<1>, g, b, 0, st, ctx_states, hidden_norm_w, (int)Hd, hidden_eps, normed);
        else if (nch <= 512)
            hipLaunchKernelGGL(ctx_hidden_norm_kernel<2>, g, b, 0, st, ctx_states, hidden_norm_w, (int)Hd, hidden_eps, normed);
        else if (nch <= 1024)
            hipLaunchKernelGGL(ctx_hidden_norm_kernel<4>, g, b, 0, st, ctx_states, hidden_norm_w, (int)Hd, hidden_eps, normed);
        else
            hipLaunchKernelGGL(ctx_hidden_norm_kernel<0>, g, b, 0, st, ctx_states, hidden_norm_w, (int)Hd, hidden_eps, normed);
    }
    const dim3 grid((unsigned)(8 * per));
#define CKV_LAUNCH(BNV, TL)                                                                                         \
    hipLaunchKernelGGL((ctx_kv_tiles<BNV, TL>), grid, dim3(GT_THREADS), 0, st, normed, W_kv, (int)num_ctx, (int)Hd, \
                       (int)N, nM, (int)ntiles, (int)Hkv, k_norm_w, k_eps, positions, cos_sin, (int)rotary_dim,       \
                       is_neox != 0, table_bf16 != 0, max_pos, slots, cp,                                              \
                       num_blocks, (int)block_size, kv_out, (int)cache_fp8, kv_scales)
    const bool tail = Hd % GT_BK != 0;
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

extern "C" int dflash_context_kv(const uint16_t* ctx_states, const uint16_t* hidden_norm_w, float hidden_eps,
                                 const uint16_t* W_kv, int64_t num_ctx, int64_t Hd, int32_t L, int32_t Hkv,
                                 int32_t D, const uint16_t* k_norm_w, float k_eps, const int64_t* positions,
                                 const float* cos_sin, int64_t max_pos, const int64_t* slots,
                                 uint16_t* const* caches, int64_t num_blocks, int32_t block_size,
                                 uint16_t* kv_out, void* ws, size_t ws_bytes, void* stream) {
    return dflash_context_kv_ex(ctx_states, hidden_norm_w, hidden_eps, W_kv, num_ctx, Hd, L, Hkv, D, k_norm_w, k_eps,
                                positions, cos_sin, max_pos, D, 1, 0, slots, caches, num_blocks, block_size,
                                FP8_NONE, nullptr, kv_out, ws, ws_bytes, stream);
}

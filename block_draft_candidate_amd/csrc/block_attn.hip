// Non-causal sliding-window attention of the draft's query block over the paged
// K/V cache (DFlash2BeamAttention: every layer is non-causal sliding-window
// attention over the block, scale head_dim ** -0.5, grouped K/V heads; the
// context K/V is already in the cache, the block's own K/V is written by the
// fused norm/RoPE kernel first).
//
// One workgroup per (request, kv head); wave w handles q head kv * G + w, i.e.
// the G heads that share the kv head read each K/V tile once from HBM.  A wave's
// 16 MFMA columns are the block's (up to 16) queries.
//   S^T = K Q^T   : v_mfma_f32_16x16x32_bf16, K rows from LDS, Q^T from registers;
//                   every lane then holds scores of a single query, so the online
//                   softmax (fp32, exp2) needs only two cross-lane steps.
//   O^T += V^T P^T: P^T comes straight from the S^T registers (bf16), V^T from an
//                   LDS tile stored transposed.
// K/V tiles of 64 keys (4 cache blocks of 16) are double-buffered in LDS with a
// register prefetch of the next tile.
#include "common.h"

namespace dflash {

constexpr int AT_D = 128;
constexpr int AT_BS = 16;      // cache block size
constexpr int AT_TK = 64;      // keys per tile
constexpr int AT_VP = 72;      // V^T row pitch (elements): conflict-free 8-byte reads

template <int G>
__global__ __launch_bounds__(64 * G) void block_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ cache, int64_t num_blocks,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ seq_lens, int Lq,
    int Hq, int Hkv, int window, float scale_log2, uint16_t* __restrict__ out) {
    constexpr int NT = 64 * G;
    constexpr int CHUNKS = (AT_TK * 2 * AT_D * 2 / 16) / NT;  // 16-byte chunks per thread per tile
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][AT_TK * AT_D];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][AT_D * AT_VP];

    const int r = blockIdx.x / Hkv;
    const int hk = blockIdx.x - r * Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hq = hk * G + wave;
    const int qi = lane & 15, g = lane >> 4;

    int L = seq_lens[r];
    L = L < 0 ? 0 : (L > max_blocks * AT_BS ? max_blocks * AT_BS : L);
    const bool qvalid = qi < Lq && L >= Lq;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    bf16x8 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        qf[s] = as_bf16x8(qvalid ? ldg16(q + (((int64_t)r * Lq + qi) * Hq + hq) * AT_D + 32 * s + 8 * g) : zero4);

    const int lo0 = max(0, L - Lq - window + 1);
    const int kstart = (lo0 / AT_BS) * AT_BS;
    const int ntiles = L > kstart ? (L - kstart + AT_TK - 1) / AT_TK : 0;
    const int qlo = L - Lq + qi - window + 1;  // lowest visible key of this lane's query
    const int32_t* bt = block_tables + (int64_t)r * max_blocks;

    u32x4 regs[CHUNKS];
    auto gload = [&](int tile) {
        const int kb = kstart + tile * AT_TK;
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = tid + NT * i;
            const int jb = c >> 9, wo = c & 511;  // cache block within the tile, 16-byte chunk within it
            const int row = wo >> 5, cc = wo & 31;
            const int key0 = kb + jb * AT_BS;
            if (key0 < L) {
                int b = bt[key0 / AT_BS];
                b = b < 0 ? 0 : (b >= num_blocks ? (int)(num_blocks - 1) : b);
                regs[i] = ldg16(cache + (((int64_t)b * Hkv + hk) * AT_BS + row) * (2 * AT_D) + cc * 8);
            } else {
                regs[i] = zero4;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = tid + NT * i;
            const int jb = c >> 9, wo = c & 511;
            const int row = wo >> 5, cc = wo & 31;
            const int key = jb * AT_BS + row;
            if (cc < 16) {
                *reinterpret_cast<u32x4*>(&sK[buf][key * AT_D + ((cc ^ (key & 7)) << 3)]) = regs[i];
            } else {
                const int d0 = (cc - 16) * 8;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sV[buf][(d0 + 2 * e) * AT_VP + key] = (uint16_t)(regs[i][e] & 0xffffu);
                    sV[buf][(d0 + 2 * e + 1) * AT_VP + key] = (uint16_t)(regs[i][e] >> 16);
                }
            }
        }
    };

    float m = -INFINITY, lsum = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (ntiles > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < ntiles) gload(tile + 1);
        const int kb = kstart + tile * AT_TK;

        // S^T = K Q^T for 4 blocks of 16 keys
        float sv[4][4];
        float mt = -INFINITY;
#pragma unroll
        for (int kblk = 0; kblk < 4; ++kblk) {
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
            const int key = kblk * 16 + qi;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ch = 4 * s + g;
                const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(&sK[buf][key * AT_D + ((ch ^ (key & 7)) << 3)]));
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], st, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kp = kb + kblk * 16 + 4 * g + e;
                const bool vis = qvalid && kp < L && kp >= qlo;
                sv[kblk][e] = vis ? st[e] * scale_log2 : -INFINITY;
                mt = fmaxf(mt, sv[kblk][e]);
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mnew = fmaxf(m, mt);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2f(m - muse);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
        float pv[4][4];
#pragma unroll
        for (int kblk = 0; kblk < 4; ++kblk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[kblk][e] = exp2f(sv[kblk][e] - muse);
                lsum += pv[kblk][e];
            }

        // O^T += V^T P^T over two 32-key steps
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            u32x4 pp;
            pp[0] = pack_bf16x2(pv[2 * s2][0], pv[2 * s2][1]);
            pp[1] = pack_bf16x2(pv[2 * s2][2], pv[2 * s2][3]);
            pp[2] = pack_bf16x2(pv[2 * s2 + 1][0], pv[2 * s2 + 1][1]);
            pp[3] = pack_bf16x2(pv[2 * s2 + 1][2], pv[2 * s2 + 1][3]);
            const bf16x8 pf = as_bf16x8(pp);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const int d = mb * 16 + qi;
                const uint16_t* vrow = &sV[buf][d * AT_VP + 32 * s2 + 4 * g];
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
                const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
                o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vv), pf, o[mb], 0, 0, 0);
            }
        }

        if (tile + 1 < ntiles) sstore(buf ^ 1);
        __syncthreads();
    }

    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    if (qi < Lq) {
        uint16_t* dst = out + (((int64_t)r * Lq + qi) * Hq + hq) * AT_D;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            u32x2 w;
            w[0] = pack_bf16x2(o[mb][0] * inv, o[mb][1] * inv);
            w[1] = pack_bf16x2(o[mb][2] * inv, o[mb][3] * inv);
            *reinterpret_cast<u32x2*>(dst + mb * 16 + 4 * g) = w;
        }
    }
}

template <int G>
static void launch_attn(const uint16_t* q, const uint16_t* cache, int64_t nblk, const int32_t* bt, int maxb,
                        const int32_t* seq, int64_t Rq, int Lq, int Hq, int Hkv, int window, float scale,
                        uint16_t* out, hipStream_t st) {
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((block_attn_kernel<G>), dim3((unsigned)(Rq * Hkv)), dim3(64 * G), 0, st, q, cache, nblk,
                       bt, maxb, seq, Lq, Hq, Hkv, window, scale_log2, out);
}

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_block_attn_workspace_size(int64_t Rq, int32_t Lq, int32_t Hq, int32_t D) {
    (void)Rq; (void)Lq; (void)Hq; (void)D;
    return 0;
}

extern "C" int dflash_block_attn(const uint16_t* q, const uint16_t* kv_cache, int64_t num_blocks,
                                 const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                 int64_t Rq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                 int32_t window, float scale, uint16_t* out, void* ws, size_t ws_bytes,
                                 void* stream) {
    (void)ws; (void)ws_bytes;
    const void* req[] = {q, kv_cache, block_tables, seq_lens, out};
    for (const void* p : req)
        if (!p || !DFLASH_ALIGNED16(p)) return DFLASH_ERR_INVALID_ARG;
    if (num_blocks < 1 || max_blocks < 1 || Rq < 1 || Lq < 1 || Hq < 1 || Hkv < 1 || window < 1 ||
        !(scale > 0.f) || !(scale < INFINITY))
        return DFLASH_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return DFLASH_ERR_INVALID_ARG;
    if (D != AT_D || block_size != AT_BS || Lq > 16) return DFLASH_ERR_UNSUPPORTED;
    if (Rq * Hkv > INT32_MAX || (int64_t)max_blocks * AT_BS > INT32_MAX || num_blocks > INT32_MAX)
        return DFLASH_ERR_UNSUPPORTED;
    const int G = Hq / Hkv;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (G) {
        case 1: launch_attn<1>(q, kv_cache, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, st); break;
        case 2: launch_attn<2>(q, kv_cache, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, st); break;
        case 4: launch_attn<4>(q, kv_cache, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, st); break;
        case 8: launch_attn<8>(q, kv_cache, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, st); break;
        default: return DFLASH_ERR_UNSUPPORTED;
    }
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

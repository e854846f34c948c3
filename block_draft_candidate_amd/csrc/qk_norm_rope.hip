// Draft-layer q/k RMSNorm + NeoX RoPE + slot-mapped K/V cache write, one pass
// (DFlash2BeamAttention.forward calls beam_qk_norm_rope with q_norm/k_norm
// weights, the rope's cos/sin cache and, when the cache is bf16, the layer's
// kv cache and slot mapping).
//
// One workgroup per token.  Sixteen lanes own one head (head_dim 128 = 16
// lanes x 8 bf16, one 16-byte load and store per lane); the 16 groups of a
// 256-thread workgroup take heads g, g + 16, ...  The token's position, slot,
// RoPE row and every head's data are loaded up front, so a workgroup pays one
// memory round trip (plus the position -> RoPE row step).  The sum of squares is
// reduced inside the 16-lane group, and the RoPE partner (i <-> i + 64) of a
// lane's 8 elements lives in lane ^ 8 of the same group.  V heads are copied to
// the cache bit for bit.
#include "fp8.h"

namespace dflash {

constexpr int QK_D = 128;
constexpr int QK_HPG = 3;  // heads per 16-lane group handled per round (48 heads: all)

// RoPE coefficients of a lane's 8 consecutive head elements [8j, 8j + 8)
// (j = lane within the head's 16-lane group), so that the rotated element is
// o[e] = y[e] * cv[e] + partner[e] * sv[e]:
//   NeoX pairs (i, i + rot/2): partner = the same element of lane src
//     (j + rot/16 in the first half, j - rot/16 in the second), sin negated in
//     the first half;
//   GPT-J pairs (2i, 2i + 1): partner = y[e ^ 1] of the same lane, sin
//     negated on even elements.
// Lanes past the rotary dim get cv = 1, sv = 0 (and src = j).  The table row
// of the position is [cos(0 .. rot/2), sin(0 .. rot/2)], fp32 or bf16.
template <bool NEOX, bool TBF16>
__device__ __forceinline__ void lane_rope_coeffs(const void* table, int64_t pos, int rot, int j,
                                                 float (&cv)[8], float (&sv)[8], int& src) {
    const int half = rot >> 1;
    src = j;
#pragma unroll
    for (int e = 0; e < 8; ++e) { cv[e] = 1.f; sv[e] = 0.f; }
    if (8 * j >= rot) return;
    const int64_t rowoff = pos * rot;
    float c[8], sn[8];
    if (NEOX) {
        const bool first = 8 * j < half;
        const int ib = first ? 8 * j : 8 * j - half;
        src = first ? j + (rot >> 4) : j - (rot >> 4);
        if (TBF16) {
            const uint16_t* tb = reinterpret_cast<const uint16_t*>(table) + rowoff;
            unpack8(ldg16(tb + ib), c);
            unpack8(ldg16(tb + half + ib), sn);
        } else {
            const float* tf = reinterpret_cast<const float*>(table) + rowoff;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(tf + ib + 4 * h);
                const f32x4 b = *reinterpret_cast<const f32x4*>(tf + half + ib + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) { c[4 * h + e] = a[e]; sn[4 * h + e] = b[e]; }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { cv[e] = c[e]; sv[e] = first ? -sn[e] : sn[e]; }
    } else {
        const int ib = 4 * j;
        float c4[4], s4[4];
        if (TBF16) {
            const uint16_t* tb = reinterpret_cast<const uint16_t*>(table) + rowoff;
            const u32x2 a = *reinterpret_cast<const u32x2*>(tb + ib);
            const u32x2 b = *reinterpret_cast<const u32x2*>(tb + half + ib);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                c4[2 * e] = __uint_as_float(a[e] << 16); c4[2 * e + 1] = __uint_as_float(a[e] & 0xffff0000u);
                s4[2 * e] = __uint_as_float(b[e] << 16); s4[2 * e + 1] = __uint_as_float(b[e] & 0xffff0000u);
            }
        } else {
            const float* tf = reinterpret_cast<const float*>(table) + rowoff;
            const f32x4 a = *reinterpret_cast<const f32x4*>(tf + ib);
            const f32x4 b = *reinterpret_cast<const f32x4*>(tf + half + ib);
#pragma unroll
            for (int e = 0; e < 4; ++e) { c4[e] = a[e]; s4[e] = b[e]; }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { cv[e] = c4[e >> 1]; sv[e] = (e & 1) ? s4[e >> 1] : -s4[e >> 1]; }
    }
}

template <bool NEOX, bool TBF16, int FP8>
__global__ __launch_bounds__(256) void qk_norm_rope_cache_kernel(
    const uint16_t* __restrict__ qkv, int64_t row_stride, int Hq, int Hkv,
    const uint16_t* __restrict__ q_w, const uint16_t* __restrict__ k_w, float eps,
    const int64_t* __restrict__ positions, const void* __restrict__ cos_sin, int rot,
    int64_t max_pos, const int64_t* __restrict__ slots, uint16_t* __restrict__ cache, int64_t num_blocks,
    int block_size, uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_out,
    const float* __restrict__ kv_scale) {
    const int NH = Hq + 2 * Hkv;
    const int64_t t = blockIdx.x;
    const int grp = threadIdx.x >> 4;
    const int j = threadIdx.x & 15;
    const uint16_t* row = qkv + t * row_stride + j * 8;

    int64_t pos = positions[t];
    pos = pos < 0 ? 0 : (pos >= max_pos ? max_pos - 1 : pos);
    int64_t cache_base = -1;  // element offset of [blk, 0, off, 0] in the cache
    if (cache != nullptr) {
        const int64_t s = slots[t];
        if (s >= 0 && s < num_blocks * block_size) {
            const int64_t blk = s / block_size, off = s - blk * block_size;
            cache_base = (blk * Hkv * block_size + off) * (2 * QK_D);
        }
    }
    const int64_t head_stride = (int64_t)block_size * 2 * QK_D;  // next kv head of the same block
    // norm weights kept packed (8 bf16 in 4 registers each), widened on use
    const u32x4 qw_raw = ldg16(q_w + j * 8);
    const u32x4 kw_raw = ldg16(k_w + j * 8);
    float cv[8], sv[8];
    int src;
    lane_rope_coeffs<NEOX, TBF16>(cos_sin, pos, rot, j, cv, sv, src);

    for (int h0 = grp; h0 < NH; h0 += 16 * QK_HPG) {
        u32x4 raw[QK_HPG];
#pragma unroll
        for (int i = 0; i < QK_HPG; ++i) {
            const int h = h0 + 16 * i;
            raw[i] = h < NH ? ldg16(row + (int64_t)h * QK_D) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < QK_HPG; ++i) {
            const int h = h0 + 16 * i;
            if (h >= NH) break;  // uniform within the 16-lane group
            if (h >= Hq + Hkv) {  // v head: copied as is (an fp8 cache: quantised)
                if (cache_base >= 0) {
                    const int64_t off = cache_base + (h - Hq - Hkv) * head_stride + QK_D + j * 8;
                    if (FP8 == FP8_NONE) {
                        stg16(cache + off, raw[i]);
                    } else {
                        float v[8];
                        unpack8(raw[i], v);
                        *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(cache) + off) =
                            pack_fp8x8<FP8>(v, kv_scale[1]);
                    }
                }
                continue;
            }
            float x[8];
            unpack8(raw[i], x);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off, 16);
            const float rinv = 1.0f / sqrtf(ss * (1.0f / QK_D) + eps);
            const bool is_q = h < Hq;
            float wv[8];
            unpack8(is_q ? qw_raw : kw_raw, wv);
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = x[e] * rinv * wv[e];
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // x1 cos - x2 sin for the first element of a pair, x2 cos + x1 sin for the second
                const float partner = NEOX ? __shfl(y[e], src, 16) : y[e ^ 1];
                o[e] = y[e] * cv[e] + partner * sv[e];
            }
            u32x4 packed;
#pragma unroll
            for (int e = 0; e < 4; ++e) packed[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
            if (is_q) {
                stg16(q_out + (t * Hq + h) * QK_D + j * 8, packed);
            } else {
                const int hk = h - Hq;
                if (k_out != nullptr) stg16(k_out + (t * Hkv + hk) * QK_D + j * 8, packed);
                if (cache_base >= 0) {
                    const int64_t off = cache_base + hk * head_stride + j * 8;
                    if (FP8 == FP8_NONE) {
                        stg16(cache + off, packed);
                    } else {  // the bf16 key, quantised
                        float kb[8];
                        unpack8(packed, kb);
                        *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(cache) + off) =
                            pack_fp8x8<FP8>(kb, kv_scale[0]);
                    }
                }
            }
        }
    }
}

// cos_sin[p, i] = cos(p * theta^(-2i/D)), cos_sin[p, D/2 + i] = sin(...), in
// fp64, rounded once to the table's type (fp32 or bf16).
__device__ __forceinline__ void store_table(float* p, double v) { *p = (float)v; }
__device__ __forceinline__ void store_table(uint16_t* p, double v) {
    // fp64 -> fp32 -> bf16, each step round to nearest even
    *p = (uint16_t)f32_to_bf16_bits((float)v);
}
template <typename TT>
__global__ void rope_cos_sin_kernel(TT* __restrict__ out, int64_t max_pos, int D, double theta) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int half = D / 2;
    if (idx >= max_pos * half) return;
    const int64_t p = idx / half;
    const int i = (int)(idx - p * half);
    const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
    const double ang = (double)p * inv_freq;
    store_table(out + p * D + i, cos(ang));
    store_table(out + p * D + half + i, sin(ang));
}

}  // namespace dflash

using namespace dflash;

template <typename TT>
static int rope_table(TT* cos_sin, int64_t max_pos, int32_t D, double theta, void* stream) {
    if (!cos_sin || max_pos < 1 || D < 2 || (D & 1) || !(theta > 0.0)) return DFLASH_ERR_INVALID_ARG;
    if (max_pos > ((int64_t)1 << 40) / D) return DFLASH_ERR_UNSUPPORTED;
    const int64_t n = max_pos * (D / 2);
    hipLaunchKernelGGL(rope_cos_sin_kernel<TT>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), cos_sin, max_pos, (int)D, theta);
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

extern "C" int dflash_rope_cos_sin(float* cos_sin, int64_t max_pos, int32_t D, double theta, void* stream) {
    return rope_table(cos_sin, max_pos, D, theta, stream);
}

extern "C" int dflash_rope_cos_sin_bf16(uint16_t* cos_sin, int64_t max_pos, int32_t rotary_dim, double theta,
                                        void* stream) {
    return rope_table(cos_sin, max_pos, rotary_dim, theta, stream);
}

extern "C" int dflash_qk_norm_rope_cache_ex(const uint16_t* qkv, int64_t row_stride, int64_t T_q, int32_t Hq,
                                            int32_t Hkv, int32_t D, const uint16_t* q_w, const uint16_t* k_w,
                                            float eps, const int64_t* positions, const void* cos_sin,
                                            int64_t max_pos, int32_t rotary_dim, int32_t is_neox,
                                            int32_t table_bf16, const int64_t* slots, uint16_t* kv_cache,
                                            int64_t num_blocks, int32_t block_size, int32_t cache_fp8,
                                            const float* kv_scale, uint16_t* q_out, uint16_t* k_out,
                                            void* stream) {
    const void* req[] = {qkv, q_w, k_w, positions, cos_sin, q_out};
    for (const void* q : req)
        if (!q || !DFLASH_ALIGNED16(q)) return DFLASH_ERR_INVALID_ARG;
    if ((slots == nullptr) != (kv_cache == nullptr)) return DFLASH_ERR_INVALID_ARG;
    if (kv_cache && (!DFLASH_ALIGNED16(kv_cache) || num_blocks < 1 || block_size < 1))
        return DFLASH_ERR_INVALID_ARG;
    if (k_out && !DFLASH_ALIGNED16(k_out)) return DFLASH_ERR_INVALID_ARG;
    if (!k_out && !kv_cache) return DFLASH_ERR_INVALID_ARG;
    if (T_q < 1 || Hq < 1 || Hkv < 1 || max_pos < 1 || !(eps >= 0.f)) return DFLASH_ERR_INVALID_ARG;
    if ((table_bf16 != 0 && table_bf16 != 1) || (is_neox != 0 && is_neox != 1)) return DFLASH_ERR_INVALID_ARG;
    if (rotary_dim < 2 || rotary_dim > D || (rotary_dim & 1)) return DFLASH_ERR_INVALID_ARG;
    if (cache_fp8 < FP8_NONE || cache_fp8 > FP8_E5M2) return DFLASH_ERR_INVALID_ARG;
    if (cache_fp8 != FP8_NONE && (!kv_cache || !kv_scale || (reinterpret_cast<uintptr_t>(kv_scale) & 3u)))
        return DFLASH_ERR_INVALID_ARG;
    if (D != QK_D) return DFLASH_ERR_UNSUPPORTED;
    if (rotary_dim % (is_neox ? 16 : 8) != 0) return DFLASH_ERR_UNSUPPORTED;
    if (row_stride < (int64_t)(Hq + 2 * Hkv) * D || row_stride % 8 != 0) return DFLASH_ERR_INVALID_ARG;
    if (T_q > INT32_MAX || (int64_t)Hq + 2 * (int64_t)Hkv > 65536) return DFLASH_ERR_UNSUPPORTED;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
#define QK_LAUNCH(NX, TB, F8)                                                                                     \
    hipLaunchKernelGGL((qk_norm_rope_cache_kernel<NX, TB, F8>), dim3((unsigned)T_q), dim3(256), 0, st, qkv,          \
                       row_stride, Hq, Hkv, q_w, k_w, eps, positions, cos_sin, (int)rotary_dim, max_pos, slots,       \
                       kv_cache, num_blocks, block_size, q_out, k_out, kv_scale)
#define QK_LAUNCH_F8(NX, TB)                                \
    do {                                                    \
        if (cache_fp8 == FP8_E4M3) QK_LAUNCH(NX, TB, FP8_E4M3); \
        else if (cache_fp8 == FP8_E5M2) QK_LAUNCH(NX, TB, FP8_E5M2); \
        else QK_LAUNCH(NX, TB, FP8_NONE);                   \
    } while (0)
    if (is_neox) {
        if (table_bf16) QK_LAUNCH_F8(true, true);
        else QK_LAUNCH_F8(true, false);
    } else {
        if (table_bf16) QK_LAUNCH_F8(false, true);
        else QK_LAUNCH_F8(false, false);
    }
#undef QK_LAUNCH_F8
#undef QK_LAUNCH
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

extern "C" int dflash_qk_norm_rope_cache(const uint16_t* qkv, int64_t row_stride, int64_t T_q, int32_t Hq,
                                         int32_t Hkv, int32_t D, const uint16_t* q_w, const uint16_t* k_w,
                                         float eps, const int64_t* positions, const float* cos_sin,
                                         int64_t max_pos, const int64_t* slots, uint16_t* kv_cache,
                                         int64_t num_blocks, int32_t block_size, uint16_t* q_out,
                                         uint16_t* k_out, void* stream) {
    return dflash_qk_norm_rope_cache_ex(qkv, row_stride, T_q, Hq, Hkv, D, q_w, k_w, eps, positions, cos_sin,
                                        max_pos, D, 1, 0, slots, kv_cache, num_blocks, block_size, FP8_NONE, nullptr,
                                        q_out, k_out, stream);
}

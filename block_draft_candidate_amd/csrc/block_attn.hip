// Non-causal sliding-window attention of the draft's query block over the paged
// K/V cache (DFlash2BeamAttention: every layer is non-causal sliding-window
// attention over the block, scale head_dim ** -0.5, grouped K/V heads; the
// context K/V is already in the cache, the block's own K/V is written by the
// fused norm/RoPE kernel first).
//
// One workgroup per (request, kv head); wave w handles q head kv * G + w, so the
// G heads that share a kv head read each K/V tile from HBM once.  A wave's 16
// MFMA columns are the block's (up to 16) queries.
//   * K/V tiles of 32 keys (2 cache blocks) go straight from HBM to LDS with
//     LDS-DMA (buffer_load_dwordx4 ... lds, nontemporal: each block is read
//     once), whole 512-byte cache rows (K | V), in a ring of AT_NST stages
//     (AT_NST - 1 tiles in flight).  K chunks are
//     XOR-swizzled by row (16-byte units), V chunks by row (16-byte units,
//     2 * (row % 8)), so both reads below are bank-conflict free.  The visible
//     part of the request's block table is copied to LDS once, so issuing a
//     tile's loads needs no scalar memory round trip.
//   * S^T = K Q^T: v_mfma_f32_16x16x32_bf16, K rows from LDS, Q^T from registers;
//     each lane then holds scores of a single query, so the online softmax
//     (fp32, exp2) needs only two cross-lane steps.
//   * O^T += V^T P^T: P^T comes straight from the S^T registers, split into two
//     bf16 parts (hi = bf16(p), lo = bf16(p - hi)) so that two MFMAs carry p to
//     2^-16 relative, the precision of the fp32 row sum that normalises it; V^T
//     comes from the row-major V tile through ds_read_b64_tr_b16 (the
//     transposing LDS read): lane p of a 16-lane group points at
//     V[key(p / 4)][d0 + 4 (p % 4)], and lane i receives V[key(j)][d0 + i],
//     j = 0..3.
//   * Tile rows at or past the request's length (the unwritten rest of its last
//     cache block, or that block again when a tile runs past it) are loaded
//     from an out-of-range offset and land as zeros: their weight is zero, and
//     a stale NaN or Inf there must not reach the output through 0 * NaN.
//   * With an fp8 cache (E4M3fn or E5M2) the LDS-DMA brings the tile's
//     256-byte fp8 rows into the ring instead (chunks swizzled by f8_swz), and
//     each wave converts its MFMA operands in registers (K from 8-byte reads,
//     V^T from the 8-bit transposing read; hardware fp8 -> bf16 conversions,
//     exact); the rest is the bf16 path.  The layer's K scale is
//     folded into the score scale and its V scale into the output.
#include "fp8.h"

namespace dflash {

constexpr int AT_D = 128;
constexpr int AT_BS = 16;      // cache block size
constexpr int AT_TK = 32;      // keys per tile
constexpr int AT_NST = 2;      // LDS ring stages (tiles): 36 KB of LDS per workgroup (bf16) lets four
                               // workgroups share a CU, which hides more than deeper rings with
                               // fewer workgroups (measured: 2 stages 194 us, 3: 256, 4: 251, 8: 409)
constexpr int AT_BTCAP = 1024; // block-table entries staged in LDS (longer spans read it from HBM)
constexpr int AT_ROW = 2 * AT_D;  // elements per cache row (K | V)

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// Two fp32 -> two bf16 packed (lo word = a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t at_cvt_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// (a, b) = hi + lo with both parts bf16: hi = bf16(x), lo = bf16(x - hi).  x - hi
// is exact in fp32 and |x - hi| <= ulp_bf16(x) / 2, so hi + lo is within
// 2^-16 |x| of x.
__device__ __forceinline__ void at_split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = at_cvt_bf16x2(a, b);
    lo = at_cvt_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ void at_fence() { asm volatile("" ::: "memory"); }

// One LDS-DMA instruction: 16 bytes per lane from the cache block at `blk`
// (one kv head's 16 rows of `row_bytes`, range-checked to that block) at byte
// offset `off`, landing at lds + 16 * lane.  Each workgroup reads its blocks
// once, so the loads carry the nontemporal hint (cache policy 2): the K/V
// stream then runs measurably closer to the HBM peak than with plain loads.
__device__ __forceinline__ void at_load_block_rows(const void* blk, int row_bytes, int off, void* lds) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)blk, (short)0, AT_BS * row_bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 2);
}

// Two fp8 codes (the low or high half of a word) -> two bf16 packed in a word,
// one v_cvt_scalef32_pk_bf16_fp8 / _bf8 with scale 1: every finite OCP E4M3 /
// E5M2 value is a bf16 number, so the conversion is exact (checked on the
// device over all 65536 code pairs of both formats and both halves against the
// fp32 conversion's top halves: bit-identical, NaNs included).
typedef __attribute__((ext_vector_type(2))) __bf16 at_bf16x2;
template <int F8, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    const at_bf16x2 r = F8 == FP8_E4M3 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI)
                                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// fp8 tiles: row r keeps its 16-byte chunk c (K: 0-7, V: 8-15) at physical chunk
// c ^ f8_swz(r).  The 16 rows a K fragment read spans, and the 8 keys a V
// transpose read spans (4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3), all get
// different values, so neither read has bank conflicts.
__device__ __forceinline__ int f8_swz(int r) { return (r & 15) ^ (((r >> 4) & 1) << 2); }
typedef __attribute__((ext_vector_type(2))) int at_v2i;

template <int G, int F8>
__global__ __launch_bounds__(64 * G) void block_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ cache, int64_t num_blocks,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ seq_lens, int Lq,
    int Hq, int Hkv, int window, float scale_log2, uint16_t* __restrict__ out, const float* __restrict__ kv_scale) {
    // LDS-DMA instructions per wave per tile: 2 bf16 rows or 4 fp8 rows each
    constexpr int NI = F8 == FP8_NONE ? AT_TK / 2 / G : AT_TK / 4 / G;
    constexpr int RB = F8 == FP8_NONE ? AT_ROW * 2 : AT_ROW;  // bytes per cache row
    static_assert(NI >= 1, "at least one LDS-DMA instruction per wave");
    // a ring of AT_NST tiles (bf16 rows, or fp8 rows at half the bytes), then
    // the staged block-table entries
    constexpr int RING = AT_NST * AT_TK * RB / 2;  // elements of uint16_t
    __shared__ __attribute__((aligned(1024))) uint16_t smem[RING + AT_BTCAP * 2];
    int32_t* const btl = reinterpret_cast<int32_t*>(smem + RING);
    uint8_t* const ring8 = reinterpret_cast<uint8_t*>(smem);
    if (F8 != FP8_NONE) scale_log2 *= kv_scale[0];

    const int r = blockIdx.x / Hkv;
    const int hk = blockIdx.x - r * Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
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
    const int nblk_req = (L + AT_BS - 1) / AT_BS;
    // cache block of block-table index i (clamped to the request's last block
    // and to the cache): from LDS when the visible span fits, else from HBM
    const int blk0 = kstart / AT_BS;
    const int nvis = nblk_req - blk0;
    const bool bt_in_lds = nvis <= AT_BTCAP;
    if (bt_in_lds)
        for (int i = tid; i < nvis; i += 64 * G) {
            int b = bt[blk0 + i];
            btl[i] = b < 0 ? 0 : (b >= num_blocks ? (int)(num_blocks - 1) : b);
        }
    __syncthreads();
    auto block_of = [&](int i) {
        i = min(i, nblk_req > 0 ? nblk_req - 1 : 0);
        if (bt_in_lds) return btl[max(i - blk0, 0)];
        int b = bt[i];
        return b < 0 ? 0 : (b >= num_blocks ? (int)(num_blocks - 1) : b);
    };

    // DMA lane layout (bf16): instruction covers tile rows 2q, 2q+1; lane i -> row
    // 2q + i/32, physical 16-byte chunk i % 32 of the 512-byte row.  Physical
    // chunk pc < 16 holds K chunk pc ^ (row % 16); pc >= 16 holds V chunk
    // (pc - 16) ^ (2 (row % 8)).  (fp8: instruction covers rows 4q .. 4q+3, lane
    // i -> row 4q + i/16, physical 16-byte chunk i % 16 of the 256-byte row,
    // holding K | V chunk i % 16 ^ f8_swz(row).)
    // Per-lane byte offsets inside a cache block (tile-independent), and per
    // tile one scalar block base per instruction.
    int loff[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        if (F8 == FP8_NONE) {
            const int rr = (2 * (wave_s * NI + j) + (lane >> 5)) & 15;  // row within the cache block
            const int pc = lane & 31;
            const int lchunk = pc < 16 ? (pc ^ rr) : (16 + ((pc - 16) ^ (2 * (rr & 7))));
            loff[j] = (rr * AT_ROW + lchunk * 8) * 2;
        } else {
            const int trow = 4 * (wave_s * NI + j) + (lane >> 4);  // tile row
            loff[j] = (trow & 15) * AT_ROW + (((lane & 15) ^ f8_swz(trow)) * 16);
        }
    }
    constexpr int RPI = F8 == FP8_NONE ? 2 : 4;  // tile rows per DMA instruction
    const int lrow = F8 == FP8_NONE ? (lane >> 5) : (lane >> 4);  // this lane's row within an instruction
    auto issue = [&](int tile, int st) {
        const int kb = kstart + tile * AT_TK;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int qd = wave_s * NI + j;
            const int b = __builtin_amdgcn_readfirstlane(block_of(kb / AT_BS + (RPI * qd) / AT_BS));
            const uint8_t* blk = reinterpret_cast<const uint8_t*>(cache) + ((int64_t)b * Hkv + hk) * AT_BS * RB;
            void* dst = F8 == FP8_NONE ? (void*)(smem + st * AT_TK * AT_ROW + qd * 512)
                                       : (void*)(ring8 + st * AT_TK * AT_ROW + qd * 1024);  // (fp8 rows: AT_ROW bytes)
            // rows at or past the request's length read as zeros (offset past the range)
            at_load_block_rows(blk, RB, kb + RPI * qd + lrow < L ? loff[j] : (int)0x80000000, dst);
        }
    };

    float m = -INFINITY, lsum = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int t = 0; t < AT_NST - 1; ++t)
        if (t < ntiles) issue(t, t);
    for (int tile = 0; tile < ntiles; ++tile) {
        const int st = tile % AT_NST;
        // this wave's loads of the tile landed (the later tiles already issued,
        // up to AT_NST - 2 of them, may still be in flight) ...
        const int ahead = min(AT_NST - 2, ntiles - 1 - tile);
        wait_stages_ahead<AT_NST - 2, NI>(ahead);
        __builtin_amdgcn_s_barrier();  // ... and every wave's; the stage of tile - 1 is free
        at_fence();
        if (tile + AT_NST - 1 < ntiles) issue(tile + AT_NST - 1, (tile + AT_NST - 1) % AT_NST);
        const uint16_t* tb = smem + st * AT_TK * AT_ROW;   // bf16 tile
        const uint8_t* t8 = ring8 + st * AT_TK * AT_ROW;     // fp8 tile (AT_ROW bytes per row)
        const int kb = kstart + tile * AT_TK;
        // every key of the tile is visible to every query of the block (the
        // highest window start is L - window, for the last query), and every
        // query lane is a real query: no masking
        const bool interior = Lq == 16 && L >= Lq && kb >= L - window && kb + AT_TK <= L;

        // S^T = K Q^T for 4 blocks of 16 keys
        constexpr int NKB = AT_TK / 16;
        float sv[NKB][4];
        float mt = -INFINITY;
#pragma unroll
        for (int kblk = 0; kblk < NKB; ++kblk) {
            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
            const int row = kblk * 16 + qi;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 kf;
                if (F8 == FP8_NONE) {
                    const int ch = (4 * s + g) ^ (row & 15);
                    kf = as_bf16x8(*reinterpret_cast<const u32x4*>(tb + row * AT_ROW + ch * 8));
                } else {
                    // 8 codes: half (g & 1) of the row's K chunk 2 s + g / 2
                    const int u = 4 * s + g;
                    const u32x2 w = *reinterpret_cast<const u32x2*>(t8 + row * AT_ROW +
                                                                    (((u >> 1) ^ f8_swz(row)) * 16) + (u & 1) * 8);
                    kf = as_bf16x8(u32x4{fp8x2_to_bf16x2<F8, false>(w[0]), fp8x2_to_bf16x2<F8, true>(w[0]),
                                         fp8x2_to_bf16x2<F8, false>(w[1]), fp8x2_to_bf16x2<F8, true>(w[1])});
                }
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sacc, 0, 0, 0);
            }
            if (interior) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sv[kblk][e] = sacc[e] * scale_log2;
                    mt = fmaxf(mt, sv[kblk][e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kp = kb + kblk * 16 + 4 * g + e;
                    const bool vis = qvalid && kp < L && kp >= qlo;
                    sv[kblk][e] = vis ? sacc[e] * scale_log2 : -INFINITY;
                    mt = fmaxf(mt, sv[kblk][e]);
                }
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mnew = fmaxf(m, mt);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        // rescale the running sums only when some query's maximum moved (after
        // the first tiles it rarely does); v_exp_f32 directly: arguments are
        // <= 0 and results below 2^-126 may flush to zero
        if (__ballot(mnew != m) != 0u) {
            const float alpha = __builtin_amdgcn_exp2f(m - muse);
            lsum *= alpha;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
        }
        m = mnew;
        float pv[NKB][4];
#pragma unroll
        for (int kblk = 0; kblk < NKB; ++kblk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[kblk][e] = __builtin_amdgcn_exp2f(sv[kblk][e] - muse);
                lsum += pv[kblk][e];
            }

        // O^T += V^T P^T over 32-key steps; K index of the MFMA for lane group g,
        // element j <-> key 32 s2 + 4 g + j (j < 4) or 32 s2 + 16 + 4 g + (j - 4).
        // P = P_hi + P_lo (two bf16 MFMAs), so the weights keep the row sum's precision.
        const int p = lane & 15;
#pragma unroll
        for (int s2 = 0; s2 < AT_TK / 32; ++s2) {
            uint32_t ph[4], pl[4];
            at_split_bf16x2(pv[2 * s2][0], pv[2 * s2][1], ph[0], pl[0]);
            at_split_bf16x2(pv[2 * s2][2], pv[2 * s2][3], ph[1], pl[1]);
            at_split_bf16x2(pv[2 * s2 + 1][0], pv[2 * s2 + 1][1], ph[2], pl[2]);
            at_split_bf16x2(pv[2 * s2 + 1][2], pv[2 * s2 + 1][3], ph[3], pl[3]);
            const bf16x8 pfh = as_bf16x8(u32x4{ph[0], ph[1], ph[2], ph[3]});
            const bf16x8 pfl = as_bf16x8(u32x4{pl[0], pl[1], pl[2], pl[3]});
            const int r1 = 32 * s2 + 4 * g + (p >> 2);
            const int r2 = r1 + 16;
            // fp8: ds_read_b64_tr_b8 gives lane 8 h + j of a 16-lane group byte j
            // of the 8 bytes read by the group's lanes h, h + 2, .., h + 14 (element
            // e from lane 2 e + h).  So lane 2 e + h of group g reads key e of the
            // group's MFMA K order (32 s2 + 4 g + e, then 32 s2 + 16 + 4 g + e - 4)
            // at V bytes 16 mb + 8 h .. + 8: lane (p, g) then holds d = 16 mb + p
            // for those 8 keys.
            const int e8 = p >> 1;
            const int rk = 32 * s2 + (e8 < 4 ? 4 * g + e8 : 16 + 4 * g + (e8 - 4));
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                u32x4 vv;
                if (F8 == FP8_NONE) {
                    // 8-byte chunk of d = 16 mb + 4 (p % 4) in the V half, swizzled by row
                    const int c8 = 4 * mb + (p & 3);
                    const int o1 = r1 * AT_ROW + AT_D + ((c8 ^ (4 * (r1 & 7))) << 2);
                    const int o2 = r2 * AT_ROW + AT_D + ((c8 ^ (4 * (r2 & 7))) << 2);
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(tb + o1));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(tb + o2));
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                    vv = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
                } else {
                    const int o = rk * AT_ROW + (((8 + mb) ^ f8_swz(rk)) * 16) + (p & 1) * 8;
                    const u32x2 w = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) at_v2i*)(t8 + o)));
                    vv = u32x4{fp8x2_to_bf16x2<F8, false>(w[0]), fp8x2_to_bf16x2<F8, true>(w[0]),
                               fp8x2_to_bf16x2<F8, false>(w[1]), fp8x2_to_bf16x2<F8, true>(w[1])};
                }
                o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vv), pfl, o[mb], 0, 0, 0);
                o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vv), pfh, o[mb], 0, 0, 0);
            }
        }
    }

    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const float inv = (lsum > 0.f ? 1.0f / lsum : 0.f) * (F8 == FP8_NONE ? 1.f : kv_scale[1]);
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
                        uint16_t* out, int f8, const float* kv_scale, hipStream_t st) {
    const float scale_log2 = scale * 1.4426950408889634f;
    const dim3 grid((unsigned)(Rq * Hkv)), block(64 * G);
    if (f8 == FP8_E4M3)
        hipLaunchKernelGGL((block_attn_kernel<G, FP8_E4M3>), grid, block, 0, st, q, cache, nblk, bt, maxb, seq, Lq,
                           Hq, Hkv, window, scale_log2, out, kv_scale);
    else if (f8 == FP8_E5M2)
        hipLaunchKernelGGL((block_attn_kernel<G, FP8_E5M2>), grid, block, 0, st, q, cache, nblk, bt, maxb, seq, Lq,
                           Hq, Hkv, window, scale_log2, out, kv_scale);
    else
        hipLaunchKernelGGL((block_attn_kernel<G, FP8_NONE>), grid, block, 0, st, q, cache, nblk, bt, maxb, seq, Lq,
                           Hq, Hkv, window, scale_log2, out, kv_scale);
}

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_block_attn_workspace_size(int64_t Rq, int32_t Lq, int32_t Hq, int32_t D) {
    (void)Rq; (void)Lq; (void)Hq; (void)D;
    return 0;
}

extern "C" int dflash_block_attn_ex(const uint16_t* q, const void* kv_cache, int64_t num_blocks,
                                    const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                    int64_t Rq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                    int32_t window, float scale, int32_t cache_fp8, const float* kv_scale,
                                    uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    (void)ws; (void)ws_bytes;
    const void* req[] = {q, kv_cache, block_tables, seq_lens, out};
    for (const void* p : req)
        if (!p || !DFLASH_ALIGNED16(p)) return DFLASH_ERR_INVALID_ARG;
    if (num_blocks < 1 || max_blocks < 1 || Rq < 1 || Lq < 1 || Hq < 1 || Hkv < 1 || window < 1 ||
        !(scale > 0.f) || !(scale < INFINITY))
        return DFLASH_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return DFLASH_ERR_INVALID_ARG;
    if (cache_fp8 < FP8_NONE || cache_fp8 > FP8_E5M2) return DFLASH_ERR_INVALID_ARG;
    if (cache_fp8 != FP8_NONE && (!kv_scale || (reinterpret_cast<uintptr_t>(kv_scale) & 3u)))
        return DFLASH_ERR_INVALID_ARG;
    if (D != AT_D || block_size != AT_BS || Lq > 16) return DFLASH_ERR_UNSUPPORTED;
    if (Rq * Hkv > INT32_MAX || (int64_t)max_blocks * AT_BS > INT32_MAX || num_blocks > INT32_MAX)
        return DFLASH_ERR_UNSUPPORTED;
    const int G = Hq / Hkv;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const uint16_t* c = reinterpret_cast<const uint16_t*>(kv_cache);
    switch (G) {
        case 1: launch_attn<1>(q, c, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, cache_fp8, kv_scale, st); break;
        case 2: launch_attn<2>(q, c, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, cache_fp8, kv_scale, st); break;
        case 4: launch_attn<4>(q, c, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, cache_fp8, kv_scale, st); break;
        case 8: launch_attn<8>(q, c, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, window, scale, out, cache_fp8, kv_scale, st); break;
        default: return DFLASH_ERR_UNSUPPORTED;
    }
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

extern "C" int dflash_block_attn(const uint16_t* q, const uint16_t* kv_cache, int64_t num_blocks,
                                 const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                 int64_t Rq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                 int32_t window, float scale, uint16_t* out, void* ws, size_t ws_bytes,
                                 void* stream) {
    return dflash_block_attn_ex(q, kv_cache, num_blocks, block_tables, max_blocks, seq_lens, Rq, Lq, Hq, Hkv, D,
                                block_size, window, scale, FP8_NONE, nullptr, out, ws, ws_bytes, stream);
}

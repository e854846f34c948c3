// LM-head top-k of the DFlash2 drafter's candidate head
// (DFlash2BeamForCausalLM.compute_candidates through its LogitsProcessor:
// scale = output_multiplier, soft cap = final_logit_softcapping).
//
// One pass over the LM-head weight W [V, Hd] computes logit tiles with bf16
// MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate) and selects top-k in the
// tile epilogue; the [T, V] logits are never written to HBM.
//
//   * A workgroup (256 threads, 4 waves in 2 x 2) owns a 256-row slice of H and
//     a contiguous run of BN-column tiles of W (its "group").  Each wave
//     computes a 128 x BN/2 block of a 256 x BN tile; the K loop streams 64-wide
//     slices of H and W through double-buffered, XOR-swizzled LDS with register
//     prefetch of the next slice.
//   * Epilogue: the tile is staged through LDS in two column halves; thread t
//     scans row t and keeps that row's running top-k of the group in registers
//     as packed words (ordered bf16 key << 16 | 0xFFFF - column-in-group), so
//     one unsigned compare orders (key desc, id asc).  A raw-accumulator
//     threshold derived from the current k-th key skips the scale/softcap work
//     for almost every column.
//   * Groups that share W columns are placed on one XCD (workgroup ids go to
//     XCDs round-robin), so the 256-row slices reuse W through that XCD's L2.
//   * A merge kernel picks the k best of the groups' partial lists per row.
#include "common.h"

namespace dflash {

constexpr int LM_BM = 256;
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

// The top-k key of one accumulator: bf16(c * tanh(s * acc / c)), or bf16(s * acc)
// without a cap.
__device__ __forceinline__ uint32_t logit_key_bits(float acc, float s, float c, float inv_c) {
    float x = s * acc;
    if (c > 0.f) x = c * tanhf(x * inv_c);
    return f32_to_bf16_bits(x);
}

// A raw-accumulator bound below which a logit's key is certainly smaller than
// the key `okey`: the value two bf16 steps below the key, mapped back through
// the cap and the scale, with a relative margin of 2^-12 at each step (far
// above the fp32 error of tanh/atanh).  Near saturation of the cap (|x| >
// 0.9 c) no bound is used.
__device__ float acc_lower_bound(uint32_t okey, float s, float c) {
    if (okey < 0x0082u) return -INFINITY;  // at or below -inf: nothing to bound
    const float xlo = bf16_bits_to_f32(unorder_key(okey - 2));
    if (!(xlo > -INFINITY)) return -INFINITY;
    float y = xlo;
    if (c > 0.f) {
        const float z = xlo / c;
        if (!(fabsf(z) < 0.9f)) return -INFINITY;
        y = c * atanhf(z);
    }
    y -= fabsf(y) * 0x1p-12f + 1e-30f;
    float a = y / s;
    a -= fabsf(a) * 0x1p-12f + 1e-30f;
    return a;
}

// Insert p into the descending list L (the smallest falls off).  A no-op when
// p <= L[n-1].
template <int N>
__device__ __forceinline__ void list_insert(uint32_t (&L)[N], uint32_t p) {
#pragma unroll
    for (int j = N - 1; j > 0; --j) L[j] = max(L[j], min(L[j - 1], p));
    L[0] = max(L[0], p);
}

template <int BN, int KCAP>
__global__ __launch_bounds__(LM_THREADS, 1) void lm_topk_tiles(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ W, int T, int V, int Hd,
    int nM, int nN, int G, int xcd_map, float s, float c, float inv_c,
    uint64_t* __restrict__ part) {
    constexpr int WN = BN / 2;              // columns per wave
    constexpr int NB = WN / 16;             // 16-column MFMA blocks per wave
    constexpr int MB = 8;                   // 16-row MFMA blocks per wave (128 rows)
    constexpr int A_CH = LM_BM * 8 / LM_THREADS;  // 16-byte chunks per thread per slice
    constexpr int B_CH = BN * 8 / LM_THREADS;
    constexpr int SP = WN + 1;              // staging pitch (floats): conflict-free row scans
    constexpr int A_ELEMS = LM_BM * LM_BK;
    constexpr int B_ELEMS = BN * LM_BK;
    constexpr int AB_BYTES = 2 * (A_ELEMS + B_ELEMS) * 2;
    constexpr int ST_BYTES = LM_BM * SP * 4;
    constexpr int LDS_BYTES = AB_BYTES > ST_BYTES ? AB_BYTES : ST_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    uint16_t* sA = reinterpret_cast<uint16_t*>(lds);
    uint16_t* sB = sA + 2 * A_ELEMS;
    float* stage = reinterpret_cast<float*>(lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int L = blockIdx.x;
    if (xcd_map) {
        const int per = gridDim.x >> 3;
        L = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    const int m_tile = L % nM;
    const int g = L / nM;
    const int n_begin = (int)((int64_t)g * nN / G);
    const int n_end = (int)((int64_t)(g + 1) * nN / G);
    const int m0 = m_tile * LM_BM;
    const int gcol0 = n_begin * BN;
    const int my_row = m0 + tid;

    uint32_t list[KCAP];
#pragma unroll
    for (int j = 0; j < KCAP; ++j) list[j] = 0u;
    float thr = -INFINITY;

    const int nK = (Hd + LM_BK - 1) / LM_BK;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    for (int nt = n_begin; nt < n_end; ++nt) {
        const int n0 = nt * BN;
        f32x4 acc[MB][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        u32x4 ga[A_CH], gb[B_CH];
        auto gload = [&](int kt) {
            const int k0 = kt * LM_BK;
#pragma unroll
            for (int i = 0; i < A_CH; ++i) {
                const int ch = tid + LM_THREADS * i;
                const int row = ch >> 3, kc = ch & 7;
                const int gr = m0 + row, gk = k0 + kc * 8;
                ga[i] = (gr < T && gk < Hd) ? ldg16(H + (int64_t)gr * Hd + gk) : zero4;
            }
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const int ch = tid + LM_THREADS * i;
                const int row = ch >> 3, kc = ch & 7;
                const int gr = n0 + row, gk = k0 + kc * 8;
                gb[i] = (gr < V && gk < Hd) ? ldg16(W + (int64_t)gr * Hd + gk) : zero4;
            }
        };
        auto sstore = [&](int buf) {
#pragma unroll
            for (int i = 0; i < A_CH; ++i) {
                const int ch = tid + LM_THREADS * i;
                const int row = ch >> 3, kc = ch & 7;
                *reinterpret_cast<u32x4*>(sA + buf * A_ELEMS + row * LM_BK + ((kc ^ (row & 7)) << 3)) = ga[i];
            }
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const int ch = tid + LM_THREADS * i;
                const int row = ch >> 3, kc = ch & 7;
                *reinterpret_cast<u32x4*>(sB + buf * B_ELEMS + row * LM_BK + ((kc ^ (row & 7)) << 3)) = gb[i];
            }
        };

        gload(0);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < nK; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nK) gload(kt + 1);
            const uint16_t* a_base = sA + buf * A_ELEMS;
            const uint16_t* b_base = sB + buf * B_ELEMS;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int ch = kk * 4 + (lane >> 4);
                bf16x8 af[MB], bfr[NB];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int row = wm * 128 + i * 16 + (lane & 15);
                    af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(a_base + row * LM_BK + ((ch ^ (row & 7)) << 3)));
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int row = wn * WN + j * 16 + (lane & 15);
                    bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(b_base + row * LM_BK + ((ch ^ (row & 7)) << 3)));
                }
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nK) sstore(buf ^ 1);
            __syncthreads();
        }

        // Epilogue: stage one column half at a time, then each thread scans its row.
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wn == pass) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = wm * 128 + i * 16 + 4 * (lane >> 4) + e;
                            const int col = j * 16 + (lane & 15);
                            stage[row * SP + col] = acc[i][j][e];
                        }
            }
            __syncthreads();
            if (my_row < T) {
                const int cbase = n0 + pass * WN;
                const int ncols = min(WN, V - cbase);
                const float* srow = stage + tid * SP;
                for (int cc = 0; cc < ncols; ++cc) {
                    const float a = srow[cc];
                    if (a >= thr) {
                        const uint32_t kb = logit_key_bits(a, s, c, inv_c);
                        const uint32_t p = (order_key(kb) << 16) | (0xffffu - (uint32_t)(cbase + cc - gcol0));
                        if (p > list[KCAP - 1]) {
                            list_insert(list, p);
                            if (list[KCAP - 1] != 0u) thr = acc_lower_bound(list[KCAP - 1] >> 16, s, c);
                        }
                    }
                }
            }
            __syncthreads();
        }
    }

    if (my_row < T) {
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

// One wave per row: k best of the row's G * KCAP partial entries
// (entry = ordered key << 32 | ~id; larger is better; 0 = empty).
template <int KCAP>
__global__ __launch_bounds__(256) void lm_topk_merge(const uint64_t* __restrict__ part, int T, int G,
                                                     int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= T) return;
    const int n = G * KCAP;
    const uint64_t* src = part + (int64_t)row * n;
    uint64_t Ls[KCAP];
#pragma unroll
    for (int j = 0; j < KCAP; ++j) Ls[j] = 0;
    for (int i = lane; i < n; i += 64) {
        const uint64_t p = src[i];
        if (p > Ls[KCAP - 1]) {
#pragma unroll
            for (int j = KCAP - 1; j > 0; --j) {
                const uint64_t lo = Ls[j - 1] < p ? Ls[j - 1] : p;
                Ls[j] = Ls[j] > lo ? Ls[j] : lo;
            }
            Ls[0] = Ls[0] > p ? Ls[0] : p;
        }
    }
    for (int r = 0; r < k; ++r) {
        uint64_t best = Ls[0];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const uint64_t o = __shfl_xor(best, off);
            best = o > best ? o : best;
        }
        if (Ls[0] == best && best != 0) {
#pragma unroll
            for (int j = 0; j < KCAP - 1; ++j) Ls[j] = Ls[j + 1];
            Ls[KCAP - 1] = 0;
        }
        if (lane == 0) {
            const uint32_t okey = (uint32_t)(best >> 32);
            ids[(int64_t)row * k + r] = (int32_t)(~(uint32_t)best);
            logits[(int64_t)row * k + r] = best ? bf16_bits_to_f32(unorder_key(okey)) : -INFINITY;
        }
    }
}

struct LmPlan {
    int BN, KCAP, nM, nN, G, xcd;
    int64_t nwg;
    size_t ws;
};

static bool lm_plan(int64_t T, int64_t V, int64_t Hd, int k, LmPlan& p) {
    (void)Hd;
    p.KCAP = k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : k <= 32 ? 32 : 64;
    p.nM = (int)((T + LM_BM - 1) / LM_BM);
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
    if ((int64_t)p.nM * p.G < target) groups(128);
    p.nwg = (int64_t)p.nM * p.G;
    if (p.nwg > (int64_t)1 << 30) return false;
    p.xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.ws = (size_t)T * (size_t)p.G * (size_t)p.KCAP * sizeof(uint64_t);
    return true;
}

template <int BN, int KCAP>
static void launch_tiles(const LmPlan& p, const uint16_t* H, const uint16_t* W, int T, int V, int Hd,
                         float s, float c, uint64_t* part, hipStream_t st) {
    const float inv_c = c > 0.f ? 1.0f / c : 0.f;
    hipLaunchKernelGGL((lm_topk_tiles<BN, KCAP>), dim3((unsigned)p.nwg), dim3(LM_THREADS), 0, st, H, W, T,
                       V, Hd, p.nM, p.nN, p.G, p.xcd, s, c, inv_c, part);
}

template <int KCAP>
static void launch_all(const LmPlan& p, const uint16_t* H, const uint16_t* W, int T, int V, int Hd, int k,
                       float s, float c, uint64_t* part, int32_t* ids, float* logits, hipStream_t st) {
    if (p.BN == 256)
        launch_tiles<256, KCAP>(p, H, W, T, V, Hd, s, c, part, st);
    else
        launch_tiles<128, KCAP>(p, H, W, T, V, Hd, s, c, part, st);
    hipLaunchKernelGGL((lm_topk_merge<KCAP>), dim3((T + 3) / 4), dim3(256), 0, st, part, T, p.G, k, ids,
                       logits);
}

}  // namespace dflash

using namespace dflash;

extern "C" size_t dflash_lm_topk_workspace_size(int64_t T, int64_t V, int64_t Hd, int32_t k) {
    LmPlan p;
    if (T < 1 || V < 1 || Hd < 1 || k < 1 || k > 64 || !lm_plan(T, V, Hd, k, p)) return 0;
    return p.ws;
}

extern "C" int dflash_lm_topk(const uint16_t* H, const uint16_t* W, int64_t T, int64_t V, int64_t Hd,
                              int32_t k, float output_multiplier, float softcap, int32_t* ids,
                              float* logits, void* ws, size_t ws_bytes, void* stream) {
    if (!H || !W || !ids || !logits || !ws) return DFLASH_ERR_INVALID_ARG;
    if (!DFLASH_ALIGNED16(H) || !DFLASH_ALIGNED16(W) || !DFLASH_ALIGNED16(ws)) return DFLASH_ERR_INVALID_ARG;
    if (T < 1 || V < 1 || Hd < 1 || k < 1 || k > V) return DFLASH_ERR_INVALID_ARG;
    if (!(output_multiplier > 0.f) || !(output_multiplier < INFINITY)) return DFLASH_ERR_INVALID_ARG;
    if (softcap != softcap || softcap == INFINITY) return DFLASH_ERR_INVALID_ARG;
    if (k > 64 || Hd % 8 != 0) return DFLASH_ERR_UNSUPPORTED;
    if (T > INT32_MAX || V > INT32_MAX || Hd > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    LmPlan p;
    if (!lm_plan(T, V, Hd, k, p)) return DFLASH_ERR_UNSUPPORTED;
    if (ws_bytes < p.ws) return DFLASH_ERR_WORKSPACE;
    const float c = softcap > 0.f ? softcap : 0.f;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint64_t* part = reinterpret_cast<uint64_t*>(ws);
    const int Ti = (int)T, Vi = (int)V, Hi = (int)Hd;
    switch (p.KCAP) {
        case 4: launch_all<4>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, st); break;
        case 8: launch_all<8>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, st); break;
        case 16: launch_all<16>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, st); break;
        case 32: launch_all<32>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, st); break;
        default: launch_all<64>(p, H, W, Ti, Vi, Hi, k, output_multiplier, c, part, ids, logits, st); break;
    }
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

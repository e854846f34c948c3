// Candidate-selector edge scores of the DFlash2 drafter
// (DFlash2BeamCandidateSelector: score = the candidate's own logit +
// <predecessor[q] * h_p, successor[c]>, h_p = the hidden state projected to the
// codebook rank, the first position's predecessor = the anchor token).
//
// Two kernels:
//   1. edges_projection: h_p = W_proj . h for every (request, step) row, a skinny
//      bf16 MFMA GEMM [T, Hd] x [R, Hd]^T.  The Hd axis is split into KS slices
//      so that enough workgroups stream H; each slice writes fp32 partial sums
//      (no atomics: the edge kernel adds the slices in a fixed order).
//   2. edges_bilinear: one wave per (request, step).  Lane group g (= lane/16)
//      owns a quarter of every rank chunk; each lane gathers its share of the
//      predecessor row (row = lane % 16 -> predecessor q) and successor row
//      (-> candidate c) straight from HBM with 8/16-byte loads, forms
//      a = P[pred] * h_p in fp32 and feeds fp32 MFMA 16x16x4 steps, so the k x k
//      block comes out of the matrix core with every product in fp32.
#include "common.h"

namespace dflash {

constexpr int PJ_ROWS = 64;   // rows of H per workgroup (4 waves x 16)
constexpr int PJ_BK = 64;     // K chunk staged in LDS
constexpr int PJ_THREADS = 256;

// part[ks][t][i] = sum over the ks-th Hd slice of H[t, j] * Wp[i, j]
template <int RB>  // R / 16
__global__ __launch_bounds__(PJ_THREADS) void edges_projection(const uint16_t* __restrict__ H,
                                                               const uint16_t* __restrict__ Wp, int T,
                                                               int Hd, int kslice,
                                                               float* __restrict__ part) {
    constexpr int R = RB * 16;
    constexpr int A_CH = PJ_ROWS * 8 / PJ_THREADS;             // 2
    constexpr int B_CH = (R * 8 + PJ_THREADS - 1) / PJ_THREADS;
    __shared__ __attribute__((aligned(16))) uint16_t sA[PJ_ROWS * PJ_BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[R * PJ_BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row0 = blockIdx.x * PJ_ROWS;
    const int ks = blockIdx.y;
    const int kbeg = ks * kslice;
    const int kend = min(Hd, kbeg + kslice);
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    f32x4 acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ga[A_CH], gb[B_CH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int ch = tid + PJ_THREADS * i;
            const int r = ch >> 3, kc = ch & 7;
            const int gr = row0 + r, gk = k0 + kc * 8;
            ga[i] = (gr < T && gk < kend) ? ldg16(H + (int64_t)gr * Hd + gk) : zero4;
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int ch = tid + PJ_THREADS * i;
            const int r = ch >> 3, kc = ch & 7;
            const int gk = k0 + kc * 8;
            gb[i] = (r < R && gk < kend) ? ldg16(Wp + (int64_t)r * Hd + gk) : zero4;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int ch = tid + PJ_THREADS * i;
            const int r = ch >> 3, kc = ch & 7;
            *reinterpret_cast<u32x4*>(sA + r * PJ_BK + ((kc ^ (r & 7)) << 3)) = ga[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int ch = tid + PJ_THREADS * i;
            const int r = ch >> 3, kc = ch & 7;
            if (r < R) *reinterpret_cast<u32x4*>(sB + r * PJ_BK + ((kc ^ (r & 7)) << 3)) = gb[i];
        }
    };

    if (kbeg < kend) {
        gload(kbeg);
        for (int k0 = kbeg; k0 < kend; k0 += PJ_BK) {
            __syncthreads();  // previous chunk's LDS reads are done
            sstore();
            __syncthreads();
            if (k0 + PJ_BK < kend) gload(k0 + PJ_BK);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int ch = kk * 4 + (lane >> 4);
                const int ar = wave * 16 + (lane & 15);
                const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(sA + ar * PJ_BK + ((ch ^ (ar & 7)) << 3)));
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    const int br = j * 16 + (lane & 15);
                    const bf16x8 bfr = as_bf16x8(*reinterpret_cast<const u32x4*>(sB + br * PJ_BK + ((ch ^ (br & 7)) << 3)));
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[j], 0, 0, 0);
                }
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

template <int VPL>
__device__ __forceinline__ void load_bf16_vec(const uint16_t* p, float (&f)[VPL]) {
    if constexpr (VPL == 8) {
        unpack8(ldg16(p), f);
    } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        f[0] = __uint_as_float(v[0] << 16);
        f[1] = __uint_as_float(v[0] & 0xffff0000u);
        f[2] = __uint_as_float(v[1] << 16);
        f[3] = __uint_as_float(v[1] & 0xffff0000u);
    }
}

// One wave per row t = r * S + p.  KB = ceil(k / 16) blocks of 16 predecessors
// and 16 candidates; VPL = rank values per lane per 4 * VPL-wide chunk.
template <int KB, int VPL>
__global__ __launch_bounds__(256) void edges_bilinear(
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Sc, const int32_t* __restrict__ ids,
    const float* __restrict__ U, const float* __restrict__ part, int KS, const int32_t* __restrict__ anchor,
    int T, int St, int k, int V, int R, float* __restrict__ E) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int r = t / St, p = t - r * St;
    const int g = lane >> 4, li = lane & 15;

    int pred[KB], cid[KB];
    bool qv[KB], cv[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const int q = b * 16 + li;
        qv[b] = q < k;
        cv[b] = q < k;
        int pr = 0, ci = 0;
        if (q < k) {
            pr = (p == 0) ? anchor[r] : ids[(int64_t)(t - 1) * k + q];
            ci = ids[(int64_t)t * k + q];
        }
        pred[b] = min(max(pr, 0), V - 1);
        cid[b] = min(max(ci, 0), V - 1);
    }

    f32x4 acc[KB][KB];
#pragma unroll
    for (int a = 0; a < KB; ++a)
#pragma unroll
        for (int b = 0; b < KB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int CH = 4 * VPL;
    for (int i0 = 0; i0 < R; i0 += CH) {
        const int ib = i0 + g * VPL;
        float h[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) h[v] = 0.f;
        for (int ks = 0; ks < KS; ++ks) {
            const float* src = part + ((int64_t)ks * T + t) * R + ib;
#pragma unroll
            for (int v = 0; v < VPL; v += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(src + v);
                h[v] += x[0];
                h[v + 1] += x[1];
                h[v + 2] += x[2];
                h[v + 3] += x[3];
            }
        }
        float a[KB][VPL], b[KB][VPL];
#pragma unroll
        for (int bq = 0; bq < KB; ++bq) {
            load_bf16_vec<VPL>(P + (int64_t)pred[bq] * R + ib, a[bq]);
#pragma unroll
            for (int v = 0; v < VPL; ++v) a[bq][v] = qv[bq] ? a[bq][v] * h[v] : 0.f;
        }
#pragma unroll
        for (int bc = 0; bc < KB; ++bc) {
            load_bf16_vec<VPL>(Sc + (int64_t)cid[bc] * R + ib, b[bc]);
#pragma unroll
            for (int v = 0; v < VPL; ++v) b[bc][v] = cv[bc] ? b[bc][v] : 0.f;
        }
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int bq = 0; bq < KB; ++bq)
#pragma unroll
                for (int bc = 0; bc < KB; ++bc)
                    acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[bq][v], b[bc][v], acc[bq][bc], 0, 0, 0);
    }

#pragma unroll
    for (int bc = 0; bc < KB; ++bc) {
        const int c = bc * 16 + li;
        if (c >= k) continue;
        const float u = U[(int64_t)t * k + c];
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

static EdgePlan edge_plan(int64_t T, int R, int64_t Hd) {
    EdgePlan p;
    const int64_t row_blocks = (T + PJ_ROWS - 1) / PJ_ROWS;
    int64_t ks = (256 + row_blocks - 1) / row_blocks;  // fill the chip with workgroups
    const int64_t max_ks = (Hd + PJ_BK - 1) / PJ_BK;
    if (ks > max_ks) ks = max_ks;
    if (ks > 16) ks = 16;
    if (ks < 1) ks = 1;
    int64_t kslice = (Hd + ks - 1) / ks;
    kslice = (kslice + PJ_BK - 1) / PJ_BK * PJ_BK;
    ks = (Hd + kslice - 1) / kslice;
    p.KS = (int)ks;
    p.kslice = (int)kslice;
    p.ws = (size_t)ks * (size_t)T * (size_t)R * sizeof(float);
    return p;
}

template <int RB>
static void launch_projection(const uint16_t* H, const uint16_t* Wp, int T, int Hd, const EdgePlan& p,
                              float* part, hipStream_t st) {
    dim3 grid((T + PJ_ROWS - 1) / PJ_ROWS, p.KS);
    hipLaunchKernelGGL((edges_projection<RB>), grid, dim3(PJ_THREADS), 0, st, H, Wp, T, Hd, p.kslice, part);
}

template <int KB>
static void launch_bilinear(const uint16_t* P, const uint16_t* Sc, const int32_t* ids, const float* U,
                            const float* part, int KS, const int32_t* anchor, int T, int St, int k, int V,
                            int R, float* E, hipStream_t st) {
    dim3 grid((T + 3) / 4);
    if (R % 32 == 0)
        hipLaunchKernelGGL((edges_bilinear<KB, 8>), grid, dim3(256), 0, st, P, Sc, ids, U, part, KS, anchor, T,
                           St, k, V, R, E);
    else
        hipLaunchKernelGGL((edges_bilinear<KB, 4>), grid, dim3(256), 0, st, P, Sc, ids, U, part, KS, anchor, T,
                           St, k, V, R, E);
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
    if (T > INT32_MAX / 64 || V > INT32_MAX || Hd > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
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
    if (KB == 1)
        launch_bilinear<1>(pred_cb, succ_cb, cand_ids, unary, part, p.KS, anchor, Ti, S, k, (int)V, R, edges, st);
    else if (KB == 2)
        launch_bilinear<2>(pred_cb, succ_cb, cand_ids, unary, part, p.KS, anchor, Ti, S, k, (int)V, R, edges, st);
    else
        launch_bilinear<4>(pred_cb, succ_cb, cand_ids, unary, part, p.KS, anchor, Ti, S, k, (int)V, R, edges, st);
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

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
constexpr int PJ_BK = 64;     // K slice staged in LDS
constexpr int PJ_THREADS = 256;
constexpr int PJ_STAGES = 3;

// Issue the LDS-DMA loads of rows [0, nrows) x columns [k0, k0 + 64) of a
// K-contiguous bf16 matrix (buffer rsrc, row pitch ld elements) into an LDS tile
// of 128-byte rows (16-byte chunks XOR-swizzled by row % 8).  Instruction q
// fills rows 8q .. 8q+7; wave w issues q = w, w + 4, ...  Columns >= kend read
// as zero.
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

// part[ks][t][i] = sum over the ks-th Hd slice of H[t, j] * Wp[i, j].  bf16 MFMA
// 16x16x32; three-stage LDS-DMA pipeline over 64-wide K slices.
template <int RB>  // R / 16
__global__ __launch_bounds__(PJ_THREADS) void edges_projection(const uint16_t* __restrict__ H,
                                                               const uint16_t* __restrict__ Wp, int T,
                                                               int Hd, int kslice,
                                                               float* __restrict__ part) {
    constexpr int R = RB * 16;
    constexpr int NQA = PJ_ROWS / 8;
    constexpr int NQB = R / 8;
    constexpr int STAGE = (PJ_ROWS + R) * PJ_BK;
    constexpr int PER_WAVE = NQA / 4 + NQB / 4;  // DMA instructions every wave issues per slice
    __shared__ __attribute__((aligned(1024))) uint16_t smem[PJ_STAGES * STAGE];

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

    auto issue = [&](int sl, int st) {
        uint16_t* base = smem + st * STAGE;
        pj_dma<NQA>(rsA, base, wave_s, lane, Hd, kbeg + sl * PJ_BK, kend);
        pj_dma<NQB>(rsB, base + PJ_ROWS * PJ_BK, wave_s, lane, Hd, kbeg + sl * PJ_BK, kend);
    };
    for (int sl = 0; sl < PJ_STAGES - 1 && sl < nS; ++sl) issue(sl, sl);
    for (int kt = 0; kt < nS; ++kt) {
        // wait for slice kt; slice kt+1 may still be in flight
        if (kt + 1 < nS) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (kt + PJ_STAGES - 1 < nS) issue(kt + PJ_STAGES - 1, (kt + PJ_STAGES - 1) % PJ_STAGES);
        const uint16_t* a_base = smem + (kt % PJ_STAGES) * STAGE;
        const uint16_t* b_base = a_base + PJ_ROWS * PJ_BK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int chs = ((kk * 4 + (lane >> 4)) ^ (lane & 7)) << 3;  // row % 8 == lane % 8
            const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(a_base + (wave * 16 + (lane & 15)) * PJ_BK + chs));
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                const bf16x8 bfr = as_bf16x8(*reinterpret_cast<const u32x4*>(b_base + (j * 16 + (lane & 15)) * PJ_BK + chs));
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

// One wave per row t = r * S + p (WAVES waves per workgroup, each with its own
// LDS region).  The row's 16 * KB predecessor and 16 * KB candidate codebook
// rows are gathered with whole-row coalesced 16-byte loads into LDS (row pitch
// 2R + 16 bytes, so that the 16 MFMA rows read different banks), h_p (the sum of
// the KS projection partials, in a fixed order) is staged once per row, then
// lane l takes predecessor row q = l % 16 (MFMA row) and candidate row c = l % 16
// (MFMA column) and lane group g = l / 16 owns a quarter of each 4 * VPL-wide rank
// chunk: a = P[pred] * h_p is formed in fp32 and the k x k block accumulates on
// v_mfma_f32_16x16x4f32, every product in fp32.
template <int KB, int R, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void edges_bilinear(
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Sc, const int32_t* __restrict__ ids,
    const float* __restrict__ U, const float* __restrict__ part, int KS, const int32_t* __restrict__ anchor,
    int T, int St, int k, int V, float* __restrict__ E) {
    constexpr int NR = 16 * KB;              // gathered rows per codebook
    constexpr int PITCH = R + 8;             // elements (2R + 16 bytes)
    constexpr int CPR = R / 8;               // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;            // rows per gather instruction
    constexpr int VPL = (R % 32 == 0) ? 8 : 4;
    constexpr int CH = 4 * VPL;
    constexpr int WAVE_ELEMS = 2 * NR * PITCH + 2 * R;  // bf16 rows + fp32 h_p
    extern __shared__ __attribute__((aligned(16))) uint16_t smem_e[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * WAVES + wave;
    const bool live = t < T;
    const int tt = live ? t : T - 1;        // dead waves mirror the last row and store nothing
    const int r = tt / St, p = tt - r * St;
    const int g = lane >> 4, li = lane & 15;
    uint16_t* sP = smem_e + wave * WAVE_ELEMS;
    uint16_t* sS = sP + NR * PITCH;
    float* sH = reinterpret_cast<float*>(sS + NR * PITCH);

    // ids of the predecessor rows (q) and candidate rows (c) this lane stands for
    int pred[KB], cid[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const int q = b * 16 + li;
        int pr = 0, ci = 0;
        if (q < k) {
            pr = (p == 0) ? anchor[r] : ids[(int64_t)(tt - 1) * k + q];
            ci = ids[(int64_t)tt * k + q];
        }
        pred[b] = min(max(pr, 0), V - 1);
        cid[b] = min(max(ci, 0), V - 1);
    }

    // h_p, the sum of the KS partials in order, one rank entry per lane per step
#pragma unroll
    for (int i = lane; i < R; i += 64) {
        float h = 0.f;
        for (int ks = 0; ks < KS; ++ks) h += part[((int64_t)ks * T + tt) * R + i];
        sH[i] = h;
    }

    // coalesced gathers: instruction j covers rows j * RPI .. j * RPI + RPI - 1,
    // CPR lanes per row; row ids come from the lanes that hold them (row % 16)
    const int gr = lane / CPR, gc = lane % CPR;
    constexpr int NJ = (NR + RPI - 1) / RPI;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int row = j * RPI + gr;
        int pid = 0, cidr = 0;
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const int x = __shfl(pred[b], row & 15);
            const int y = __shfl(cid[b], row & 15);
            if ((row >> 4) == b) { pid = x; cidr = y; }
        }
        if (gr < RPI && row < NR) {
            const u32x4 pv = ldg16(P + (int64_t)pid * R + gc * 8);
            const u32x4 sv = ldg16(Sc + (int64_t)cidr * R + gc * 8);
            *reinterpret_cast<u32x4*>(sP + row * PITCH + gc * 8) = pv;
            *reinterpret_cast<u32x4*>(sS + row * PITCH + gc * 8) = sv;
        }
    }
    __syncthreads();

    f32x4 acc[KB][KB];
#pragma unroll
    for (int a = 0; a < KB; ++a)
#pragma unroll
        for (int b = 0; b < KB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i0 = 0; i0 < R; i0 += CH) {
        const int ib = i0 + g * VPL;
        float h[VPL];
#pragma unroll
        for (int v = 0; v < VPL; v += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(sH + ib + v);
            h[v] = x[0]; h[v + 1] = x[1]; h[v + 2] = x[2]; h[v + 3] = x[3];
        }
        float a[KB][VPL], b[KB][VPL];
#pragma unroll
        for (int bq = 0; bq < KB; ++bq) {
            const bool qv = bq * 16 + li < k;
            if constexpr (VPL == 8) {
                unpack8(*reinterpret_cast<const u32x4*>(sP + (bq * 16 + li) * PITCH + ib), a[bq]);
                unpack8(*reinterpret_cast<const u32x4*>(sS + (bq * 16 + li) * PITCH + ib), b[bq]);
            } else {
                const u32x2 x = *reinterpret_cast<const u32x2*>(sP + (bq * 16 + li) * PITCH + ib);
                const u32x2 y = *reinterpret_cast<const u32x2*>(sS + (bq * 16 + li) * PITCH + ib);
                a[bq][0] = __uint_as_float(x[0] << 16); a[bq][1] = __uint_as_float(x[0] & 0xffff0000u);
                a[bq][2] = __uint_as_float(x[1] << 16); a[bq][3] = __uint_as_float(x[1] & 0xffff0000u);
                b[bq][0] = __uint_as_float(y[0] << 16); b[bq][1] = __uint_as_float(y[0] & 0xffff0000u);
                b[bq][2] = __uint_as_float(y[1] << 16); b[bq][3] = __uint_as_float(y[1] & 0xffff0000u);
            }
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                a[bq][v] = qv ? a[bq][v] * h[v] : 0.f;
                b[bq][v] = qv ? b[bq][v] : 0.f;
            }
        }
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
            for (int bq = 0; bq < KB; ++bq)
#pragma unroll
                for (int bc = 0; bc < KB; ++bc)
                    acc[bq][bc] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[bq][v], b[bc][v], acc[bq][bc], 0, 0, 0);
    }

    if (!live) return;
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

template <int KB, int R>
static void launch_bilinear_r(const uint16_t* P, const uint16_t* Sc, const int32_t* ids, const float* U,
                              const float* part, int KS, const int32_t* anchor, int T, int St, int k, int V,
                              float* E, hipStream_t st) {
    constexpr size_t wave_bytes = (size_t)(2 * 16 * KB * (R + 8) + 2 * R) * 2;
    constexpr int WAVES = wave_bytes * 4 <= 64 * 1024 ? 4 : 1;
    if (wave_bytes * WAVES > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&edges_bilinear<KB, R, WAVES>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)(wave_bytes * WAVES));
    hipLaunchKernelGGL((edges_bilinear<KB, R, WAVES>), dim3((T + WAVES - 1) / WAVES), dim3(64 * WAVES),
                       wave_bytes * WAVES, st, P, Sc, ids, U, part, KS, anchor, T, St, k, V, E);
}

template <int KB>
static bool launch_bilinear(const uint16_t* P, const uint16_t* Sc, const int32_t* ids, const float* U,
                            const float* part, int KS, const int32_t* anchor, int T, int St, int k, int V,
                            int R, float* E, hipStream_t st) {
    switch (R) {
#define BL_CASE(n) \
    case n: launch_bilinear_r<KB, n>(P, Sc, ids, U, part, KS, anchor, T, St, k, V, E, st); return true;
        BL_CASE(16) BL_CASE(32) BL_CASE(48) BL_CASE(64) BL_CASE(80) BL_CASE(96) BL_CASE(112) BL_CASE(128)
        BL_CASE(144) BL_CASE(160) BL_CASE(176) BL_CASE(192) BL_CASE(208) BL_CASE(224) BL_CASE(240) BL_CASE(256)
#undef BL_CASE
        default: return false;
    }
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

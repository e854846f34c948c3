// Bias-free bf16 linear Y = X . W^T with a bf16 output, for the draft layer's
// projections around its attention (DFlash2BeamAttention: qkv_proj before the
// fused q/k norm + RoPE + cache write, o_proj after the attention).
//
// The 256 x BN tile of gemm_tile.h (BN = 256, 192 or 128, whichever fills the
// CUs in the fewest width-weighted rounds); the epilogue stages each column
// group of the tile (128 columns, or 96 at BN = 192) row-major in LDS, and
// thread t rounds row t's fp32 sums once to bf16 and stores them with 16-byte
// writes.  Columns past N are computed on zero rows of W and never stored.
#include "gemm_tile.h"

namespace dflash {

template <int BN, bool TAIL>
__global__ __launch_bounds__(GT_THREADS, 1) void linear_tiles(const uint16_t* __restrict__ X,
                                                              const uint16_t* __restrict__ W, int M, int N, int K,
                                                              int nM, int ntiles, uint16_t* __restrict__ Y,
                                                              int64_t ldy) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[GT_SMEM];
    float* stage = reinterpret_cast<float*>(smem);
    int m_tile, n_tile;
    if (!gemm_tile_index(ntiles, nM, m_tile, n_tile)) return;
    const int m0 = m_tile * GT_BM;
    const int n0 = n_tile * BN;
    const int my_row = m0 + (int)threadIdx.x;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(X + (int64_t)m0 * K), (short)0, min(GT_BM, M - m0) * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (int64_t)n0 * K), (short)0, min(BN, N - n0) * K * 2, 0x00020000);
    f32x16 acc[4][BN / 64];
    gemm_tile_mainloop<BN, TAIL>(smem, rsA, rsB, K, acc);

    constexpr int GW = gemm_tile_group<BN>();
#pragma unroll
    for (int pass = 0; pass < BN / GW; ++pass) {
        const int c0 = n0 + pass * GW;
        if (c0 >= N) break;  // uniform: the tile's last groups past N
        gemm_tile_stage<BN>(stage, acc, pass);
        if (my_row < M) {
            const float* rowp = stage + threadIdx.x * GT_SP;
            uint16_t* dst = Y + (int64_t)my_row * ldy + c0;
            const int nch = min(GW, N - c0) / 8;  // N % 8 == 0
#pragma unroll 4
            for (int c = 0; c < nch; ++c) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(rowp + 8 * c);
                const f32x4 b = *reinterpret_cast<const f32x4*>(rowp + 8 * c + 4);
                stg16(dst + 8 * c, u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                                         pack_bf16x2(b[2], b[3])});
            }
        }
        gemm_tile_pass_done();
    }
}

}  // namespace dflash

using namespace dflash;

extern "C" int dflash_linear(const uint16_t* X, const uint16_t* W, int64_t M, int64_t N, int64_t K, uint16_t* Y,
                             int64_t ldy, void* stream) {
    if (!X || !W || !Y || !DFLASH_ALIGNED16(X) || !DFLASH_ALIGNED16(W) || !DFLASH_ALIGNED16(Y))
        return DFLASH_ERR_INVALID_ARG;
    if (M < 1 || N < 1 || K < 1 || ldy < N) return DFLASH_ERR_INVALID_ARG;
    if (N % 8 != 0 || K % 8 != 0 || ldy % 8 != 0) return DFLASH_ERR_UNSUPPORTED;
    if (M > INT32_MAX || N > INT32_MAX || (int64_t)GT_BM * K * 2 > INT32_MAX) return DFLASH_ERR_UNSUPPORTED;
    const int BN = gemm_tile_width(M, N, true);
    const int nM = (int)((M + GT_BM - 1) / GT_BM);
    const int64_t ntiles = (int64_t)nM * ((N + BN - 1) / BN);
    if (ntiles > (int64_t)1 << 28) return DFLASH_ERR_UNSUPPORTED;
    const int per = (int)((ntiles + 7) / 8);
    const dim3 grid((unsigned)(8 * per));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
#define LIN_LAUNCH(BNV, TL)                                                                                   \
    hipLaunchKernelGGL((linear_tiles<BNV, TL>), grid, dim3(GT_THREADS), 0, st, X, W, (int)M, (int)N, (int)K, \
                       nM, (int)ntiles, Y, ldy)
    const bool tail = K % GT_BK != 0;
    if (BN == 256) {
        if (tail) LIN_LAUNCH(256, true);
        else LIN_LAUNCH(256, false);
    } else if (BN == 192) {
        if (tail) LIN_LAUNCH(192, true);
        else LIN_LAUNCH(192, false);
    } else {
        if (tail) LIN_LAUNCH(128, true);
        else LIN_LAUNCH(128, false);
    }
#undef LIN_LAUNCH
    DFLASH_LAUNCH_CHECK();
    return DFLASH_OK;
}

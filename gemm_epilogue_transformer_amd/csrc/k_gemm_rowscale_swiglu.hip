// Second GEMM of the chain with the deferred RMSNorm row scale and the SwiGLU pairwise
// transform in its epilogue.
//
//   z = sw * (h . W^T)  (gamma already folded into W)
//   NONE:   y[m,n] = bf16_rne( r[m] * z[m,n] )
//   SWIGLU: g = r[m] z[m,j],  u = r[m] z[m,F+j],  y[m,j] = bf16_rne( g sigmoid(g) u )
//
// The per-row scale r commutes with the matrix product, so it is applied at the end of
// this GEMM instead of to its input (kucoin page, section "CODA: El epilogo esconde un
// tesoro"); SiLU(gate)*up pairs column j with column F+j, so each block tile loads the
// gate rows [j0, j0+BN/2) AND the up rows [F+j0, F+j0+BN/2) of W: every lane then holds
// the gate and up accumulators of the same (m, j) and the pairwise op is lane-local.
// r multiplies both accumulators BEFORE the SiLU (it commutes with the GEMM, not with
// the nonlinearity).
//
// 8-bit weights (weight-only): W is e4m3 in HBM and decoded exactly to bf16 while it is
// staged into LDS; the MFMA is the bf16 one and sw is applied in the epilogue.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace coda {

template <int BM, int BN, int WAVES_M, int WAVES_N, bool SWIGLU, bool WFP8>
__global__ void __launch_bounds__(kThreads, 2)
k_gemm_rowscale_swiglu(const uint8_t* __restrict__ H, const uint8_t* __restrict__ W,
                       const float* __restrict__ w_scale, const float* __restrict__ R,
                       uint16_t* __restrict__ Y, int M, int N_out, int K, int tiles_m,
                       int tiles_n) {
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    static_assert(!SWIGLU || (TN % 2 == 0), "SwiGLU pairs gate and up blocks");
    // output columns covered by one block tile / one wave
    constexpr int BNO = SWIGLU ? BN / 2 : BN;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BM + BN) * kRowBytes];

    int tile_m, tile_n;
    tile_coords<8>(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, j0 = tile_n * BNO;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const int kbytes = K * 2;                                    // bf16 bytes of a row
    const size_t h_row = static_cast<size_t>(K) * 2;
    const size_t w_row = static_cast<size_t>(K) * (WFP8 ? 1 : 2);
    auto a_ptr = [&](int r) -> const uint8_t* {
        const int m = m0 + r;
        return m < M ? H + static_cast<size_t>(m) * h_row : nullptr;
    };
    auto b_ptr = [&](int r) -> const uint8_t* {
        if (SWIGLU) {
            const int j = j0 + (r < BN / 2 ? r : r - BN / 2);
            if (j >= N_out) return nullptr;
            const int n = r < BN / 2 ? j : N_out + j;
            return W + static_cast<size_t>(n) * w_row;
        }
        const int n = j0 + r;
        return n < N_out ? W + static_cast<size_t>(n) * w_row : nullptr;
    };
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    // SWIGLU: blocks [0, TN/2) = gate rows of this wave, [TN/2, TN) = the matching up rows
    auto b_row = [&](int tn) {
        if (SWIGLU) {
            constexpr int TH = TN / 2;
            return (tn < TH ? 0 : BN / 2) + wn * TH * 32 + (tn % TH) * 32;
        }
        return wn * WN + tn * 32;
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    using BStage = typename std::conditional<WFP8, PanelStageE4m3ToBf16<BN>, PanelStage<BN>>::type;
    PanelStage<BM> sa;
    BStage sb;
    const int nk = (kbytes + kRowBytes - 1) / kRowBytes;
    if (nk > 0) {
        sa.load(a_ptr, 0, kbytes);
        sb.load(b_ptr, 0, kbytes);
        sa.store(smem[0]);
        sb.store(smem[0] + BM * kRowBytes);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            sa.load(a_ptr, (kt + 1) * kRowBytes, kbytes);
            sb.load(b_ptr, (kt + 1) * kRowBytes, kbytes);
        }
        WaveMma<Elt::BF16, TM, TN>::run(acc, smem[cur], smem[cur] + BM * kRowBytes, a_row, b_row);
        if (kt + 1 < nk) {
            sa.store(smem[cur ^ 1]);
            sb.store(smem[cur ^ 1] + BM * kRowBytes);
        }
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue ----
    const float sw = w_scale ? *w_scale : 1.0f;
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        float rr[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + wm * WM + tm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
            rr[i] = m < M ? R[m] * sw : 0.0f;
        }
        if (SWIGLU) {
            constexpr int TH = TN / 2;
#pragma unroll
            for (int g = 0; g < TH; ++g) {
                const int j = j0 + wn * TH * 32 + g * 32 + lr;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + wm * WM + tm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                    if (m < M && j < N_out) {
                        const float gv = acc[tm][g][i] * rr[i];
                        const float uv = acc[tm][g + TH][i] * rr[i];
                        const float silu = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
                        Y[static_cast<size_t>(m) * N_out + j] = f32_to_bf16_bits(silu * uv);
                    }
                }
            }
        } else {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int n = j0 + wn * WN + tn * 32 + lr;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + wm * WM + tm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                    if (m < M && n < N_out)
                        Y[static_cast<size_t>(m) * N_out + n] = f32_to_bf16_bits(acc[tm][tn][i] * rr[i]);
                }
            }
        }
    }
}

constexpr int BM3 = 128, BN3 = 128;

int64_t gemm3_tiles(int64_t M, int64_t N_out, bool swiglu) {
    const int64_t bno = swiglu ? BN3 / 2 : BN3;
    return ((M + BM3 - 1) / BM3) * ((N_out + bno - 1) / bno);
}

template <bool SWIGLU, bool WFP8>
static hipError_t launch3(int M, int N_out, int K, const void* h, const void* W,
                          const float* w_scale, const float* r, void* y, hipStream_t stream) {
    constexpr int BNO = SWIGLU ? BN3 / 2 : BN3;
    const int tiles_m = (M + BM3 - 1) / BM3, tiles_n = (N_out + BNO - 1) / BNO;
    const dim3 grid(tiles_m * tiles_n), block(kThreads);
    hipLaunchKernelGGL((k_gemm_rowscale_swiglu<BM3, BN3, 2, 2, SWIGLU, WFP8>), grid, block, 0,
                       stream, static_cast<const uint8_t*>(h), static_cast<const uint8_t*>(W),
                       w_scale, r, static_cast<uint16_t*>(y), M, N_out, K, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_gemm_rowscale_swiglu(int M, int N_out, int K, bool swiglu, const void* h,
                                       const void* W, bool w_fp8, const float* w_scale,
                                       const float* r, void* y, hipStream_t stream) {
    if (swiglu)
        return w_fp8 ? launch3<true, true>(M, N_out, K, h, W, w_scale, r, y, stream)
                     : launch3<true, false>(M, N_out, K, h, W, w_scale, r, y, stream);
    return w_fp8 ? launch3<false, true>(M, N_out, K, h, W, w_scale, r, y, stream)
                 : launch3<false, false>(M, N_out, K, h, W, w_scale, r, y, stream);
}

}  // namespace coda

// First GEMM of the chain with its residual + partial-RMS epilogue.
//
//   v[m,n] = sa*sw * sum_k A[m,k] W[n,k] + x_res[m,n];   h = bf16_rne(v)
//   P[m,t] = sum over the tile's columns n of h[m,n]^2   (one fp32 partial per row and
//            N-tile, reduced in a fixed order: in lane, across the 32 lanes of a row,
//            then across the waves that share the row)
//
// The output tile never leaves the chip between the accumulate and the epilogue (kucoin
// page, section "CODA: El epilogo esconde un tesoro": the matrix product's result still
// lives in registers when the epilogue runs; RMSNorm only needs a PARTIAL root mean
// square at the end of the first GEMM, here the combinable sum of squares).
#include "gemm_core.hpp"
#include "launch.hpp"

namespace coda {

template <int BM, int BN, int WAVES_M, int WAVES_N, Elt E>
__global__ void __launch_bounds__(kThreads, 2)
k_gemm_resid_partialrms(const uint8_t* __restrict__ A, const uint8_t* __restrict__ W,
                        const float* __restrict__ a_scale, const float* __restrict__ w_scale,
                        const uint16_t* x_res, uint16_t* h, float* __restrict__ P,
                        int M, int N, int K, int tiles_m, int tiles_n) {
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int EB = EltInfo<E>::kBytes;
    static_assert(WAVES_M * WAVES_N * kWave == kThreads, "4 waves");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BM + BN) * kRowBytes];
    __shared__ float red[WAVES_N][BM];

    int tile_m, tile_n;
    tile_coords<8>(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const size_t kbytes_row = static_cast<size_t>(K) * EB;
    const int kbytes = K * EB;
    auto a_ptr = [&](int r) -> const uint8_t* {
        const int m = m0 + r;
        return m < M ? A + static_cast<size_t>(m) * kbytes_row : nullptr;
    };
    auto b_ptr = [&](int r) -> const uint8_t* {
        const int n = n0 + r;
        return n < N ? W + static_cast<size_t>(n) * kbytes_row : nullptr;
    };
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    auto b_row = [&](int tn) { return wn * WN + tn * 32; };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    PanelStage<BM> sa;
    PanelStage<BN> sb;
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
        WaveMma<E, TM, TN>::run(acc, smem[cur], smem[cur] + BM * kRowBytes, a_row, b_row);
        if (kt + 1 < nk) {
            sa.store(smem[cur ^ 1]);
            sb.store(smem[cur ^ 1] + BM * kRowBytes);
        }
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue ----
    const float scale = (a_scale ? *a_scale : 1.0f) * (w_scale ? *w_scale : 1.0f);
    const int lr = lane & 31, lh = lane >> 5;
    float rs[TM][16];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) rs[tm][i] = 0.0f;

#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int n = n0 + wn * WN + tn * 32 + lr;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + wm * WM + tm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                if (m < M && n < N) {
                    const size_t off = static_cast<size_t>(m) * N + n;
                    float v = acc[tm][tn][i] * scale;
                    if (x_res) v += bf16_bits_to_f32(x_res[off]);
                    const uint16_t hb = f32_to_bf16_bits(v);
                    h[off] = hb;
                    const float q = bf16_bits_to_f32(hb);
                    rs[tm][i] += q * q;
                }
            }
        }
    // sum over the 32 lanes that hold one row's columns
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v = rs[tm][i];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 8, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 1, 64);
            rs[tm][i] = v;
        }
    if (lr == 0) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red[wn][wm * WM + tm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3)] = rs[tm][i];
    }
    __syncthreads();
    const int T = tiles_n;
    for (int r = threadIdx.x; r < BM; r += kThreads) {
        const int m = m0 + r;
        if (m < M) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES_N; ++w) s += red[w][r];
            P[static_cast<size_t>(m) * T + tile_n] = s;
        }
    }
}

// Tile configuration of the first GEMM.  The partial count per row is the number of
// N-tiles, so it is fixed by BN1.
constexpr int BM1 = 128, BN1 = 128;

int64_t partials_per_row(int64_t N) { return N < 1 ? -1 : (N + BN1 - 1) / BN1; }

int64_t gemm1_tiles(int64_t M, int64_t N) { return ((M + BM1 - 1) / BM1) * ((N + BN1 - 1) / BN1); }

hipError_t launch_gemm_resid_partialrms(int M, int N, int K, const void* A, bool fp8,
                                        const float* a_scale, const void* W,
                                        const float* w_scale, const void* x_res, void* h,
                                        float* P, hipStream_t stream) {
    const int tiles_m = (M + BM1 - 1) / BM1, tiles_n = (N + BN1 - 1) / BN1;
    const dim3 grid(tiles_m * tiles_n), block(kThreads);
    if (fp8) {
        hipLaunchKernelGGL((k_gemm_resid_partialrms<BM1, BN1, 2, 2, Elt::E4M3>), grid, block, 0,
                           stream, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(W),
                           a_scale, w_scale, static_cast<const uint16_t*>(x_res),
                           static_cast<uint16_t*>(h), P, M, N, K, tiles_m, tiles_n);
    } else {
        hipLaunchKernelGGL((k_gemm_resid_partialrms<BM1, BN1, 2, 2, Elt::BF16>), grid, block, 0,
                           stream, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(W),
                           a_scale, w_scale, static_cast<const uint16_t*>(x_res),
                           static_cast<uint16_t*>(h), P, M, N, K, tiles_m, tiles_n);
    }
    return hipGetLastError();
}

}  // namespace coda

// Input-gradient GEMM of the MLP-input block with the RMSNorm backward in its epilogue.
//
//   acc[m,n] = sum_k dz[m,k] W'[k,n]           (dz = r * dL/dz from the SwiGLU backward,
//                                               W'^T passed K-contiguous as Wt[n,k])
//   dh[m,n]  = bf16_rne( acc[m,n] + q[m] * h[m,n] + dh_res[m,n] )
//
// with q = -(r^3/N) * dL/dr from the light reduction.  Through the row scale the
// gradient of h has a per-row rank-one correction along h itself; like the forward's
// row scale it is applied in the epilogue of the GEMM that produces the other term
// (kucoin page, section "CODA: El epilogo esconde un tesoro": the reparameterisation
// holds for the backward pass).  dh_res is the gradient that reaches h through the
// residual stream (may be NULL).  With h and q both NULL the same kernel is the plain
// product C = A . B^T (+ C_res) in bf16: the first GEMM's input gradient.  Mainloop and tiles as the first GEMM; per 32-row slab
// the accumulators are staged row-major in LDS and every lane takes runs of 8 columns:
// 16-byte loads of h and dh_res (one slab ahead), fp32 arithmetic, one bf16 rounding,
// one 16-byte store.  RING: the mainloop on LDS stage rings (three stages of the dz
// panel, which streams from HBM, two of the weight panel; mainloop_dma_ring), whose 160 KB
// then also hold the epilogue's slabs.
#include "epilogue.hpp"
#include "gemm_pipeline.hpp"
#include "launch.hpp"

namespace coda {

// Tile-rows per group of the tile walk (tile_coords): 4 rather than 8 was 1-4 % faster on
// the 16K-token shapes (11 % on the 8-bit first GEMM); outputs do not depend on the walk.
#ifndef CODA_B2_GROUP
#define CODA_B2_GROUP 4
#endif

template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int RB, int SPREAD, int OCC, bool RING>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, OCC)
k_gemm_rmsnorm_bwd(const uint8_t* __restrict__ DZ, const uint8_t* __restrict__ WT, const uint16_t* Hb,
                   const float* __restrict__ Q, const uint16_t* DHres, uint16_t* DH, int M, int N, int K,
                   int tiles_m, int tiles_n) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;

    constexpr int kStage = (BM + BN) * RB;
    using S = Slab<TN>;
    const int wave = threadIdx.x >> 6;
    uint8_t* st[NS];          // shared stages (RING = false)
    uint8_t* sa[3];           // the rings (RING = true)
    uint8_t* sb[2];
    uint8_t* slab;            // this wave's epilogue slab
    if constexpr (RING) {
        __shared__ __attribute__((aligned(1024))) uint8_t rings[3 * BM * RB + 2 * BN * RB];
        static_assert(NW * S::kBytes <= 3 * BM * RB + 2 * BN * RB, "the slabs fit the rings");
#pragma unroll
        for (int i = 0; i < 3; ++i) sa[i] = rings + i * BM * RB;
#pragma unroll
        for (int i = 0; i < 2; ++i) sb[i] = rings + 3 * BM * RB + i * BN * RB;
        slab = rings + wave * S::kBytes;
    } else {
        __shared__ __attribute__((aligned(1024))) uint8_t stages[NS][kStage];
#pragma unroll
        for (int i = 0; i < NS; ++i) st[i] = stages[i];
        slab = slab_region<NS, NW, kStage, S::kBytes>(st, wave);
    }

    int tile_m, tile_n;
    tile_coords<CODA_B2_GROUP>(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // q of this wave's rows (lane l: rows l, 64 + l, ...); rows past M hold 0
    static_assert(WM % 64 == 0, "each lane holds WM / 64 row coefficients");
    float qv[WM / 64];
#pragma unroll
    for (int i = 0; i < WM / 64; ++i) {
        const int m = m0 + wm * WM + 64 * i + (threadIdx.x & 63);
        qv[i] = (Q != nullptr && m < M) ? Q[m] : 0.0f;
    }

    const int kbytes = K * 2;
    DmaPanel<BM, BM, NW, RB> pa;
    DmaPanel<BN, BN, NW, RB> pb;
    const uint8_t* a0 = DZ + static_cast<size_t>(m0) * kbytes;
    const uint8_t* b0 = WT + static_cast<size_t>(n0) * kbytes;
    pa.init(a0, min(BM, M - m0), a0, 0, kbytes);
    pb.init(b0, min(BN, N - n0), b0, 0, kbytes);
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    auto b_row = [&](int tn) { return wn * WN + tn * 32; };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if constexpr (RING)
        mainloop_dma_ring<Elt::BF16, BM, BN, NW, RB, SPREAD>(acc, pa, pb, kbytes, sa, sb, a_row, b_row);
    else
        mainloop_dma<Elt::BF16, BM, BN, BN, NS, NW, RB, SPREAD>(acc, pa, pb, kbytes, st, a_row, b_row);

    const int valid_rows = min(BM, M - m0);
    const uint32_t row_bytes = static_cast<uint32_t>(N) * 2;
    const size_t tile_off = static_cast<size_t>(m0) * N;
    const __amdgpu_buffer_rsrc_t h_rsrc =
        make_buffer_rsrc(Hb ? Hb + tile_off : DH + tile_off, Hb ? valid_rows * row_bytes : 0u);
    const __amdgpu_buffer_rsrc_t r_rsrc =
        make_buffer_rsrc(DHres ? DHres + tile_off : Hb + tile_off, DHres ? valid_rows * row_bytes : 0u);
    const __amdgpu_buffer_rsrc_t o_rsrc = make_buffer_rsrc(DH + tile_off, valid_rows * row_bytes);
    auto seg_voff = [&](int tm, int j) -> uint32_t {
        const int tr = wm * WM + tm * 32 + S::seg_row(j);
        const int n = n0 + wn * WN + S::seg_col(j);
        return n < N ? static_cast<uint32_t>(tr) * row_bytes + static_cast<uint32_t>(n) * 2 : kOobOffset;
    };
    i32x4_t hv[2][S::kSegPerLane], gv[2][S::kSegPerLane];
    acc_read_fence();
#pragma unroll
    for (int j = 0; j < S::kSegPerLane; ++j) {
        hv[0][j] = __builtin_amdgcn_raw_buffer_load_b128(h_rsrc, seg_voff(0, j), 0, 0);
        gv[0][j] = __builtin_amdgcn_raw_buffer_load_b128(r_rsrc, seg_voff(0, j), 0, 0);
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        if (tm + 1 < TM) {
#pragma unroll
            for (int j = 0; j < S::kSegPerLane; ++j) {
                hv[(tm + 1) & 1][j] = __builtin_amdgcn_raw_buffer_load_b128(h_rsrc, seg_voff(tm + 1, j), 0, 0);
                gv[(tm + 1) & 1][j] = __builtin_amdgcn_raw_buffer_load_b128(r_rsrc, seg_voff(tm + 1, j), 0, 0);
            }
        }
        float v[TN][16];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[tn][i] = acc_read(acc[tm][tn][i]);
        S::put(slab, v);
#pragma unroll
        for (int j = 0; j < S::kSegPerLane; ++j) {
            float t[8];
            S::get(slab, j, t);
            const int row = tm * 32 + S::seg_row(j);
            const float q = __shfl(qv[row / 64], row % 64);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = static_cast<uint32_t>(hv[tm & 1][j][e]);
                const uint32_t y = static_cast<uint32_t>(gv[tm & 1][j][e]);
                const float a0v = t[2 * e] + q * bf16_bits_to_f32(static_cast<uint16_t>(x & 0xFFFFu)) +
                                  bf16_bits_to_f32(static_cast<uint16_t>(y & 0xFFFFu));
                const float a1v = t[2 * e + 1] + q * bf16_bits_to_f32(static_cast<uint16_t>(x >> 16)) +
                                  bf16_bits_to_f32(static_cast<uint16_t>(y >> 16));
                o[e] = pack_bf16x2(a0v, a1v);
            }
            __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(o[0]), int(o[1]), int(o[2]), int(o[3])}, o_rsrc,
                                                   seg_voff(tm, j), 0, 0);
        }
    }
}

// Tile configuration (the first GEMM's).
#ifndef CODA_B2_BM
#define CODA_B2_BM 256
#define CODA_B2_BN 256
#define CODA_B2_WM 2
#define CODA_B2_WN 2
#define CODA_B2_NS 2
#define CODA_B2_RB 128
#define CODA_B2_SPREAD 3
#define CODA_B2_OCC 1
#endif
// Contractions of at least this many k run on the stage rings: where dz streams from HBM
// (16384 tokens x 16384 of K: 0.836 against 0.861 ms; K = 128256: 6.46 against 6.66 ms),
// and with the rings' wider DMA spread also at K = 2048 (dA: 0.1245-0.1248 against
// 0.1297-0.1302 ms) and 3072 (0.184 against 0.189 ms); shorter ones keep the two shared
// stages.  Both give the same bits.
#ifndef CODA_B2_RING_MIN_K
#define CODA_B2_RING_MIN_K 2048
#endif
// k-steps a k-tile's DMA is spread over on the rings (on the shared stages: CODA_B2_SPREAD;
// 4 there made dA 7 % slower, 4 on the rings is 0.2-0.8 % faster than 3)
#ifndef CODA_B2_SPREAD_RING
#define CODA_B2_SPREAD_RING 4
#endif
constexpr int BMB = CODA_B2_BM, BNB = CODA_B2_BN;

int64_t gemm_bwd2_tiles(int64_t M, int64_t N) { return ((M + BMB - 1) / BMB) * ((N + BNB - 1) / BNB); }

hipError_t launch_gemm_rmsnorm_bwd(int M, int N, int K, const void* dz, const void* Wt, const void* h,
                                   const float* q, const void* dh_res, void* dh, hipStream_t stream) {
    const int tiles_m = (M + BMB - 1) / BMB, tiles_n = (N + BNB - 1) / BNB;
    const dim3 grid(tiles_m * tiles_n), block(64 * CODA_B2_WM * CODA_B2_WN);
    if (K >= CODA_B2_RING_MIN_K)
        hipLaunchKernelGGL((k_gemm_rmsnorm_bwd<BMB, BNB, CODA_B2_WM, CODA_B2_WN, CODA_B2_NS, CODA_B2_RB,
                                               CODA_B2_SPREAD_RING, CODA_B2_OCC, true>),
                           grid, block, 0, stream, static_cast<const uint8_t*>(dz), static_cast<const uint8_t*>(Wt),
                           static_cast<const uint16_t*>(h), q, static_cast<const uint16_t*>(dh_res),
                           static_cast<uint16_t*>(dh), M, N, K, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((k_gemm_rmsnorm_bwd<BMB, BNB, CODA_B2_WM, CODA_B2_WN, CODA_B2_NS, CODA_B2_RB,
                                               CODA_B2_SPREAD, CODA_B2_OCC, false>),
                           grid, block, 0, stream, static_cast<const uint8_t*>(dz), static_cast<const uint8_t*>(Wt),
                           static_cast<const uint16_t*>(h), q, static_cast<const uint16_t*>(dh_res),
                           static_cast<uint16_t*>(dh), M, N, K, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace coda

// First GEMM of the chain with its residual + partial-RMS epilogue.
//
//   v[m,n] = sa*sw * sum_k A[m,k] W[n,k] + x_res[m,n];   h = bf16_rne(v)
//   P[m,t] = sum over the tile's columns n of h[m,n]^2   (one fp32 partial per row and
//            N-tile, reduced in a fixed order: 8 columns in lane, a DPP all-reduce over the
//            lanes that hold one row of a wave's slab, then the waves sharing the row)
//
// The output tile never leaves the chip between the accumulate and the epilogue (kucoin
// page, section "CODA: El epilogo esconde un tesoro": the matrix product's result still
// lives in registers when the epilogue runs; RMSNorm only needs a PARTIAL root mean
// square at the end of the first GEMM, here the combinable sum of squares).
#include "epilogue.hpp"
#include "gemm_pipeline.hpp"
#include "launch.hpp"

namespace coda {

// Tile-rows per group of the tile walk (tile_coords): 4 rather than 8 was 1-4 % faster on
// the 16K-token shapes (11 % on the 8-bit first GEMM); outputs do not depend on the walk.
// The residual prefetch on the stage rings (XresPrefetchRing): off.  With the walk in
// groups of 4 tile-rows it no longer pays (one machine each, alternating, bits equal): the
// 16K-token attention output 0.1248-0.1252 against 0.1250-0.1251 ms without and with it,
// the 8192-deep MLP output 0.4115-0.4125 against 0.4163-0.4166 ms, the 8-bit form
// 0.0740-0.0748 against 0.0755-0.0756 ms.
#ifndef CODA_G1_XPF
#define CODA_G1_XPF 0
#endif
#ifndef CODA_G1_GROUP
#define CODA_G1_GROUP 4
#endif

// Prefetch of the residual tile during the mainloop.  In the epilogue every workgroup
// reads its 256 x 256 residual tile (128 KB) at the same moment, a burst from HBM that no
// MFMA work overlaps; read once during the last k-tiles instead (into a junk LDS block:
// only the cache fill matters), the epilogue finds it in the last-level cache.  Wave w
// takes tile rows 64w .. 64w+63, two rows (1 KB) per instruction, P instructions per k-tile
// over the last 32 / P k-tiles; on earlier k-tiles, and without a residual, the
// instructions address past the descriptor's range (zeros, no traffic), so that every
// k-tile issues the same count.
template <int P>
struct XresPrefetch {
    static constexpr int kOps = P;
    static constexpr int kInst = 32;      // instructions per wave for 64 rows of 512 bytes
    u32x4_t rsrc;
    uint32_t lane_off;                    // this lane's byte offset in instruction 0
    uint32_t inst_step;                   // bytes between instructions (two rows)
    uint32_t junk;                        // LDS address of the wave's junk block
    __device__ __forceinline__ void issue(int kt, int nk) const {
        const int i0 = (kt - (nk - kInst / P)) * P;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = i0 + p;
            const uint32_t voff = (i >= 0 && i < kInst) ? lane_off + static_cast<uint32_t>(i) * inst_step : kOob;
            dma16(rsrc, voff, junk);
        }
    }
    // The same loads into a freed A stage of the ring mainloop: load p into the 1 KB that
    // this wave's A DMA instruction p fills (rows (NW p + wave) * 8 of 128-byte rows).
    template <int NW>
    __device__ __forceinline__ void issue_stage(int kt, int nk, uint8_t* stage) const {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int i0 = (kt - (nk - kInst / P)) * P;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = i0 + p;
            const uint32_t voff = (i >= 0 && i < kInst) ? lane_off + static_cast<uint32_t>(i) * inst_step : kOob;
            dma16(rsrc, voff, lds_addr(stage + (NW * p + wave) * 1024));
        }
    }
};

// XresPrefetch for the ring mainloop (its hook names the stage).
template <int P, int NW>
struct XresPrefetchRing : XresPrefetch<P> {
    __device__ __forceinline__ void issue_into(int kt, int nk, uint8_t* stage) const {
        this->template issue_stage<NW>(kt, nk, stage);
    }
};

// RING: the mainloop with three A stages and two B stages (mainloop_dma_ring), which take
// the whole LDS: the residual prefetch then loads into the A stage each crossing frees
// (XresPrefetchRing), and the epilogue's row sums live behind the slabs in the stage
// memory.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int RB, int SPREAD, int OCC, bool RING, Elt E>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, OCC)
k_gemm_resid_partialrms(const uint8_t* __restrict__ A, const uint8_t* __restrict__ W,
                        const float* __restrict__ a_scale, const float* __restrict__ w_scale,
                        const uint16_t* x_res, uint16_t* h, float* __restrict__ P,
                        int M, int N, int K, int tiles_m, int tiles_n) {
    constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int EB = EltInfo<E>::kBytes;

    constexpr int kStage = (BM + BN) * RB;
    using S = Slab<TN>;
    uint8_t* st[NS];          // shared stages (RING = false)
    uint8_t* sa[3];           // the rings (RING = true)
    uint8_t* sb[2];
    float* red;               // [WAVES_N][BM] row sums of the epilogue
    uint8_t* slab;            // this wave's epilogue slab
    uint8_t* junk = nullptr;  // this wave's 1 KB block for the residual prefetch
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if constexpr (RING) {
        __shared__ __attribute__((aligned(1024))) uint8_t rings[3 * BM * RB + 2 * BN * RB];
        static_assert(NW * S::kBytes + WAVES_N * BM * 4 <= 3 * BM * RB + 2 * BN * RB, "slabs and row sums fit");
#pragma unroll
        for (int i = 0; i < 3; ++i) sa[i] = rings + i * BM * RB;
#pragma unroll
        for (int i = 0; i < 2; ++i) sb[i] = rings + 3 * BM * RB + i * BN * RB;
        slab = rings + wave * S::kBytes;
        red = reinterpret_cast<float*>(rings + NW * S::kBytes);
    } else {
        __shared__ __attribute__((aligned(1024))) uint8_t stages[NS][kStage];
        __shared__ float red_s[WAVES_N][BM];
        __shared__ __attribute__((aligned(1024))) uint8_t junk_s[NW][1024];
#pragma unroll
        for (int i = 0; i < NS; ++i) st[i] = stages[i];
        slab = slab_region<NS, NW, kStage, S::kBytes>(st, wave);
        red = &red_s[0][0];
        junk = junk_s[wave];
    }

    int tile_m, tile_n;
    tile_coords<CODA_G1_GROUP>(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const int kbytes = K * EB;
    DmaPanel<BM, BM, NW, RB> pa;
    DmaPanel<BN, BN, NW, RB> pb;
    const uint8_t* a0 = A + static_cast<size_t>(m0) * kbytes;
    const uint8_t* b0 = W + static_cast<size_t>(n0) * kbytes;
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

    // the residual tile's cache fill during the last k-tiles (1 KB per wave and k-tile for
    // bf16 operands, 2 KB for the 8-bit ones, whose k-tiles are half as many)
    static_assert(BM == 64 * NW && BN == 256, "the prefetch covers 256 columns of 64 rows per wave");
    XresPrefetchRing<E == Elt::E4M3 ? 2 : 1, NW> xpf;
    {
        const uint32_t rb = static_cast<uint32_t>(N) * 2;
        xpf.rsrc = make_rsrc(x_res ? x_res + static_cast<size_t>(m0) * N : h,
                             x_res ? static_cast<uint32_t>(min(BM, M - m0)) * rb : 0u);
        xpf.lane_off = static_cast<uint32_t>(64 * wave + (lane >> 5)) * rb + static_cast<uint32_t>(n0) * 2u +
                       static_cast<uint32_t>(lane & 31) * 16u;
        xpf.inst_step = __builtin_amdgcn_readfirstlane(2u * rb);
        if constexpr (!RING) xpf.junk = __builtin_amdgcn_readfirstlane(lds_addr(junk));
    }
    if constexpr (RING && CODA_G1_XPF)
        mainloop_dma_ring<E, BM, BN, NW, RB, SPREAD>(acc, pa, pb, kbytes, sa, sb, a_row, b_row, xpf);
    else if constexpr (RING)
        mainloop_dma_ring<E, BM, BN, NW, RB, SPREAD>(acc, pa, pb, kbytes, sa, sb, a_row, b_row, NoExtra{});
    else
        mainloop_dma<E, BM, BN, BN, NS, NW, RB, SPREAD>(acc, pa, pb, kbytes, st, a_row, b_row, xpf);

    // ---------------------------------------------------------------- epilogue ----
    // Per 32-row slab of this wave: stage scale*acc row-major in the wave's own (now
    // free) LDS stage, then each lane takes runs of 8 columns: 16-byte residual load,
    // fp32 add, one bf16 rounding, 16-byte store of h, and the sum of the 8 squares.
    // Row sums: 16 lanes hold one slab row -> DPP all-reduce over them -> per-wave partial in
    // `red`, then the WAVES_N waves sharing a row are added in a fixed order.
    const float scale = (a_scale ? *a_scale : 1.0f) * (w_scale ? *w_scale : 1.0f);
    const int valid_rows = min(BM, M - m0);
    const uint32_t row_bytes = static_cast<uint32_t>(N) * 2;
    const size_t tile_off = static_cast<size_t>(m0) * N;
    const __amdgpu_buffer_rsrc_t xr_rsrc =
        make_buffer_rsrc(x_res ? x_res + tile_off : h + tile_off, x_res ? valid_rows * row_bytes : 0u);
    const __amdgpu_buffer_rsrc_t h_rsrc = make_buffer_rsrc(h + tile_off, valid_rows * row_bytes);
    // residual loads of slab tm+1 are in flight while slab tm is processed
    auto seg_voff = [&](int tm, int j) -> uint32_t {
        const int tr = wm * WM + tm * 32 + S::seg_row(j);
        const int n = n0 + wn * WN + S::seg_col(j);
        return n < N ? static_cast<uint32_t>(tr) * row_bytes + static_cast<uint32_t>(n) * 2 : kOobOffset;
    };
    // accumulators are read at their use (acc_read): plain reads had the compiler spill 8
    // of them after the mainloop, and the reloads' vmcnt waits in the last slab then
    // waited for every h store and residual load before them
    acc_read_fence();
    i32x4_t xr[2][S::kSegPerLane];
#pragma unroll
    for (int j = 0; j < S::kSegPerLane; ++j)
        xr[0][j] = __builtin_amdgcn_raw_buffer_load_b128(xr_rsrc, seg_voff(0, j), 0, 0);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        if (tm + 1 < TM) {
#pragma unroll
            for (int j = 0; j < S::kSegPerLane; ++j)
                xr[(tm + 1) & 1][j] = __builtin_amdgcn_raw_buffer_load_b128(xr_rsrc, seg_voff(tm + 1, j), 0, 0);
        }
        float v[TN][16];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[tn][i] = acc_read(acc[tm][tn][i]) * scale;
        S::put(slab, v);
#pragma unroll
        for (int j = 0; j < S::kSegPerLane; ++j) {
            float t[8];
            S::get(slab, j, t);
            float sq = 0.0f;
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = static_cast<uint32_t>(xr[tm & 1][j][e]);
                o[e] = pack_bf16x2(t[2 * e] + bf16_bits_to_f32(static_cast<uint16_t>(x & 0xFFFFu)),
                                   t[2 * e + 1] + bf16_bits_to_f32(static_cast<uint16_t>(x >> 16)));
                const float q0 = __uint_as_float(o[e] << 16), q1 = __uint_as_float(o[e] & 0xFFFF0000u);
                sq += q0 * q0;
                sq += q1 * q1;
            }
            __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(o[0]), int(o[1]), int(o[2]), int(o[3])},
                                                   h_rsrc, seg_voff(tm, j), 0, 0);
            // columns past N contribute nothing (their residual reads and sums are zero)
            sq = group_allreduce<S::kSegPerRow>(sq, AddOp());
            if ((lane & (S::kSegPerRow - 1)) == 0) red[wn * BM + wm * WM + tm * 32 + S::seg_row(j)] = sq;
        }
    }
    __syncthreads();
    const int T = tiles_n;
    for (int r = threadIdx.x; r < BM; r += NT) {
        const int m = m0 + r;
        if (m < M) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES_N; ++w) s += red[w * BM + r];
            P[static_cast<size_t>(m) * T + tile_n] = s;
        }
    }
}

// Tile configuration of the first GEMM (compile-time).  The partial count per row is the
// number of N-tiles, so it is fixed by BN1.
#ifndef CODA_G1_BM
#define CODA_G1_BM 256
#define CODA_G1_BN 256
#define CODA_G1_WM 2
#define CODA_G1_WN 2
#define CODA_G1_NS 2
#define CODA_G1_RB 128
#define CODA_G1_OCC 1
#endif
// k-steps a k-tile's DMA is spread over (on the rings 4: 135.8-138.1 against 139.4-140.8 us
// for 3 and 145.8-147.2 for 2 inside the chain; the 8-bit k-tiles have two k-steps)
#ifndef CODA_G1_SPREAD
#define CODA_G1_SPREAD 4
#endif
#ifndef CODA_G1_RING
#define CODA_G1_RING 1
#endif
constexpr int BM1 = CODA_G1_BM, BN1 = CODA_G1_BN, NS1 = CODA_G1_NS, OCC1 = CODA_G1_OCC;
constexpr int RB1 = CODA_G1_RB;
// the 8-bit mainloop has one MFMA k-step per 64-byte k-tile: it needs an even stage count
constexpr int NS1_8 = (RB1 == 64 && NS1 % 2) ? NS1 + 1 : NS1;
constexpr int WM1 = CODA_G1_WM, WN1 = CODA_G1_WN;
// k-steps the DMA of a k-tile is spread over (at most the k-steps of a k-tile: RB/32 for
// bf16, RB/64 for e4m3)
constexpr int SP1 = CODA_G1_SPREAD, SP1_8 = SP1 < RB1 / 64 ? SP1 : RB1 / 64;

int64_t partials_per_row(int64_t N) { return N < 1 ? -1 : (N + BN1 - 1) / BN1; }

int64_t gemm1_tiles(int64_t M, int64_t N) { return ((M + BM1 - 1) / BM1) * ((N + BN1 - 1) / BN1); }

hipError_t launch_gemm_resid_partialrms(int M, int N, int K, const void* A, bool fp8,
                                        const float* a_scale, const void* W,
                                        const float* w_scale, const void* x_res, void* h,
                                        float* P, hipStream_t stream) {
    const int tiles_m = (M + BM1 - 1) / BM1, tiles_n = (N + BN1 - 1) / BN1;
    const dim3 grid(tiles_m * tiles_n), block(64 * WM1 * WN1);
    if (fp8) {
        hipLaunchKernelGGL((k_gemm_resid_partialrms<BM1, BN1, WM1, WN1, NS1_8, RB1, SP1_8, OCC1, CODA_G1_RING != 0, Elt::E4M3>), grid, block, 0,
                           stream, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(W),
                           a_scale, w_scale, static_cast<const uint16_t*>(x_res),
                           static_cast<uint16_t*>(h), P, M, N, K, tiles_m, tiles_n);
    } else {
        hipLaunchKernelGGL((k_gemm_resid_partialrms<BM1, BN1, WM1, WN1, NS1, RB1, SP1, OCC1, CODA_G1_RING != 0, Elt::BF16>), grid, block, 0,
                           stream, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(W),
                           a_scale, w_scale, static_cast<const uint16_t*>(x_res),
                           static_cast<uint16_t*>(h), P, M, N, K, tiles_m, tiles_n);
    }
    return hipGetLastError();
}

}  // namespace coda

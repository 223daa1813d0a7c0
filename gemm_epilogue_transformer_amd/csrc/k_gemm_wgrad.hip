// Weight-gradient GEMM (a sum over the tokens) with a column-scale epilogue and the
// column partials of the RMSNorm-weight gradient.
//
//   G[j,k]   = sum_m At[j,m] Bt[k,m]            (At = (r * dL/dz)^T, Bt = h^T: both passed
//                                                token-contiguous, so the mainloop is the
//                                                forward's)
//   dW[j,k]  = gamma[k] * G[j,k]                 (fp32; gamma NULL: 1)
//   Pg[t,k]  = sum over the rows j of tile t of W[j,k] * G[j,k]   (only when W is given)
//
// For the block y = SwiGLU(RMSNorm(h) . W^T) with the folded weight W' = gamma * W,
// dL/dW = gamma * G and dL/dgamma[k] = sum_j W[j,k] G[j,k]: the vector operand gamma is
// broadcast over the columns and the gamma gradient is a block reduction in the
// epilogue, the forward's primitives (kucoin page, section "Cinco bloques y un lenguaje
// LEGO"; section "CODA: El epilogo esconde un tesoro": the backward pass inherits the
// forward's structure).  Per 32-row slab: accumulators staged row-major in LDS, each
// lane takes runs of 8 columns; the column sums run over the lane's rows, the 4 lanes
// holding the same columns, then the waves sharing them, in a fixed order.
#include <algorithm>
#include <mutex>

#include "epilogue.hpp"
#include "gemm_pipeline.hpp"
#include "launch.hpp"

namespace coda {

// Tile-rows per group of the tile walk (tile_coords): 4 rather than 8 was 1-4 % faster on
// the 16K-token shapes (11 % on the 8-bit first GEMM); outputs do not depend on the walk.
#ifndef CODA_WG_GROUP
#define CODA_WG_GROUP 4
#endif

// Split over the tokens (S > 1): block (s, tile) sums tokens [s * k_split,
// min((s + 1) * k_split, K)) and writes its raw sums (no gamma) to slice s of dW, which
// is then the [S, NR, NC] workspace, and (with W) its partial rows to slice s of an
// [S, tiles_m, NC] workspace region; k_splitk_reduce adds up each in a fixed order.
//
// TOK: the operands are token-major, X [K, lda] and Y [K, ldb] (the activations as the
// forward and backward store them, NR and NC of their columns used), read through LDS
// transpose reads (DmaPanelTok / FragsTok); otherwise token-contiguous At [NR, K] and
// Bt [NC, K] (lda, ldb unused).
template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int RB, int SPREAD, int OCC, bool TOK, bool RING>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, OCC)
k_gemm_wgrad(const uint8_t* __restrict__ At, const uint8_t* __restrict__ Bt, const float* __restrict__ gamma,
             const uint16_t* __restrict__ Wraw, float* __restrict__ dW, float* __restrict__ Pg, int NR, int NC,
             int K, int tiles_m, int tiles_n, int k_split, int lda, int ldb) {
    constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;

    constexpr int kStage = (BM + BN) * RB;
    using S = Slab<TN>;
    static_assert(!RING || TOK, "the stage rings run the token-major panels");
    uint8_t* st[NS];          // shared stages (RING = false)
    uint8_t* sa[3];           // the rings (RING = true): three stages of the A panel, two of B
    uint8_t* sb[2];
    uint8_t* slab;            // this wave's epilogue slab
    float* red;               // [WAVES_M][BN] column partials of the epilogue
    {
        const int w = threadIdx.x >> 6;
        if constexpr (RING) {
            __shared__ __attribute__((aligned(1024))) uint8_t rings[3 * BM * RB + 2 * BN * RB];
            static_assert(NW * S::kBytes + WAVES_M * BN * 4 <= 3 * BM * RB + 2 * BN * RB, "slabs and partials fit");
#pragma unroll
            for (int i = 0; i < 3; ++i) sa[i] = rings + i * BM * RB;
#pragma unroll
            for (int i = 0; i < 2; ++i) sb[i] = rings + 3 * BM * RB + i * BN * RB;
            slab = rings + w * S::kBytes;
            red = reinterpret_cast<float*>(rings + NW * S::kBytes);
        } else {
            __shared__ __attribute__((aligned(1024))) uint8_t stages[NS][kStage];
            __shared__ float red_s[WAVES_M][BN];
#pragma unroll
            for (int i = 0; i < NS; ++i) st[i] = stages[i];
            slab = slab_region<NS, NW, kStage, S::kBytes>(st, w);
            red = &red_s[0][0];
        }
    }

    const int tiles = tiles_m * tiles_n;
    const int split = blockIdx.x / tiles;
    int tile_m, tile_n;
    tile_coords<CODA_WG_GROUP>(blockIdx.x - split * tiles, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const int k0 = split * k_split, ktok = min(k_split, K - k0);   // this block's tokens
    const int kext = ktok * 2;
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    auto b_row = [&](int tn) { return wn * WN + tn * 32; };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if constexpr (TOK) {
        static_assert(BM == 256 && BN == 256 && RB == 128, "token-major panels are 256 columns x 64 tokens");
        // token row k0 of X, column m0 (and of Y, column n0); rows past this block's
        // tokens are outside the descriptors and read zeros
        DmaPanelTok<NW> pa, pb;
        pa.init(At + (static_cast<size_t>(k0) * lda + m0) * 2, ktok, lda * 2, NR - m0);
        pb.init(Bt + (static_cast<size_t>(k0) * ldb + n0) * 2, ktok, ldb * 2, NC - n0);
        if constexpr (RING)
            mainloop_dma_ring_fp<FragPair<FragsTok<TM, TN>>, NW, RB, SPREAD>(acc, pa, pb, kext, sa, sb, a_row, b_row);
        else
            mainloop_dma_fp<FragPair<FragsTok<TM, TN>>, BM, BN, BN, NS, NW, RB, RB, SPREAD>(acc, pa, pb, kext, kext,
                                                                                          st, a_row, b_row);
    } else {
        // rows are K tokens apart; this block reads tokens [k0, k0 + ktok) of each (the
        // descriptors start at token k0, the mainloop stops at kext)
        const int kbytes = K * 2;
        DmaPanel<BM, BM, NW, RB> pa;
        DmaPanel<BN, BN, NW, RB> pb;
        const uint8_t* a0 = At + static_cast<size_t>(m0) * kbytes + static_cast<size_t>(k0) * 2;
        const uint8_t* b0 = Bt + static_cast<size_t>(n0) * kbytes + static_cast<size_t>(k0) * 2;
        pa.init(a0, min(BM, NR - m0), a0, 0, kbytes);
        pb.init(b0, min(BN, NC - n0), b0, 0, kbytes);
        mainloop_dma<Elt::BF16, BM, BN, BN, NS, NW, RB, SPREAD>(acc, pa, pb, kext, st, a_row, b_row);
    }
    dW += static_cast<size_t>(split) * NR * NC;
    if (Wraw) Pg += static_cast<size_t>(split) * tiles_m * NC;   // a token split's own partial rows

    static_assert(64 % S::kSegPerRow == 0, "a lane's segments share their columns");
    const int valid_rows = min(BM, NR - m0);
    const uint32_t wrow = static_cast<uint32_t>(NC) * 2, orow = static_cast<uint32_t>(NC) * 4;
    const __amdgpu_buffer_rsrc_t w_rsrc =
        make_buffer_rsrc(Wraw ? Wraw + static_cast<size_t>(m0) * NC : nullptr, Wraw ? valid_rows * wrow : 0u);
    const __amdgpu_buffer_rsrc_t o_rsrc = make_buffer_rsrc(dW + static_cast<size_t>(m0) * NC, valid_rows * orow);
    const __amdgpu_buffer_rsrc_t g_rsrc = make_buffer_rsrc(gamma, gamma ? static_cast<uint32_t>(NC) * 4 : 0u);
    // this lane's 8 columns (the same for all its segments) and their gamma
    const int col = n0 + wn * WN + (lane % S::kSegPerRow) * 8;
    const bool col_in = col < NC;
    float gm[8];
    {
        const uint32_t go = col_in ? static_cast<uint32_t>(col) * 4 : kOobOffset;
        const f32x4_t g0 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, go, 0, 0));
        const f32x4_t g1 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, go + 16, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gm[e] = gamma ? g0[e] : 1.0f;
            gm[4 + e] = gamma ? g1[e] : 1.0f;
        }
    }
    float cs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // raw W of this lane's segments, loaded one 32-row slab ahead (double-buffered) so
    // that its latency overlaps the previous slab's work
    auto w_off = [&](int tm, int j) -> uint32_t {
        const uint32_t tr = static_cast<uint32_t>(wm * WM + tm * 32 + S::seg_row(j));
        return col_in ? tr * wrow + col * 2u : kOobOffset;
    };
    i32x4_t wb[2][S::kSegPerLane];
    acc_read_fence();
    if (Wraw) {
#pragma unroll
        for (int j = 0; j < S::kSegPerLane; ++j) wb[0][j] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_off(0, j), 0, 0);
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        if (Wraw && tm + 1 < TM) {
#pragma unroll
            for (int j = 0; j < S::kSegPerLane; ++j)
                wb[(tm + 1) & 1][j] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_off(tm + 1, j), 0, 0);
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
            const uint32_t tr = static_cast<uint32_t>(wm * WM + tm * 32 + S::seg_row(j));
            const i32x4_t wv = Wraw ? wb[tm & 1][j] : i32x4_t{0, 0, 0, 0};
            f32x4_t o0, o1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o0[e] = gm[e] * t[e];
                o1[e] = gm[4 + e] * t[4 + e];
            }
            const uint32_t oo = col_in ? tr * orow + col * 4u : kOobOffset;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, o0), o_rsrc, oo, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, o1), o_rsrc, oo + 16, 0, 0);
            if (Wraw) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = static_cast<uint32_t>(wv[e]);
                    cs[2 * e] += bf16_bits_to_f32(static_cast<uint16_t>(x & 0xFFFFu)) * t[2 * e];
                    cs[2 * e + 1] += bf16_bits_to_f32(static_cast<uint16_t>(x >> 16)) * t[2 * e + 1];
                }
            }
        }
    }
    if (Wraw) {
        // the lanes that hold the same columns: lane % kSegPerRow equal
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int off = S::kSegPerRow; off < 64; off <<= 1) cs[e] += __shfl_xor(cs[e], off);
        if (lane < S::kSegPerRow) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wm * BN + wn * WN + lane * 8 + e] = cs[e];
        }
        __syncthreads();
        for (int c = threadIdx.x; c < BN; c += NT) {
            const int k = n0 + c;
            if (k < NC) {
                float s = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES_M; ++w) s += red[w * BN + c];
                Pg[static_cast<size_t>(tile_m) * NC + k] = s;
            }
        }
    }
}

// dW[i] = gamma[i % NC] * sum_s ws[s, i]  (fixed order s = 0, 1, ...; fp32), 4 per thread
__global__ void __launch_bounds__(256)
k_splitk_reduce(const f32x4_t* __restrict__ ws, const float* __restrict__ gamma, f32x4_t* __restrict__ dW,
                int64_t n4, int NC4, int S) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        f32x4_t a = ws[i];
        for (int s = 1; s < S; ++s) a += ws[static_cast<int64_t>(s) * n4 + i];
        if (gamma) {
            const int c = static_cast<int>(i % NC4) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] *= gamma[c + e];
        }
        dW[i] = a;
    }
}

// dgamma[k] = fl32( sum_t Pg[t, k] )  (fp64, fixed order): a block takes 32 columns; its
// 8 row groups g add rows t = g, g + 8, ... (coalesced 128-byte column runs), then group
// 0 adds the 8 group sums in order
__global__ void __launch_bounds__(256)
k_colsum_reduce(const float* __restrict__ Pg, float* __restrict__ out, int T, int NC) {
    __shared__ double part[8][32];
    const int c = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int k = blockIdx.x * 32 + c;
    double s = 0.0;
    if (k < NC)
        for (int t = g; t < T; t += 8) s += static_cast<double>(Pg[static_cast<size_t>(t) * NC + k]);
    part[g][c] = s;
    __syncthreads();
    if (g == 0 && k < NC) {
        double a = part[0][c];
#pragma unroll
        for (int i = 1; i < 8; ++i) a += part[i][c];
        out[k] = static_cast<float>(a);
    }
}

// dst[0, n) = 0 (the gradient of an empty token batch); a kernel rather than a memset so
// that the call may be captured in a graph
__global__ void __launch_bounds__(256) k_fill_zero_f32(float* __restrict__ dst, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        dst[i] = 0.0f;
}

#ifndef CODA_WG_BM
#define CODA_WG_BM 256
#define CODA_WG_BN 256
#define CODA_WG_WM 2
#define CODA_WG_WN 2
#define CODA_WG_NS 2
#define CODA_WG_RB 128
#define CODA_WG_SPREAD 2
#define CODA_WG_OCC 1
#endif
// Token-major weight gradients whose blocks each sum at least this many tokens run on the
// LDS stage rings (three stages of the A panel, two of B; mainloop_dma_ring_fp): dz, the A
// panel, streams from HBM there (16384 tokens x 16384 columns: 0.833-0.840 against
// 0.841-0.847 ms); a token split's shorter blocks keep the two shared stages.  Same bits.
#ifndef CODA_WG_RING_MIN_K
#define CODA_WG_RING_MIN_K 8192
#endif
// k-steps a k-tile's DMA is spread over on the rings (on the shared stages: CODA_WG_SPREAD;
// 4 there made the split dWo 9 % slower, 4 on the rings is 1-2.5 % faster than 2)
#ifndef CODA_WG_SPREAD_RING
#define CODA_WG_SPREAD_RING 4
#endif
constexpr int BMW = CODA_WG_BM, BNW = CODA_WG_BN;

int64_t wgrad_tiles(int64_t NR, int64_t NC) { return ((NR + BMW - 1) / BMW) * ((NC + BNW - 1) / BNW); }
int64_t wgrad_partials_rows(int64_t NR) { return NR < 1 ? -1 : (NR + BMW - 1) / BMW; }

// Token splits for a problem of `tiles` output tiles, each split at least
// kMinSplitTokens tokens: the S that minimises the estimated time of the rounds of
// blocks the 256 CUs run (one 256 x 256 tile each at a time; a round costs the block's
// tokens at ~30 ns per token and tile) plus the fp32 slices the split writes and its
// reduce reads back (2 S NR NC 4 bytes at ~5 TB/s).  A partly filled last round costs
// as much as a full one, so S is chosen against it, not just to reach 256 blocks.
constexpr int kMinSplitTokens = 2048, kMaxSplits = 16;
int wgrad_splits(int64_t NR, int64_t NC, int64_t K) {
    const int64_t tiles = wgrad_tiles(NR, NC);
    const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(kMaxSplits, K / kMinSplitTokens));
    constexpr double kNsPerTileToken = 30.5, kBytesPerNs = 5000.0;
    int best = 1;
    double best_ns = 0.0;
    for (int64_t S = 1; S <= smax; ++S) {
        const int64_t rounds = (tiles * S + 255) / 256;
        const double ns = static_cast<double>(rounds) * static_cast<double>((K + S - 1) / S) * kNsPerTileToken +
                          (S > 1 ? 2.0 * static_cast<double>(S) * NR * NC * 4 / kBytesPerNs : 0.0);
        if (S == 1 || ns < best_ns) {
            best = static_cast<int>(S);
            best_ns = ns;
        }
    }
    return best;
}
// the split's dW slices [S, NR, NC], then its gamma-gradient partial slices [S, tiles_m, NC]
int64_t wgrad_workspace_bytes(int64_t NR, int64_t NC, int64_t K) {
    const int S = wgrad_splits(NR, NC, K);
    return S > 1 ? static_cast<int64_t>(S) * (NR + (NR + BMW - 1) / BMW) * NC * 4 : 0;
}

// Splits and tokens per split: the time model's choice (wgrad_splits).  Token-major
// operands are addressed per 64-token k-tile (the descriptor is rebased on every
// k-tile), so their leading dimension puts no limit on a split's token count.
WgradPlan wgrad_plan(int64_t NR, int64_t NC, int64_t K) {
    if (K <= 0) return {1, 0};
    int64_t S = wgrad_splits(NR, NC, K);
    const int64_t k_split = S > 1 ? ((K + S - 1) / S + 63) / 64 * 64 : K;
    S = (K + k_split - 1) / k_split;
    return {static_cast<int>(S), static_cast<int>(k_split)};
}

template <bool TOK>
static hipError_t launch_wgrad(int NR, int NC, int K, const void* At, int lda, const void* Bt, int ldb,
                               const float* gamma, const void* Wraw, float* dW, float* Pg, float* ws,
                               int64_t ws_bytes, hipStream_t stream) {
    const int tiles_m = (NR + BMW - 1) / BMW, tiles_n = (NC + BNW - 1) / BNW;
    const WgradPlan plan = wgrad_plan(NR, NC, K);
    int S = plan.S, k_split = plan.k_split;                  // tokens per split: a multiple of 64
    auto need = [&](int s) { return static_cast<int64_t>(s) * (NR + (Wraw ? tiles_m : 0)) * NC * 4; };
    if (S > 1 && (ws == nullptr || ws_bytes < need(S))) {
        // without room for the split: one block per tile
        S = 1;
        k_split = K;
    }
    // split: dW slices, then (with W) the partial slices, in the workspace
    float* ws_p = S > 1 ? ws + static_cast<int64_t>(S) * NR * NC : nullptr;
    const dim3 grid(tiles_m * tiles_n * S), block(64 * CODA_WG_WM * CODA_WG_WN);
    if (TOK && k_split >= CODA_WG_RING_MIN_K)
        hipLaunchKernelGGL((k_gemm_wgrad<BMW, BNW, CODA_WG_WM, CODA_WG_WN, CODA_WG_NS, CODA_WG_RB,
                                         CODA_WG_SPREAD_RING, CODA_WG_OCC, TOK, TOK>),
                           grid, block, 0, stream, static_cast<const uint8_t*>(At), static_cast<const uint8_t*>(Bt),
                           S > 1 ? nullptr : gamma, static_cast<const uint16_t*>(Wraw), S > 1 ? ws : dW,
                           S > 1 && Wraw ? ws_p : Pg, NR, NC, K, tiles_m, tiles_n, k_split, lda, ldb);
    else
        hipLaunchKernelGGL((k_gemm_wgrad<BMW, BNW, CODA_WG_WM, CODA_WG_WN, CODA_WG_NS, CODA_WG_RB, CODA_WG_SPREAD,
                                         CODA_WG_OCC, TOK, false>),
                           grid, block, 0, stream, static_cast<const uint8_t*>(At), static_cast<const uint8_t*>(Bt),
                           S > 1 ? nullptr : gamma, static_cast<const uint16_t*>(Wraw), S > 1 ? ws : dW,
                           S > 1 && Wraw ? ws_p : Pg, NR, NC, K, tiles_m, tiles_n, k_split, lda, ldb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    const int64_t n4 = static_cast<int64_t>(NR) * NC / 4;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(k_splitk_reduce, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       reinterpret_cast<const f32x4_t*>(ws), gamma, reinterpret_cast<f32x4_t*>(dW), n4, NC / 4, S);
    e = hipGetLastError();
    if (e != hipSuccess || !Wraw) return e;
    // the gamma-gradient partials: the splits' rows added in the same fixed order (the
    // sums are linear in G, so adding per-split partials equals partials of the sum)
    const int64_t p4 = static_cast<int64_t>(tiles_m) * NC / 4;
    hipLaunchKernelGGL(k_splitk_reduce, dim3(static_cast<unsigned>(std::min<int64_t>((p4 + 255) / 256, 4096))),
                       dim3(256), 0, stream, reinterpret_cast<const f32x4_t*>(ws_p), nullptr,
                       reinterpret_cast<f32x4_t*>(Pg), p4, NC / 4, S);
    return hipGetLastError();
}

hipError_t launch_gemm_wgrad(int NR, int NC, int K, const void* At, const void* Bt, const float* gamma,
                             const void* Wraw, float* dW, float* Pg, float* ws, int64_t ws_bytes,
                             hipStream_t stream) {
    return launch_wgrad<false>(NR, NC, K, At, 0, Bt, 0, gamma, Wraw, dW, Pg, ws, ws_bytes, stream);
}

hipError_t launch_gemm_wgrad_tok(int NR, int NC, int K, const void* X, int lda, const void* Y, int ldb,
                                 const float* gamma, const void* Wraw, float* dW, float* Pg, float* ws,
                                 int64_t ws_bytes, hipStream_t stream) {
    return launch_wgrad<true>(NR, NC, K, X, lda, Y, ldb, gamma, Wraw, dW, Pg, ws, ws_bytes, stream);
}

// Scratch of the allocation-free entry point: the token split's dW slices and partial
// slices, in a file-scope device array of kNoAllocScratchBytes that every GPU the library
// runs on holds from the module's load to the end of the process.  In host code the
// array's name is only a host-side stand-in; its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that address is used.
// Calls on one device share the array: two such calls that overlap in time race.  Every
// element the split reduce reads is written by the GEMM of the same call first, so
// nothing needs clearing between calls.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float*>(g_scratch_ptr[dev]);
    return hipSuccess;
}
}  // namespace

hipError_t launch_gemm_wgrad_tok_noalloc(int NR, int NC, int K, const void* X, int lda, const void* Y, int ldb,
                                         const float* gamma, const void* Wraw, float* dW, float* Pg,
                                         hipStream_t stream) {
    float* ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_wgrad<true>(NR, NC, K, X, lda, Y, ldb, gamma, Wraw, dW, Pg, ws, kNoAllocScratchBytes, stream);
}

hipError_t launch_colsum_reduce(int T, int NC, const float* Pg, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(k_colsum_reduce, dim3((NC + 31) / 32), dim3(256), 0, stream, Pg, out, T, NC);
    return hipGetLastError();
}

hipError_t launch_fill_zero_f32(int64_t n, float* dst, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_fill_zero_f32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, dst, n);
    return hipGetLastError();
}

}  // namespace coda

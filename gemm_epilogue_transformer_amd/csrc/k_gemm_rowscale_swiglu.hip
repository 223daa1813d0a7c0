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
// RoPE (kucoin page, same section, last paragraph: the reparameterisation covers RoPE
// too): act NONE's product, then in every Q/K head of 64 columns value i and value i+32
// turn by pos[m] * theta_i (cos / sin from a table).  A head's two halves are the wave's
// blocks b and b+1 (b even) in the same lane and rows, so the rotation is lane-local,
// like the gate/up pairing of SwiGLU.
//
// 8-bit weights (weight-only): W is e4m3 in HBM and in LDS (half the bytes of a bf16
// panel) and is converted exactly to bf16 in registers after the LDS read; the MFMA is
// the bf16 one and sw is applied in the epilogue.
#include <algorithm>
#include <atomic>

#include "epilogue.hpp"
#include "gemm_pipeline.hpp"
#include "launch.hpp"

#ifndef CODA_G3_TC
#define CODA_G3_TC 1      // 0: the forward SwiGLU epilogue stages through LDS like the others
#endif
#ifndef CODA_G3_TC_CE
#define CODA_G3_TC_CE 1   // the loss statistics and their backward from transposed blocks too
#endif

namespace coda {

// Tile-rows per group of the tile walks (tile_coords): the one-tile-per-workgroup kernel
// (4 rather than 8: 1-3 % faster on the 16K-token shapes) and the overlapped loss kernel
// (no difference measured); the overlapped row-scale kernels take theirs at launch.
// Outputs do not depend on the walk.
#ifndef CODA_G3_NP_GROUP
#define CODA_G3_NP_GROUP 4
#endif
#ifndef CODA_G3_CE_GROUP
#define CODA_G3_CE_GROUP 8
#endif
#ifndef CODA_G3_OVL_SMALL_K
#define CODA_G3_OVL_SMALL_K 2048
#endif

enum { kActNone = 0, kActSwiglu = 1, kActRope = 2, kActCe = 3, kActSwigluBwd = 4, kActSwigluSave = 5, kActCeBwd = 6 };

// RoPE operands (unused by the other activations).
struct RopeArgs {
    const int32_t* pos;       // [M] positions
    const float* cos;         // [table_rows, 32]
    const float* sin;         // [table_rows, 32]
    int table_rows;
    int rot_cols;             // leading rotated columns (whole 64-column heads)
};

// hook.at<P>() runs after part P of an epilogue (a block pair of the SwiGLU epilogue, a
// block row of the loss epilogue): a persistent kernel issues a share of the next tile's
// DMA there.
struct NoEpiHook {
    template <int P>
    __device__ __forceinline__ void at() const {}
};

// Cross-entropy operands (unused by the other activations).
struct CeArgs {
    const int32_t* targets;   // [M]
    float* partials;          // [M, T, 2]: (max, sum exp(z - max)) per 256-column tile
    float* tgt_logit;         // [M]: z[m, targets[m]], written by the tile holding it
    int T;                    // tiles per row = ceil(V / 256)
    const float* lse;         // backward: [M] the forward's log-sum-exp
    const float* gw;          // backward: [M] d(total loss) / d(loss of row m)
};

// Cross-entropy epilogue (kucoin page, section "Cinco bloques y un lenguaje LEGO": a
// block log-sum-exp and the max / sum-exp state of online normalisation, in the epilogue
// of the LM-head product; section "CODA: El epilogo esconde un tesoro": the
// reparameterisation covers the cross-entropy loss).  The logits z = r*sw*acc never
// leave the chip: per 32-row slab they are staged row-major in LDS like the other
// epilogues; each lane takes 8 consecutive columns of one row (columns >= V masked),
// its max, a DPP all-reduce max over the lanes of the row, the sum of exp(z - max), a
// DPP all-reduce sum; the waves sharing a row are combined in a fixed order; one (max,
// sum-exp) pair per row and tile.  The lane whose 8 columns hold the row's target
// writes that logit.
template <int BM, int BN, int WAVES_M, int WAVES_N, int TM, int TN>
__device__ __forceinline__ void ce_epilogue(const f32x16_t (&acc)[TM][TN], const float (&rv)[BM / WAVES_M / 64],
                                            const int (&tv)[BM / WAVES_M / 64], float sw, const CeArgs& ce,
                                            int M, int V, int m0, int j0, int tile_n, int wm, int wn,
                                            uint8_t* slab, float* red) {
    acc_read_fence();                       // accumulators are read with acc_read
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, NT = 64 * WAVES_M * WAVES_N;
    using S = Slab<TN>;
    const int lane = threadIdx.x & 63;
    const int lh = lane >> 5;
    const float ninf = -__builtin_inff();
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        float rr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rr[4 * g + e] = __shfl(rv[tm / 2], (tm % 2) * 32 + 8 * g + 4 * lh + e) * sw;
        float v[TN][16];
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[b][i] = acc_read(acc[tm][b][i]) * rr[i];
        S::put(slab, v);
#pragma unroll
        for (int j = 0; j < S::kSegPerLane; ++j) {
            float t[8];
            S::get(slab, j, t);
            const int rl = tm * 32 + S::seg_row(j);            // row within the wave
            const int n = j0 + wn * WN + S::seg_col(j);         // first column of the 8
            float mx = ninf;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < V) mx = fmaxf(mx, t[e]);
            mx = group_allreduce<S::kSegPerRow>(mx, MaxOp());
            float sum = 0.0f;
            if (mx > ninf) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n + e < V) sum += __expf(t[e] - mx);
            }
            sum = group_allreduce<S::kSegPerRow>(sum, AddOp());
            const int tg = __shfl(tv[rl / 64], rl % 64);
            if (tg >= n && tg < n + 8 && tg < V) {
                float z = t[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) z = (tg - n == e) ? t[e] : z;
                ce.tgt_logit[m0 + wm * WM + rl] = z;
            }
            if ((lane & (S::kSegPerRow - 1)) == 0) {
                red[2 * (wn * BM + wm * WM + rl)] = mx;
                red[2 * (wn * BM + wm * WM + rl) + 1] = sum;
            }
        }
    }
    __syncthreads();
    for (int r = threadIdx.x; r < BM; r += NT) {
        const int m = m0 + r;
        if (m < M) {
            float mt = ninf;
#pragma unroll
            for (int w = 0; w < WAVES_N; ++w) mt = fmaxf(mt, red[2 * (w * BM + r)]);
            float st = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES_N; ++w) {
                const float mw = red[2 * (w * BM + r)];
                if (mw > ninf) st += red[2 * (w * BM + r) + 1] * __expf(mw - mt);
            }
            float* pp = ce.partials + (static_cast<size_t>(m) * ce.T + tile_n) * 2;
            pp[0] = mt;
            pp[1] = st;
        }
    }
}

// Sum / max of a value over lane l and lane l ^ 32: v_permlane32_swap on two copies of
// it (one result holds the lower half-wave's value in every lane, the other the
// upper's), the same operation order in both lanes.  Both the second operand and the
// two results pass through empty asm statements: used directly in arithmetic, the
// compiler at hand reads the instruction's first result register for both results.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    uint32_t v = u;
    asm volatile("" : "+v"(v));
    const auto p = __builtin_amdgcn_permlane32_swap(u, v, false, false);
    uint32_t a = p[0], b = p[1];
    asm volatile("" : "+v"(a), "+v"(b));
    lo = __builtin_bit_cast(float, a);
    hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float halves_max(float x) {
    float lo, hi;
    halves(x, lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float halves_sum(float x) {
    float lo, hi;
    halves(x, lo, hi);
    return lo + hi;
}

// Cross-entropy epilogue on transposed accumulator blocks (the mainloop's MFMA took the
// W fragment first): in block (tm, b) lane l holds logits of row 32*tm + l%32 of the
// wave, columns 32*b + 8*(i/4) + 4*(l/32) + i%4 of the wave's columns in register i.  So
// a row's max and sum of exponentials over the wave's columns are in-lane reductions
// over 16*TN values and one exchange between the two half-waves, with no LDS staging;
// the waves sharing a row combine in a fixed order as in ce_epilogue.  rt[tm], tt[tm]:
// r and the target of the lane's row (0 and -1 past M).  The lane holding a row's target
// column writes that logit.
template <int BM, int BN, int WAVES_M, int WAVES_N, int TM, int TN, class Hook = NoEpiHook>
__device__ __forceinline__ void ce_epilogue_tc(const f32x16_t (&acc)[TM][TN], const float (&rt)[TM],
                                               const int (&tt)[TM], float sw, const CeArgs& ce, int M, int V,
                                               int m0, int j0, int tile_n, int wm, int wn, float* red,
                                               const Hook& hook = Hook()) {
    acc_read_fence();                       // accumulators are read with acc_read
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, NT = 64 * WAVES_M * WAVES_N;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int lr = lane & 31, lh = lane >> 5;
    const float ninf = -__builtin_inff();
    const int nw = j0 + wn * WN;                    // first column of the wave
    const bool full = nw + WN <= V;                 // wave-uniform: no column past V
    static_for<TM>([&](auto TMc) {
        constexpr int tm = decltype(TMc)::value;
        const float rr = rt[tm] * sw;
        // logits; past V (only in the last column tile) -inf, which adds nothing below
        float z[TN][16];
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) z[b][i] = acc_read(acc[tm][b][i]) * rr;
        if (!full) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (nw + 32 * b + 8 * (i >> 2) + 4 * lh + (i & 3) >= V) z[b][i] = ninf;
        }
        float mx = ninf;
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, z[b][i]);
        mx = halves_max(mx);
        float sum = 0.0f;
        if (mx > ninf) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) sum += __expf(z[b][i] - mx);
        }
        sum = halves_sum(sum);
        const int rl = wm * WM + tm * 32 + lr;      // row within the block tile
        const int tg = tt[tm];
        const int o = tg - nw;
        if (o >= 0 && o < WN && tg < V) {
            const int c = o & 31;
            if (((c >> 2) & 1) == lh) {
                const int k = (o >> 5) * 16 + ((c >> 3) << 2) + (c & 3);
                float zt = 0.0f;
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) zt = (k == 16 * b + i) ? z[b][i] : zt;
                ce.tgt_logit[m0 + rl] = zt;
            }
        }
        if (lh == 0) {
            red[2 * (wn * BM + rl)] = mx;
            red[2 * (wn * BM + rl) + 1] = sum;
        }
        hook.template at<tm>();
        __builtin_amdgcn_sched_barrier(0);
    });
    __syncthreads();
    for (int r = threadIdx.x; r < BM; r += NT) {
        const int m = m0 + r;
        if (m < M) {
            float mt = ninf;
#pragma unroll
            for (int w = 0; w < WAVES_N; ++w) mt = fmaxf(mt, red[2 * (w * BM + r)]);
            float st = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES_N; ++w) {
                const float mw = red[2 * (w * BM + r)];
                if (mw > ninf) st += red[2 * (w * BM + r) + 1] * __expf(mw - mt);
            }
            float* pp = ce.partials + (static_cast<size_t>(m) * ce.T + tile_n) * 2;
            pp[0] = mt;
            pp[1] = st;
        }
    }
}

// Backward operands (unused by the forward activations).
struct BwdArgs {
    const uint16_t* dy;       // [M, F] bf16: upstream gradient of y
    uint16_t* dz;             // [M, 2F] bf16: r * dL/dz (gate columns, then up columns)
    float* partials;          // [M, T]: sum over the tile's columns of dL/dz * acc
    int T;                    // tiles per row = ceil(F / (BN/2))
};

// SwiGLU backward epilogue (kucoin page, section "CODA: El epilogo esconde un tesoro":
// the reparameterisation holds for the backward pass).  The mainloop has recomputed the
// forward product acc (gate and up blocks of the same (m, j) in one lane, as in the
// forward); with g = r*acc_g, u = r*acc_u, s = sigmoid(g) and the upstream dy:
//   dL/dg = dy u s (1 + g (1 - s)),   dL/du = dy g s
//   dz = r * (dL/dg, dL/du)  (bf16: the gradient at the accumulator, the next GEMM's A)
//   partial c = sum over the tile's columns of dL/dz * acc  (= dL/dr, fp32)
// The accumulators are staged row-major in LDS; each lane takes 8 gate columns of one
// row and the matching 8 up columns, loads dy as one 16-byte vector, stores two 16-byte
// vectors of dz; c: DPP all-reduce over the 8 lanes of the row, then the waves sharing it.
template <int BM, int BN, int WAVES_M, int WAVES_N, int TM, int TN>
__device__ __forceinline__ void swiglu_bwd_epilogue(const f32x16_t (&acc)[TM][TN],
                                                    const float (&rv)[BM / WAVES_M / 64], const BwdArgs& bw,
                                                    int M, int F, int m0, int j0, int tile_n, int wm, int wn,
                                                    uint8_t* slab, float* red) {
    acc_read_fence();                       // accumulators are read with acc_read
    constexpr int WM = BM / WAVES_M, NT = 64 * WAVES_M * WAVES_N;
    constexpr int NB = TN / 2;                       // gate (= up) blocks per wave
    constexpr int kGseg = NB * 4;                    // 8-column gate segments per row
    constexpr int kSegPerLane = 32 * kGseg / 64;
    static_assert(kGseg == 8, "8 lanes per row: the all-reduce below");
    using S = Slab<TN>;
    const int lane = threadIdx.x & 63;
    const int valid_rows = min(BM, M - m0);
    const uint32_t dy_row = static_cast<uint32_t>(F) * 2, dz_row = static_cast<uint32_t>(F) * 4;
    const __amdgpu_buffer_rsrc_t dy_rsrc =
        make_buffer_rsrc(bw.dy + static_cast<size_t>(m0) * F, static_cast<uint32_t>(valid_rows) * dy_row);
    const __amdgpu_buffer_rsrc_t dz_rsrc =
        make_buffer_rsrc(bw.dz + static_cast<size_t>(m0) * 2 * F, static_cast<uint32_t>(valid_rows) * dz_row);
    // dy of segment jj of slab tm (16 bytes: 8 gate columns of one row), loaded one slab
    // ahead so that its latency overlaps the previous slab's arithmetic and stores
    auto dy_off = [&](int tm, int jj) -> uint32_t {
        const int q = lane + 64 * jj;
        const int col = j0 + wn * NB * 32 + (q % kGseg) * 8;
        const uint32_t trow = static_cast<uint32_t>(wm * WM + tm * 32 + q / kGseg);
        return col < F ? trow * dy_row + static_cast<uint32_t>(col) * 2 : kOobOffset;
    };
    i32x4_t dyb[2][kSegPerLane];
#pragma unroll
    for (int jj = 0; jj < kSegPerLane; ++jj) dyb[0][jj] = __builtin_amdgcn_raw_buffer_load_b128(dy_rsrc, dy_off(0, jj), 0, 0);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        if (tm + 1 < TM) {
#pragma unroll
            for (int jj = 0; jj < kSegPerLane; ++jj)
                dyb[(tm + 1) & 1][jj] = __builtin_amdgcn_raw_buffer_load_b128(dy_rsrc, dy_off(tm + 1, jj), 0, 0);
        }
        float v[TN][16];
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[b][i] = acc_read(acc[tm][b][i]);
        S::put(slab, v);
#pragma unroll
        for (int jj = 0; jj < kSegPerLane; ++jj) {
            const int q = lane + 64 * jj;
            const int row = q / kGseg, gcol = (q % kGseg) * 8;
            const int rw = tm * 32 + row;                          // row within the wave
            const int col = j0 + wn * NB * 32 + gcol;              // output column (gate j)
            const float rr = __shfl(rv[tm / 2], (tm % 2) * 32 + row);
            const uint8_t* sp = slab + row * S::kStride;
            const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(sp + gcol * 4);
            const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(sp + gcol * 4 + 16);
            const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(sp + (NB * 32 + gcol) * 4);
            const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(sp + (NB * 32 + gcol) * 4 + 16);
            const float ag[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            const float au[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
            const uint32_t in_range = col < F;
            const uint32_t trow = static_cast<uint32_t>(wm * WM + rw);
            const i32x4_t dyv = dyb[tm & 1][jj];
            float c = 0.0f;
            uint32_t og[4], ou[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = static_cast<uint32_t>(dyv[e]);
                float dgo[2], duo[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = 2 * e + hh;
                    const float d = bf16_bits_to_f32(static_cast<uint16_t>(hh ? x >> 16 : x & 0xFFFFu));
                    const float g = ag[k] * rr, u = au[k] * rr;
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                    const float dg = d * u * sg * (1.0f + g * (1.0f - sg));
                    const float du = d * g * sg;
                    c += dg * ag[k] + du * au[k];
                    dgo[hh] = rr * dg;
                    duo[hh] = rr * du;
                }
                og[e] = pack_bf16x2(dgo[0], dgo[1]);
                ou[e] = pack_bf16x2(duo[0], duo[1]);
            }
            const uint32_t vg = in_range ? trow * dz_row + static_cast<uint32_t>(col) * 2 : kOobOffset;
            const uint32_t vu = in_range ? trow * dz_row + static_cast<uint32_t>(F + col) * 2 : kOobOffset;
            __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(og[0]), int(og[1]), int(og[2]), int(og[3])},
                                                   dz_rsrc, vg, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(ou[0]), int(ou[1]), int(ou[2]), int(ou[3])},
                                                   dz_rsrc, vu, 0, 0);
            c = group_allreduce<kGseg>(c, AddOp());
            if ((lane & (kGseg - 1)) == 0) red[wn * BM + wm * WM + rw] = c;
        }
    }
    __syncthreads();
    for (int r = threadIdx.x; r < BM; r += NT) {
        const int m = m0 + r;
        if (m < M) {
            float c = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES_N; ++w) c += red[w * BM + r];
            bw.partials[static_cast<size_t>(m) * bw.T + tile_n] = c;
        }
    }
}

// Cross-entropy backward epilogue (kucoin page, section "CODA: El epilogo esconde un
// tesoro", last paragraph: the reparameterisation covers the loss and holds for the
// backward pass).  The mainloop has recomputed the LM-head product acc (bf16 weights);
// with z = r*acc, the forward's log-sum-exp lse, the target t and the row's weight g
// (the gradient of the total loss with respect to the row's loss):
//   dL/dz[m, v] = g (exp(z - lse) - [v == t])      (0 for a row whose t lies outside
//                                                    [0, V): its loss is the constant 0)
//   dz = bf16( r dL/dz )                  (the input-gradient and weight-gradient GEMMs' operand)
//   partial c = sum over the wave's 128 columns of dL/dz * acc   (fp32, one per row and wave)
// Per 32-row slab the accumulators are staged row-major in LDS; each lane takes 8
// columns of one row (16 lanes per row), its row's values shuffled from the registers
// that hold them (lane l: rows l, 64 + l of the wave), one 16-byte store of dz, and c
// through a 16-lane DPP all-reduce.  Partial column 2 * tile_n + wn of T = ceil(V/128).
template <int BM, int BN, int WAVES_M, int WAVES_N, int TM, int TN>
__device__ __forceinline__ void ce_bwd_epilogue(const f32x16_t (&acc)[TM][TN],
                                                const float (&rv)[BM / WAVES_M / 64],
                                                const int (&tv)[BM / WAVES_M / 64],
                                                const float (&lv)[BM / WAVES_M / 64],
                                                const float (&gv)[BM / WAVES_M / 64], const BwdArgs& bw,
                                                int M, int V, int m0, int j0, int tile_n, int wm, int wn,
                                                uint8_t* slab) {
    acc_read_fence();                       // accumulators are read with acc_read
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    using S = Slab<TN>;
    static_assert(S::kSegPerRow == 16, "16 lanes per row: the all-reduce below");
    const int lane = threadIdx.x & 63;
    const int valid_rows = min(BM, M - m0);
    const uint32_t dz_row = static_cast<uint32_t>(V) * 2;
    const __amdgpu_buffer_rsrc_t dz_rsrc =
        make_buffer_rsrc(bw.dz + static_cast<size_t>(m0) * V, static_cast<uint32_t>(valid_rows) * dz_row);
    const int pcol = 2 * tile_n + wn;                       // this wave's partial column
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        float v[TN][16];
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[b][i] = acc_read(acc[tm][b][i]);
        S::put(slab, v);
#pragma unroll
        for (int j = 0; j < S::kSegPerLane; ++j) {
            float t[8];
            S::get(slab, j, t);
            const int rl = tm * 32 + S::seg_row(j);            // row within the wave
            const int n = j0 + wn * WN + S::seg_col(j);         // first column of the 8
            const float rr = __shfl(rv[rl / 64], rl % 64);
            const float ls = __shfl(lv[rl / 64], rl % 64);
            const float gg = __shfl(gv[rl / 64], rl % 64);
            const int tg = __shfl(tv[rl / 64], rl % 64);
            const float gr = (tg >= 0 && tg < V) ? gg : 0.0f;  // an ignored row: no gradient
            float c = 0.0f;
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float dzo[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = 2 * e + hh;
                    const float p = __expf(rr * t[k] - ls);
                    const float dl = (n + k < V) ? gr * (p - (n + k == tg ? 1.0f : 0.0f)) : 0.0f;
                    c += dl * t[k];
                    dzo[hh] = rr * dl;
                }
                o[e] = pack_bf16x2(dzo[0], dzo[1]);
            }
            const uint32_t trow = static_cast<uint32_t>(wm * WM + rl);
            const uint32_t voff = n < V ? trow * dz_row + static_cast<uint32_t>(n) * 2 : kOobOffset;
            __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(o[0]), int(o[1]), int(o[2]), int(o[3])}, dz_rsrc,
                                                   voff, 0, 0);
            c = group_allreduce<16>(c, AddOp());
            const int m = m0 + wm * WM + rl;
            if ((lane & 15) == 0 && m < M && pcol < bw.T) bw.partials[static_cast<size_t>(m) * bw.T + pcol] = c;
        }
    }
}

// Backward of the loss epilogue on transposed accumulator blocks (the layout of
// ce_epilogue_tc): per lane and block row the 16*TN logits of one row, so the row's
// r, lse, weight and target are per-lane values, dz leaves as 16-byte stores after one
// half-wave exchange per pair of 4-column groups (as in swiglu_epilogue_tc), and the
// partial sum of dL/dz * acc over the wave's 128 columns is an in-lane sum plus one
// exchange.  rt, tt, lt, gt: r, target, lse and weight of the lane's row in each block
// row (0, -1, 0, 0 past M).
template <int BM, int BN, int WAVES_M, int WAVES_N, int TM, int TN>
__device__ __forceinline__ void ce_bwd_epilogue_tc(const f32x16_t (&acc)[TM][TN], const float (&rt)[TM],
                                                   const int (&tt)[TM], const float (&lt)[TM], const float (&gt)[TM],
                                                   const BwdArgs& bw, int M, int V, int m0, int j0, int tile_n,
                                                   int wm, int wn) {
    acc_read_fence();                       // accumulators are read with acc_read
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static_assert(WN == 128, "one partial per wave and row: 128 columns");
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int lr = lane & 31, lh = lane >> 5;
    const int valid_rows = min(BM, M - m0);
    const uint32_t dz_row = static_cast<uint32_t>(V) * 2;
    const __amdgpu_buffer_rsrc_t dz_rsrc =
        make_buffer_rsrc(bw.dz + static_cast<size_t>(m0) * V, static_cast<uint32_t>(valid_rows) * dz_row);
    const int pcol = 2 * tile_n + wn;                       // this wave's partial column
    const int nw = j0 + wn * WN;                            // first column of the wave
    const bool full = nw + WN <= V;                         // wave-uniform: no column past V
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const float rr = rt[tm], ls = lt[tm];
        const int tg = tt[tm];
        const float gr = (tg >= 0 && tg < V) ? gt[tm] : 0.0f;  // an ignored row: no gradient
        const int rl = wm * WM + tm * 32 + lr;                 // row within the block tile
        const uint32_t row_off = static_cast<uint32_t>(rl) * dz_row;
        float c = 0.0f;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            // dL/dz of the block's 16 columns; past V (only in the last column tile) 0
            float dl[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int n = nw + 32 * b + 8 * (i >> 2) + 4 * lh + (i & 3);
                const float p = __expf(rr * acc_read(acc[tm][b][i]) - ls);
                dl[i] = gr * (p - (n == tg ? 1.0f : 0.0f));
            }
            if (!full) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (nw + 32 * b + 8 * (i >> 2) + 4 * lh + (i & 3) >= V) dl[i] = 0.0f;
            }
            uint32_t pk[4][2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float dzo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    c += dl[4 * g + e] * acc_read(acc[tm][b][4 * g + e]);
                    dzo[e] = rr * dl[4 * g + e];
                }
                pk[g][0] = pack_bf16x2(dzo[0], dzo[1]);
                pk[g][1] = pack_bf16x2(dzo[2], dzo[3]);
            }
            const int nb = nw + 32 * b;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const auto sw2 = __builtin_amdgcn_permlane32_swap(pk[2 * q][h], pk[2 * q + 1][h], false, false);
                    w[h] = sw2[0];
                    w[2 + h] = sw2[1];
                }
                const int n = nb + 16 * q + 8 * lh;
                const uint32_t voff = n < V ? row_off + static_cast<uint32_t>(n) * 2 : kOobOffset;
                __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(w[0]), int(w[1]), int(w[2]), int(w[3])}, dz_rsrc,
                                                       voff, 0, 0);
            }
        }
        c = halves_sum(c);
        const int m = m0 + rl;
        if (lh == 0 && m < M && pcol < bw.T) bw.partials[static_cast<size_t>(m) * bw.T + pcol] = c;
    }
}

// SwiGLU forward that also keeps the pre-activation for a backward without recompute:
// y = silu(g) * u as in the plain SwiGLU epilogue (the same fp32 operations, so the same
// bits) and z = [g | u] = r * (h . W'^T) rounded to bf16, z [M, 2F] (gate columns, then
// up).  The unscaled accumulators are staged in LDS; each lane takes 8 gate columns of a
// row and the matching 8 up columns (the backward epilogue's walk): three 16-byte stores.
template <int BM, int BN, int WAVES_M, int TM, int TN>
__device__ __forceinline__ void swiglu_save_epilogue(const f32x16_t (&acc)[TM][TN],
                                                     const float (&rv)[BM / WAVES_M / 64], float sw,
                                                     uint16_t* __restrict__ Y, uint16_t* __restrict__ Z, int M,
                                                     int F, int m0, int j0, int wm, int wn, uint8_t* slab) {
    acc_read_fence();                       // accumulators are read with acc_read
    constexpr int WM = BM / WAVES_M;
    constexpr int NB = TN / 2;
    constexpr int kGseg = NB * 4;
    constexpr int kSegPerLane = 32 * kGseg / 64;
    using S = Slab<TN>;
    const int lane = threadIdx.x & 63;
    const int valid_rows = min(BM, M - m0);
    const uint32_t y_row = static_cast<uint32_t>(F) * 2, z_row = static_cast<uint32_t>(F) * 4;
    const __amdgpu_buffer_rsrc_t y_rsrc =
        make_buffer_rsrc(Y + static_cast<size_t>(m0) * F, static_cast<uint32_t>(valid_rows) * y_row);
    const __amdgpu_buffer_rsrc_t z_rsrc =
        make_buffer_rsrc(Z + static_cast<size_t>(m0) * 2 * F, static_cast<uint32_t>(valid_rows) * z_row);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        float v[TN][16];
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[b][i] = acc_read(acc[tm][b][i]);
        S::put(slab, v);
#pragma unroll
        for (int jj = 0; jj < kSegPerLane; ++jj) {
            const int q = lane + 64 * jj;
            const int row = q / kGseg, gcol = (q % kGseg) * 8;
            const int col = j0 + wn * NB * 32 + gcol;
            const float rr = __shfl(rv[tm / 2], (tm % 2) * 32 + row) * sw;
            const uint8_t* sp = slab + row * S::kStride;
            const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(sp + gcol * 4);
            const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(sp + gcol * 4 + 16);
            const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(sp + (NB * 32 + gcol) * 4);
            const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(sp + (NB * 32 + gcol) * 4 + 16);
            const float ag[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            const float au[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
            float yv[8], gv[8], uv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                gv[k] = ag[k] * rr;
                uv[k] = au[k] * rr;
                yv[k] = gv[k] * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[k])) * uv[k];
            }
            const bool in_range = col < F;
            const uint32_t trow = static_cast<uint32_t>(wm * WM + tm * 32 + row);
            const uint32_t vy = in_range ? trow * y_row + static_cast<uint32_t>(col) * 2 : kOobOffset;
            const uint32_t vg = in_range ? trow * z_row + static_cast<uint32_t>(col) * 2 : kOobOffset;
            const uint32_t vu = in_range ? trow * z_row + static_cast<uint32_t>(F + col) * 2 : kOobOffset;
            __builtin_amdgcn_raw_buffer_store_b128(
                i32x4_t{int(pack_bf16x2(yv[0], yv[1])), int(pack_bf16x2(yv[2], yv[3])),
                        int(pack_bf16x2(yv[4], yv[5])), int(pack_bf16x2(yv[6], yv[7]))},
                y_rsrc, vy, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(
                i32x4_t{int(pack_bf16x2(gv[0], gv[1])), int(pack_bf16x2(gv[2], gv[3])),
                        int(pack_bf16x2(gv[4], gv[5])), int(pack_bf16x2(gv[6], gv[7]))},
                z_rsrc, vg, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(
                i32x4_t{int(pack_bf16x2(uv[0], uv[1])), int(pack_bf16x2(uv[2], uv[3])),
                        int(pack_bf16x2(uv[4], uv[5])), int(pack_bf16x2(uv[6], uv[7]))},
                z_rsrc, vu, 0, 0);
        }
    }
}

// Epilogue shared by the bf16 and 8-bit weight instantiations.  Wave (wm, wn) holds TM x TN 32x32 accumulator blocks;
// with SwiGLU, blocks [0, TN/2) are gate columns and [TN/2, TN) the matching up columns.
// Per 32-row slab: r (times sw) is applied lane-locally to both accumulators before the
// SiLU; the finished fp32 outputs are staged row-major in the wave's LDS region `slab`
// and written as 16-byte runs of 8 bf16.  Rows / columns outside y are masked by the
// buffer range check.
//
// r of the wave's WM rows lives in registers: lane l holds rows l, 64 + l, ... of the
// wave (rv[WM / 64]), loaded before the mainloop; the epilogue fetches the rows it needs
// with cross-lane permutes, so r takes no LDS (the stages may fill all of it).
//
// RoPE: pv holds the positions of the wave's rows like rv holds r; per slab each lane
// loads cos / sin of its 16 rows at frequency lane % 32 (range-checked: a position
// outside the table reads 0).
template <int BM, int BN, int WAVES_M, int TM, int TN, int ACT>
__device__ __forceinline__ void rowscale_epilogue(const f32x16_t (&acc)[TM][TN],
                                                  const float (&rv)[BM / WAVES_M / 64],
                                                  const int (&pv)[BM / WAVES_M / 64], const RopeArgs& rope,
                                                  float sw, uint16_t* __restrict__ Y, int M, int N_out,
                                                  int m0, int j0, int wm, int wn, uint8_t* slab) {
    acc_read_fence();                       // accumulators are read with acc_read
    constexpr bool SWIGLU = ACT == kActSwiglu;
    constexpr int WM = BM / WAVES_M;
    constexpr int NB = SWIGLU ? TN / 2 : TN;          // output blocks per wave
    static_assert(ACT != kActRope || NB % 2 == 0, "a head's halves are blocks b and b+1 of one wave");
    using S = Slab<NB>;
    const int lane = threadIdx.x & 63;
    const int lh = lane >> 5;
    const int valid_rows = min(BM, M - m0);
    const uint32_t row_bytes = static_cast<uint32_t>(N_out) * 2;
    const __amdgpu_buffer_rsrc_t y_rsrc =
        make_buffer_rsrc(Y + static_cast<size_t>(m0) * N_out, static_cast<uint32_t>(valid_rows) * row_bytes);
    // RoPE: first column of the wave; heads whose first column is below rot_cols turn
    const int n_wave = j0 + wn * NB * 32;
    const bool any_rot = ACT == kActRope && n_wave < rope.rot_cols;
    const uint32_t tbytes = ACT == kActRope ? static_cast<uint32_t>(rope.table_rows) * 128u : 0u;
    const __amdgpu_buffer_rsrc_t cos_rsrc = make_buffer_rsrc(rope.cos, tbytes);
    const __amdgpu_buffer_rsrc_t sin_rsrc = make_buffer_rsrc(rope.sin, tbytes);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        // r of the 16 rows this lane holds: rows 8g + 4*lh + (0..3), g = 0..3
        float rr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rr[4 * g + e] = __shfl(rv[tm / 2], (tm % 2) * 32 + 8 * g + 4 * lh + e) * sw;
        float v[NB][16];
        if constexpr (ACT == kActRope) {
            float cs[16] = {}, sn[16] = {};
            if (any_rot) {
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int p = __shfl(pv[tm / 2], (tm % 2) * 32 + 8 * g + 4 * lh + e);
                        const uint32_t off = (p >= 0 && p < rope.table_rows)
                                                 ? static_cast<uint32_t>(p) * 128u + static_cast<uint32_t>(lane & 31) * 4u
                                                 : kOobOffset;
                        cs[4 * g + e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cos_rsrc, off, 0, 0));
                        sn[4 * g + e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sin_rsrc, off, 0, 0));
                    }
            }
#pragma unroll
            for (int b = 0; b < NB; b += 2) {
                if (n_wave + b * 32 < rope.rot_cols) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float x1 = acc_read(acc[tm][b][i]) * rr[i], x2 = acc_read(acc[tm][b + 1][i]) * rr[i];
                        v[b][i] = x1 * cs[i] - x2 * sn[i];
                        v[b + 1][i] = x2 * cs[i] + x1 * sn[i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        v[b][i] = acc_read(acc[tm][b][i]) * rr[i];
                        v[b + 1][i] = acc_read(acc[tm][b + 1][i]) * rr[i];
                    }
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if constexpr (SWIGLU) {
                        const float gv = acc_read(acc[tm][b][i]) * rr[i];
                        const float uv = acc_read(acc[tm][b + NB][i]) * rr[i];
                        v[b][i] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
                    } else {
                        v[b][i] = acc_read(acc[tm][b][i]) * rr[i];
                    }
                }
        }
        S::put(slab, v);
#pragma unroll
        for (int j = 0; j < S::kSegPerLane; ++j) {
            const int tr = wm * WM + tm * 32 + S::seg_row(j);
            const int n = j0 + wn * NB * 32 + S::seg_col(j);
            const uint32_t voff =
                n < N_out ? static_cast<uint32_t>(tr) * row_bytes + static_cast<uint32_t>(n) * 2 : kOobOffset;
            float t[8];
            S::get(slab, j, t);
            __builtin_amdgcn_raw_buffer_store_b128(
                i32x4_t{int(pack_bf16x2(t[0], t[1])), int(pack_bf16x2(t[2], t[3])),
                        int(pack_bf16x2(t[4], t[5])), int(pack_bf16x2(t[6], t[7]))},
                y_rsrc, voff, 0, 0);
        }
    }
}

// SwiGLU epilogue on transposed accumulator blocks (the mainloop's MFMA took the W
// fragment first; rt[tm]: r of the lane's row 32*tm + l%32 of the wave, 0 past M): in
// block (tm, b) lane l holds row 32*tm + l%32 of the wave and, in
// register i, column 8*(i/4) + 4*(l/32) + i%4 of the block.  So r is one value per lane
// and block row, and every group of 4 registers is 4 consecutive output columns of one
// row; one cross-half lane swap per pair of groups makes them 8, stored with one 16-byte
// store, with no LDS staging.  Same fp32 operations per element, in the same order, as
// rowscale_epilogue.
template <int BM, int BN, int WAVES_M, int TM, int TN, class Hook = NoEpiHook>
__device__ __forceinline__ void swiglu_epilogue_tc(const f32x16_t (&acc)[TM][TN], const float (&rt)[TM], float sw,
                                                   uint16_t* __restrict__ Y, int M, int N_out, int m0, int j0,
                                                   int wm, int wn, const Hook& hook = Hook()) {
    constexpr int WM = BM / WAVES_M;
    constexpr int NB = TN / 2;
    // lane-derived addresses are formed here, not hoisted out of a persistent kernel's
    // tile loop (where they would stay live through the mainloop)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int lr = lane & 31, lh = lane >> 5;
    const int valid_rows = min(BM, M - m0);
    const uint32_t row_bytes = static_cast<uint32_t>(N_out) * 2;
    const __amdgpu_buffer_rsrc_t y_rsrc =
        make_buffer_rsrc(Y + static_cast<size_t>(m0) * N_out, static_cast<uint32_t>(valid_rows) * row_bytes);
    acc_read_fence();
    static_for<TM>([&](auto TMc) {
        constexpr int tm = decltype(TMc)::value;
        const float rr = rt[tm] * sw;
        const uint32_t row_off = static_cast<uint32_t>(wm * WM + tm * 32 + lr) * row_bytes;
        static_for<NB>([&](auto Bc) {
            constexpr int b = decltype(Bc)::value;
            uint32_t pk[4][2];    // group g: columns 8g + 4lh .. +3 as two bf16 pairs
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gv = acc_read(acc[tm][b][4 * g + e]) * rr;
                    const float uv = acc_read(acc[tm][b + NB][4 * g + e]) * rr;
                    v[e] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
                }
                pk[g][0] = pack_bf16x2(v[0], v[1]);
                pk[g][1] = pack_bf16x2(v[2], v[3]);
            }
            // groups 2q and 2q+1: the upper half-wave's group 2q and the lower's group 2q+1
            // trade places (v_permlane32_swap), so lane l < 32 holds columns 16q .. 16q+7
            // and lane l + 32 columns 16q+8 .. 16q+15 of its row: 16-byte stores
            const int nb = j0 + wn * NB * 32 + b * 32;
            static_for<2>([&](auto Qc) {
                constexpr int q = decltype(Qc)::value;
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const auto sw2 = __builtin_amdgcn_permlane32_swap(pk[2 * q][h], pk[2 * q + 1][h], false, false);
                    w[h] = sw2[0];
                    w[2 + h] = sw2[1];
                }
                const int n = nb + 16 * q + 8 * lh;
                const uint32_t voff = n < N_out ? row_off + static_cast<uint32_t>(n) * 2 : kOobOffset;
                __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(w[0]), int(w[1]), int(w[2]), int(w[3])}, y_rsrc,
                                                       voff, 0, 0);
            });
            hook.template at<tm * NB + b>();
            __builtin_amdgcn_sched_barrier(0);
        });
    });
}

// Direct-to-LDS mainloop (PIPE 1: the register-staged one, bf16 weights only; PIPE 2: the
// register-staged one with the RMSNorm weight gfold folded into a raw W on its way to
// LDS, bit-identical to a pre-folded W').  W8: the
// weights are e4m3, RB is the k-tile depth of a bf16 h row and a W row holds RB/2 bytes.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int RB, int SPREAD, int PIPE, int OCC, int ACT,
          bool W8, bool RING = false>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, OCC)
k_gemm_rowscale_swiglu(const uint8_t* __restrict__ H, const uint8_t* __restrict__ W,
                       const float* __restrict__ w_scale, const float* __restrict__ R,
                       uint16_t* __restrict__ Y, int M, int N_out, int K, int tiles_m,
                       int tiles_n, RopeArgs rope, CeArgs ce, BwdArgs bw, const float* __restrict__ gfold) {
    // the backward recomputes the forward's gate / up product: same B panel layout
    constexpr bool SWIGLU = ACT == kActSwiglu || ACT == kActSwigluBwd || ACT == kActSwigluSave;
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    static_assert(!SWIGLU || (TN % 2 == 0), "SwiGLU pairs gate and up blocks");
    constexpr int BNO = SWIGLU ? BN / 2 : BN;       // output columns of one block tile
    // transposed accumulator blocks (16-byte stores straight from registers) for the
    // forward SwiGLU on the bf16 DMA mainloop
    constexpr bool TC = CODA_G3_TC && (ACT == kActSwiglu || ((ACT == kActCe || ACT == kActCeBwd) && CODA_G3_TC_CE)) &&
                        !W8 && PIPE == 0;
    constexpr bool TC_CE = TC && (ACT == kActCe || ACT == kActCeBwd);

    constexpr int RBB = W8 ? RB / 2 : RB;            // bytes of a W row per k-tile
    constexpr int kStage = BM * RB + BN * RBB;
    static_assert(!W8 || (RB == 128 && PIPE == 0), "8-bit weights: DMA mainloop, 64-k tiles");
    // RING: the mainloop on LDS stage rings (three h stages, two weight stages), which take
    // the whole LDS; the epilogue's slabs and row partials then live in the ring memory
    static_assert(!RING || (!W8 && PIPE == 0 && (ACT == kActSwigluBwd || ACT == kActCeBwd || ACT == kActRope)),
                  "rings: the bf16 SwiGLU and loss backward, RoPE");
    constexpr int kSlabBytes = Slab<(ACT == kActSwiglu) ? TN / 2 : TN>::kBytes;
    constexpr int kRed = ACT == kActCe ? 2 * WAVES_N * BM : (ACT == kActSwigluBwd ? WAVES_N * BM : 1);
    uint8_t* st[NS];
    uint8_t* sa[3];
    uint8_t* sb[2];
    float* ce_red;            // cross-entropy: (max, sum-exp) of every row for each of the WAVES_N column halves
    uint8_t* slab;            // this wave's epilogue slab
    if constexpr (RING) {
        __shared__ __attribute__((aligned(1024))) uint8_t rings[3 * BM * RB + 2 * BN * RBB];
        static_assert(NW * kSlabBytes + kRed * 4 <= 3 * BM * RB + 2 * BN * RBB, "slabs and partials fit");
#pragma unroll
        for (int i = 0; i < 3; ++i) sa[i] = rings + i * BM * RB;
#pragma unroll
        for (int i = 0; i < 2; ++i) sb[i] = rings + 3 * BM * RB + i * BN * RBB;
        slab = rings + (threadIdx.x >> 6) * kSlabBytes;
        ce_red = reinterpret_cast<float*>(rings + NW * kSlabBytes);
    } else {
        __shared__ __attribute__((aligned(1024))) uint8_t stages[NS][kStage];
        __shared__ float ce_red_s[kRed];
#pragma unroll
        for (int i = 0; i < NS; ++i) st[i] = stages[i];
        slab = slab_region<NS, NW, kStage, kSlabBytes>(st, threadIdx.x >> 6);
        ce_red = ce_red_s;
    }

    int tile_m, tile_n;
    tile_coords<CODA_G3_NP_GROUP>(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, j0 = tile_n * BNO;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // r of this wave's rows (lane l: rows l, 64 + l, ...), loaded now so that its latency
    // hides behind the mainloop; rows past M hold 0
    static_assert(WM % 64 == 0, "each lane holds WM / 64 row scales");
    float rv[WM / 64];
    int pv[WM / 64];                                // RoPE: positions of the same rows
    int tv[WM / 64];                                // cross-entropy: their targets (-1 past M)
    float lv[WM / 64], gv[WM / 64];                 // cross-entropy backward: lse and row weight
#pragma unroll
    for (int i = 0; i < WM / 64; ++i) {
        const int m = m0 + wm * WM + 64 * i + (threadIdx.x & 63);
        rv[i] = m < M ? R[m] : 0.0f;
        pv[i] = 0;
        tv[i] = -1;
        if constexpr (ACT == kActRope) pv[i] = (m < M && rope.rot_cols > 0) ? rope.pos[m] : 0;
        if constexpr (ACT == kActCe || ACT == kActCeBwd) tv[i] = m < M ? ce.targets[m] : -1;
        lv[i] = 0.0f;
        gv[i] = 0.0f;
        if constexpr (ACT == kActCeBwd) {
            lv[i] = m < M ? ce.lse[m] : 0.0f;
            gv[i] = m < M ? ce.gw[m] : 0.0f;
        }
    }

    // transposed layout: r and the target of the lane's row in each block row
    float rt[TM], lt[TM], gt[TM];
    int tt[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WM + 32 * i + (threadIdx.x & 31);
        rt[i] = (TC_CE && m < M) ? R[m] : 0.0f;
        tt[i] = (TC_CE && m < M) ? ce.targets[m] : -1;
        lt[i] = (TC_CE && ACT == kActCeBwd && m < M) ? ce.lse[m] : 0.0f;
        gt[i] = (TC_CE && ACT == kActCeBwd && m < M) ? ce.gw[m] : 0.0f;
    }

    const int kbytes = K * 2;                       // bytes of an h row
    const int kbytes_b = W8 ? K : K * 2;            // bytes of a W row
    using PanelA = std::conditional_t<PIPE >= 1, RegPanel<BM, BM, NW, RB>, DmaPanel<BM, BM, NW, RB>>;
    using PanelB = std::conditional_t<PIPE >= 1, RegPanel<BN, SWIGLU ? BN / 2 : BN, NW, RB>,
                                      DmaPanel<BN, SWIGLU ? BN / 2 : BN, NW, RBB>>;
    PanelA pa;
    PanelB pb;
    const uint8_t* a0 = H + static_cast<size_t>(m0) * kbytes;
    pa.init(a0, min(BM, M - m0), a0, 0, kbytes);
    const uint8_t* g0 = W + static_cast<size_t>(j0) * kbytes_b;
    if constexpr (SWIGLU) {
        const uint8_t* u0 = W + static_cast<size_t>(N_out + j0) * kbytes_b;
        pb.init(g0, min(BN / 2, N_out - j0), u0, min(BN / 2, N_out - j0), kbytes_b);
    } else {
        pb.init(g0, min(BN, N_out - j0), g0, 0, kbytes_b);
    }
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    // SWIGLU: blocks [0, TN/2) = this wave's gate rows, [TN/2, TN) = the matching up rows
    auto b_row = [&](int tn) {
        if constexpr (SWIGLU) {
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

    if constexpr (W8) {
        mainloop_dma_fp<FragsW8<TM, TN>, BM, BN, (SWIGLU ? BN / 2 : BN), NS, NW, RB, RBB, SPREAD>(
            acc, pa, pb, kbytes, kbytes_b, st, a_row, b_row);
    } else if constexpr (PIPE == 1) {
        static_assert(NS == 2, "the register-staged mainloop has two LDS stages");
        mainloop_reg<Elt::BF16, BM, BN, (SWIGLU ? BN / 2 : BN), NW, RB>(acc, pa, pb, kbytes, st, a_row, b_row);
    } else if constexpr (PIPE == 2) {
        static_assert(NS == 2, "the register-staged mainloop has two LDS stages");
        mainloop_reg<Elt::BF16, BM, BN, (SWIGLU ? BN / 2 : BN), NW, RB>(acc, pa, pb, kbytes, st, a_row, b_row,
                                                                         GammaFold<RB>(gfold, K));
    } else if constexpr (RING) {
        mainloop_dma_ring_fp<FragPair<Frags<Elt::BF16, TM, TN, RB, TC>>, NW, RB, SPREAD>(acc, pa, pb, kbytes, sa, sb,
                                                                                       a_row, b_row);
    } else {
        mainloop_dma<Elt::BF16, BM, BN, (SWIGLU ? BN / 2 : BN), NS, NW, RB, SPREAD, TC>(acc, pa, pb, kbytes, st, a_row,
                                                                                     b_row);
    }

    const float sw = w_scale ? *w_scale : 1.0f;
    if constexpr (ACT == kActCe && TC)
        ce_epilogue_tc<BM, BN, WAVES_M, WAVES_N, TM, TN>(acc, rt, tt, sw, ce, M, N_out, m0, j0, tile_n, wm, wn,
                                                         ce_red);
    else if constexpr (ACT == kActCe)
        ce_epilogue<BM, BN, WAVES_M, WAVES_N, TM, TN>(acc, rv, tv, sw, ce, M, N_out, m0, j0, tile_n, wm, wn, slab,
                                                      ce_red);
    else if constexpr (ACT == kActSwigluBwd)
        swiglu_bwd_epilogue<BM, BN, WAVES_M, WAVES_N, TM, TN>(acc, rv, bw, M, N_out, m0, j0, tile_n, wm, wn, slab,
                                                              ce_red);
    else if constexpr (ACT == kActCeBwd && TC)
        ce_bwd_epilogue_tc<BM, BN, WAVES_M, WAVES_N, TM, TN>(acc, rt, tt, lt, gt, bw, M, N_out, m0, j0, tile_n, wm,
                                                             wn);
    else if constexpr (ACT == kActCeBwd)
        ce_bwd_epilogue<BM, BN, WAVES_M, WAVES_N, TM, TN>(acc, rv, tv, lv, gv, bw, M, N_out, m0, j0, tile_n, wm, wn,
                                                          slab);
    else if constexpr (TC) {
        float rt[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) rt[tm] = __shfl(rv[tm / 2], (tm % 2) * 32 + (threadIdx.x & 31));
        swiglu_epilogue_tc<BM, BN, WAVES_M, TM, TN>(acc, rt, sw, Y, M, N_out, m0, j0, wm, wn);
    }
    else if constexpr (ACT == kActSwigluSave)
        swiglu_save_epilogue<BM, BN, WAVES_M, TM, TN>(acc, rv, sw, Y, bw.dz, M, N_out, m0, j0, wm, wn, slab);
    else
        rowscale_epilogue<BM, BN, WAVES_M, TM, TN, ACT>(acc, rv, pv, rope, sw, Y, M, N_out, m0, j0, wm, wn, slab);
}

// Epilogue hook of the persistent kernel: after block pair P of PARTS, share P of the next
// tile's prologue DMA (when there is a next tile).
template <class Pro, int PARTS>
struct ProHook {
    const Pro& pro;
    bool more;
    template <int P>
    __device__ __forceinline__ void at() const {
        if (more) pro.template issue_share<P, PARTS>();
    }
};

// Persistent form of the forward SwiGLU GEMM (bf16 weights, transposed accumulator
// blocks, the epilogue of swiglu_epilogue_tc): a grid of at most one workgroup per CU
// walks tiles blockIdx.x, blockIdx.x + gridDim.x, ... in the XCD-aware order of the
// one-tile-per-workgroup launch (with gridDim.x a multiple of 8, tile t still runs on XCD
// t mod 8).  The epilogue touches no LDS, so the next tile's first k-tiles are issued
// into the stages during it, a share after each block pair's stores (one burst of them
// stalls the issuing wave once the address queue is full), and their latency hides
// behind the rest of the epilogue; the next tile's row scales are loaded after it (the
// mainloop's first wait leaves those loads in flight).
template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int RB, int SPREAD>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1)
k_gemm_swiglu_persistent(const uint8_t* __restrict__ H, const uint8_t* __restrict__ W,
                         const float* __restrict__ w_scale, const float* __restrict__ R, uint16_t* __restrict__ Y,
                         int M, int N_out, int K, int tiles_m, int tiles_n) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int BNO = BN / 2;                      // output columns of one block tile
    static_assert(TN % 2 == 0, "SwiGLU pairs gate and up blocks");
    constexpr int kStage = BM * RB + BN * RB;
    __shared__ __attribute__((aligned(1024))) uint8_t stages[NS][kStage];
    uint8_t* st[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) st[i] = stages[i];
    using FP = FragPair<Frags<Elt::BF16, TM, TN, RB, true>>;
    using PanelA = DmaPanel<BM, BM, NW, RB>;
    using PanelB = DmaPanel<BN, BN / 2, NW, RB>;

    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int kbytes = K * 2;
    const int ntiles = tiles_m * tiles_n;
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    // blocks [0, TN/2) = this wave's gate rows, [TN/2, TN) = the matching up rows
    auto b_row = [&](int tn) {
        constexpr int TH = TN / 2;
        return (tn < TH ? 0 : BN / 2) + wn * TH * 32 + (tn % TH) * 32;
    };
    PanelA pa;
    PanelB pb;
    int m0 = 0, j0 = 0;
    float rv[TM];                                    // r of the lane's row in each block row
    // panels of tile t
    auto setup = [&](int t) {
        int tile_m, tile_n;
        tile_coords<8>(t, tiles_m, tiles_n, tile_m, tile_n);
        m0 = tile_m * BM;
        j0 = tile_n * BNO;
        const uint8_t* a0 = H + static_cast<size_t>(m0) * kbytes;
        pa.init(a0, min(BM, M - m0), a0, 0, kbytes);
        const uint8_t* g0 = W + static_cast<size_t>(j0) * kbytes;
        const uint8_t* u0 = W + static_cast<size_t>(N_out + j0) * kbytes;
        pb.init(g0, min(BN / 2, N_out - j0), u0, min(BN / 2, N_out - j0), kbytes);
    };
    // row scales of the tile set up last (rows past M: 0, through the descriptor's range
    // check); TM loads, issued after its prologue DMA: the mainloop's first wait leaves
    // exactly TM loads in flight after the prologue, so every wave issues all of them
    // (a load guarded by a row check would be skipped by waves whose rows all lie past M)
    const __amdgpu_buffer_rsrc_t r_rsrc = make_buffer_rsrc(R, static_cast<uint32_t>(M) * 4u);
    auto load_r = [&]() {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t m = static_cast<uint32_t>(m0 + wm * WM + 32 * i + (threadIdx.x & 31));
            rv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, m * 4u, 0, 0));
        }
    };
    using Pro = DmaPrologue<FP, BM, NS, RB, SPREAD, TM, TN, PanelA, PanelB>;
    const Pro pro{pa, pb, kbytes, kbytes, st};
    const float sw = w_scale ? *w_scale : 1.0f;
    int t = blockIdx.x;                              // the grid holds at most ntiles workgroups
    setup(t);
    static_for<Pro::kOps>([&](auto Q) { pro.template issue<decltype(Q)::value>(); });
    auto pend = pro.template pending<TM>();
    load_r();
    for (; t < ntiles; t += gridDim.x) {
        f32x16_t acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
        mainloop_dma_run<FP, BM, BN, BN / 2, NS, NW, RB, RB, SPREAD>(acc, pa, pb, kbytes, kbytes, st, a_row, b_row,
                                                                     pend);
        // the mainloop ended with every DMA drained and a barrier: the stages are free
        const int cm0 = m0, cj0 = j0;
        float rc[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) rc[i] = rv[i];
        const bool more = t + static_cast<int>(gridDim.x) < ntiles;     // uniform over the workgroup
        if (more) setup(t + gridDim.x);
        swiglu_epilogue_tc<BM, BN, WAVES_M, TM, TN>(acc, rc, sw, Y, M, N_out, cm0, cj0, wm, wn,
                                                    ProHook<Pro, TM * (TN / 2)>{pro, more});
        if (more) {
            pend = pro.template pending<TM>();
            load_r();
        }
    }
}

// Output staging of the overlapped GEMMs: one wave's slab in LDS (two halves of 4 KB), each
// half 32 rows x 64 output columns (128 bytes per row): with SwiGLU a half is one block row
// of the tile (the wave's 64 output columns), without an activation a block row's 128
// output columns fill both halves (col_off 0 and 64).  16-byte chunk c of slab row r lies
// at r*128 + (c ^ ((r >> 1) & 7))*16, so both the epilogue's row-wise writes (16 rows at one
// chunk per 16 lanes) and the line-wise reads (2 rows x 8 chunks) are conflict-free.  A
// half is stored by four instructions, store i covering rows 8i .. 8i+7 with 8 lanes per
// 128-byte row (lane l: row 8i + l/8, chunk l%8); the transposed accumulator layout alone
// would give 32 rows x 32 bytes per instruction.
struct YSlab {
    uint8_t* ys;                     // this wave's slab
    __amdgpu_buffer_rsrc_t rsrc;     // y rows [m0, m0 + valid rows) of the tile
    uint32_t row_bytes;
    int row0, col0, n_out;           // the wave's first row (tile-relative) and output column
    __device__ __forceinline__ static int off(int hf, int r, int c) {
        return hf * 4096 + r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
    }
    // store i of block row tm from half hf, whose first column is col0 + col_off
    __device__ __forceinline__ void store(int hf, int tm, int i, int col_off) const {
        const int lane = threadIdx.x & 63;
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(ys + off(hf, r, c));
        const uint32_t row_off = static_cast<uint32_t>(row0 + tm * 32 + r) * row_bytes;
        const int n = col0 + col_off + c * 8;
        const uint32_t voff = n < n_out ? row_off + static_cast<uint32_t>(n) * 2 : kOobOffset;
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, voff, 0, 0);
    }
};

// One tile boundary of the overlapped persistent GEMM with the row-scale epilogue
// (k_gemm_rowscale_ovl), SWIGLU: y = SiLU(r s acc_gate) * r s acc_up from gate/up block
// pairs (blocks b and b + TN/2), else y = r s acc from pairs of adjacent column blocks
// (2b, 2b + 1):
// EPI: the epilogue of the tile whose sums acc holds (row scales rt, origin m0, j0), the
// arithmetic of swiglu_epilogue_tc / the staged plain epilogue in the same order, its
// output through the slab (YSlab);
// MMA: the next tile's k-tile 0 (stage 0; its first k-step's fragments in f.f[0], the
// other k-steps read here) multiplied into acc block pair by block pair, each pair right
// after the epilogue has read its accumulators out (a zero C operand starts the pair), so
// the matrix cores run while the epilogue's VALU work does; the rest of the next tile's
// k-tile 1 DMA (instructions kPer .. kPerTile-1, offsets o) is issued over the first
// pairs, and after pair HOLD-1 the wave waits for it (vmcnt 0: no store has been issued
// yet, the first HOLD / 2 block rows wait in the slab) and passes a barrier, so that
// k-tile 1 has landed for every wave when the next mainloop starts; the later block rows
// leave as soon as they are complete.
template <bool SWIGLU, bool EPI, bool MMA, int BM, int BN, int WAVES_M, int TM, int TN, int RB, int SPREAD, int HOLD,
          class FP, class PA, class PB, class Off, class ARow, class BRow>
__device__ __forceinline__ void rowscale_epilogue_ovl(f32x16_t (&acc)[TM][TN], const FP& f, const float (&rt)[TM],
                                                      float sw, uint16_t* __restrict__ Y, int M, int N_out, int m0,
                                                      int j0, int wm, int wn, const PA& pa, const PB& pb,
                                                      const Off& o, uint8_t* const (&st)[2], uint8_t* ys,
                                                      const ARow& a_row, const BRow& b_row) {
    using D = DmaSched<FP, 2, SPREAD, TM, TN, PA, PB>;
    constexpr int KS = D::KS, kPer = D::kPer0, kPerTile = D::kPerTile, nA = D::nA;   // kPer0 went out at the crossing
    constexpr int kRest = kPerTile - kPer;          // DMA instructions of k-tile 1 still to issue
    constexpr int kRestParts = HOLD < 3 ? HOLD : 3; // ... spread over the first pairs
    constexpr int WM = BM / WAVES_M;
    constexpr int NB = TN / 2;                      // pairs per block row
    constexpr int NP = TM * NB;                     // block pairs
    constexpr int kHalves = SWIGLU ? 1 : 2;         // slab halves per block row
    constexpr int kHeldRows = HOLD / NB;            // block rows stored after the wait
    static_assert(!MMA || (HOLD >= kRestParts && HOLD <= NP), "the wait follows the last DMA share");
    static_assert(NB == 2 && HOLD % NB == 0 && kHeldRows * kHalves <= 2,
                  "a block row fills kHalves slab halves; the held block rows fit the two halves");
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int lr = lane & 31, lh = lane >> 5;
    const int valid_rows = min(BM, M - m0);
    const uint32_t row_bytes = static_cast<uint32_t>(N_out) * 2;
    const YSlab ysl{ys,
                    make_buffer_rsrc(Y + static_cast<size_t>(m0) * N_out,
                                     EPI ? static_cast<uint32_t>(valid_rows) * row_bytes : 0u),
                    row_bytes, wm * WM, j0 + wn * NB * 32 * kHalves, N_out};
    // block row tm's output from the slab
    auto store_row = [&](int tm) {
        static_for<kHalves>([&](auto Hc) {
            constexpr int hx = decltype(Hc)::value;
            const int hf = SWIGLU ? (tm & 1) : hx;
            static_for<4>([&](auto Ic) { ysl.store(hf, tm, Ic, hx * 64); });
        });
    };
    // fragments of k-steps 1 .. KS-1 of the next tile's k-tile 0: every B block, A per block row
    const uint8_t* sA = st[0];
    const uint8_t* sB = st[0] + BM * RB;
    bf16x8_t bq[KS - 1][TN], aq[KS - 1];
    if constexpr (MMA) {
        static_for<KS - 1>([&](auto Sc) {
            constexpr int s = decltype(Sc)::value + 1;
            static_for<TN>([&](auto Tc) {
                constexpr int tn = decltype(Tc)::value;
                bq[s - 1][tn] = *reinterpret_cast<const bf16x8_t*>(sB + swz<RB>(b_row(tn) + lr, 2 * s + lh));
            });
        });
    }
    if constexpr (EPI) acc_read_fence();
    static_for<TM>([&](auto TMc) {
        constexpr int tm = decltype(TMc)::value;
        if constexpr (MMA) {
            static_for<KS - 1>([&](auto Sc) {
                constexpr int s = decltype(Sc)::value + 1;
                aq[s - 1] = *reinterpret_cast<const bf16x8_t*>(sA + swz<RB>(a_row(tm) + lr, 2 * s + lh));
            });
        }
        const float rr = EPI ? rt[tm] * sw : 0.0f;
        static_for<NB>([&](auto Bc) {
            constexpr int b = decltype(Bc)::value;
            constexpr int p = tm * NB + b;
            constexpr int x0 = SWIGLU ? b : 2 * b, x1 = SWIGLU ? b + NB : 2 * b + 1;   // the pair's blocks
            float gv[16], uv[16];
            if constexpr (EPI) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    gv[i] = acc_read(acc[tm][x0][i]);
                    uv[i] = acc_read(acc[tm][x1][i]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (MMA) {
                // the pair's blocks of the next tile: k-step 0 from f.f[0], then aq / bq
                static_for<KS>([&](auto Sc) {
                    constexpr int s = decltype(Sc)::value;
                    static_for<2>([&](auto Xc) {
                        constexpr int x = decltype(Xc)::value == 0 ? x0 : x1;
                        const bf16x8_t av = s == 0 ? f.f[0].a[tm] : aq[s - 1 < 0 ? 0 : s - 1];
                        const bf16x8_t bv = s == 0 ? f.f[0].b[x] : bq[s - 1 < 0 ? 0 : s - 1][x];
                        acc[tm][x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, av, s == 0 ? f32x16_t{} : acc[tm][x],
                                                                             0, 0, 0);
                    });
                });
            }
            if constexpr (EPI) {
                // lane (row lr, half lh) ends with 16-byte chunks of its slab row: SwiGLU
                // 4b + 2q + lh of half tm & 1; plain, block x0 / x1 give 2q + lh / 4 + 2q + lh
                // of half b
                auto put = [&](const uint32_t (&pk)[4][2], int hf, int c0) {
                    static_for<2>([&](auto Qc) {
                        constexpr int q = decltype(Qc)::value;
                        uint32_t w[4];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const auto sw2 =
                                __builtin_amdgcn_permlane32_swap(pk[2 * q][h], pk[2 * q + 1][h], false, false);
                            w[h] = sw2[0];
                            w[2 + h] = sw2[1];
                        }
                        *reinterpret_cast<i32x4_t*>(ys + YSlab::off(hf, lr, c0 + 2 * q + lh)) =
                            i32x4_t{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
                    });
                };
                if constexpr (SWIGLU) {
                    uint32_t pk[4][2];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float gs = gv[4 * g + e] * rr;
                            const float us = uv[4 * g + e] * rr;
                            v[e] = gs * __builtin_amdgcn_rcpf(1.0f + __expf(-gs)) * us;
                        }
                        pk[g][0] = pack_bf16x2(v[0], v[1]);
                        pk[g][1] = pack_bf16x2(v[2], v[3]);
                    }
                    put(pk, tm & 1, 4 * b);
                } else {
                    uint32_t pk0[4][2], pk1[4][2];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        pk0[g][0] = pack_bf16x2(gv[4 * g] * rr, gv[4 * g + 1] * rr);
                        pk0[g][1] = pack_bf16x2(gv[4 * g + 2] * rr, gv[4 * g + 3] * rr);
                        pk1[g][0] = pack_bf16x2(uv[4 * g] * rr, uv[4 * g + 1] * rr);
                        pk1[g][1] = pack_bf16x2(uv[4 * g + 2] * rr, uv[4 * g + 3] * rr);
                    }
                    put(pk0, b, 0);
                    put(pk1, b, 4);
                }
                // a complete block row leaves at once unless it is held for the wait
                if constexpr (b == NB - 1 && !(MMA && tm < kHeldRows)) store_row(tm);
            }
            if constexpr (MMA) {
                static_for<kRest>([&](auto Qc) {
                    constexpr int q = decltype(Qc)::value;
                    if constexpr (q * kRestParts / kRest == p) {
                        constexpr int qq = kPer + q;
                        if constexpr (qq < nA) pa.issue_one(qq, st[1], o.a);
                        else pb.issue_one(qq - nA, st[1] + BM * RB, o.b);
                    }
                });
                if constexpr (p == HOLD - 1) {
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // k-tile 1 landed (no store issued yet)
                    __syncthreads();                               // ... for every wave
                    if constexpr (EPI) static_for<kHeldRows>([&](auto Tc) { store_row(decltype(Tc)::value); });
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    });
}

// Persistent GEMM with the row-scale epilogue overlapped (bf16 weights, transposed
// accumulator blocks; SWIGLU: gate/up panels and the SwiGLU epilogue, else one weight
// panel and y = r s acc): the tile walk of k_gemm_swiglu_persistent, the DMA stream running
// across tiles (mainloop_dma_cont loads the next tile's k-tiles 0 and 1 in the current
// tile's last two crossings), and each tile's epilogue fused with the next tile's k-tile 0
// (rowscale_epilogue_ovl).  The first tile's k-tile 0 runs alone, the last tile's epilogue
// alone.  A tile's row scales load once its predecessor's epilogue is done.  Needs at
// least 3 k-tiles (K > 128); when this workgroup has no next tile the "next" panels are
// the current ones (their loads are in bounds and never used).  LDS: the two 64 KB stages
// and four 8 KB output slabs, the whole 160 KB.
template <bool SWIGLU, int BM, int BN, int WAVES_M, int WAVES_N, int RB, int SPREAD, int HOLD>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1)
k_gemm_rowscale_ovl(const uint8_t* __restrict__ H, const uint8_t* __restrict__ W, const float* __restrict__ w_scale,
                    const float* __restrict__ R, uint16_t* __restrict__ Y, int M, int N_out, int K, int tiles_m,
                    int tiles_n, int group) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int BNO = SWIGLU ? BN / 2 : BN;       // output columns of one block tile
    static_assert(TN % 2 == 0, "block pairs");
    static_assert(WN == 128, "a wave's output columns are one (SwiGLU) or two 128-byte row segments");
    constexpr int kStage = BM * RB + BN * RB;
    __shared__ __attribute__((aligned(1024))) uint8_t stages[2][kStage];
    __shared__ __attribute__((aligned(16))) uint8_t yslab[NW][8192];
    uint8_t* st[2] = {stages[0], stages[1]};
    using FP = FragPair<Frags<Elt::BF16, TM, TN, RB, true>>;
    using PanelA = DmaPanel<BM, BM, NW, RB>;
    using PanelB = DmaPanel<BN, SWIGLU ? BN / 2 : BN, NW, RB>;
    using D = DmaSched<FP, 2, SPREAD, TM, TN, PanelA, PanelB>;

    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    uint8_t* ys = yslab[wave];
    const int kbytes = K * 2;
    const int ntiles = tiles_m * tiles_n;
    const int G = gridDim.x;
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    // SWIGLU: blocks [0, TN/2) = this wave's gate rows, [TN/2, TN) = the matching up rows
    auto b_row = [&](int tn) {
        if constexpr (SWIGLU) {
            constexpr int TH = TN / 2;
            return (tn < TH ? 0 : BN / 2) + wn * TH * 32 + (tn % TH) * 32;
        }
        return wn * WN + tn * 32;
    };
    auto setup = [&](int t, PanelA& A, PanelB& B, int& tm0, int& tj0) {
        int tile_m, tile_n;
        tile_coords_g(t, tiles_m, tiles_n, group, tile_m, tile_n);
        tm0 = tile_m * BM;
        tj0 = tile_n * BNO;
        const uint8_t* a0 = H + static_cast<size_t>(tm0) * kbytes;
        A.init(a0, min(BM, M - tm0), a0, 0, kbytes);
        const uint8_t* g0 = W + static_cast<size_t>(tj0) * kbytes;
        if constexpr (SWIGLU) {
            const uint8_t* u0 = W + static_cast<size_t>(N_out + tj0) * kbytes;
            B.init(g0, min(BNO, N_out - tj0), u0, min(BNO, N_out - tj0), kbytes);
        } else {
            B.init(g0, min(BNO, N_out - tj0), g0, 0, kbytes);
        }
    };
    const __amdgpu_buffer_rsrc_t r_rsrc = make_buffer_rsrc(R, static_cast<uint32_t>(M) * 4u);
    float rv[TM];
    auto load_r = [&](int tm0) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t m = static_cast<uint32_t>(tm0 + wm * WM + 32 * i + (threadIdx.x & 31));
            rv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, m * 4u, 0, 0));
        }
    };
    const float sw = w_scale ? *w_scale : 1.0f;
    PanelA pa, na;
    PanelB pb, nb;
    int m0 = 0, j0 = 0, nm0 = 0, nj0 = 0;
    int t = blockIdx.x;                              // the grid holds at most ntiles workgroups
    setup(t, pa, pb, m0, j0);
    if (t + G < ntiles) setup(t + G, na, nb, nm0, nj0);
    else { na = pa; nb = pb; }
    // k-tile 0 of the first tile and the first share of its k-tile 1
    using Off = DmaPending<decltype(pa.base_offset(0, kbytes)), decltype(pb.base_offset(0, kbytes))>;
    {
        const Off o0{pa.base_offset(0, kbytes), pb.base_offset(0, kbytes)};
        static_for<D::kPerTile>([&](auto Qc) {
            constexpr int q = decltype(Qc)::value;
            if constexpr (q < D::nA) pa.issue_one(q, st[0], o0.a);
            else pb.issue_one(q - D::nA, st[0] + BM * RB, o0.b);
        });
    }
    Off o{pa.base_offset(1, kbytes), pb.base_offset(1, kbytes)};
    static_for<D::kPer0>([&](auto Qc) {
        constexpr int q = decltype(Qc)::value;
        if constexpr (q < D::nA) pa.issue_one(q, st[1], o.a);
        else pb.issue_one(q - D::nA, st[1] + BM * RB, o.b);
    });
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(D::kPer0));   // k-tile 0 landed
    __syncthreads();
    FP f;
    f.load(0, st[0], st[0] + BM * RB, 0, a_row, b_row);
    f32x16_t acc[TM][TN];
    rowscale_epilogue_ovl<SWIGLU, false, true, BM, BN, WAVES_M, TM, TN, RB, SPREAD, HOLD>(
        acc, f, rv, sw, Y, M, N_out, m0, j0, wm, wn, pa, pb, o, st, ys, a_row, b_row);
    load_r(m0);
    for (;;) {
        o = mainloop_dma_cont<FP, BM, RB, SPREAD, TM, TN>(acc, f, pa, pb, na, nb, kbytes, st, a_row, b_row);
        const int cm0 = m0, cj0 = j0;                // the tile whose sums acc holds
        t += G;
        if (t >= ntiles) break;                      // uniform over the workgroup
        pa = na;
        pb = nb;
        m0 = nm0;
        j0 = nj0;
        if (t + G < ntiles) setup(t + G, na, nb, nm0, nj0);
        rowscale_epilogue_ovl<SWIGLU, true, true, BM, BN, WAVES_M, TM, TN, RB, SPREAD, HOLD>(
            acc, f, rv, sw, Y, M, N_out, cm0, cj0, wm, wn, pa, pb, o, st, ys, a_row, b_row);
        load_r(m0);
    }
    rowscale_epilogue_ovl<SWIGLU, true, false, BM, BN, WAVES_M, TM, TN, RB, SPREAD, HOLD>(
        acc, f, rv, sw, Y, M, N_out, m0, j0, wm, wn, pa, pb, o, st, ys, a_row, b_row);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));       // the unused loads of the last crossings
}

// Persistent form of the LM-head GEMM with the loss epilogue (bf16 weights, transposed
// accumulator blocks, ce_epilogue_tc), the same tile walk and prologue overlap as the
// persistent SwiGLU GEMM: the next tile's DMA goes out in four shares, one after each of
// the epilogue's block rows, and the next tile's row scales and targets load after the
// epilogue (both through buffer descriptors over [0, M), so every wave issues all of
// them; a target past M is replaced by -1 after the load).
template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int RB, int SPREAD>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1)
k_gemm_ce_persistent(const uint8_t* __restrict__ H, const uint8_t* __restrict__ W,
                     const float* __restrict__ w_scale, const float* __restrict__ R, CeArgs ce, int M, int V,
                     int K, int tiles_m, int tiles_n) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int kStage = BM * RB + BN * RB;
    __shared__ __attribute__((aligned(1024))) uint8_t stages[NS][kStage];
    __shared__ float ce_red[2 * WAVES_N * BM];
    uint8_t* st[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) st[i] = stages[i];
    using FP = FragPair<Frags<Elt::BF16, TM, TN, RB, true>>;
    using PanelA = DmaPanel<BM, BM, NW, RB>;
    using PanelB = DmaPanel<BN, BN, NW, RB>;

    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int kbytes = K * 2;
    const int ntiles = tiles_m * tiles_n;
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    auto b_row = [&](int tn) { return wn * WN + tn * 32; };
    PanelA pa;
    PanelB pb;
    int m0 = 0, j0 = 0, tn0 = 0;
    float rv[TM];                                    // r and target of the lane's row in each block row
    int tv[TM];
    auto setup = [&](int t) {
        int tile_m, tile_n;
        tile_coords<CODA_G3_CE_GROUP>(t, tiles_m, tiles_n, tile_m, tile_n);
        m0 = tile_m * BM;
        j0 = tile_n * BN;
        tn0 = tile_n;
        const uint8_t* a0 = H + static_cast<size_t>(m0) * kbytes;
        pa.init(a0, min(BM, M - m0), a0, 0, kbytes);
        const uint8_t* b0 = W + static_cast<size_t>(j0) * kbytes;
        pb.init(b0, min(BN, V - j0), b0, 0, kbytes);
    };
    const __amdgpu_buffer_rsrc_t r_rsrc = make_buffer_rsrc(R, static_cast<uint32_t>(M) * 4u);
    const __amdgpu_buffer_rsrc_t t_rsrc = make_buffer_rsrc(ce.targets, static_cast<uint32_t>(M) * 4u);
    auto load_rows = [&]() {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm * WM + 32 * i + (threadIdx.x & 31);
            const uint32_t off = static_cast<uint32_t>(m) * 4u;
            rv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, off, 0, 0));
            const int x = __builtin_amdgcn_raw_buffer_load_b32(t_rsrc, off, 0, 0);
            tv[i] = m < M ? x : -1;
        }
    };
    using Pro = DmaPrologue<FP, BM, NS, RB, SPREAD, TM, TN, PanelA, PanelB>;
    const Pro pro{pa, pb, kbytes, kbytes, st};
    const float sw = w_scale ? *w_scale : 1.0f;
    int t = blockIdx.x;                              // the grid holds at most ntiles workgroups
    setup(t);
    static_for<Pro::kOps>([&](auto Q) { pro.template issue<decltype(Q)::value>(); });
    auto pend = pro.template pending<2 * TM>();
    load_rows();
    for (; t < ntiles; t += gridDim.x) {
        f32x16_t acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
        mainloop_dma_run<FP, BM, BN, BN, NS, NW, RB, RB, SPREAD>(acc, pa, pb, kbytes, kbytes, st, a_row, b_row, pend);
        const int cm0 = m0, cj0 = j0, ctn = tn0;
        float rc[TM];
        int tc[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            rc[i] = rv[i];
            tc[i] = tv[i];
        }
        const bool more = t + static_cast<int>(gridDim.x) < ntiles;     // uniform over the workgroup
        if (more) setup(t + gridDim.x);
        ce_epilogue_tc<BM, BN, WAVES_M, WAVES_N, TM, TN>(acc, rc, tc, sw, ce, M, V, cm0, cj0, ctn, wm, wn, ce_red,
                                                         ProHook<Pro, TM>{pro, more});
        if (more) {
            pend = pro.template pending<2 * TM>();
            load_rows();
        }
    }
}

// One tile boundary of the overlapped LM-head GEMM with the loss epilogue (k_gemm_ce_ovl),
// as rowscale_epilogue_ovl for the SwiGLU GEMM:
// EPI: the loss statistics of the tile whose sums acc holds (ce_epilogue_tc's arithmetic
// in the same order: per block row the logits r*s*acc, columns past V at -inf, the row's
// max and sum of exponentials over the wave's columns, the target's logit; then across the
// waves of a row through red, one (max, sum) partial per row and tile);
// MMA: the next tile's k-tile 0 multiplied into acc block row by block row, each right
// after the epilogue has read that block row out, and the rest of the next tile's k-tile 1
// DMA issued over the first block rows; the barrier that precedes the cross-wave step
// follows a wait for that DMA (vmcnt 0: only the rare target-logit stores can be in
// flight), so k-tile 1 has landed for every wave when the next mainloop starts.
template <bool EPI, bool MMA, int BM, int BN, int WAVES_M, int WAVES_N, int TM, int TN, int RB, int SPREAD,
          class FP, class PA, class PB, class Off, class ARow, class BRow>
__device__ __forceinline__ void ce_epilogue_ovl(f32x16_t (&acc)[TM][TN], const FP& f, const float (&rt)[TM],
                                                const int (&tt)[TM], float sw, const CeArgs& ce, int M, int V,
                                                int m0, int j0, int tile_n, int wm, int wn, float* red, const PA& pa,
                                                const PB& pb, const Off& o, uint8_t* const (&st)[2],
                                                const ARow& a_row, const BRow& b_row) {
    using D = DmaSched<FP, 2, SPREAD, TM, TN, PA, PB>;
    constexpr int KS = D::KS, kPer = D::kPer0, kPerTile = D::kPerTile, nA = D::nA;   // kPer0 went out at the crossing
    constexpr int kRest = kPerTile - kPer;
    constexpr int kRestParts = TM < 3 ? TM : 3;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, NT = 64 * WAVES_M * WAVES_N;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int lr = lane & 31, lh = lane >> 5;
    const float ninf = -__builtin_inff();
    const int nw = j0 + wn * WN;                    // first column of the wave
    const bool full = nw + WN <= V;                 // wave-uniform: no column past V
    const uint8_t* sA = st[0];
    const uint8_t* sB = st[0] + BM * RB;
    if constexpr (EPI) acc_read_fence();
    static_for<TM>([&](auto TMc) {
        constexpr int tm = decltype(TMc)::value;
        const float rr = EPI ? rt[tm] * sw : 0.0f;
        float z[TN][16];
        if constexpr (EPI) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) z[b][i] = acc_read(acc[tm][b][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MMA) {
            // fragments read per k-step from stage 0 (the logits hold 64 registers here, so
            // none are kept across block rows; f's copy of k-step 0 is not used)
            static_for<KS>([&](auto Sc) {
                constexpr int s = decltype(Sc)::value;
                const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(sA + swz<RB>(a_row(tm) + lr, 2 * s + lh));
                static_for<TN>([&](auto Bc) {
                    constexpr int b = decltype(Bc)::value;
                    const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(sB + swz<RB>(b_row(b) + lr, 2 * s + lh));
                    acc[tm][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, av, s == 0 ? f32x16_t{} : acc[tm][b],
                                                                         0, 0, 0);
                });
            });
            // a k-step's five reads, then its four MFMAs (no reads hoisted further ahead:
            // the logits hold 64 registers here)
            static_for<KS>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1 + TN, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
            });
        }
        if constexpr (EPI) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) z[b][i] *= rr;
            if (!full) {
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (nw + 32 * b + 8 * (i >> 2) + 4 * lh + (i & 3) >= V) z[b][i] = ninf;
            }
            float mx = ninf;
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, z[b][i]);
            mx = halves_max(mx);
            float sum = 0.0f;
            if (mx > ninf) {
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sum += __expf(z[b][i] - mx);
            }
            sum = halves_sum(sum);
            const int rl = wm * WM + tm * 32 + lr;      // row within the block tile
            const int tg = tt[tm];
            const int ot = tg - nw;
            if (ot >= 0 && ot < WN && tg < V) {
                const int c = ot & 31;
                if (((c >> 2) & 1) == lh) {
                    const int k = (ot >> 5) * 16 + ((c >> 3) << 2) + (c & 3);
                    float zt = 0.0f;
#pragma unroll
                    for (int b = 0; b < TN; ++b)
#pragma unroll
                        for (int i = 0; i < 16; ++i) zt = (k == 16 * b + i) ? z[b][i] : zt;
                    ce.tgt_logit[m0 + rl] = zt;
                }
            }
            if (lh == 0) {
                red[2 * (wn * BM + rl)] = mx;
                red[2 * (wn * BM + rl) + 1] = sum;
            }
        }
        if constexpr (MMA) {
            static_for<kRest>([&](auto Qc) {
                constexpr int q = decltype(Qc)::value;
                if constexpr (q * kRestParts / kRest == tm) {
                    constexpr int qq = kPer + q;
                    if constexpr (qq < nA) pa.issue_one(qq, st[1], o.a);
                    else pb.issue_one(qq - nA, st[1] + BM * RB, o.b);
                }
            });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (MMA) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));     // k-tile 1 landed
    __syncthreads();                                                   // ... and red is complete
    if constexpr (EPI) {
        for (int r = threadIdx.x; r < BM; r += NT) {
            const int m = m0 + r;
            if (m < M) {
                float mt = ninf;
#pragma unroll
                for (int w = 0; w < WAVES_N; ++w) mt = fmaxf(mt, red[2 * (w * BM + r)]);
                float st_ = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES_N; ++w) {
                    const float mw = red[2 * (w * BM + r)];
                    if (mw > ninf) st_ += red[2 * (w * BM + r) + 1] * __expf(mw - mt);
                }
                float* pp = ce.partials + (static_cast<size_t>(m) * ce.T + tile_n) * 2;
                pp[0] = mt;
                pp[1] = st_;
            }
        }
    }
}

// Overlapped form of the LM-head GEMM with the loss epilogue (bf16 weights, transposed
// accumulator blocks): k_gemm_ce_persistent's tile walk with the DMA stream running across
// tiles (mainloop_dma_cont) and each tile's loss statistics fused with the next tile's
// k-tile 0 (ce_epilogue_ovl).  A tile's row scales and targets load once its predecessor's
// epilogue is done (through descriptors over [0, M); a target past M becomes -1).  Needs
// at least 4 k-tiles (K > 128).
template <int BM, int BN, int WAVES_M, int WAVES_N, int RB, int SPREAD>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1)
k_gemm_ce_ovl(const uint8_t* __restrict__ H, const uint8_t* __restrict__ W, const float* __restrict__ w_scale,
              const float* __restrict__ R, CeArgs ce, int M, int V, int K, int tiles_m, int tiles_n) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int kStage = BM * RB + BN * RB;
    __shared__ __attribute__((aligned(1024))) uint8_t stages[2][kStage];
    __shared__ float ce_red[2 * WAVES_N * BM];
    uint8_t* st[2] = {stages[0], stages[1]};
    using FP = FragPair<Frags<Elt::BF16, TM, TN, RB, true>>;
    using PanelA = DmaPanel<BM, BM, NW, RB>;
    using PanelB = DmaPanel<BN, BN, NW, RB>;
    using D = DmaSched<FP, 2, SPREAD, TM, TN, PanelA, PanelB>;

    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int kbytes = K * 2;
    const int ntiles = tiles_m * tiles_n;
    const int G = gridDim.x;
    auto a_row = [&](int tm) { return wm * WM + tm * 32; };
    auto b_row = [&](int tn) { return wn * WN + tn * 32; };
    auto setup = [&](int t, PanelA& A, PanelB& B, int& tm0, int& tj0, int& ttn) {
        int tile_m, tile_n;
        tile_coords<8>(t, tiles_m, tiles_n, tile_m, tile_n);
        tm0 = tile_m * BM;
        tj0 = tile_n * BN;
        ttn = tile_n;
        const uint8_t* a0 = H + static_cast<size_t>(tm0) * kbytes;
        A.init(a0, min(BM, M - tm0), a0, 0, kbytes);
        const uint8_t* b0 = W + static_cast<size_t>(tj0) * kbytes;
        B.init(b0, min(BN, V - tj0), b0, 0, kbytes);
    };
    const __amdgpu_buffer_rsrc_t r_rsrc = make_buffer_rsrc(R, static_cast<uint32_t>(M) * 4u);
    const __amdgpu_buffer_rsrc_t t_rsrc = make_buffer_rsrc(ce.targets, static_cast<uint32_t>(M) * 4u);
    float rv[TM];
    int tv[TM];
    auto load_rows = [&](int tm0) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = tm0 + wm * WM + 32 * i + (threadIdx.x & 31);
            const uint32_t off = static_cast<uint32_t>(m) * 4u;
            rv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, off, 0, 0));
            const int x = __builtin_amdgcn_raw_buffer_load_b32(t_rsrc, off, 0, 0);
            tv[i] = m < M ? x : -1;
        }
    };
    const float sw = w_scale ? *w_scale : 1.0f;
    PanelA pa, na;
    PanelB pb, nb;
    int m0 = 0, j0 = 0, tn0 = 0, nm0 = 0, nj0 = 0, ntn = 0;
    int t = blockIdx.x;                              // the grid holds at most ntiles workgroups
    setup(t, pa, pb, m0, j0, tn0);
    if (t + G < ntiles) setup(t + G, na, nb, nm0, nj0, ntn);
    else { na = pa; nb = pb; }
    using Off = DmaPending<decltype(pa.base_offset(0, kbytes)), decltype(pb.base_offset(0, kbytes))>;
    {
        const Off o0{pa.base_offset(0, kbytes), pb.base_offset(0, kbytes)};
        static_for<D::kPerTile>([&](auto Qc) {
            constexpr int q = decltype(Qc)::value;
            if constexpr (q < D::nA) pa.issue_one(q, st[0], o0.a);
            else pb.issue_one(q - D::nA, st[0] + BM * RB, o0.b);
        });
    }
    Off o{pa.base_offset(1, kbytes), pb.base_offset(1, kbytes)};
    static_for<D::kPer0>([&](auto Qc) {
        constexpr int q = decltype(Qc)::value;
        if constexpr (q < D::nA) pa.issue_one(q, st[1], o.a);
        else pb.issue_one(q - D::nA, st[1] + BM * RB, o.b);
    });
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(D::kPer0));   // k-tile 0 landed
    __syncthreads();
    FP f;
    f.load(0, st[0], st[0] + BM * RB, 0, a_row, b_row);
    f32x16_t acc[TM][TN];
    ce_epilogue_ovl<false, true, BM, BN, WAVES_M, WAVES_N, TM, TN, RB, SPREAD>(
        acc, f, rv, tv, sw, ce, M, V, m0, j0, tn0, wm, wn, ce_red, pa, pb, o, st, a_row, b_row);
    load_rows(m0);
    for (;;) {
        o = mainloop_dma_cont<FP, BM, RB, SPREAD, TM, TN>(acc, f, pa, pb, na, nb, kbytes, st, a_row, b_row);
        const int cm0 = m0, cj0 = j0, ctn = tn0;     // the tile whose sums acc holds
        t += G;
        if (t >= ntiles) break;                      // uniform over the workgroup
        pa = na;
        pb = nb;
        m0 = nm0;
        j0 = nj0;
        tn0 = ntn;
        if (t + G < ntiles) setup(t + G, na, nb, nm0, nj0, ntn);
        ce_epilogue_ovl<true, true, BM, BN, WAVES_M, WAVES_N, TM, TN, RB, SPREAD>(
            acc, f, rv, tv, sw, ce, M, V, cm0, cj0, ctn, wm, wn, ce_red, pa, pb, o, st, a_row, b_row);
        load_rows(m0);
    }
    ce_epilogue_ovl<true, false, BM, BN, WAVES_M, WAVES_N, TM, TN, RB, SPREAD>(
        acc, f, rv, tv, sw, ce, M, V, m0, j0, tn0, wm, wn, ce_red, pa, pb, o, st, a_row, b_row);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));       // the unused loads of the last crossings
}

// Tile configurations of the second GEMM (compile-time).
#ifndef CODA_G3_BM
#define CODA_G3_BM 256
#define CODA_G3_BN 256
#define CODA_G3_WM 2
#define CODA_G3_WN 2
#define CODA_G3_NS 2
#define CODA_G3_RB 128
#define CODA_G3_OCC 1
#endif
#ifndef CODA_G3_SPREAD
#define CODA_G3_SPREAD 3
#endif
// The one-tile-per-workgroup GEMM on LDS stage rings (three h stages, two weight stages,
// mainloop_dma_ring_fp) for the recomputing SwiGLU backward (0.968-0.982 against 0.976-0.992
// ms on the 16K-token MLP input) and the loss backward (7.20-7.21 against 7.28 ms on the
// 128256-token LM head), whose operands the backward's other kernels have pushed out of the
// last-level cache, and for RoPE (with the rings' DMA spread of 4: 0.1905-0.1910 against
// 0.1936-0.1962 ms on the 16K-token QKV projection).  The same bits either way.
#ifndef CODA_G3_RING_BWD
#define CODA_G3_RING_BWD 1
#endif
// k-steps a k-tile's DMA is spread over on the rings (4: SwiGLU backward 0.8 %, loss
// backward 1.4 % faster than 3)
#ifndef CODA_G3_SPREAD_RING
#define CODA_G3_SPREAD_RING 4
#endif
#ifndef CODA_G3_RING_CEBWD
#define CODA_G3_RING_CEBWD 1
#endif
#ifndef CODA_G3_RING_ROPE
#define CODA_G3_RING_ROPE 1
#endif
#ifndef CODA_G3_PIPE
#define CODA_G3_PIPE 0
#endif
#ifndef CODA_G3_NS8
#define CODA_G3_NS8 2
#endif
#ifndef CODA_G3_OVL
#define CODA_G3_OVL 1       // ... with the epilogue overlapped (K > 128)
#endif
#ifndef CODA_G3_HOLD
#define CODA_G3_HOLD 4      // block pairs whose stores wait for the next tile's k-tile 1
#endif
#ifndef CODA_G3_PERSIST
#define CODA_G3_PERSIST 1   // forward SwiGLU on bf16 weights: the persistent kernel
#endif
#ifndef CODA_G3_PERSIST_CE
#define CODA_G3_PERSIST_CE 1   // the loss epilogue on bf16 weights: the persistent kernel
#endif
constexpr int BM3 = CODA_G3_BM, BN3 = CODA_G3_BN, NS3 = CODA_G3_NS, OCC3 = CODA_G3_OCC;
constexpr int WM3 = CODA_G3_WM, WN3 = CODA_G3_WN, RB3 = CODA_G3_RB, SP3 = CODA_G3_SPREAD, PIPE3 = CODA_G3_PIPE;
// 8-bit weights: a stage is 3/4 of a bf16 one, so a third stage fits where two do
constexpr int NS3_8 = CODA_G3_NS8;

int64_t gemm3_tiles(int64_t M, int64_t N_out, bool swiglu) {
    const int64_t bno = swiglu ? BN3 / 2 : BN3;
    return ((M + BM3 - 1) / BM3) * ((N_out + bno - 1) / bno);
}

// Tile-rows per group of the overlapped row-scale kernels' walk.  The 32 tiles an XCD runs
// at once cover G tile-rows x 32/G tile-columns.  With 1 MB K-panels (K <= 2048) G = 4
// touches the same 12 panels per round as G = 8 and writes y in 2 KB row runs (workload
// 2: -2.0 %, the QKV projection -4.0 % against G = 8).  G = 2 was another 1.3 % faster
// there but moved 2.70 instead of 1.89 GB through the L2 per launch (18 panels per round);
// with larger panels G = 8 is the best (K = 4096: G = 4 +1.2 %, G = 2 +4.3 %).
static int ovl_group(int K) { return K <= CODA_G3_OVL_SMALL_K ? 4 : 8; }

// Compute units of the current device, queried once per device (the persistent grid size).
static hipError_t cu_count(int* cus) {
    static std::atomic<int> cache[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return hipSuccess;
}

template <int ACT, bool WFP8, bool GFOLD = false, bool RING = false>
static hipError_t launch3(int M, int N_out, int K, const void* h, const void* W,
                          const float* w_scale, const float* r, void* y, const RopeArgs& rope,
                          const CeArgs& ce, const BwdArgs& bw, hipStream_t stream,
                          const float* gfold = nullptr) {
    constexpr int BNO = (ACT == kActSwiglu || ACT == kActSwigluBwd || ACT == kActSwigluSave) ? BN3 / 2 : BN3;
    const int tiles_m = (M + BM3 - 1) / BM3, tiles_n = (N_out + BNO - 1) / BNO;
    const dim3 grid(tiles_m * tiles_n), block(64 * WM3 * WN3);
    static_assert(!(GFOLD && WFP8), "the in-kernel fold takes a bf16 weight");
    constexpr int PIPE = GFOLD ? 2 : (WFP8 ? 0 : PIPE3);
    hipLaunchKernelGGL((k_gemm_rowscale_swiglu<BM3, BN3, WM3, WN3, WFP8 ? NS3_8 : NS3, RB3,
                                               RING ? CODA_G3_SPREAD_RING : SP3, PIPE, OCC3, ACT, WFP8, RING>),
                       grid, block, 0, stream, static_cast<const uint8_t*>(h), static_cast<const uint8_t*>(W),
                       w_scale, r, static_cast<uint16_t*>(y), M, N_out, K, tiles_m, tiles_n, rope, ce, bw, gfold);
    return hipGetLastError();
}

hipError_t launch_gemm_rowscale_gfold(int M, int N_out, int K, bool swiglu, const void* h, const void* W_raw,
                                      const float* gamma, const float* r, void* y, hipStream_t stream) {
    const RopeArgs none{nullptr, nullptr, nullptr, 0, 0};
    const CeArgs no_ce{nullptr, nullptr, nullptr, 0};
    const BwdArgs no_bw{nullptr, nullptr, nullptr, 0};
    return swiglu ? launch3<kActSwiglu, false, true>(M, N_out, K, h, W_raw, nullptr, r, y, none, no_ce, no_bw,
                                                     stream, gamma)
                  : launch3<kActNone, false, true>(M, N_out, K, h, W_raw, nullptr, r, y, none, no_ce, no_bw,
                                                   stream, gamma);
}

hipError_t launch_gemm_rowscale_swiglu(int M, int N_out, int K, bool swiglu, const void* h,
                                       const void* W, bool w_fp8, const float* w_scale,
                                       const float* r, void* y, hipStream_t stream) {
    const RopeArgs none{nullptr, nullptr, nullptr, 0, 0};
    const CeArgs no_ce{nullptr, nullptr, nullptr, 0};
    const BwdArgs no_bw{nullptr, nullptr, nullptr, 0};
    if (!swiglu && !w_fp8 && CODA_G3_OVL && NS3 == 2 && PIPE3 == 0 && 2 * K > 2 * RB3) {
        // plain row-scaled output: the overlapped persistent kernel, one block row held
        const int tiles_m = (M + BM3 - 1) / BM3, tiles_n = (N_out + BN3 - 1) / BN3;
        int cus = 0;
        const hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
        const int grid = std::min(tiles_m * tiles_n, std::max(cus, 1));
        hipLaunchKernelGGL((k_gemm_rowscale_ovl<false, BM3, BN3, WM3, WN3, RB3, SP3, 2>), dim3(grid),
                           dim3(64 * WM3 * WN3), 0, stream, static_cast<const uint8_t*>(h),
                           static_cast<const uint8_t*>(W), w_scale, r, static_cast<uint16_t*>(y), M, N_out, K, tiles_m,
                           tiles_n, ovl_group(K));
        return hipGetLastError();
    }
    if (swiglu && !w_fp8 && CODA_G3_PERSIST && CODA_G3_TC && PIPE3 == 0) {
        const int tiles_m = (M + BM3 - 1) / BM3, tiles_n = (N_out + BN3 / 2 - 1) / (BN3 / 2);
        int cus = 0;
        const hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
        const int grid = std::min(tiles_m * tiles_n, std::max(cus, 1));
        if (CODA_G3_OVL && NS3 == 2 && 2 * K > 2 * RB3) {     // at least 3 k-tiles (4 padded)
            hipLaunchKernelGGL((k_gemm_rowscale_ovl<true, BM3, BN3, WM3, WN3, RB3, SP3, CODA_G3_HOLD>), dim3(grid),
                               dim3(64 * WM3 * WN3), 0, stream, static_cast<const uint8_t*>(h),
                               static_cast<const uint8_t*>(W), w_scale, r, static_cast<uint16_t*>(y), M, N_out, K,
                               tiles_m, tiles_n, ovl_group(K));
            return hipGetLastError();
        }
        hipLaunchKernelGGL((k_gemm_swiglu_persistent<BM3, BN3, WM3, WN3, NS3, RB3, SP3>), dim3(grid),
                           dim3(64 * WM3 * WN3), 0, stream, static_cast<const uint8_t*>(h),
                           static_cast<const uint8_t*>(W), w_scale, r, static_cast<uint16_t*>(y), M, N_out, K, tiles_m,
                           tiles_n);
        return hipGetLastError();
    }
    if (swiglu)
        return w_fp8 ? launch3<kActSwiglu, true>(M, N_out, K, h, W, w_scale, r, y, none, no_ce, no_bw, stream)
                     : launch3<kActSwiglu, false>(M, N_out, K, h, W, w_scale, r, y, none, no_ce, no_bw, stream);
    return w_fp8 ? launch3<kActNone, true>(M, N_out, K, h, W, w_scale, r, y, none, no_ce, no_bw, stream)
                 : launch3<kActNone, false>(M, N_out, K, h, W, w_scale, r, y, none, no_ce, no_bw, stream);
}

hipError_t launch_gemm_rowscale_rope(int M, int N_out, int K, const void* h, const void* W,
                                     bool w_fp8, const float* w_scale, const float* r,
                                     const int32_t* pos, const float* cos, const float* sin,
                                     int table_rows, int rot_cols, void* y, hipStream_t stream) {
    const RopeArgs rope{pos, cos, sin, table_rows, rot_cols};
    const CeArgs no_ce{nullptr, nullptr, nullptr, 0};
    const BwdArgs no_bw{nullptr, nullptr, nullptr, 0};
    return w_fp8 ? launch3<kActRope, true>(M, N_out, K, h, W, w_scale, r, y, rope, no_ce, no_bw, stream)
                 : launch3<kActRope, false, false, CODA_G3_RING_ROPE != 0>(M, N_out, K, h, W, w_scale, r, y, rope,
                                                                         no_ce, no_bw, stream);
}

int64_t ce_partials_per_row(int64_t V) { return V < 1 ? -1 : (V + BN3 - 1) / BN3; }

hipError_t launch_gemm_rowscale_ce(int M, int V, int K, const void* h, const void* W, bool w_fp8,
                                   const float* w_scale, const float* r, const int32_t* targets,
                                   float* partials, float* tgt_logit, hipStream_t stream) {
    const RopeArgs none{nullptr, nullptr, nullptr, 0, 0};
    const CeArgs ce{targets, partials, tgt_logit, static_cast<int>(ce_partials_per_row(V))};
    const BwdArgs no_bw{nullptr, nullptr, nullptr, 0};
    if (!w_fp8 && CODA_G3_PERSIST_CE && CODA_G3_TC && CODA_G3_TC_CE && PIPE3 == 0) {
        const int tiles_m = (M + BM3 - 1) / BM3, tiles_n = (V + BN3 - 1) / BN3;
        int cus = 0;
        const hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
        const int grid = std::min(tiles_m * tiles_n, std::max(cus, 1));
        if (CODA_G3_OVL && NS3 == 2 && 2 * K > 2 * RB3) {     // at least 3 k-tiles (4 padded)
            hipLaunchKernelGGL((k_gemm_ce_ovl<BM3, BN3, WM3, WN3, RB3, SP3>), dim3(grid), dim3(64 * WM3 * WN3), 0,
                               stream, static_cast<const uint8_t*>(h), static_cast<const uint8_t*>(W), w_scale, r,
                               ce, M, V, K, tiles_m, tiles_n);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((k_gemm_ce_persistent<BM3, BN3, WM3, WN3, NS3, RB3, SP3>), dim3(grid),
                           dim3(64 * WM3 * WN3), 0, stream, static_cast<const uint8_t*>(h),
                           static_cast<const uint8_t*>(W), w_scale, r, ce, M, V, K, tiles_m, tiles_n);
        return hipGetLastError();
    }
    return w_fp8 ? launch3<kActCe, true>(M, V, K, h, W, w_scale, r, nullptr, none, ce, no_bw, stream)
                 : launch3<kActCe, false>(M, V, K, h, W, w_scale, r, nullptr, none, ce, no_bw, stream);
}

hipError_t launch_gemm_rowscale_swiglu_save(int M, int F, int K, const void* h, const void* W, const float* r,
                                            void* y, void* z, hipStream_t stream) {
    const RopeArgs none{nullptr, nullptr, nullptr, 0, 0};
    const CeArgs no_ce{nullptr, nullptr, nullptr, 0};
    const BwdArgs save{nullptr, static_cast<uint16_t*>(z), nullptr, 0};   // dz carries z
    return launch3<kActSwigluSave, false>(M, F, K, h, W, nullptr, r, y, none, no_ce, save, stream);
}

int64_t swiglu_bwd_partials_per_row(int64_t F) { return F < 1 ? -1 : (F + BN3 / 2 - 1) / (BN3 / 2); }

hipError_t launch_gemm_ce_bwd(int M, int V, int K, const void* h, const void* W, const float* r,
                              const int32_t* targets, const float* lse, const float* gw, void* dz, float* partials,
                              hipStream_t stream) {
    const RopeArgs none{nullptr, nullptr, nullptr, 0, 0};
    const CeArgs ce{targets, nullptr, nullptr, 0, lse, gw};
    // partials per row and 128 columns (a wave's share of a 256-column tile)
    const BwdArgs bw{nullptr, static_cast<uint16_t*>(dz), partials, static_cast<int>(swiglu_bwd_partials_per_row(V))};
    return launch3<kActCeBwd, false, false, CODA_G3_RING_CEBWD != 0>(M, V, K, h, W, nullptr, r, nullptr, none, ce,
                                                                      bw, stream);
}

hipError_t launch_gemm_swiglu_bwd(int M, int F, int K, const void* h, const void* W, const float* r,
                                  const void* dy, void* dz, float* partials, hipStream_t stream) {
    const RopeArgs none{nullptr, nullptr, nullptr, 0, 0};
    const CeArgs no_ce{nullptr, nullptr, nullptr, 0};
    const BwdArgs bw{static_cast<const uint16_t*>(dy), static_cast<uint16_t*>(dz), partials,
                     static_cast<int>(swiglu_bwd_partials_per_row(F))};
    return launch3<kActSwigluBwd, false, false, CODA_G3_RING_BWD != 0>(M, F, K, h, W, nullptr, r, nullptr, none,
                                                                        no_ce, bw, stream);
}

}  // namespace coda

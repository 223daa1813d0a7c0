// MFMA mainloop shared by the chain's two GEMM kernels (gfx950, wave64).
//
// Both operands stream K-contiguous rows: A[m, k] (activations) and B[n, k] (weights
// in the nn.Linear layout), so every global load is a 16-byte vector along K and every
// LDS fragment read is one 16-byte ds_read per lane.
//
// Block tile BM x BN, 256 threads = 4 waves arranged WAVES_M x WAVES_N; each wave owns
// a (BM/WAVES_M) x (BN/WAVES_N) sub-tile made of 32x32 MFMA blocks.  One k-tile is 128
// BYTES of every row (64 bf16 or 128 e4m3 values).  LDS holds two k-tiles (double
// buffer).  Inside a row the eight 16-byte chunks are XOR-swizzled with ((row >> 1) & 7)
// (see lds_off), so fragment reads are free of bank conflicts.
//
// MFMA output layout (32x32 blocks): lane l, accumulator i holds
//   row (A side) = 8*(i/4) + 4*(l/32) + (i%4),   column (B side) = l % 32.
#pragma once

#include "device_common.hpp"

namespace coda {

constexpr int kRowBytes = 128;   // bytes of one row per k-tile
constexpr int kThreads = 256;

// 16-byte chunk c of a 128-byte row r sits in slot c ^ ((r >> 1) & 7): the 16 lanes the
// 64-bank LDS serves together read 16 consecutive rows at one chunk and hit 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Operand kinds -------------------------------------------------------------------
enum class Elt { BF16, E4M3 };

// One k-tile = 128 bytes per row; number of elements per row-tile.
template <Elt E> struct EltInfo;
template <> struct EltInfo<Elt::BF16> { static constexpr int kBytes = 2; static constexpr int kPerTile = 64; };
template <> struct EltInfo<Elt::E4M3> { static constexpr int kBytes = 1; static constexpr int kPerTile = 128; };

// Global -> register staging of one k-tile of a ROWS x 128-byte panel.
// Chunk q (0 .. ROWS*8-1) = (row q/8, 16-byte chunk q%8); thread t handles chunks
// t, t+256, ...  `row_ptr(r)` returns the global address of panel row r's first byte
// (nullptr if the row is outside the matrix).  Chunks past the row's K bytes read 0.
template <int ROWS>
struct PanelStage {
    static constexpr int kPer = ROWS * 8 / kThreads;
    static_assert(kPer * kThreads == ROWS * 8, "panel rows must be a multiple of 32");
    i32x4_t v[kPer];

    template <class RowPtr>
    __device__ __forceinline__ void load(const RowPtr& row_ptr, int kbyte0, int kbytes) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int q = threadIdx.x + j * kThreads;
            const int r = q >> 3, c = q & 7;
            const uint8_t* p = row_ptr(r);
            const int kb = kbyte0 + c * 16;
            if (p != nullptr && kb < kbytes) {
                v[j] = *reinterpret_cast<const i32x4_t*>(p + kb);
            } else {
                v[j] = i32x4_t{0, 0, 0, 0};
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int q = threadIdx.x + j * kThreads;
            *reinterpret_cast<i32x4_t*>(lds + lds_off(q >> 3, q & 7)) = v[j];
        }
    }
};

// Same as PanelStage, but the global panel is e4m3 and LDS receives bf16: each 16-byte
// LDS chunk (8 bf16) comes from 8 global bytes, decoded exactly.
template <int ROWS>
struct PanelStageE4m3ToBf16 {
    static constexpr int kPer = ROWS * 8 / kThreads;
    static_assert(kPer * kThreads == ROWS * 8, "panel rows must be a multiple of 32");
    i32x2_t v[kPer];

    // kbyte0/kbytes are in units of the bf16 LDS row (2 bytes per element).
    template <class RowPtr>
    __device__ __forceinline__ void load(const RowPtr& row_ptr, int kbyte0, int kbytes) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int q = threadIdx.x + j * kThreads;
            const int r = q >> 3, c = q & 7;
            const uint8_t* p = row_ptr(r);
            const int kb = kbyte0 + c * 16;
            if (p != nullptr && kb < kbytes) {
                v[j] = *reinterpret_cast<const i32x2_t*>(p + (kb >> 1));
            } else {
                v[j] = i32x2_t{0, 0};
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int q = threadIdx.x + j * kThreads;
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t x = static_cast<uint32_t>(v[j][h]);
                w[2 * h + 0] = e4m3_to_bf16_bits(x & 0xFFu) | (uint32_t(e4m3_to_bf16_bits((x >> 8) & 0xFFu)) << 16);
                w[2 * h + 1] = e4m3_to_bf16_bits((x >> 16) & 0xFFu) | (uint32_t(e4m3_to_bf16_bits(x >> 24)) << 16);
            }
            *reinterpret_cast<i32x4_t*>(lds + lds_off(q >> 3, q & 7)) =
                i32x4_t{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
        }
    }
};

// MFMA step over one LDS k-tile for a wave's TM x TN blocks.
// a_row(tm) / b_row(tn): LDS panel row of the block's first row.
template <Elt E, int TM, int TN>
struct WaveMma;

template <int TM, int TN>
struct WaveMma<Elt::BF16, TM, TN> {
    template <class ARow, class BRow>
    __device__ __forceinline__ static void run(f32x16_t (&acc)[TM][TN], const uint8_t* sA,
                                               const uint8_t* sB, const ARow& a_row,
                                               const BRow& b_row) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int s = 0; s < 4; ++s) {          // 4 x k16 per 128-byte k-tile
            bf16x8_t a[TM], b[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                a[tm] = *reinterpret_cast<const bf16x8_t*>(sA + lds_off(a_row(tm) + lr, 2 * s + lh));
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                b[tn] = *reinterpret_cast<const bf16x8_t*>(sB + lds_off(b_row(tn) + lr, 2 * s + lh));
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
        }
    }
};

template <int TM, int TN>
struct WaveMma<Elt::E4M3, TM, TN> {
    template <class ARow, class BRow>
    __device__ __forceinline__ static void run(f32x16_t (&acc)[TM][TN], const uint8_t* sA,
                                               const uint8_t* sB, const ARow& a_row,
                                               const BRow& b_row) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int s = 0; s < 2; ++s) {          // 2 x k64 per 128-byte k-tile
            i32x8_t a[TM], b[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int row = a_row(tm) + lr;
                const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(sA + lds_off(row, 4 * s + 2 * lh));
                const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(sA + lds_off(row, 4 * s + 2 * lh + 1));
                a[tm] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int row = b_row(tn) + lr;
                const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(sB + lds_off(row, 4 * s + 2 * lh));
                const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(sB + lds_off(row, 4 * s + 2 * lh + 1));
                b[tn] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    // formats 0/0 = e4m3 x e4m3; block scales 127 = 2^0 (unscaled)
                    acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a[tm], b[tn], acc[tm][tn], 0, 0, 0, 127, 0, 127);
        }
    }
};

}  // namespace coda

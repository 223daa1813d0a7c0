// Epilogue building blocks shared by the chain's GEMM kernels (gfx950).
//
// After the mainloop the LDS stages are free.  Each wave re-lays its accumulators out
// through its own LDS region one 32-row slab at a time: the MFMA layout (lane = column,
// registers = rows) is written as a row-major fp32 slab and read back as runs of 8
// consecutive columns, so every global access of the epilogue is one 16-byte buffer
// load or store (8 bf16), and rows / columns outside the matrix are masked by the buffer
// range check instead of per-element branches.
#pragma once

#include "device_common.hpp"

namespace coda {

// Buffer descriptor (the builtin type, for buffer load/store builtins) of
// [base, base + bytes); fields forced wave-uniform so it lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buffer_rsrc(const void* base,
                                                                   uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, static_cast<int>(n), 0x00020000);
}

constexpr uint32_t kOobOffset = 0x80000000u;   // beyond every epilogue descriptor range

// A 32 x (NB*32) fp32 slab in LDS, row stride NB*128 + 32 bytes (the pad puts the two
// half-waves' rows of a write on different bank halves).
template <int NB>
struct Slab {
    static constexpr int kStride = NB * 128 + 32;
    static constexpr int kBytes = 32 * kStride;
    static constexpr int kSegPerRow = NB * 4;            // 8-column segments per row
    static constexpr int kSegPerLane = 32 * kSegPerRow / 64;

    // Write NB 32x32 blocks (MFMA layout: lane l, register i -> row 8*(i/4) + 4*(l/32) +
    // i%4, column 32*b + l%32) as a row-major slab.
    __device__ __forceinline__ static void put(uint8_t* buf, const float (&v)[NB][16]) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 8 * (i >> 2) + 4 * lh + (i & 3);
                *reinterpret_cast<float*>(buf + r * kStride + (32 * b + lr) * 4) = v[b][i];
            }
    }
    // Segment j of this lane: row and first column of its 8 consecutive columns.
    __device__ __forceinline__ static int seg_row(int j) { return ((threadIdx.x & 63) + 64 * j) / kSegPerRow; }
    __device__ __forceinline__ static int seg_col(int j) { return (((threadIdx.x & 63) + 64 * j) % kSegPerRow) * 8; }
    __device__ __forceinline__ static void get(const uint8_t* buf, int j, float (&out)[8]) {
        const f32x4_t* p = reinterpret_cast<const f32x4_t*>(buf + seg_row(j) * kStride + seg_col(j) * 4);
        const f32x4_t a = p[0], b = p[1];
        out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
        out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
    }
};

// All-reduce over aligned groups of W = 8 or 16 lanes (lanes W*k .. W*k + W-1, inside
// one 16-lane DPP row) with VALU data-parallel moves instead of LDS permutes: quad
// permutes pair lanes 1 and 2 apart, the 8-lane mirror pairs the two 4-lane halves of an
// 8-group, the 16-lane mirror the two 8-lane halves of a row.  Every lane of the group
// ends with the reduction of its W lanes.
__device__ __forceinline__ float dpp_quad_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                                 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                                 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_half_mirror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                                 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_mirror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                                 0x140, 0xF, 0xF, false));
}
template <int W, class Op>
__device__ __forceinline__ float group_allreduce(float x, Op op) {
    static_assert(W == 8 || W == 16, "groups of 8 or 16 lanes");
    x = op(x, dpp_quad_xor1(x));
    x = op(x, dpp_quad_xor2(x));
    x = op(x, dpp_half_mirror(x));
    if constexpr (W == 16) x = op(x, dpp_row_mirror(x));
    return x;
}
struct AddOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};


}  // namespace coda

// Device-side helpers shared by the chain's kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace coda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16 ----------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}

// Two round-to-nearest-even conversions in one v_cvt_pk_bf16_f32 (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}

// ------------------------------------------------------------ accumulators ------
// One accumulator element read out of its AGPR right here (v_accvgpr_read_b32).  Plain
// reads let the compiler copy all 256 accumulators of a finished tile into VGPRs in one
// block after the mainloop, which in a persistent kernel spills, and the spill reloads'
// full vmcnt waits then also wait for the next tile's DMA.  The MFMA that wrote the
// element must be done: callers run acc_read_fence() once between the last MFMA and the
// first read (the read is inline asm, so the compiler inserts no wait states for it).
__device__ __forceinline__ float acc_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}
// 32 wait states: more than the 32x32 MFMA's result latency requires
__device__ __forceinline__ void acc_read_fence() {
    __builtin_amdgcn_sched_barrier(0);       // no MFMA is moved below the wait states
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
}

// ------------------------------------------------------------------ e4m3 ----------
// OCP E4M3FN: bias 7, 3 mantissa bits, max 448, no infinities, NaN = S.1111.111.

// Saturating round-to-nearest-even of an fp32 value (bit manipulation on the fp32
// encoding; subnormal range via an exact scaling by 2^9 and rint).
__device__ __forceinline__ uint8_t f32_to_e4m3_sat(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7F;                       // NaN
    if (a >= 0x43E00000u) return static_cast<uint8_t>(sign | 0x7Eu);   // >= 448: saturate
    if (a >= 0x3C800000u) {                                 // >= 2^-6: normal range
        uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // keep 3 mantissa bits, RNE
        return static_cast<uint8_t>(sign | (r - (120u << 3)));  // rebias 127 -> 7
    }
    float s = __uint_as_float(a) * 512.0f;                  // subnormal units of 2^-9, exact
    uint32_t q = static_cast<uint32_t>(rintf(s));           // 0..8 (8 = min normal 0x08)
    return static_cast<uint8_t>(sign | q);
}

// Exact e4m3 -> bf16 bits (every finite e4m3 value is a bf16 value).
__device__ __forceinline__ uint16_t e4m3_to_bf16_bits(uint32_t c) {
    uint32_t s = (c & 0x80u) << 8;
    uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    if (e == 0xFu && m == 7u) return static_cast<uint16_t>(s | 0x7FC0u);
    if (e != 0) return static_cast<uint16_t>(s | ((e + 120u) << 7) | (m << 4));
    float v = static_cast<float>(m) * (1.0f / 512.0f);      // subnormal, exact
    return static_cast<uint16_t>(s | (__float_as_uint(v) >> 16));
}

// ------------------------------------------------------------ tile mapping --------
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on XCD i % 8,
// each XCD with its own L2).  Give every XCD one contiguous range of the linear tile
// order, then walk that order in groups of `G` tile-rows so that the tiles resident at
// the same time on one XCD share A row-panels and B column-panels in its L2.
// (G a runtime value: tile_coords_g, for a kernel that picks the group by its shape.)
template <class GT>
__device__ __forceinline__ void tile_coords_impl(int pid, int tiles_m, int tiles_n, GT gt, int& tm, int& tn) {
    const int G = gt;
    const int total = tiles_m * tiles_n;
    const int xcd = pid & 7, local = pid >> 3;
    const int q = total >> 3, rem = total & 7;
    const int lin = (xcd < rem) ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
    const int group = lin / (G * tiles_n);
    const int first_m = group * G;
    const int gsize = min(tiles_m - first_m, G);
    const int in = lin - group * G * tiles_n;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

template <int G>
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
    tile_coords_impl(pid, tiles_m, tiles_n, std::integral_constant<int, G>{}, tm, tn);
}

__device__ __forceinline__ void tile_coords_g(int pid, int tiles_m, int tiles_n, int G, int& tm, int& tn) {
    tile_coords_impl(pid, tiles_m, tiles_n, G, tm, tn);
}

}  // namespace coda

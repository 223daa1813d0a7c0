// Weight preparation (once per weight update, not part of the chain's timed path).
//
// gamma fold: RMSNorm's weight gamma scales the reduction dimension k of the second
// GEMM, so it is a diagonal that moves into the second weight (kucoin page, section
// "Cinco bloques y un lenguaje LEGO": RMSNorm weights are a broadcast vector operand;
// the row scale r is what stays per token):  Wp[n,k] = bf16_rne(fl32(gamma[k] W[n,k])).
//
// e4m3 quantisation with a per-tensor fp32 scale (the 8-bit variant):
//   amax = max |x|,  s = fl32(amax/448) (1 if amax == 0),  q = e4m3_sat_rne(fl32(x/s)),
// with x = fl32(gamma[k] X[n,k]) for the second weight (fold BEFORE quantising) and
// x = X for the activations and the first weight.  The max is order-independent, so
// an atomic max over non-negative fp32 bit patterns is deterministic.
#include "device_common.hpp"
#include "launch.hpp"

namespace coda {

// 8 elements (one 16-byte bf16 vector) per thread and grid-stride step.
__global__ void __launch_bounds__(256)
k_fold_bf16(const i32x4_t* __restrict__ W, const float* __restrict__ gamma,
            i32x4_t* __restrict__ Wp, int64_t n_vec, int64_t k_vec) {
    for (int64_t v = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; v < n_vec;
         v += int64_t(gridDim.x) * blockDim.x) {
        const int64_t k0 = (v % k_vec) * 8;
        const i32x4_t x = W[v];
        i32x4_t o;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t u = static_cast<uint32_t>(x[h]);
            const float g0 = gamma ? gamma[k0 + 2 * h] : 1.0f;
            const float g1 = gamma ? gamma[k0 + 2 * h + 1] : 1.0f;
            const float p0 = g0 * bf16_bits_to_f32(static_cast<uint16_t>(u & 0xFFFFu));
            const float p1 = g1 * bf16_bits_to_f32(static_cast<uint16_t>(u >> 16));
            o[h] = static_cast<int>(pack_bf16x2(p0, p1));
        }
        Wp[v] = o;
    }
}

__global__ void k_clear_amax(float* amax_scale) {
    if (threadIdx.x == 0) amax_scale[0] = 0.0f;
}

__device__ __forceinline__ float folded(uint16_t b, const float* gamma, int64_t k) {
    const float x = bf16_bits_to_f32(b);
    return gamma ? gamma[k] * x : x;
}

__global__ void __launch_bounds__(256)
k_amax(const i32x4_t* __restrict__ X, const float* __restrict__ gamma, float* amax_scale,
       int64_t n_vec, int64_t k_vec) {
    float m = 0.0f;
    for (int64_t v = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; v < n_vec;
         v += int64_t(gridDim.x) * blockDim.x) {
        const int64_t k0 = (v % k_vec) * 8;
        const i32x4_t x = X[v];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t u = static_cast<uint32_t>(x[h]);
            m = fmaxf(m, fabsf(folded(static_cast<uint16_t>(u & 0xFFFFu), gamma, k0 + 2 * h)));
            m = fmaxf(m, fabsf(folded(static_cast<uint16_t>(u >> 16), gamma, k0 + 2 * h + 1)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float wmax[4];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float b = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        // non-negative fp32 values order like their bit patterns
        atomicMax(reinterpret_cast<unsigned int*>(amax_scale), __float_as_uint(b));
    }
}

// 16 elements (two bf16 vectors in, one 16-byte e4m3 vector out) per step.
__global__ void __launch_bounds__(256)
k_quant(const i32x4_t* __restrict__ X, const float* __restrict__ gamma, float* amax_scale,
        i32x4_t* __restrict__ Q, int64_t n_out_vec, int64_t k_out_vec) {
    const float amax = amax_scale[0];
    const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) amax_scale[1] = s;
    for (int64_t v = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; v < n_out_vec;
         v += int64_t(gridDim.x) * blockDim.x) {
        const int64_t k0 = (v % k_out_vec) * 16;
        uint32_t out[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const i32x4_t x = X[2 * v + half];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t u = static_cast<uint32_t>(x[h]);
                const int64_t k = k0 + half * 8 + 2 * h;
                const uint32_t q0 = f32_to_e4m3_sat(folded(static_cast<uint16_t>(u & 0xFFFFu), gamma, k) / s);
                const uint32_t q1 = f32_to_e4m3_sat(folded(static_cast<uint16_t>(u >> 16), gamma, k + 1) / s);
                const int idx = half * 8 + 2 * h;          // byte index in the 16-byte vector
                if ((idx & 3) == 0) out[idx >> 2] = 0;
                out[idx >> 2] |= (q0 | (q1 << 8)) << (8 * (idx & 3));
            }
        }
        Q[v] = i32x4_t{int(out[0]), int(out[1]), int(out[2]), int(out[3])};
    }
}

static unsigned grid_for(int64_t n_vec) {
    const int64_t blocks = (n_vec + 255) / 256;
    return static_cast<unsigned>(blocks < 8192 ? (blocks < 1 ? 1 : blocks) : 8192);
}

// RoPE angle table: cos / sin of p * base^(-2i/64) for p < rows, i < 32, in fp64, one
// rounding to fp32.  One thread per (p, i).
__global__ void __launch_bounds__(256)
k_rope_table(int rows, double base, float* __restrict__ cos_t, float* __restrict__ sin_t) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<int64_t>(rows) * 32) return;
    const int p = static_cast<int>(idx >> 5), i = static_cast<int>(idx & 31);
    const double theta = pow(base, -2.0 * static_cast<double>(i) / 64.0);
    const double ang = static_cast<double>(p) * theta;
    cos_t[idx] = static_cast<float>(cos(ang));
    sin_t[idx] = static_cast<float>(sin(ang));
}

hipError_t launch_rope_table(int rows, double base, float* cos_t, float* sin_t, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(rows) * 32;
    hipLaunchKernelGGL(k_rope_table, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, rows,
                       base, cos_t, sin_t);
    return hipGetLastError();
}

// dst[c, r] = src[r, c] for a bf16 [R, C] matrix, through a 64x64 LDS tile (padded
// rows against bank conflicts); 256 threads, each moves 16 elements.
__global__ void __launch_bounds__(256)
k_transpose_bf16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t R, int64_t C,
                 int64_t tiles_c) {
    __shared__ uint16_t t[64][66];
    const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
    const int64_t r0 = tr * 64, c0 = tc * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = r0 + ty + 4 * i, c = c0 + tx;
        t[ty + 4 * i][tx] = (r < R && c < C) ? src[r * C + c] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t c = c0 + ty + 4 * i, r = r0 + tx;
        if (c < C && r < R) dst[c * R + r] = t[tx][ty + 4 * i];
    }
}

// The same for R % 8 == 0 and C % 8 == 0 (16-byte rows on both sides): a 128 x 64 tile,
// 16-byte loads of 8 columns of a source row, 16-byte stores of 8 rows of a destination
// row (the destination row's 128 tile rows = 256 contiguous bytes per tile).  LDS rows
// padded to 72 elements (16-byte aligned); the transposed reads of a wave take one
// element from each of 64 consecutive columns of a row: conflict-free.
constexpr int kTrR = 128, kTrC = 64, kTrPad = 72;
__global__ void __launch_bounds__(256)
k_transpose16_bf16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t R, int64_t C,
                   int64_t tiles_c) {
    __shared__ __attribute__((aligned(16))) uint16_t t[kTrR][kTrPad];
    const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
    const int64_t r0 = tr * kTrR, c0 = tc * kTrC;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kTrR * kTrC / 8 / 256; ++i) {
        const int idx = tid + 256 * i;
        const int rr = idx >> 3, ch = idx & 7;       // tile row, 8-column chunk
        const int64_t r = r0 + rr, c = c0 + 8 * ch;
        i32x4_t v = {0, 0, 0, 0};
        if (r < R && c < C) v = *reinterpret_cast<const i32x4_t*>(src + r * C + c);
        *reinterpret_cast<i32x4_t*>(&t[rr][8 * ch]) = v;
    }
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t c = c0 + lane;
#pragma unroll
    for (int i = 0; i < kTrR / 8 / 4; ++i) {
        const int rc = wave + 4 * i;                 // 8-row chunk of the tile
        const int64_t r = r0 + 8 * rc;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = static_cast<uint32_t>(t[8 * rc + 2 * e][lane]) |
                   (static_cast<uint32_t>(t[8 * rc + 2 * e + 1][lane]) << 16);
        if (c < C && r < R)
            *reinterpret_cast<i32x4_t*>(dst + c * R + r) = i32x4_t{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
    }
}

hipError_t launch_transpose_bf16(int64_t R, int64_t C, const void* src, void* dst, hipStream_t stream) {
    if (R % 8 == 0 && C % 8 == 0) {
        const int64_t tiles_r = (R + kTrR - 1) / kTrR, tiles_c = (C + kTrC - 1) / kTrC;
        hipLaunchKernelGGL(k_transpose16_bf16, dim3(static_cast<unsigned>(tiles_r * tiles_c)), dim3(256), 0,
                           stream, static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), R, C, tiles_c);
        return hipGetLastError();
    }
    const int64_t tiles_r = (R + 63) / 64, tiles_c = (C + 63) / 64;
    hipLaunchKernelGGL(k_transpose_bf16, dim3(static_cast<unsigned>(tiles_r * tiles_c)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), R, C, tiles_c);
    return hipGetLastError();
}

hipError_t launch_fold_bf16(int64_t N, int64_t K, const void* W, const float* gamma, void* Wp,
                            hipStream_t stream) {
    const int64_t k_vec = K / 8, n_vec = N * k_vec;
    hipLaunchKernelGGL(k_fold_bf16, dim3(grid_for(n_vec)), dim3(256), 0, stream,
                       static_cast<const i32x4_t*>(W), gamma, static_cast<i32x4_t*>(Wp), n_vec, k_vec);
    return hipGetLastError();
}

hipError_t launch_quantize_e4m3(int64_t N, int64_t K, const void* X, const float* gamma,
                                void* Q, float* amax_scale, hipStream_t stream) {
    const int64_t k_vec = K / 8, n_vec = N * k_vec;
    hipLaunchKernelGGL(k_clear_amax, dim3(1), dim3(64), 0, stream, amax_scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_amax, dim3(grid_for(n_vec)), dim3(256), 0, stream,
                       static_cast<const i32x4_t*>(X), gamma, amax_scale, n_vec, k_vec);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t k_out = K / 16, n_out = N * k_out;
    hipLaunchKernelGGL(k_quant, dim3(grid_for(n_out)), dim3(256), 0, stream,
                       static_cast<const i32x4_t*>(X), gamma, amax_scale, static_cast<i32x4_t*>(Q),
                       n_out, k_out);
    return hipGetLastError();
}

}  // namespace coda

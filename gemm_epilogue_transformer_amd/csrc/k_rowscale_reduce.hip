// The light reduction between the two GEMMs: the per-tile partial sums of squares of
// each row are combined into the RMSNorm row scale
//   r[m] = fl32( 1 / sqrt( (sum_t P[m,t]) / N + eps ) )
// (kucoin page, section "CODA: El epilogo esconde un tesoro": the partial root mean
// square of the first GEMM's end is merged by an extremely light reduction kernel).
// The sum runs in a fixed order in fp64, the sqrt and divide in fp64, one final
// rounding to fp32: cheap, since this kernel moves only M*(T+1) floats.
#include "device_common.hpp"
#include "launch.hpp"

namespace coda {

// One thread per row.  The partials are loaded eight at a time before they are added (a
// load per add would put T memory latencies in series); the additions keep the order
// t = 0, 1, ..., T-1.  64-thread blocks spread the rows over every CU.
__global__ void __launch_bounds__(64)
k_rowscale_reduce(const float* __restrict__ P, float* __restrict__ r, int M, int T,
                  double n, double eps) {
    const int m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    const float* p = P + static_cast<size_t>(m) * T;
    double s = 0.0;
    int t = 0;
    for (; t + 8 <= T; t += 8) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = p[t + e];
#pragma unroll
        for (int e = 0; e < 8; ++e) s += static_cast<double>(v[e]);
    }
    for (; t < T; ++t) s += static_cast<double>(p[t]);
    r[m] = static_cast<float>(1.0 / sqrt(s / n + eps));
}

hipError_t launch_rowscale_reduce(int M, int N, int T, const float* P, float eps, float* r,
                                  hipStream_t stream) {
    const dim3 block(64), grid((M + 63) / 64);
    hipLaunchKernelGGL(k_rowscale_reduce, grid, block, 0, stream, P, r, M, T, static_cast<double>(N),
                       static_cast<double>(eps));
    return hipGetLastError();
}

// The row scale of a stored h (the backward may recompute it instead of saving it):
//   r[m] = fl32( 1 / sqrt( sum_n h[m,n]^2 / N + eps ) )
// one wave per row, 16-byte loads, the squares (exact in fp32 for bf16 h) summed in fp64
// in a fixed order (lane-strided, then a fixed butterfly).
__global__ void __launch_bounds__(256)
k_rowscale_from_h(const uint16_t* __restrict__ h, float* __restrict__ r, int M, int N, double eps) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;                       // wave-uniform
    const i32x4_t* p = reinterpret_cast<const i32x4_t*>(h + static_cast<size_t>(row) * N);
    double s = 0.0;
    for (int v = lane; v < N / 8; v += 64) {
        const i32x4_t q = p[v];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t x = static_cast<uint32_t>(q[e]);
            const float a = bf16_bits_to_f32(static_cast<uint16_t>(x & 0xFFFFu));
            const float b = bf16_bits_to_f32(static_cast<uint16_t>(x >> 16));
            s += static_cast<double>(a * a) + static_cast<double>(b * b);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) r[row] = static_cast<float>(1.0 / sqrt(s / static_cast<double>(N) + eps));
}

hipError_t launch_rowscale_from_h(int M, int N, const void* h, float eps, float* r, hipStream_t stream) {
    const dim3 block(256), grid((M + 3) / 4);
    hipLaunchKernelGGL(k_rowscale_from_h, grid, block, 0, stream, static_cast<const uint16_t*>(h), r, M, N,
                       static_cast<double>(eps));
    return hipGetLastError();
}

// Backward of the row scale: q[m] = fl32( -(r[m]^3 / N) * sum_t P[m,t] ), the partials
// being sum_j dL/dz_j * acc_j = dL/dr over the tiles of the recomputed product (fixed
// order, fp64).  With it the input gradient is dh = r * (dz . W') + q * h: the second
// term is the RMSNorm backward through r = (mean(h^2) + eps)^(-1/2), dr/dh = -r^3 h / N.
__global__ void __launch_bounds__(256)
k_rmsnorm_bwd_reduce(const float* __restrict__ P, const float* __restrict__ r, float* __restrict__ q, int M,
                     int T, double n) {
    // one wave per row: lane l adds t = l, l + 64, ... in fp64 (coalesced 256-byte rows of
    // partials), then an xor butterfly over the 64 lanes in a fixed pattern (addition
    // commutes, so every lane ends with the same bits)
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= M) return;                                  // whole waves
    const float* p = P + static_cast<size_t>(m) * T;
    double s = 0.0;
    for (int t = lane; t < T; t += 64) s += static_cast<double>(p[t]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) {
        const double rr = static_cast<double>(r[m]);
        q[m] = static_cast<float>(-(rr * rr * rr / n) * s);
    }
}

hipError_t launch_rmsnorm_bwd_reduce(int M, int N, int T, const float* P, const float* r, float* q,
                                     hipStream_t stream) {
    const dim3 block(256), grid((M + 3) / 4);
    hipLaunchKernelGGL(k_rmsnorm_bwd_reduce, grid, block, 0, stream, P, r, q, M, T, static_cast<double>(N));
    return hipGetLastError();
}

}  // namespace coda

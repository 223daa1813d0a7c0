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

__global__ void __launch_bounds__(256)
k_rowscale_reduce(const float* __restrict__ P, float* __restrict__ r, int M, int T,
                  double n, double eps) {
    const int m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    const float* p = P + static_cast<size_t>(m) * T;
    double s = 0.0;
    for (int t = 0; t < T; ++t) s += static_cast<double>(p[t]);
    r[m] = static_cast<float>(1.0 / sqrt(s / n + eps));
}

hipError_t launch_rowscale_reduce(int M, int N, int T, const float* P, float eps, float* r,
                                  hipStream_t stream) {
    const dim3 block(256), grid((M + 255) / 256);
    hipLaunchKernelGGL(k_rowscale_reduce, grid, block, 0, stream, P, r, M, T, static_cast<double>(N),
                       static_cast<double>(eps));
    return hipGetLastError();
}

}  // namespace coda

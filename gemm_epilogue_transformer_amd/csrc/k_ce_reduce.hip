// The light reduction after the LM-head GEMM: each row's per-tile (max, sum-exp) pairs
// are merged into the log-sum-exp and the loss
//   lse[m]  = fl32( M + log( sum_t s_t * exp(m_t - M) ) ),  M = max_t m_t
//   loss[m] = fl32( lse - z[m, target] )   for a target in [0, V), else 0
// (kucoin page, section "Cinco bloques y un lenguaje LEGO": the max / sum-exp state of
// online normalisation, merged outside the GEMM like the partial RMS).  One wave per
// row: lane l folds the tiles l, l+64, ... in order (online max / rescale in fp64),
// then a fixed butterfly merges the 64 lane states; deterministic.
#include "device_common.hpp"
#include "launch.hpp"

namespace coda {

__device__ __forceinline__ void lse_merge(double& m, double& s, double m2, double s2) {
    // (m, s) represents s * exp(m); an empty state has m = -inf, s = 0
    if (m2 == -__builtin_inf()) return;
    if (m == -__builtin_inf()) { m = m2; s = s2; return; }
    if (m2 > m) { s = s * exp(m - m2) + s2; m = m2; }
    else { s += s2 * exp(m2 - m); }
}

__global__ void __launch_bounds__(256)
k_ce_reduce(const float* __restrict__ P, const int32_t* __restrict__ targets,
            const float* __restrict__ tgt_logit, float* __restrict__ lse, float* __restrict__ loss,
            int M, int T, int V) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;                       // wave-uniform
    const float* p = P + static_cast<size_t>(row) * T * 2;
    double m = -__builtin_inf(), s = 0.0;
    for (int t = lane; t < T; t += 64) {
        const float mt = p[2 * t], st = p[2 * t + 1];
        if (mt > -__builtin_inff()) lse_merge(m, s, static_cast<double>(mt), static_cast<double>(st));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
        lse_merge(m, s, m2, s2);
    }
    if (lane == 0) {
        const double l = m + log(s);
        const int tg = targets[row];
        lse[row] = static_cast<float>(l);
        loss[row] = (tg >= 0 && tg < V) ? static_cast<float>(l - static_cast<double>(tgt_logit[row])) : 0.0f;
    }
}

hipError_t launch_ce_reduce(int M, int V, int T, const float* partials, const int32_t* targets,
                            const float* tgt_logit, float* lse, float* loss, hipStream_t stream) {
    const dim3 block(256), grid((M + 3) / 4);
    hipLaunchKernelGGL(k_ce_reduce, grid, block, 0, stream, partials, targets, tgt_logit, lse, loss, M, T, V);
    return hipGetLastError();
}

}  // namespace coda

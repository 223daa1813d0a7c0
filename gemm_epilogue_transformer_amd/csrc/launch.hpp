// Host-side launchers of the chain's kernels (internal to the library).  Arguments are
// validated by the C ABI layer before any of these is called; each launcher only
// configures the grid and enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coda {

int64_t partials_per_row(int64_t N);

// Number of workgroups (tiles) each GEMM launches; the ABI checks them against the grid
// limit before launching.
int64_t gemm1_tiles(int64_t M, int64_t N);
int64_t gemm3_tiles(int64_t M, int64_t N_out, bool swiglu);

hipError_t launch_gemm_resid_partialrms(int M, int N, int K, const void* A, bool fp8,
                                        const float* a_scale, const void* W,
                                        const float* w_scale, const void* x_res, void* h,
                                        float* P, hipStream_t stream);

hipError_t launch_rowscale_reduce(int M, int N, int T, const float* P, float eps, float* r,
                                  hipStream_t stream);

hipError_t launch_gemm_rowscale_swiglu(int M, int N_out, int K, bool swiglu, const void* h,
                                       const void* W, bool w_fp8, const float* w_scale,
                                       const float* r, void* y, hipStream_t stream);

// Row scale + RoPE epilogue (no activation); pos / cos / sin may be NULL when
// rot_cols == 0.
hipError_t launch_gemm_rowscale_rope(int M, int N_out, int K, const void* h, const void* W,
                                     bool w_fp8, const float* w_scale, const float* r,
                                     const int32_t* pos, const float* cos, const float* sin,
                                     int table_rows, int rot_cols, void* y, hipStream_t stream);

hipError_t launch_rope_table(int rows, double base, float* cos, float* sin, hipStream_t stream);

// Cross-entropy: LM-head GEMM with the block log-sum-exp epilogue, then the reduction.
int64_t ce_partials_per_row(int64_t V);
hipError_t launch_gemm_rowscale_ce(int M, int V, int K, const void* h, const void* W, bool w_fp8,
                                   const float* w_scale, const float* r, const int32_t* targets,
                                   float* partials, float* tgt_logit, hipStream_t stream);
hipError_t launch_ce_reduce(int M, int V, int T, const float* partials, const int32_t* targets,
                            const float* tgt_logit, float* lse, float* loss, hipStream_t stream);

// Backward of the MLP-input block (input gradient): recompute + SwiGLU-backward epilogue,
// the row coefficient reduction, the input-gradient GEMM with the RMSNorm-backward
// epilogue, and the weight transpose it reads.
int64_t swiglu_bwd_partials_per_row(int64_t F);
hipError_t launch_gemm_swiglu_bwd(int M, int F, int K, const void* h, const void* W, const float* r,
                                  const void* dy, void* dz, float* partials, hipStream_t stream);
hipError_t launch_rowscale_from_h(int M, int N, const void* h, float eps, float* r, hipStream_t stream);
hipError_t launch_rmsnorm_bwd_reduce(int M, int N, int T, const float* partials, const float* r, float* q,
                                     hipStream_t stream);
int64_t gemm_bwd2_tiles(int64_t M, int64_t N);
hipError_t launch_gemm_rmsnorm_bwd(int M, int N, int K, const void* dz, const void* Wt, const void* h,
                                   const float* q, const void* dh_res, void* dh, hipStream_t stream);
hipError_t launch_transpose_bf16(int64_t R, int64_t C, const void* src, void* dst, hipStream_t stream);

// The second GEMM reading the raw weight and folding gamma in while staging it.
hipError_t launch_gemm_rowscale_gfold(int M, int N_out, int K, bool swiglu, const void* h, const void* W_raw,
                                      const float* gamma, const float* r, void* y, hipStream_t stream);

// SwiGLU forward that keeps the pre-activation, and the backward that starts from it.
hipError_t launch_gemm_rowscale_swiglu_save(int M, int F, int K, const void* h, const void* W, const float* r,
                                            void* y, void* z, hipStream_t stream);
hipError_t launch_gemm_ce_bwd(int M, int V, int K, const void* h, const void* W, const float* r,
                              const int32_t* targets, const float* lse, const float* gw, void* dz, float* partials,
                              hipStream_t stream);
hipError_t launch_rope_bwd(int M, int N, const void* dy, const void* y, const float* r, const int32_t* pos,
                           const float* cos, const float* sin, int table_rows, int rot_cols, void* dz,
                           float* partials, hipStream_t stream);
hipError_t launch_swiglu_bwd_saved(int M, int F, const void* z, const void* dy, const float* r, void* dz,
                                   void* dzt, float* partials, hipStream_t stream);

// Weight gradients: token-contracting GEMM with the gamma column scale and the column
// partials of the gamma gradient, and their fixed-order column sum.
int64_t wgrad_tiles(int64_t NR, int64_t NC);
int64_t wgrad_partials_rows(int64_t NR);
int64_t wgrad_workspace_bytes(int64_t NR, int64_t NC, int64_t K);
struct WgradPlan {
    int S;          // token splits
    int k_split;    // tokens per split
};
WgradPlan wgrad_plan(int64_t NR, int64_t NC, int64_t K);
hipError_t launch_gemm_wgrad(int NR, int NC, int K, const void* At, const void* Bt, const float* gamma,
                             const void* Wraw, float* dW, float* Pg, float* ws, int64_t ws_bytes,
                             hipStream_t stream);
hipError_t launch_gemm_wgrad_tok(int NR, int NC, int K, const void* X, int lda, const void* Y, int ldb,
                                 const float* gamma, const void* Wraw, float* dW, float* Pg, float* ws,
                                 int64_t ws_bytes, hipStream_t stream);
// The same, with the token split's slices in the library's static per-device scratch
// (kNoAllocScratchBytes) instead of a caller workspace: nothing is allocated.  The
// caller has checked wgrad_workspace_bytes(NR, NC, K) <= kNoAllocScratchBytes.
constexpr int64_t kNoAllocScratchBytes = int64_t(128) << 20;
hipError_t launch_gemm_wgrad_tok_noalloc(int NR, int NC, int K, const void* X, int lda, const void* Y, int ldb,
                                         const float* gamma, const void* Wraw, float* dW, float* Pg,
                                         hipStream_t stream);
hipError_t launch_colsum_reduce(int T, int NC, const float* Pg, float* out, hipStream_t stream);
hipError_t launch_fill_zero_f32(int64_t n, float* dst, hipStream_t stream);

hipError_t launch_fold_bf16(int64_t N, int64_t K, const void* W, const float* gamma, void* Wp,
                            hipStream_t stream);

hipError_t launch_quantize_e4m3(int64_t N, int64_t K, const void* X, const float* gamma,
                                void* Q, float* amax_scale, hipStream_t stream);

}  // namespace coda

// C ABI of the chain (declared in include/coda.h): host-side validation, then one
// launcher per call.  Nothing here allocates device memory or synchronises; every
// check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include <algorithm>

#include "../../include/coda.h"
#include "launch.hpp"

namespace {

static_assert(CODA_NOALLOC_SCRATCH_BYTES == coda::kNoAllocScratchBytes, "the header states the scratch size");

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = INT32_MAX;
// The kernels address one block tile (up to 256 rows) of any operand through a 32-bit
// buffer offset range below 2^31, so row lengths are capped at 2^22 elements.
constexpr int64_t kMaxRow = int64_t(1) << 22;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) {
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int64_t v, int64_t lo) { return v >= lo && v <= kMaxDim; }

bool prod_ok(int64_t a, int64_t b) {  // a*b elements addressable and below 2^62
    return a == 0 || b <= (int64_t(1) << 62) / a;
}

coda_status hip_status(hipError_t e) {
    if (e == hipSuccess) return CODA_OK;
    g_last_hip_error = static_cast<int>(e);
    return CODA_ERR_HIP;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* coda_version(void) { return "coda-mi355x 0.1 (gfx950)"; }

const char* coda_status_string(coda_status s) {
    switch (s) {
        case CODA_OK: return "ok";
        case CODA_ERR_NULL: return "a required pointer is NULL";
        case CODA_ERR_SHAPE: return "invalid shape (sign, zero, size limit or granule)";
        case CODA_ERR_DTYPE: return "unsupported dtype or activation";
        case CODA_ERR_VALUE: return "invalid value (eps must be finite and >= 0)";
        case CODA_ERR_ALIAS: return "an output overlaps an input or another output";
        case CODA_ERR_HIP: return "HIP launch failed (see coda_last_hip_error)";
        case CODA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    }
    return "unknown status";
}

int coda_last_hip_error(void) { return g_last_hip_error; }

int64_t coda_partials_per_row(int64_t N) { return coda::partials_per_row(N); }

coda_status coda_prepare_weight_bf16(int64_t N, int64_t K, const void* W, const float* gamma,
                                     void* Wp, void* stream) {
    if (!W || !Wp) return CODA_ERR_NULL;
    if (!dim_ok(N, 1) || !dim_ok(K, 1) || K % 8 != 0 || !prod_ok(N, K)) return CODA_ERR_SHAPE;
    if (!aligned16(W) || !aligned16(Wp) || (gamma && !aligned16(gamma))) return CODA_ERR_ALIGN;
    const Range out = span(Wp, N * K * 2);
    if (overlap(out, span(W, N * K * 2)) || (gamma && overlap(out, span(gamma, K * 4))))
        return CODA_ERR_ALIAS;
    return hip_status(coda::launch_fold_bf16(N, K, W, gamma, Wp, as_stream(stream)));
}

coda_status coda_quantize_e4m3(int64_t N, int64_t K, const void* X, const float* gamma, void* Q,
                               float* amax_scale, void* stream) {
    if (!X || !Q || !amax_scale) return CODA_ERR_NULL;
    if (!dim_ok(N, 1) || !dim_ok(K, 1) || K % 16 != 0 || !prod_ok(N, K)) return CODA_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(Q) || (gamma && !aligned16(gamma)) || !aligned16(amax_scale))
        return CODA_ERR_ALIGN;
    const Range q = span(Q, N * K), sc = span(amax_scale, 8);
    const Range x = span(X, N * K * 2);
    if (overlap(q, x) || overlap(sc, x) || overlap(q, sc)) return CODA_ERR_ALIAS;
    if (gamma) {
        const Range g = span(gamma, K * 4);
        if (overlap(q, g) || overlap(sc, g)) return CODA_ERR_ALIAS;
    }
    return hip_status(coda::launch_quantize_e4m3(N, K, X, gamma, Q, amax_scale, as_stream(stream)));
}

coda_status coda_gemm_resid_partialrms(int64_t M, int64_t N, int64_t K, const void* A,
                                       coda_dtype ab_dtype, const float* a_scale, const void* W,
                                       const float* w_scale, const void* x_res, void* h,
                                       float* partials, void* stream) {
    if (ab_dtype != CODA_BF16 && ab_dtype != CODA_E4M3) return CODA_ERR_DTYPE;
    const bool fp8 = ab_dtype == CODA_E4M3;
    if (!dim_ok(M, 0) || !dim_ok(N, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (N % 8 != 0 || K % (fp8 ? 16 : 8) != 0 || N > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    if (!prod_ok(M, K) || !prod_ok(N, K) || !prod_ok(M, N)) return CODA_ERR_SHAPE;
    const int64_t T = coda::partials_per_row(N);
    if (coda::gemm1_tiles(M, N) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;  // empty problem: nothing to enqueue, empty tensors may be NULL
    if (!A || !W || !h || !partials) return CODA_ERR_NULL;
    if (fp8 && (!a_scale || !w_scale)) return CODA_ERR_NULL;
    if (!aligned16(A) || !aligned16(W) || !aligned16(h) || !aligned16(partials) ||
        (x_res && !aligned16(x_res)))
        return CODA_ERR_ALIGN;
    const int64_t eb = fp8 ? 1 : 2;
    const Range rh = span(h, M * N * 2), rp = span(partials, M * T * 4);
    const Range ra = span(A, M * K * eb), rw = span(W, N * K * eb);
    if (overlap(rh, rp) || overlap(rh, ra) || overlap(rh, rw) || overlap(rp, ra) || overlap(rp, rw))
        return CODA_ERR_ALIAS;
    if (x_res) {
        const Range rx = span(x_res, M * N * 2);
        if (overlap(rp, rx) || (x_res != h && overlap(rh, rx))) return CODA_ERR_ALIAS;
    }
    for (const float* s : {a_scale, w_scale})
        if (s && (overlap(rh, span(s, 4)) || overlap(rp, span(s, 4)))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_resid_partialrms(int(M), int(N), int(K), A, fp8, a_scale, W,
                                                         w_scale, x_res, h, partials,
                                                         as_stream(stream)));
}

coda_status coda_rowscale_reduce(int64_t M, int64_t N, const float* partials, float eps, float* r,
                                 void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(N, 1)) return CODA_ERR_SHAPE;
    const int64_t T = coda::partials_per_row(N);
    if (!prod_ok(M, T)) return CODA_ERR_SHAPE;
    if (!std::isfinite(eps) || eps < 0.0f) return CODA_ERR_VALUE;
    if (M == 0) return CODA_OK;
    if (!partials || !r) return CODA_ERR_NULL;
    if (!aligned16(partials) || !aligned16(r)) return CODA_ERR_ALIGN;
    if (overlap(span(partials, M * T * 4), span(r, M * 4))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_rowscale_reduce(int(M), int(N), int(T), partials, eps, r,
                                                   as_stream(stream)));
}

coda_status coda_gemm_rowscale_swiglu(int64_t M, int64_t N_out, int64_t K, coda_act act,
                                      const void* h, const void* W, coda_dtype w_dtype,
                                      const float* w_scale, const float* r, void* y,
                                      void* stream) {
    if (act != CODA_ACT_NONE && act != CODA_ACT_SWIGLU) return CODA_ERR_DTYPE;
    if (w_dtype != CODA_BF16 && w_dtype != CODA_E4M3) return CODA_ERR_DTYPE;
    const bool fp8 = w_dtype == CODA_E4M3;
    const bool swiglu = act == CODA_ACT_SWIGLU;
    if (!dim_ok(M, 0) || !dim_ok(N_out, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (N_out % 8 != 0 || K % (fp8 ? 16 : 8) != 0 || N_out > kMaxRow || K > kMaxRow)
        return CODA_ERR_SHAPE;
    const int64_t n_w = swiglu ? 2 * N_out : N_out;
    if (n_w > kMaxDim || !prod_ok(M, K) || !prod_ok(n_w, K) || !prod_ok(M, N_out))
        return CODA_ERR_SHAPE;
    if (coda::gemm3_tiles(M, N_out, swiglu) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;  // empty problem: nothing to enqueue, empty tensors may be NULL
    if (!h || !W || !r || !y) return CODA_ERR_NULL;
    if (fp8 && !w_scale) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(W) || !aligned16(r) || !aligned16(y)) return CODA_ERR_ALIGN;
    const Range ry = span(y, M * N_out * 2);
    if (overlap(ry, span(h, M * K * 2)) || overlap(ry, span(W, n_w * K * (fp8 ? 1 : 2))) ||
        overlap(ry, span(r, M * 4)) || (w_scale && overlap(ry, span(w_scale, 4))))
        return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_rowscale_swiglu(int(M), int(N_out), int(K), swiglu, h, W, fp8,
                                                        w_scale, r, y, as_stream(stream)));
}

coda_status coda_rope_table(int64_t rows, double base, float* cos, float* sin, void* stream) {
    if (rows < 1 || rows >= (int64_t(1) << 24)) return CODA_ERR_SHAPE;
    if (!std::isfinite(base) || !(base > 1.0)) return CODA_ERR_VALUE;
    if (!cos || !sin) return CODA_ERR_NULL;
    if (!aligned16(cos) || !aligned16(sin)) return CODA_ERR_ALIGN;
    if (overlap(span(cos, rows * 32 * 4), span(sin, rows * 32 * 4))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_rope_table(int(rows), base, cos, sin, as_stream(stream)));
}

coda_status coda_gemm_rowscale_rope(int64_t M, int64_t N_out, int64_t K, const void* h,
                                    const void* W, coda_dtype w_dtype, const float* w_scale,
                                    const float* r, const int32_t* pos, const float* cos,
                                    const float* sin, int64_t table_rows, int64_t rot_cols,
                                    void* y, void* stream) {
    if (w_dtype != CODA_BF16 && w_dtype != CODA_E4M3) return CODA_ERR_DTYPE;
    const bool fp8 = w_dtype == CODA_E4M3;
    if (!dim_ok(M, 0) || !dim_ok(N_out, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (N_out % 8 != 0 || K % (fp8 ? 16 : 8) != 0 || N_out > kMaxRow || K > kMaxRow)
        return CODA_ERR_SHAPE;
    if (rot_cols < 0 || rot_cols > N_out || rot_cols % 64 != 0) return CODA_ERR_SHAPE;
    const bool rot = rot_cols > 0;
    if (rot && (table_rows < 1 || table_rows >= (int64_t(1) << 24))) return CODA_ERR_SHAPE;
    if (!prod_ok(M, K) || !prod_ok(N_out, K) || !prod_ok(M, N_out)) return CODA_ERR_SHAPE;
    if (coda::gemm3_tiles(M, N_out, false) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!h || !W || !r || !y) return CODA_ERR_NULL;
    if (fp8 && !w_scale) return CODA_ERR_NULL;
    if (rot && (!pos || !cos || !sin)) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(W) || !aligned16(r) || !aligned16(y)) return CODA_ERR_ALIGN;
    if (rot && (!aligned16(pos) || !aligned16(cos) || !aligned16(sin))) return CODA_ERR_ALIGN;
    const Range ry = span(y, M * N_out * 2);
    if (overlap(ry, span(h, M * K * 2)) || overlap(ry, span(W, N_out * K * (fp8 ? 1 : 2))) ||
        overlap(ry, span(r, M * 4)) || (w_scale && overlap(ry, span(w_scale, 4))))
        return CODA_ERR_ALIAS;
    if (rot && (overlap(ry, span(pos, M * 4)) || overlap(ry, span(cos, table_rows * 128)) ||
                overlap(ry, span(sin, table_rows * 128))))
        return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_rowscale_rope(int(M), int(N_out), int(K), h, W, fp8, w_scale, r,
                                                      rot ? pos : nullptr, cos, sin, int(rot ? table_rows : 0),
                                                      int(rot_cols), y, as_stream(stream)));
}

int64_t coda_ce_partials_per_row(int64_t V) { return V < 1 || V > kMaxRow ? -1 : coda::ce_partials_per_row(V); }

coda_status coda_gemm_rowscale_ce(int64_t M, int64_t V, int64_t K, const void* h, const void* W,
                                  coda_dtype w_dtype, const float* w_scale, const float* r,
                                  const int32_t* targets, float* partials, float* tgt_logit,
                                  void* stream) {
    if (w_dtype != CODA_BF16 && w_dtype != CODA_E4M3) return CODA_ERR_DTYPE;
    const bool fp8 = w_dtype == CODA_E4M3;
    if (!dim_ok(M, 0) || !dim_ok(V, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (K % (fp8 ? 16 : 8) != 0 || V > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    const int64_t T = coda::ce_partials_per_row(V);
    if (!prod_ok(M, K) || !prod_ok(V, K) || !prod_ok(M, 2 * T)) return CODA_ERR_SHAPE;
    if (coda::gemm3_tiles(M, V, false) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!h || !W || !r || !targets || !partials || !tgt_logit) return CODA_ERR_NULL;
    if (fp8 && !w_scale) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(W) || !aligned16(r) || !aligned16(targets) || !aligned16(partials) ||
        !aligned16(tgt_logit))
        return CODA_ERR_ALIGN;
    const Range rp = span(partials, M * T * 8), rt = span(tgt_logit, M * 4);
    const Range ins[] = {span(h, M * K * 2), span(W, V * K * (fp8 ? 1 : 2)), span(r, M * 4), span(targets, M * 4),
                         w_scale ? span(w_scale, 4) : Range{0, 0}};
    if (overlap(rp, rt)) return CODA_ERR_ALIAS;
    for (const Range& in : ins)
        if (overlap(rp, in) || overlap(rt, in)) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_rowscale_ce(int(M), int(V), int(K), h, W, fp8, w_scale, r, targets, partials,
                                                    tgt_logit, as_stream(stream)));
}

coda_status coda_ce_reduce(int64_t M, int64_t V, const float* partials, const int32_t* targets,
                           const float* tgt_logit, float* lse, float* loss, void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(V, 1) || V > kMaxRow) return CODA_ERR_SHAPE;
    const int64_t T = coda::ce_partials_per_row(V);
    if (!prod_ok(M, 2 * T)) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!partials || !targets || !tgt_logit || !lse || !loss) return CODA_ERR_NULL;
    if (!aligned16(partials) || !aligned16(targets) || !aligned16(tgt_logit) || !aligned16(lse) || !aligned16(loss))
        return CODA_ERR_ALIGN;
    const Range rl = span(lse, M * 4), rs = span(loss, M * 4);
    const Range ins[] = {span(partials, M * T * 8), span(targets, M * 4), span(tgt_logit, M * 4)};
    if (overlap(rl, rs)) return CODA_ERR_ALIAS;
    for (const Range& in : ins)
        if (overlap(rl, in) || overlap(rs, in)) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_ce_reduce(int(M), int(V), int(T), partials, targets, tgt_logit, lse, loss,
                                             as_stream(stream)));
}

coda_status coda_rowscale_from_h(int64_t M, int64_t N, const void* h, float eps, float* r, void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(N, 1) || N % 8 != 0 || N > kMaxRow || !prod_ok(M, N)) return CODA_ERR_SHAPE;
    if (!std::isfinite(eps) || eps < 0.0f) return CODA_ERR_VALUE;
    if (M == 0) return CODA_OK;
    if (!h || !r) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(r)) return CODA_ERR_ALIGN;
    if (overlap(span(r, M * 4), span(h, M * N * 2))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_rowscale_from_h(int(M), int(N), h, eps, r, as_stream(stream)));
}

coda_status coda_transpose_bf16(int64_t R, int64_t C, const void* src, void* dst, void* stream) {
    if (!dim_ok(R, 1) || !dim_ok(C, 1) || !prod_ok(R, C)) return CODA_ERR_SHAPE;
    if (!src || !dst) return CODA_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return CODA_ERR_ALIGN;
    if (overlap(span(src, R * C * 2), span(dst, R * C * 2))) return CODA_ERR_ALIAS;
    if ((R + 63) / 64 * ((C + 63) / 64) > kMaxDim) return CODA_ERR_SHAPE;
    return hip_status(coda::launch_transpose_bf16(R, C, src, dst, as_stream(stream)));
}

int64_t coda_swiglu_bwd_partials_per_row(int64_t F) {
    return F < 1 || F > kMaxRow / 2 ? -1 : coda::swiglu_bwd_partials_per_row(F);
}

coda_status coda_gemm_swiglu_bwd(int64_t M, int64_t F, int64_t K, const void* h, const void* W,
                                 const float* r, const void* dy, void* dz, float* partials,
                                 void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(F, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (F % 8 != 0 || K % 8 != 0 || 2 * F > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    const int64_t T = coda::swiglu_bwd_partials_per_row(F);
    if (!prod_ok(M, K) || !prod_ok(2 * F, K) || !prod_ok(M, 2 * F) || !prod_ok(M, T)) return CODA_ERR_SHAPE;
    if (coda::gemm3_tiles(M, F, true) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!h || !W || !r || !dy || !dz || !partials) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(W) || !aligned16(r) || !aligned16(dy) || !aligned16(dz) || !aligned16(partials))
        return CODA_ERR_ALIGN;
    const Range rz = span(dz, M * 2 * F * 2), rp = span(partials, M * T * 4);
    const Range ins[] = {span(h, M * K * 2), span(W, 2 * F * K * 2), span(r, M * 4), span(dy, M * F * 2)};
    if (overlap(rz, rp)) return CODA_ERR_ALIAS;
    for (const Range& in : ins)
        if (overlap(rz, in) || overlap(rp, in)) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_swiglu_bwd(int(M), int(F), int(K), h, W, r, dy, dz, partials,
                                                   as_stream(stream)));
}

coda_status coda_gemm_ce_bwd(int64_t M, int64_t V, int64_t K, const void* h, const void* W, const float* r,
                             const int32_t* targets, const float* lse, const float* g, void* dz, float* partials,
                             void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(V, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (V % 8 != 0 || K % 8 != 0 || 2 * V > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    const int64_t T = coda::swiglu_bwd_partials_per_row(V);
    if (!prod_ok(M, K) || !prod_ok(V, K) || !prod_ok(M, V) || !prod_ok(M, T)) return CODA_ERR_SHAPE;
    if (coda::gemm3_tiles(M, V, false) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!h || !W || !r || !targets || !lse || !g || !dz || !partials) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(W) || !aligned16(r) || !aligned16(dz) || !aligned16(partials))
        return CODA_ERR_ALIGN;
    const Range rz = span(dz, M * V * 2), rp = span(partials, M * T * 4);
    const Range ins[] = {span(h, M * K * 2), span(W, V * K * 2), span(r, M * 4), span(targets, M * 4),
                         span(lse, M * 4), span(g, M * 4)};
    if (overlap(rz, rp)) return CODA_ERR_ALIAS;
    for (const Range& in : ins)
        if (overlap(rz, in) || overlap(rp, in)) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_ce_bwd(int(M), int(V), int(K), h, W, r, targets, lse, g, dz, partials,
                                               as_stream(stream)));
}

coda_status coda_rmsnorm_bwd_reduce(int64_t M, int64_t N, int64_t F, const float* partials,
                                    const float* r, float* q, void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(N, 1) || !dim_ok(F, 1) || 2 * F > kMaxRow) return CODA_ERR_SHAPE;
    const int64_t T = coda::swiglu_bwd_partials_per_row(F);
    if (!prod_ok(M, T)) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!partials || !r || !q) return CODA_ERR_NULL;
    if (!aligned16(partials) || !aligned16(r) || !aligned16(q)) return CODA_ERR_ALIGN;
    const Range rq = span(q, M * 4);
    if (overlap(rq, span(partials, M * T * 4)) || overlap(rq, span(r, M * 4))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_rmsnorm_bwd_reduce(int(M), int(N), int(T), partials, r, q, as_stream(stream)));
}

coda_status coda_gemm_rmsnorm_bwd(int64_t M, int64_t N, int64_t K, const void* dz, const void* Wt,
                                  const void* h, const float* q, const void* dh_res, void* dh,
                                  void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(N, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (N % 8 != 0 || K % 8 != 0 || N > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    if (!prod_ok(M, K) || !prod_ok(N, K) || !prod_ok(M, N)) return CODA_ERR_SHAPE;
    if (coda::gemm_bwd2_tiles(M, N) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!dz || !Wt || !h || !q || !dh) return CODA_ERR_NULL;
    if (!aligned16(dz) || !aligned16(Wt) || !aligned16(h) || !aligned16(q) || !aligned16(dh) ||
        (dh_res && !aligned16(dh_res)))
        return CODA_ERR_ALIGN;
    const Range ro = span(dh, M * N * 2);
    if (overlap(ro, span(dz, M * K * 2)) || overlap(ro, span(Wt, N * K * 2)) || overlap(ro, span(h, M * N * 2)) ||
        overlap(ro, span(q, M * 4)))
        return CODA_ERR_ALIAS;
    if (dh_res && dh_res != dh && overlap(ro, span(dh_res, M * N * 2))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_rmsnorm_bwd(int(M), int(N), int(K), dz, Wt, h, q, dh_res, dh,
                                                    as_stream(stream)));
}

coda_status coda_gemm_rowscale_gfold(int64_t M, int64_t N_out, int64_t K, coda_act act, const void* h,
                                     const void* W, const float* gamma, const float* r, void* y, void* stream) {
    if (act != CODA_ACT_NONE && act != CODA_ACT_SWIGLU) return CODA_ERR_DTYPE;
    const bool swiglu = act == CODA_ACT_SWIGLU;
    if (!dim_ok(M, 0) || !dim_ok(N_out, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (N_out % 8 != 0 || K % 8 != 0 || N_out > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    const int64_t n_w = swiglu ? 2 * N_out : N_out;
    if (n_w > kMaxDim || !prod_ok(M, K) || !prod_ok(n_w, K) || !prod_ok(M, N_out)) return CODA_ERR_SHAPE;
    if (coda::gemm3_tiles(M, N_out, swiglu) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!h || !W || !gamma || !r || !y) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(W) || !aligned16(gamma) || !aligned16(r) || !aligned16(y)) return CODA_ERR_ALIGN;
    const Range ry = span(y, M * N_out * 2);
    if (overlap(ry, span(h, M * K * 2)) || overlap(ry, span(W, n_w * K * 2)) || overlap(ry, span(gamma, K * 4)) ||
        overlap(ry, span(r, M * 4)))
        return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_rowscale_gfold(int(M), int(N_out), int(K), swiglu, h, W, gamma, r, y,
                                                       as_stream(stream)));
}

coda_status coda_gemm_rowscale_swiglu_save(int64_t M, int64_t F, int64_t K, const void* h, const void* W,
                                           const float* r, void* y, void* z, void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(F, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (F % 8 != 0 || K % 8 != 0 || 2 * F > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    if (!prod_ok(M, K) || !prod_ok(2 * F, K) || !prod_ok(M, 2 * F)) return CODA_ERR_SHAPE;
    if (coda::gemm3_tiles(M, F, true) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!h || !W || !r || !y || !z) return CODA_ERR_NULL;
    if (!aligned16(h) || !aligned16(W) || !aligned16(r) || !aligned16(y) || !aligned16(z)) return CODA_ERR_ALIGN;
    const Range ry = span(y, M * F * 2), rz = span(z, M * 2 * F * 2);
    if (overlap(ry, rz)) return CODA_ERR_ALIAS;
    const Range ins[] = {span(h, M * K * 2), span(W, 2 * F * K * 2), span(r, M * 4)};
    for (const Range& in : ins)
        if (overlap(ry, in) || overlap(rz, in)) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_rowscale_swiglu_save(int(M), int(F), int(K), h, W, r, y, z,
                                                             as_stream(stream)));
}

coda_status coda_swiglu_bwd_saved(int64_t M, int64_t F, const void* z, const void* dy, const float* r, void* dz,
                                  void* dzt, float* partials, void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(F, 1) || F % 8 != 0 || 2 * F > kMaxRow) return CODA_ERR_SHAPE;
    if (dzt && M % 8 != 0) return CODA_ERR_SHAPE;
    const int64_t T = coda::swiglu_bwd_partials_per_row(F);
    if (!prod_ok(M, 2 * F) || !prod_ok(M, T) || ((M + 63) / 64) * T > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!z || !dy || !r || !dz || !partials) return CODA_ERR_NULL;
    if (!aligned16(z) || !aligned16(dy) || !aligned16(dz) || (dzt && !aligned16(dzt))) return CODA_ERR_ALIGN;
    const Range rd = span(dz, M * 2 * F * 2), rp = span(partials, M * T * 4);
    const Range rt = dzt ? span(dzt, M * 2 * F * 2) : span(nullptr, 0);
    if (overlap(rd, rp) || overlap(rd, rt) || overlap(rp, rt)) return CODA_ERR_ALIAS;
    const Range ins[] = {span(z, M * 2 * F * 2), span(dy, M * F * 2), span(r, M * 4)};
    for (const Range& in : ins)
        if (overlap(rd, in) || overlap(rp, in) || overlap(rt, in)) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_swiglu_bwd_saved(int(M), int(F), z, dy, r, dz, dzt, partials,
                                                    as_stream(stream)));
}

coda_status coda_rope_bwd(int64_t M, int64_t N, const void* dy, const void* y, const float* r, const int32_t* pos,
                          const float* cos, const float* sin, int64_t table_rows, int64_t rot_cols, void* dz,
                          float* partials, void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(N, 1) || N % 8 != 0 || N > kMaxRow) return CODA_ERR_SHAPE;
    if (rot_cols < 0 || rot_cols > N || rot_cols % 64 != 0) return CODA_ERR_SHAPE;
    const bool rot = rot_cols > 0;
    if (rot && (table_rows < 1 || table_rows >= (int64_t(1) << 24))) return CODA_ERR_SHAPE;
    const int64_t T = coda::swiglu_bwd_partials_per_row(N);
    if (!prod_ok(M, N) || !prod_ok(M, T) || ((M + 63) / 64) * T > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!dy || !y || !r || !dz || !partials) return CODA_ERR_NULL;
    if (rot && (!pos || !cos || !sin)) return CODA_ERR_NULL;
    if (!aligned16(dy) || !aligned16(y) || !aligned16(dz)) return CODA_ERR_ALIGN;
    if (rot && (!aligned16(cos) || !aligned16(sin))) return CODA_ERR_ALIGN;
    const Range rd = span(dz, M * N * 2), rp = span(partials, M * T * 4);
    if (overlap(rd, rp)) return CODA_ERR_ALIAS;
    const Range ins[] = {span(dy, M * N * 2), span(y, M * N * 2), span(r, M * 4),
                         span(rot ? pos : nullptr, rot ? M * 4 : 0),
                         span(rot ? cos : nullptr, rot ? table_rows * 128 : 0),
                         span(rot ? sin : nullptr, rot ? table_rows * 128 : 0)};
    for (const Range& in : ins)
        if (overlap(rd, in) || overlap(rp, in)) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_rope_bwd(int(M), int(N), dy, y, r, rot ? pos : nullptr, rot ? cos : nullptr,
                                            rot ? sin : nullptr, int(rot ? table_rows : 0), int(rot_cols), dz,
                                            partials, as_stream(stream)));
}

coda_status coda_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* Bt, const void* c_res,
                           void* C, void* stream) {
    if (!dim_ok(M, 0) || !dim_ok(N, 1) || !dim_ok(K, 1)) return CODA_ERR_SHAPE;
    if (N % 8 != 0 || K % 8 != 0 || N > kMaxRow || K > kMaxRow) return CODA_ERR_SHAPE;
    if (!prod_ok(M, K) || !prod_ok(N, K) || !prod_ok(M, N)) return CODA_ERR_SHAPE;
    if (coda::gemm_bwd2_tiles(M, N) > kMaxDim) return CODA_ERR_SHAPE;
    if (M == 0) return CODA_OK;
    if (!A || !Bt || !C) return CODA_ERR_NULL;
    if (!aligned16(A) || !aligned16(Bt) || !aligned16(C) || (c_res && !aligned16(c_res))) return CODA_ERR_ALIGN;
    const Range ro = span(C, M * N * 2);
    if (overlap(ro, span(A, M * K * 2)) || overlap(ro, span(Bt, N * K * 2))) return CODA_ERR_ALIAS;
    if (c_res && c_res != C && overlap(ro, span(c_res, M * N * 2))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_gemm_rmsnorm_bwd(int(M), int(N), int(K), A, Bt, nullptr, nullptr, c_res, C,
                                                    as_stream(stream)));
}

int64_t coda_wgrad_partials_rows(int64_t NR) { return NR < 1 || NR > kMaxDim ? -1 : coda::wgrad_partials_rows(NR); }

int64_t coda_wgrad_tok_workspace_bytes(int64_t NR, int64_t NC, int64_t K, int64_t lda, int64_t ldb) {
    if (!dim_ok(NR, 1) || !dim_ok(NC, 1) || !dim_ok(K, 0) || lda < NR || ldb < NC || lda > kMaxRow || ldb > kMaxRow ||
        !prod_ok(NR, NC))
        return -1;
    return coda::wgrad_workspace_bytes(NR, NC, K);
}

int64_t coda_wgrad_workspace_bytes(int64_t NR, int64_t NC, int64_t K) {
    if (!dim_ok(NR, 1) || !dim_ok(NC, 1) || !dim_ok(K, 0) || !prod_ok(NR, NC)) return -1;
    return coda::wgrad_workspace_bytes(NR, NC, K);
}

coda_status coda_gemm_wgrad(int64_t NR, int64_t NC, int64_t K, const void* At, const void* Bt,
                            const float* gamma, const void* W, float* dW, float* partials,
                            void* workspace, int64_t workspace_bytes, void* stream) {
    if (!dim_ok(NR, 1) || !dim_ok(NC, 1) || !dim_ok(K, 0)) return CODA_ERR_SHAPE;
    if (NC % 8 != 0 || K % 8 != 0 || K > kMaxRow || NC > kMaxRow / 2) return CODA_ERR_SHAPE;
    const int64_t T = coda::wgrad_partials_rows(NR);
    if (!prod_ok(NR, K) || !prod_ok(NC, K) || !prod_ok(NR, NC) || !prod_ok(T, NC)) return CODA_ERR_SHAPE;
    if (coda::wgrad_tiles(NR, NC) > kMaxDim) return CODA_ERR_SHAPE;
    if (!dW || (W && !partials) || (K > 0 && (!At || !Bt))) return CODA_ERR_NULL;
    if (!aligned16(dW) || (W && !aligned16(W)) || (gamma && !aligned16(gamma)) || (partials && !aligned16(partials)) ||
        (K > 0 && (!aligned16(At) || !aligned16(Bt))))
        return CODA_ERR_ALIGN;
    if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return CODA_ERR_VALUE;
    if (workspace && !aligned16(workspace)) return CODA_ERR_ALIGN;
    const Range ro = span(dW, NR * NC * 4), rp = W ? span(partials, T * NC * 4) : span(nullptr, 0);
    const Range rw = workspace ? span(workspace, workspace_bytes) : span(nullptr, 0);
    if ((W && overlap(ro, rp)) || overlap(ro, rw) || overlap(rp, rw)) return CODA_ERR_ALIAS;
    const Range ins[] = {K > 0 ? span(At, NR * K * 2) : span(nullptr, 0), K > 0 ? span(Bt, NC * K * 2) : span(nullptr, 0),
                         gamma ? span(gamma, NC * 4) : span(nullptr, 0), W ? span(W, NR * NC * 2) : span(nullptr, 0)};
    for (const Range& in : ins)
        if (overlap(ro, in) || (W && overlap(rp, in)) || overlap(rw, in)) return CODA_ERR_ALIAS;
    hipStream_t s = as_stream(stream);
    if (K == 0) {
        hipError_t e = coda::launch_fill_zero_f32(NR * NC, dW, s);
        if (e == hipSuccess && W) e = coda::launch_fill_zero_f32(T * NC, partials, s);
        return hip_status(e);
    }
    return hip_status(coda::launch_gemm_wgrad(int(NR), int(NC), int(K), At, Bt, gamma, W, dW, W ? partials : nullptr,
                                              static_cast<float*>(workspace), workspace_bytes, s));
}

}  // extern "C"

namespace {

// Checks of the token-major weight gradient shared by its two entry points: the caller's
// workspace (caller_workspace), or the library's static scratch, which must hold the
// split the call plans (else CODA_ERR_SHAPE, before anything is touched).
coda_status check_wgrad_tok(int64_t NR, int64_t NC, int64_t K, const void* X, int64_t lda, const void* Y,
                            int64_t ldb, const float* gamma, const void* W, float* dW, float* partials,
                            void* workspace, int64_t workspace_bytes, bool caller_workspace) {
    if (!dim_ok(NR, 1) || !dim_ok(NC, 1) || !dim_ok(K, 0)) return CODA_ERR_SHAPE;
    if (NC % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0 || lda < NR || ldb < NC) return CODA_ERR_SHAPE;
    if (lda > kMaxRow || ldb > kMaxRow || NC > kMaxRow / 2) return CODA_ERR_SHAPE;
    const int64_t T = coda::wgrad_partials_rows(NR);
    if (!prod_ok(NR, NC) || !prod_ok(T, NC)) return CODA_ERR_SHAPE;
    if (coda::wgrad_tiles(NR, NC) > kMaxDim) return CODA_ERR_SHAPE;
    if (!caller_workspace && coda::wgrad_workspace_bytes(NR, NC, K) > coda::kNoAllocScratchBytes)
        return CODA_ERR_SHAPE;
    if (!dW || (W && !partials) || (K > 0 && (!X || !Y))) return CODA_ERR_NULL;
    if (!aligned16(dW) || (W && !aligned16(W)) || (gamma && !aligned16(gamma)) || (partials && !aligned16(partials)) ||
        (K > 0 && (!aligned16(X) || !aligned16(Y))))
        return CODA_ERR_ALIGN;
    if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return CODA_ERR_VALUE;
    if (workspace && !aligned16(workspace)) return CODA_ERR_ALIGN;
    const Range ro = span(dW, NR * NC * 4), rp = W ? span(partials, T * NC * 4) : span(nullptr, 0);
    const Range rw = workspace ? span(workspace, workspace_bytes) : span(nullptr, 0);
    if ((W && overlap(ro, rp)) || overlap(ro, rw) || overlap(rp, rw)) return CODA_ERR_ALIAS;
    const Range ins[] = {K > 0 ? span(X, K * lda * 2) : span(nullptr, 0), K > 0 ? span(Y, K * ldb * 2) : span(nullptr, 0),
                         gamma ? span(gamma, NC * 4) : span(nullptr, 0), W ? span(W, NR * NC * 2) : span(nullptr, 0)};
    for (const Range& in : ins)
        if (overlap(ro, in) || (W && overlap(rp, in)) || overlap(rw, in)) return CODA_ERR_ALIAS;
    return CODA_OK;
}

// K = 0: zeros in dW (and the partials); no scratch involved.
coda_status wgrad_zero(int64_t NR, int64_t NC, const void* W, float* dW, float* partials, hipStream_t s) {
    hipError_t e = coda::launch_fill_zero_f32(NR * NC, dW, s);
    if (e == hipSuccess && W) e = coda::launch_fill_zero_f32(coda::wgrad_partials_rows(NR) * NC, partials, s);
    return hip_status(e);
}

}  // namespace

extern "C" {

coda_status coda_gemm_wgrad_tok(int64_t NR, int64_t NC, int64_t K, const void* X, int64_t lda, const void* Y,
                                int64_t ldb, const float* gamma, const void* W, float* dW, float* partials,
                                void* workspace, int64_t workspace_bytes, void* stream) {
    const coda_status st = check_wgrad_tok(NR, NC, K, X, lda, Y, ldb, gamma, W, dW, partials, workspace,
                                           workspace_bytes, true);
    if (st != CODA_OK) return st;
    hipStream_t s = as_stream(stream);
    if (K == 0) return wgrad_zero(NR, NC, W, dW, partials, s);
    return hip_status(coda::launch_gemm_wgrad_tok(int(NR), int(NC), int(K), X, int(lda), Y, int(ldb), gamma, W, dW,
                                                  W ? partials : nullptr, static_cast<float*>(workspace),
                                                  workspace_bytes, s));
}

coda_status coda_gemm_wgrad_tok_noalloc(int64_t NR, int64_t NC, int64_t K, const void* X, int64_t lda,
                                        const void* Y, int64_t ldb, const float* gamma, const void* W, float* dW,
                                        float* partials, void* stream) {
    const coda_status st = check_wgrad_tok(NR, NC, K, X, lda, Y, ldb, gamma, W, dW, partials, nullptr, 0, false);
    if (st != CODA_OK) return st;
    hipStream_t s = as_stream(stream);
    if (K == 0) return wgrad_zero(NR, NC, W, dW, partials, s);
    return hip_status(coda::launch_gemm_wgrad_tok_noalloc(int(NR), int(NC), int(K), X, int(lda), Y, int(ldb), gamma,
                                                          W, dW, W ? partials : nullptr, s));
}

coda_status coda_colsum_reduce(int64_t T, int64_t NC, const float* partials, float* out, void* stream) {
    if (!dim_ok(T, 1) || !dim_ok(NC, 1) || !prod_ok(T, NC)) return CODA_ERR_SHAPE;
    if (!partials || !out) return CODA_ERR_NULL;
    if (overlap(span(out, NC * 4), span(partials, T * NC * 4))) return CODA_ERR_ALIAS;
    return hip_status(coda::launch_colsum_reduce(int(T), int(NC), partials, out, as_stream(stream)));
}

}  // extern "C"

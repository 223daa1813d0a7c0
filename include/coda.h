/*
 * coda.h -- C ABI of the MI355X (gfx950) GEMM-epilogue chain
 *
 *     h = x_res + A . Wo^T                 (first GEMM, residual add in its epilogue)
 *     r = 1 / sqrt(mean_n(h^2) + eps)      (RMSNorm row scale, from per-tile partials)
 *     y = act( r * (h . W'^T) )            (second GEMM, row scale + SwiGLU epilogue)
 *
 * with W'[n,k] = gamma[k] * W[n,k] (RMSNorm weight folded into the second weight).
 *
 * The chain is the GEMM -> residual -> RMSNorm -> GEMM pattern of the kucoin page
 * "CODA: new research optimizes Transformer training with GEMM-epilogue programming",
 * section "CODA: El epilogo esconde un tesoro": the per-row RMSNorm scale r commutes
 * with the second matrix product, so it is applied at the END of the second GEMM; the
 * first GEMM's end only produces partial sums of squares, combined by a very light
 * reduction kernel.  SwiGLU is applied as a pairwise transform in the second GEMM's
 * epilogue (same section, last paragraph; q2bstudio page: "pairwise transformations").
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or keeps them.  Row-major storage.  Weights are K-contiguous,
 *    i.e. [out_features, in_features] (the torch.nn.Linear layout).
 *  - Every tensor pointer must be 16-byte aligned (CODA_ERR_ALIGN otherwise).
 *  - bf16 = IEEE binary32 truncated to its upper 16 bits (8-bit exponent); e4m3 =
 *    OCP 8-bit "E4M3FN" (bias 7, max 448, no infinities, NaN = S.1111.111).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only ENQUEUES
 *    work on that stream and returns; ordering between calls comes from the stream.
 *    The library never synchronises.
 *  - Arguments are validated on the host BEFORE anything is enqueued; on any error the
 *    call returns a non-zero status and enqueues nothing.  A failed launch returns
 *    CODA_ERR_HIP (the hipError_t is kept per thread, see coda_last_hip_error).  Device
 *    faults surface at the caller's next synchronisation.  No C++ exception crosses
 *    this interface.
 *  - Calls are stateless and may be issued from several host threads.
 *  - Size limits: M <= 2^31 - 1; the row lengths N, N_out and K of the GEMM calls are
 *    at most 2^22 (4194304) elements; M = 0 is a valid empty problem
 *    (nothing is enqueued, and the M-sized tensors may then be NULL), every other
 *    dimension must be >= 1.
 *  - Checks run in the order: dtype/activation codes, shapes, values, (M == 0 ->
 *    CODA_OK), NULL pointers, alignment, overlap.
 */
#ifndef CODA_H_
#define CODA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enumerations get int as their fixed underlying type, so that any int a C
 * caller passes (a value outside the enumerators included) is a valid value of the
 * parameter's type and is rejected by the checks instead of being undefined. */
#ifdef __cplusplus
#define CODA_ENUM_INT : int
#else
#define CODA_ENUM_INT
#endif

typedef enum CODA_ENUM_INT {
    CODA_OK = 0,
    CODA_ERR_NULL = 1,   /* a required pointer is NULL                                   */
    CODA_ERR_SHAPE = 2,  /* a dimension is negative, zero where >= 1 is needed, too large,
                            or not a multiple of the granule the call states             */
    CODA_ERR_DTYPE = 3,  /* unsupported dtype / activation code or combination           */
    CODA_ERR_VALUE = 4,  /* eps < 0 or not finite                                         */
    CODA_ERR_ALIAS = 5,  /* an output overlaps an input or another output (other than an
                            alias the call explicitly allows)                             */
    CODA_ERR_HIP = 6,    /* the HIP runtime rejected a launch                             */
    CODA_ERR_ALIGN = 7   /* a tensor pointer is not 16-byte aligned                       */
} coda_status;

typedef enum CODA_ENUM_INT { CODA_BF16 = 0, CODA_E4M3 = 1 } coda_dtype;
typedef enum CODA_ENUM_INT { CODA_ACT_NONE = 0, CODA_ACT_SWIGLU = 1 } coda_act;

/* ------------------------------------------------------------ weight preparation ----
 * The RMSNorm weight gamma multiplies the second GEMM's reduction dimension, so it is
 * a diagonal that folds into the second weight once per weight update (kucoin page,
 * section "Cinco bloques y un lenguaje LEGO": RMSNorm weights are a broadcast vector
 * operand).  These calls are the preparation step; they are not part of the chain.
 */

/* Wp[n,k] = bf16_rne( fl32(gamma[k] * W[n,k]) )   (gamma == NULL: Wp = W)
 *   W     [N, K] bf16, device, read
 *   gamma [K] fp32, device, read, or NULL
 *   Wp    [N, K] bf16, device, written; must not overlap W or gamma
 * Granule: K % 8 == 0.                                                               */
coda_status coda_prepare_weight_bf16(int64_t N, int64_t K, const void* W, const float* gamma,
                                     void* Wp, void* stream);

/* Per-tensor e4m3 quantisation with an fp32 scale (the 8-bit variant of the chain;
 * kucoin page, section "El impuesto a la pereza para entrenar modelos grandes": 8-bit
 * formats speed up the products and raise the share of the memory-bound work around
 * them):
 *   x[n,k]  = fl32(gamma[k] * X[n,k])        (gamma == NULL: x = X)
 *   amax    = max |x|;   scale = fl32(amax / 448)   (amax == 0: scale = 1)
 *   Q[n,k]  = e4m3_saturate_rne( fl32(x[n,k] / scale) )
 *   X          [N, K] bf16, device, read
 *   gamma      [K] fp32, device, or NULL (used to fold gamma into the second weight
 *              BEFORE quantising it)
 *   Q          [N, K] e4m3 (one byte each), device, written
 *   amax_scale [2] fp32, device, written: {amax, scale}.  Pass &amax_scale[1] as the
 *              scale argument of the GEMM calls.
 * Granule: K % 16 == 0.  Enqueues three kernels (clear, max-reduce, quantise).        */
coda_status coda_quantize_e4m3(int64_t N, int64_t K, const void* X, const float* gamma,
                               void* Q, float* amax_scale, void* stream);

/* -------------------------------------------------------------------- the chain ---- */

/* Number of per-row partial sums the first GEMM writes for a hidden size N; the caller
 * sizes `partials` as M * coda_partials_per_row(N) floats.  Returns -1 if N < 1.      */
int64_t coda_partials_per_row(int64_t N);

/* First GEMM with residual + partial-RMS epilogue (kucoin page, section "CODA: El
 * epilogo esconde un tesoro": residual add, then only a PARTIAL root-mean-square at the
 * end of the first GEMM; the combinable partial is the sum of squares over the tile).
 *   v[m,n]  = sa * sw * sum_k A[m,k] * W[n,k]  +  x_res[m,n]      (fp32 accumulation)
 *   h[m,n]  = bf16_rne(v[m,n])
 *   P[m,t]  = sum over the columns n of tile t of h[m,n]^2       (fp32, fixed order)
 *   A       [M, K]  bf16 or e4m3 (ab_dtype), device
 *   a_scale device fp32 scalar sa, or NULL (= 1; required for e4m3)
 *   W       [N, K]  same dtype as A, device
 *   w_scale device fp32 scalar sw, or NULL (= 1; required for e4m3)
 *   x_res   [M, N]  bf16, device, or NULL (= 0).  May be EXACTLY equal to h (in place).
 *   h       [M, N]  bf16, device, written
 *   partials[M, coda_partials_per_row(N)] fp32, device, written
 * Granules: N % 8 == 0; K % 8 == 0 (bf16) or K % 16 == 0 (e4m3).                      */
coda_status coda_gemm_resid_partialrms(int64_t M, int64_t N, int64_t K,
                                       const void* A, coda_dtype ab_dtype, const float* a_scale,
                                       const void* W, const float* w_scale,
                                       const void* x_res, void* h, float* partials,
                                       void* stream);

/* The light reduction that turns the partials into the row scale (kucoin page, section
 * "CODA: El epilogo esconde un tesoro": the partial sums are combined by a very light
 * reduction kernel between the two GEMMs):
 *   r[m] = fl32( 1 / sqrt( (sum_t P[m,t]) / N + eps ) )   (sum and sqrt in fp64)
 *   partials [M, coda_partials_per_row(N)] fp32, device;  r [M] fp32, device, written.
 * eps must be finite and >= 0.  A row whose sum and eps are both 0 yields +inf.       */
coda_status coda_rowscale_reduce(int64_t M, int64_t N, const float* partials, float eps,
                                 float* r, void* stream);

/* Second GEMM with row-scale (+SwiGLU) epilogue (kucoin page, section "CODA: El epilogo
 * esconde un tesoro": r commutes with the next product and is applied at its end; the
 * same reparameterisation covers SwiGLU).  z = sw * (h . W^T), with gamma already
 * folded into W:
 *   CODA_ACT_NONE:   W [N_out, K];   y[m,n] = bf16_rne( r[m] * z[m,n] )
 *   CODA_ACT_SWIGLU: W [2*N_out, K], rows [0, N_out) = gate, [N_out, 2*N_out) = up;
 *                    g = r[m]*z[m,j], u = r[m]*z[m,N_out+j],
 *                    y[m,j] = bf16_rne( g / (1 + exp(-g)) * u )
 *   (r multiplies both halves BEFORE the SiLU: it commutes with the GEMM, not with SiLU.)
 *   h       [M, K] bf16, device (the first call's output)
 *   W       bf16 or e4m3 (w_dtype; e4m3 = weight-only 8-bit, decoded exactly to bf16)
 *   w_scale device fp32 scalar sw, or NULL (= 1; required for e4m3)
 *   r       [M] fp32, device
 *   y       [M, N_out] bf16, device, written; must not overlap any input
 * Granules: K % 8 == 0 (bf16 W) or K % 16 == 0 (e4m3 W); N_out % 8 == 0.              */
coda_status coda_gemm_rowscale_swiglu(int64_t M, int64_t N_out, int64_t K, coda_act act,
                                      const void* h, const void* W, coda_dtype w_dtype,
                                      const float* w_scale, const float* r, void* y,
                                      void* stream);

/* ------------------------------------------------------------------------ RoPE ----
 * Rotary position embedding as the pairwise epilogue of the QKV GEMM (kucoin page,
 * section "CODA: El epilogo esconde un tesoro", last paragraph: the reparameterisation
 * also covers RoPE; section "Cinco bloques y un lenguaje LEGO": an element-wise
 * transform).  LLaMA layout: the output columns are heads of 64 values, Q heads then K
 * heads then V heads; in a rotated head value i pairs with value i + 32 (i < 32) and
 * the pair turns by the angle pos * theta_i, theta_i = base^(-2i/64).
 */

/* cos / sin table of the angles:  cos[p*32 + i] = fl32( cos(p * base^(-2i/64)) ),
 * sin likewise, for positions p in [0, rows), i in [0, 32) (angles and cosines in
 * fp64, one rounding to fp32).
 *   cos, sin [rows, 32] fp32, device, written; must not overlap.
 * rows in [1, 2^24); base finite and > 1 (CODA_ERR_VALUE otherwise).                   */
coda_status coda_rope_table(int64_t rows, double base, float* cos, float* sin, void* stream);

/* Second GEMM with row-scale + RoPE epilogue (no activation; the RoPE passages cited
 * above).  z = sw * (h . W^T):
 *   x[m,n] = r[m] * z[m,n];
 *   for a column n < rot_cols in head c = n / 64 at offset i = n % 64 < 32, with
 *   p = pos[m], C = cos[p*32 + i], S = sin[p*32 + i]:
 *     y[m, 64c + i]      = bf16_rne( x[m, 64c + i] * C - x[m, 64c + i + 32] * S )
 *     y[m, 64c + i + 32] = bf16_rne( x[m, 64c + i + 32] * C + x[m, 64c + i] * S )
 *   columns n >= rot_cols (V):  y[m,n] = bf16_rne( x[m,n] ).
 *   h, W, w_dtype, w_scale, r as for coda_gemm_rowscale_swiglu with CODA_ACT_NONE
 *             (W [N_out, K])
 *   pos       [M] int32, device: the row's position.  A position outside
 *             [0, table_rows) reads cos = sin = 0 (the table lookups are range-checked),
 *             i.e. zeros in that row's rotated columns -- not an error.
 *   cos, sin  [table_rows, 32] fp32, device (coda_rope_table)
 *   rot_cols  number of leading rotated columns (Q and K heads): a multiple of 64,
 *             0 <= rot_cols <= N_out.  With rot_cols == 0 pos / cos / sin may be NULL.
 *   y         [M, N_out] bf16, device, written; must not overlap any input
 * Granules: as coda_gemm_rowscale_swiglu with CODA_ACT_NONE; table_rows in [1, 2^24)
 * when rot_cols > 0.                                                                  */
coda_status coda_gemm_rowscale_rope(int64_t M, int64_t N_out, int64_t K, const void* h,
                                    const void* W, coda_dtype w_dtype, const float* w_scale,
                                    const float* r, const int32_t* pos, const float* cos,
                                    const float* sin, int64_t table_rows, int64_t rot_cols,
                                    void* y, void* stream);

/* --------------------------------------------------------------- cross-entropy ----
 * The LM-head GEMM with the loss in its epilogue (kucoin page, section "CODA: El
 * epilogo esconde un tesoro", last paragraph: the reparameterisation covers the
 * cross-entropy loss; section "Cinco bloques y un lenguaje LEGO": a block log-sum-exp
 * and the max / sum-exp state of online normalisation).  The logits never reach
 * memory: the GEMM writes one (max, sum-exp) pair per row and 256-column tile, and a
 * light reduction turns them into the log-sum-exp and the loss.
 */

/* Tiles per row of the cross-entropy partials for a vocabulary of V columns; the caller
 * sizes `partials` as M * coda_ce_partials_per_row(V) * 2 floats.  -1 if V < 1.       */
int64_t coda_ce_partials_per_row(int64_t V);

/* LM-head GEMM with row scale + block log-sum-exp epilogue (the cross-entropy passages
 * cited above: block log-sum-exp, max / sum-exp state).  z = r[m] * sw * (h . W^T):
 *   partials[m, t, 0] = max over the columns v of tile t (v in [256t, 256t+256) and
 *                       v < V) of z[m, v]                                   (fp32)
 *   partials[m, t, 1] = sum over the same columns of exp(z[m, v] - that max)  (fp32)
 *   tgt_logit[m]      = z[m, targets[m]]  if 0 <= targets[m] < V (written by the tile
 *                       that holds the column); left untouched otherwise.
 *   h, W, w_dtype, w_scale, r as for coda_gemm_rowscale_swiglu with CODA_ACT_NONE,
 *             W [V, K] (the LM-head weight with the final RMSNorm's gamma folded in)
 *   targets   [M] int32, device
 *   partials  [M, coda_ce_partials_per_row(V), 2] fp32, device, written
 *   tgt_logit [M] fp32, device, written (see above)
 * V in [1, 2^22]; granule of K as coda_gemm_rowscale_swiglu.  Outputs must not overlap
 * each other or any input.                                                            */
coda_status coda_gemm_rowscale_ce(int64_t M, int64_t V, int64_t K, const void* h, const void* W,
                                  coda_dtype w_dtype, const float* w_scale, const float* r,
                                  const int32_t* targets, float* partials, float* tgt_logit,
                                  void* stream);

/* The reduction of the partials (the light reduction after the loss epilogue, as
 * cited above):
 *   lse[m]  = fl32( Mx + log( sum_t partials[m,t,1] * exp(partials[m,t,0] - Mx) ) ),
 *             Mx = max_t partials[m,t,0]                           (fp64 inside)
 *   loss[m] = fl32( lse - tgt_logit[m] )  if 0 <= targets[m] < V, else 0 (an ignored
 *             row, e.g. targets[m] = -100)
 *   partials, targets, tgt_logit as written / read by coda_gemm_rowscale_ce
 *   lse, loss [M] fp32, device, written; must not overlap the inputs or each other.  */
coda_status coda_ce_reduce(int64_t M, int64_t V, const float* partials, const int32_t* targets,
                           const float* tgt_logit, float* lse, float* loss, void* stream);

/* ------------------------------------------------ backward of the MLP input block ----
 * Input gradient of  y = SwiGLU( RMSNorm(h) . W^T )  (kucoin page, section "CODA: El
 * epilogo esconde un tesoro", last paragraph: the reparameterisation holds for the
 * backward pass).  With acc = h . W'^T (W' = gamma-folded), r the forward's row scale,
 * z = r * acc, g = z[:, :F], u = z[:, F:], s = sigmoid(g) and the upstream gradient dy:
 *   dL/dg = dy u s (1 + g (1 - s)),   dL/du = dy g s,   c[m] = sum_j dL/dz[m,j] acc[m,j]
 *   dh = r * ((dL/dz) . W') - (r^3 / N) * c * h   (+ the residual stream's gradient)
 * Three calls: the recomputed forward product with the SwiGLU backward in its epilogue
 * (writes r * dL/dz and per-tile partials of c), the reduction of c into the row
 * coefficient q = -(r^3/N) c, and the input-gradient GEMM whose epilogue adds q * h.
 * The second GEMM reduces over 2F, so it reads W' transposed (coda_transpose_bf16,
 * once per weight update).  bf16 weights only.
 */

/* The row scale of a stored h, for a backward that recomputes it instead of saving it
 * (the RMSNorm row scale of the kucoin page, section "CODA: El epilogo esconde un
 * tesoro", from h directly):
 *   r[m] = fl32( 1 / sqrt( sum_n h[m,n]^2 / N + eps ) )     (fp64 inside)
 *   h [M, N] bf16, device;  r [M] fp32, device, written, must not overlap h.
 * Granule: N % 8 == 0.  eps finite and >= 0.                                         */
coda_status coda_rowscale_from_h(int64_t M, int64_t N, const void* h, float eps, float* r,
                                 void* stream);

/* dst[c, r] = src[r, c] for bf16 [R, C] matrices; R, C in [1, 2^31); no overlap.  A
 * layout utility (W'^T for the input-gradient GEMM), no operation of the pages.       */
coda_status coda_transpose_bf16(int64_t R, int64_t C, const void* src, void* dst, void* stream);

/* Partials per row written by coda_gemm_swiglu_bwd for F gate columns; -1 if F < 1.    */
int64_t coda_swiglu_bwd_partials_per_row(int64_t F);

/* Recomputed gate/up product with the SwiGLU-backward epilogue (the backward passage
 * cited above; the SwiGLU derivative is the epilogue's element-wise transform):
 *   h   [M, K] bf16 (the block input the forward read);  W [2F, K] bf16 (W', gate rows
 *       then up rows);  r [M] fp32 (the forward's row scale);  dy [M, F] bf16
 *   dz  [M, 2F] bf16, written: bf16_rne( r[m] * dL/dz[m, j] )  (gate columns, then up)
 *   partials [M, coda_swiglu_bwd_partials_per_row(F)] fp32, written: per tile of 128 gate
 *       (and the matching 128 up) columns, sum of dL/dz * acc   (fp32)
 * Granules: K % 8 == 0, F % 8 == 0; F <= 2^21.  Outputs must not overlap the inputs.  */
coda_status coda_gemm_swiglu_bwd(int64_t M, int64_t F, int64_t K, const void* h, const void* W,
                                 const float* r, const void* dy, void* dz, float* partials,
                                 void* stream);

/* The light reduction of the backward (cited above): the RMSNorm backward's row
 * coefficient
 * q[m] = fl32( -(r[m]^3 / N) * sum_t partials[m, t] )   (fp64 inside; N = hidden size,
 * F = the gate width the partials were written for).  q must not overlap the inputs.  */
coda_status coda_rmsnorm_bwd_reduce(int64_t M, int64_t N, int64_t F, const float* partials,
                                    const float* r, float* q, void* stream);

/* Input-gradient GEMM with the RMSNorm-backward epilogue (the backward passage cited
 * above: the row-scale term q * h is applied at the end of the product):
 *   dh[m,n] = bf16_rne( sum_k dz[m,k] Wt[n,k] + q[m] h[m,n] + dh_res[m,n] )
 *   dz [M, K] bf16 (K = 2F);  Wt [N, K] bf16 = W'^T;  h [M, N] bf16;  q [M] fp32
 *   dh_res [M, N] bf16 or NULL (= 0); may be EXACTLY equal to dh (in place)
 *   dh [M, N] bf16, written; must not overlap any other input
 * Granules: N % 8 == 0, K % 8 == 0.                                                   */
coda_status coda_gemm_rmsnorm_bwd(int64_t M, int64_t N, int64_t K, const void* dz, const void* Wt,
                                  const void* h, const float* q, const void* dh_res, void* dh,
                                  void* stream);

/* The second GEMM from the RAW weight, with gamma folded in on chip (no weight
 * preparation pass, no W' copy): each 16-byte chunk of W is multiplied by its 8 gamma
 * values and rounded, bf16_rne(fl32(gamma[k] W[n,k])), between the registers and LDS --
 * the arithmetic of coda_prepare_weight_bf16, so y is bit-identical to
 * coda_gemm_rowscale_swiglu with the prepared W'.  (kucoin page, section "Cinco bloques y
 * un lenguaje LEGO": the RMSNorm weight is a broadcast vector operand.)
 *   act NONE or SWIGLU as coda_gemm_rowscale_swiglu;  W [n_w, K] bf16 raw weight;
 *   gamma [K] fp32 (16-byte aligned);  h, r, y as there.
 * Granules: N_out % 8 == 0, K % 8 == 0.  y must not overlap the inputs.               */
coda_status coda_gemm_rowscale_gfold(int64_t M, int64_t N_out, int64_t K, coda_act act, const void* h,
                                     const void* W, const float* gamma, const float* r, void* y, void* stream);

/* ------------------------------ backward from a saved pre-activation ---- */
/* A forward that keeps the pre-activation lets the backward skip the recomputed gate/up
 * product (memory for time: z is M x 2F bf16).  Same block and same gradients as above
 * (kucoin page, section "Cinco bloques y un lenguaje LEGO": the matrix-block store
 * primitive keeps intermediate activations for the backward pass).                     */

/* The SwiGLU second GEMM of coda_gemm_rowscale_swiglu (bf16 weights) that also writes
 *   z [M, 2F] bf16 = bf16_rne( r[m] * sum_k h[m,k] W[j,k] )   (gate columns, then up)
 * y [M, F] is bit-identical to coda_gemm_rowscale_swiglu's.  h [M, K], W [2F, K] bf16,
 * r [M] fp32.  Granules: K % 8 == 0, F % 8 == 0.  y, z must not overlap each other or
 * the inputs.                                                                          */
coda_status coda_gemm_rowscale_swiglu_save(int64_t M, int64_t F, int64_t K, const void* h, const void* W,
                                           const float* r, void* y, void* z, void* stream);

/* SwiGLU backward from the saved z, with g = z[m, j], u = z[m, F+j], d = dy[m, j]:
 *   dz [M, 2F] bf16, written: bf16_rne( r[m] * dL/dz )  (as coda_gemm_swiglu_bwd)
 *   dzt [2F, M] bf16 or NULL: the transpose of dz (the weight gradient's operand);
 *       needs M % 8 == 0
 *   partials [M, coda_swiglu_bwd_partials_per_row(F)] fp32: per tile of 128 gate
 *       columns, (1/r[m]) * sum of dL/dz * z, the layout coda_rmsnorm_bwd_reduce takes
 * Granule: F % 8 == 0.  Outputs must not overlap each other or the inputs.            */
coda_status coda_swiglu_bwd_saved(int64_t M, int64_t F, const void* z, const void* dy, const float* r, void* dz,
                                  void* dzt, float* partials, void* stream);

/* -------------------------------------- backward of the cross-entropy epilogue ----
 * Input side of the backward of the LM-head block  loss_m = CE( RMSNorm(h) . W^T, t_m )
 * (kucoin page, section "CODA: El epilogo esconde un tesoro", last paragraph: the
 * reparameterisation covers the cross-entropy loss and holds for the backward pass).  As
 * the SwiGLU backward, it recomputes the product and turns it into the input-gradient
 * GEMM's operand in the epilogue; the rest is coda_rmsnorm_bwd_reduce (with F = V),
 * coda_gemm_rmsnorm_bwd (K = V, Wt = W'^T [d, V]) and coda_gemm_wgrad_tok +
 * coda_colsum_reduce on dz and h, unchanged.  With acc = h . W'^T and z = r * acc:
 *   dL/dz[m, v] = g[m] * ( exp(z[m, v] - lse[m]) - [v == targets[m]] ),  and 0 for a row
 *       whose target lies outside [0, V) (its loss is the constant 0)
 *   dz [M, V] bf16, written: bf16_rne( r[m] * dL/dz[m, v] )
 *   partials [M, coda_swiglu_bwd_partials_per_row(V)] fp32, written: per 128 columns,
 *       sum of dL/dz * acc  (fp32)
 *   h [M, K] bf16;  W [V, K] bf16 (W', gamma folded);  r [M] fp32 (the forward's row
 *   scale);  targets [M] int32;  lse [M] fp32 (the forward's log-sum-exp, coda_ce_reduce);
 *   g [M] fp32 = d(total loss) / d(loss of row m), e.g. 1/n for a mean over n rows
 * Granules: K % 8 == 0, V % 8 == 0, V <= 2^21.  Outputs must not overlap each other or
 * the inputs.  bf16 weights only.                                                      */
coda_status coda_gemm_ce_bwd(int64_t M, int64_t V, int64_t K, const void* h, const void* W, const float* r,
                             const int32_t* targets, const float* lse, const float* g, void* dz, float* partials,
                             void* stream);

/* ------------------------------------------ backward of the RoPE epilogue ----
 * Input side of the backward of the QKV block  y = RoPE( RMSNorm(h) . W^T )  (kucoin
 * page, section "CODA: El epilogo esconde un tesoro", last paragraph: the
 * reparameterisation covers RoPE and holds for the backward pass).  The rotation's
 * gradient is its transpose and needs no recomputed product; the rest of the block's
 * backward is coda_rmsnorm_bwd_reduce (with F = N), coda_gemm_rmsnorm_bwd (K = N) and
 * coda_gemm_wgrad_tok + coda_colsum_reduce on dz and h, unchanged.
 *   dL/dz = RoPE^T(dy): in a rotated head, for i < 32 with C, S the table's cos / sin at
 *     (pos[m], i):  dL/dz[64c+i] = dy[64c+i] C + dy[64c+i+32] S,
 *                   dL/dz[64c+i+32] = dy[64c+i+32] C - dy[64c+i] S;  dL/dz = dy past rot_cols
 *   dz [M, N] bf16, written: bf16_rne( r[m] * dL/dz[m, j] )
 *   partials [M, coda_swiglu_bwd_partials_per_row(N)] fp32, written: per tile of 128
 *       columns, (1/r[m]) * sum of dy * y  (= sum of dL/dz * acc, acc = z / r: the
 *       rotation is orthogonal and a tile holds whole heads)
 *   dy [M, N] bf16 (upstream gradient);  y [M, N] bf16 (the forward's output, as
 *       coda_gemm_rowscale_rope wrote it);  r [M] fp32 (the forward's row scale)
 *   pos, cos, sin, table_rows, rot_cols as for coda_gemm_rowscale_rope (a position
 *       outside the table reads zero angles there, so its rotated columns' gradient is
 *       0, the derivative of that forward); cos and sin 16-byte aligned
 * Granule: N % 8 == 0.  Outputs must not overlap each other or the inputs.             */
coda_status coda_rope_bwd(int64_t M, int64_t N, const void* dy, const void* y, const float* r, const int32_t* pos,
                          const float* cos, const float* sin, int64_t table_rows, int64_t rot_cols, void* dz,
                          float* partials, void* stream);

/* Plain product with an optional residual, bf16 out (the first GEMM's input gradient,
 * the backward of the chain: kucoin page, section "CODA: El epilogo esconde un tesoro",
 * last paragraph;
 * dA = dh . Wo, with Bt = Wo^T passed K-contiguous; the same kernel as
 * coda_gemm_rmsnorm_bwd without the row-scale term):
 *   C[m,n] = bf16_rne( sum_k A[m,k] Bt[n,k] + c_res[m,n] )    (fp32 MFMA sums)
 *   A [M, K] bf16;  Bt [N, K] bf16;  c_res [M, N] bf16 or NULL, may be EXACTLY C
 *   C [M, N] bf16, written; must not overlap A or Bt
 * Granules: N % 8 == 0, K % 8 == 0.                                                   */
coda_status coda_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* Bt, const void* c_res,
                           void* C, void* stream);

/* --------------------------------------------- backward: weight gradients ---- */
/* Weight gradients of the same block (kucoin page, section "CODA: El epilogo esconde un
 * tesoro": the backward inherits the forward's structure; section "Cinco bloques y un
 * lenguaje LEGO": a broadcast vector operand and a block reduction in the epilogue).
 * With G = (r * dL/dz)^T h summed over the tokens, dL/dW = gamma * G (gamma broadcast
 * over the columns) and dL/dgamma[k] = sum_j W[j,k] G[j,k] with the raw weight W.  The
 * reduction runs over the tokens, so both operands are passed token-contiguous (the
 * outputs of coda_transpose_bf16 of dz and of h).  With gamma = NULL and W = NULL the
 * same call is the plain weight gradient of a linear layer (the first GEMM's).
 */

/* Partial rows written by coda_gemm_wgrad for NR gradient rows; -1 if NR < 1.          */
int64_t coda_wgrad_partials_rows(int64_t NR);

/* Workspace bytes that let coda_gemm_wgrad split the K tokens over more blocks when the
 * NR x NC output has too few 256 x 256 tiles to fill the GPU (room for the split's dW
 * slices and, with W, its gamma-gradient partial slices); 0 when no split helps; -1 for
 * invalid sizes.                                                                       */
int64_t coda_wgrad_workspace_bytes(int64_t NR, int64_t NC, int64_t K);

/* Weight-gradient GEMM, contraction over K tokens (the weight-gradient passages cited
 * above):
 *   At [NR, K] bf16 (e.g. (r * dL/dz)^T, NR = 2F);  Bt [NC, K] bf16 (e.g. h^T, NC = d)
 *   gamma [NC] fp32 or NULL (= 1);  W [NR, NC] bf16 raw weight or NULL (no partials)
 *   dW [NR, NC] fp32, written: fl32( gamma[k] * sum_m At[j,m] Bt[k,m] )  (fp32 MFMA sums)
 *   partials [coda_wgrad_partials_rows(NR), NC] fp32, written when W is given: per tile
 *       of 256 rows j, sum of W[j,k] * G[j,k] (fixed order); may be NULL when W is NULL
 *   workspace: device scratch of workspace_bytes (NULL / 0 for none), 16-byte aligned.
 *       With at least coda_wgrad_workspace_bytes(NR, NC, K) bytes, the tokens are split
 *       over several blocks per tile whose fp32 sums (and, with W, partial rows) are
 *       added in a fixed order (then gamma applied): the result is reproducible for the
 *       same arguments but its last bits depend on whether the split was taken.
 * K = 0 (no tokens) writes zeros.  Granules: K % 8 == 0, NC % 8 == 0; K <= 2^22,
 * NC <= 2^21.  Outputs and workspace must not overlap each other or the inputs.
 * CODA_ERR_VALUE: workspace_bytes < 0, or > 0 with a NULL workspace.                 */
coda_status coda_gemm_wgrad(int64_t NR, int64_t NC, int64_t K, const void* At, const void* Bt,
                            const float* gamma, const void* W, float* dW, float* partials,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes for coda_gemm_wgrad_tok: the same as coda_wgrad_workspace_bytes (token
 * rows are addressed per 64-token k-tile, so the leading dimensions need no split of
 * their own); -1 for invalid sizes (lda < NR, ldb < NC, or either above 2^22).        */
int64_t coda_wgrad_tok_workspace_bytes(int64_t NR, int64_t NC, int64_t K, int64_t lda, int64_t ldb);

/* The same weight-gradient GEMM (cited above) on token-major operands, as the
 * activations are stored (no transposes): the contraction runs down the rows of
 *   X [K, lda] bf16, its first NR columns (e.g. r * dL/dz [M, 2F]: lda = NR = 2F)
 *   Y [K, ldb] bf16, its first NC columns (e.g. h [M, d]: ldb = NC = d)
 *   dW[j,k] = fl32( gamma[k] * sum_m X[m,j] Y[m,k] ); gamma, W, partials, workspace and the
 *   token split exactly as coda_gemm_wgrad (workspace sized by coda_wgrad_workspace_bytes).
 * The tiles are read through LDS transpose reads; the result is bit-identical to
 * coda_gemm_wgrad on the transposed operands with the same split.  Any K (K = 0 writes
 * zeros).  Granules: NC % 8 == 0, lda % 8 == 0, ldb % 8 == 0, lda >= NR, ldb >= NC.
 * Operands of any size (above 4 GB too): every 64-token k-tile is addressed from its own
 * base.  Without workspace (or with less than the split needs) one block per tile.     */
coda_status coda_gemm_wgrad_tok(int64_t NR, int64_t NC, int64_t K, const void* X, int64_t lda, const void* Y,
                                int64_t ldb, const float* gamma, const void* W, float* dW, float* partials,
                                void* workspace, int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): coda_gemm_wgrad_tok without the
 * workspace arguments.  The token split, when the call's plan takes one, keeps its
 * slices in a static device array of the library (CODA_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's load to the end of the process); nothing is allocated, freed
 * or cleared by the call.  Arguments, result and determinism as coda_gemm_wgrad_tok
 * with a sufficient workspace (bit-identical to it).
 * CODA_ERR_SHAPE (nothing enqueued) when coda_wgrad_workspace_bytes(NR, NC, K) exceeds
 * CODA_NOALLOC_SCRATCH_BYTES, besides the checks of coda_gemm_wgrad_tok.
 * Calls on the same GPU share the array: two calls that overlap in time (on different
 * streams, or from different threads without ordering) race and give wrong results.  */
#define CODA_NOALLOC_SCRATCH_BYTES (128ll << 20)
coda_status coda_gemm_wgrad_tok_noalloc(int64_t NR, int64_t NC, int64_t K, const void* X, int64_t lda,
                                        const void* Y, int64_t ldb, const float* gamma, const void* W, float* dW,
                                        float* partials, void* stream);

/* The block reduction's final sum (cited above):
 * out[k] = fl32( sum_t partials[t, k] )  (fixed order, fp64 inside), T >= 1 rows of NC
 * columns: the gamma gradient from coda_gemm_wgrad's partials.  out must not overlap.  */
coda_status coda_colsum_reduce(int64_t T, int64_t NC, const float* partials, float* out,
                               void* stream);

/* ------------------------------------------------------------------- utilities ---- */
const char* coda_status_string(coda_status s);
int coda_last_hip_error(void);      /* hipError_t of this thread's last CODA_ERR_HIP      */
const char* coda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CODA_H_ */

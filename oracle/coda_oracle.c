/*
 * Plain, slow, fp64 CPU oracle of the GEMM -> residual -> RMSNorm -> GEMM(+SwiGLU)
 * chain.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the bench's
 * CPU-baseline leg may load it.  It shares no code with the HIP library.
 *
 * What it computes, in the order the pages state it (kucoin "CODA: new research
 * optimizes Transformer training..." section "CODA: El epilogo esconde un tesoro"):
 * a matrix product, a residual add, RMS normalisation, a second matrix product, and
 * (same section, last paragraph; section "Resultados del experimento") SwiGLU, or
 * (same paragraph) RoPE on the QKV product (orc_rope) or the cross-entropy loss of the
 * LM-head product (orc_cross_entropy), both applied to the act-NONE output.
 * It is the UNFUSED definition: no tiling, no partial sums, no deferred row scale.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - RMSNorm: r = 1/sqrt(mean_n(hb^2) + eps), mean over the whole hidden dim, then
 *    each element times gamma[k];
 *  - the residual stream h is a bf16 tensor: hb = bf16_rne(h) feeds the norm;
 *  - gate = first half of the second product's columns, up = second half;
 *    y = silu(gate) * up with silu(g) = g / (1 + exp(-g));
 *  - the second weight the chain holds is the gamma-folded, rounded W'; the unfused
 *    weight that represents exactly the same function is W_or[n,k] = W'[n,k]/gamma[k]
 *    (formed in fp64 here) -- the weight preparation is computed by this file's own
 *    orc_fold_* routines, never taken from the GPU;
 *  - e4m3 is the OCP "E4M3FN" 8-bit format (bias 7, max 448, no infinities,
 *    NaN = S.1111.111); quantisation uses a per-tensor scale s = amax/448 and
 *    saturating round-to-nearest-even.
 *
 * Rounding decisions that produce integer codes (the fold's bf16 rounding, e4m3
 * codes, the quantisation scale) are taken in fp32 arithmetic, the precision the
 * weight preparation is specified in; everything else is fp64.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_E4M3 = 1 };
enum { ORC_ACT_NONE = 0, ORC_ACT_SWIGLU = 1 };

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- bf16 ---- */

/* bf16 layout: sign(1) exponent(8, bias 127) mantissa(7).  Decoded by the formula. */
double orc_bf16_decode(uint16_t c) {
    int s = (c >> 15) & 1, e = (c >> 7) & 0xFF, m = c & 0x7F;
    double v;
    if (e == 0xFF) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -126 - 7);          /* subnormal: m * 2^-133 */
    else v = ldexp(128.0 + m, e - 127 - 7);                     /* (1 + m/128) * 2^(e-127) */
    return s ? -v : v;
}

/* Bits of a magnitude that is exactly representable in bf16. */
static uint16_t bf16_bits_of_exact(double v) {
    if (v == 0.0) return 0;
    if (v < ldexp(1.0, -126)) return (uint16_t)(v / ldexp(1.0, -133));   /* subnormal */
    int E;
    double f = frexp(v, &E);              /* v = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                        /* v in [2^e, 2^(e+1)) */
    int m = (int)((ldexp(f, 1) - 1.0) * 128.0);
    return (uint16_t)(((e + 127) << 7) | m);
}

/* Round-to-nearest-even of any double to bf16 (single rounding). */
uint16_t orc_bf16_encode_rne(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int E;
    frexp(a, &E);                          /* a in [2^(E-1), 2^E) */
    int qexp = (E - 1) - 7;                /* spacing of bf16 values in that binade */
    if (qexp < -133) qexp = -133;          /* subnormal spacing */
    double q = nearbyint(ldexp(a, -qexp)); /* exact scaling, then ties-to-even */
    double v = ldexp(q, qexp);
    double max_bf16 = ldexp(255.0, 127 - 7);
    if (v > max_bf16) return sign | 0x7F80;
    return sign | bf16_bits_of_exact(v);
}

/* ---------------------------------------------------------------- e4m3 ---- */

/* OCP E4M3FN decode by the formula: normal (1 + m/8) * 2^(e-7), subnormal m/8 * 2^-6. */
double orc_e4m3_decode(uint8_t c) {
    int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
    if (e == 0xF && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return s ? -v : v;
}

/* Saturating round-to-nearest-even into E4M3FN.  The 127 non-negative finite codes
 * 0x00..0x7E decode to increasing values; pick the nearest, ties to the even code. */
uint8_t orc_e4m3_encode_sat_rne(double x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 0x7E;                 /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double dl = a - orc_e4m3_decode((uint8_t)lo), dh = orc_e4m3_decode((uint8_t)hi) - a;
    int c = (dl < dh) ? lo : (dh < dl) ? hi : ((lo % 2 == 0) ? lo : hi);
    return sign | (uint8_t)c;
}

/* ----------------------------------------------------- weight preparation ---- */

/* gamma fold into the second weight, bf16 result:
 *   out[n,k] = bf16_rne( fl32(gamma[k] * W[n,k]) )                               */
void orc_fold_bf16(int64_t N, int64_t K, const uint16_t* W, const float* gamma, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float w = (float)orc_bf16_decode(W[n * K + k]);
            float g = gamma ? gamma[k] : 1.0f;
            float p = g * w;                                   /* one fp32 rounding */
            out[n * K + k] = orc_bf16_encode_rne((double)p);
        }
}

/* Per-tensor e4m3 quantisation (optionally of the gamma-folded weight):
 *   x[n,k]  = fl32(gamma[k] * W[n,k])   (gamma == NULL: x = W)
 *   amax    = max |x|;  scale = fl32(amax / 448)  (amax == 0: scale = 1)
 *   out     = e4m3_sat_rne( fl32(x / scale) )                                     */
void orc_quant_e4m3(int64_t N, int64_t K, const uint16_t* W, const float* gamma,
                    uint8_t* out, float* amax_out, float* scale_out) {
    float amax = 0.0f;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float g = gamma ? gamma[k] : 1.0f;
            float x = g * (float)orc_bf16_decode(W[n * K + k]);
            float ax = fabsf(x);
            if (ax > amax) amax = ax;
        }
    float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float g = gamma ? gamma[k] : 1.0f;
            float x = g * (float)orc_bf16_decode(W[n * K + k]);
            float q = x / scale;                               /* one fp32 rounding */
            out[n * K + k] = orc_e4m3_encode_sat_rne((double)q);
        }
    *amax_out = amax;
    *scale_out = scale;
}

/* ---------------------------------------------------------------- chain ---- */

static double decode(const void* p, int dt, int64_t i) {
    return dt == ORC_BF16 ? orc_bf16_decode(((const uint16_t*)p)[i])
                          : orc_e4m3_decode(((const uint8_t*)p)[i]);
}

/*
 * The unfused chain for the rows rows[0..R) of an M-row problem.
 *   A    [M, K1]   codes (bf16 or e4m3), value = decode * a_scale
 *   Wo   [d, K1]   first weight, nn.Linear layout (Wo[n,k] multiplies A[m,k])
 *   xres [M, d]    bf16 residual, or NULL (residual 0)
 *   gamma[d]       RMSNorm weight
 *   Wp   [N2w, d]  prepared (gamma-folded) second weight codes, value = decode * wp_scale
 * Outputs per computed row i (row m = rows[i]):
 *   h[i, d]   = xres[m,:] + A[m,:] . Wo^T                 (fp64, unrounded)
 *   hb[i, d]  = bf16_rne(h)                                (bits)
 *   S[i]      = sum_n hb^2,  r[i] = 1/sqrt(S/d + eps)
 *   y[i, n_out]: z = (hb * r * gamma) . W_or^T with W_or = Wp/gamma;
 *                NONE: y = z;  SWIGLU: y = silu(z[:, :F]) * z[:, F:], F = N2w/2
 */
int orc_chain(int64_t R, const int64_t* rows,
              int64_t K1, int64_t d, int64_t N2w, int act,
              const void* A, int a_dt, double a_scale,
              const void* Wo, int wo_dt, double wo_scale,
              const uint16_t* xres, const float* gamma,
              const void* Wp, int wp_dt, double wp_scale, double eps,
              double* h_out, uint16_t* hb_out, double* S_out, double* r_out, double* y_out) {
    if (act == ORC_ACT_SWIGLU && (N2w % 2)) return 1;
    int64_t n_out = (act == ORC_ACT_SWIGLU) ? N2w / 2 : N2w;

    double* wo = (double*)malloc(sizeof(double) * (size_t)(d * K1));
    double* wor = (double*)malloc(sizeof(double) * (size_t)(N2w * d));
    if (!wo || !wor) { free(wo); free(wor); return 2; }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < d; ++n)
        for (int64_t k = 0; k < K1; ++k) wo[n * K1 + k] = decode(Wo, wo_dt, n * K1 + k) * wo_scale;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N2w; ++n)
        for (int64_t k = 0; k < d; ++k)
            wor[n * d + k] = decode(Wp, wp_dt, n * d + k) * wp_scale / (double)gamma[k];

    int fail = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)K1);
        double* hb = (double*)malloc(sizeof(double) * (size_t)d);
        double* nrm = (double*)malloc(sizeof(double) * (size_t)d);
        double* z = (double*)malloc(sizeof(double) * (size_t)N2w);
        if (!a || !hb || !nrm || !z) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < R; ++i) {
                int64_t m = rows ? rows[i] : i;
                for (int64_t k = 0; k < K1; ++k) a[k] = decode(A, a_dt, m * K1 + k) * a_scale;
                /* GEMM 1 and the residual add */
                for (int64_t n = 0; n < d; ++n) {
                    double t = 0.0;
                    for (int64_t k = 0; k < K1; ++k) t += a[k] * wo[n * K1 + k];
                    double h = (xres ? orc_bf16_decode(xres[m * d + n]) : 0.0) + t;
                    uint16_t hbits = orc_bf16_encode_rne(h);
                    h_out[i * d + n] = h;
                    hb_out[i * d + n] = hbits;
                    hb[n] = orc_bf16_decode(hbits);
                }
                /* RMSNorm */
                double S = 0.0;
                for (int64_t n = 0; n < d; ++n) S += hb[n] * hb[n];
                double r = 1.0 / sqrt(S / (double)d + eps);
                S_out[i] = S;
                r_out[i] = r;
                for (int64_t k = 0; k < d; ++k) nrm[k] = hb[k] * r * (double)gamma[k];
                /* GEMM 2 */
                for (int64_t n = 0; n < N2w; ++n) {
                    double s = 0.0;
                    for (int64_t k = 0; k < d; ++k) s += nrm[k] * wor[n * d + k];
                    z[n] = s;
                }
                /* activation */
                for (int64_t n = 0; n < n_out; ++n) {
                    if (act == ORC_ACT_SWIGLU) {
                        double g = z[n], u = z[n_out + n];
                        y_out[i * n_out + n] = g / (1.0 + exp(-g)) * u;
                    } else {
                        y_out[i * n_out + n] = z[n];
                    }
                }
            }
        }
        free(a); free(hb); free(nrm); free(z);
    }
    free(wo);
    free(wor);
    return fail ? 2 : 0;
}

/* ----------------------------------------------------------------- RoPE ---- */

/*
 * Rotary position embedding as a pairwise epilogue of the QKV product (kucoin page,
 * section "CODA: El epilogo esconde un tesoro", last paragraph: the same
 * reparameterisation holds for RoPE; section "Cinco bloques y un lenguaje LEGO": RoPE
 * is an element-wise transform).  The pages do not define it; the reading used is the
 * LLaMA one (listed in the design notes):
 *   columns [0, rot_cols) are heads of head_dim values (Q heads, then K heads); in each
 *   head, value i pairs with value i + head_dim/2 (i < head_dim/2) and the pair is
 *   rotated by the angle pos * theta_i, theta_i = base^(-2 i / head_dim):
 *     x1' = x1 cos - x2 sin,   x2' = x2 cos + x1 sin;
 *   columns [rot_cols, ncols) (V heads) pass through.
 * In place on y [R, ncols] (fp64, the unrounded chain output); pos[i] is row i's
 * position.  fp64 throughout, cos/sin from the C library.
 */
int orc_rope(int64_t R, int64_t ncols, double* y, const int32_t* pos, double base,
             int64_t head_dim, int64_t rot_cols) {
    if (head_dim < 2 || head_dim % 2 || rot_cols % head_dim || rot_cols > ncols) return 1;
    int64_t half = head_dim / 2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i) {
        double p = (double)pos[i];
        for (int64_t h0 = 0; h0 < rot_cols; h0 += head_dim) {
            for (int64_t j = 0; j < half; ++j) {
                double theta = pow(base, -2.0 * (double)j / (double)head_dim);
                double ang = p * theta;
                double c = cos(ang), sn = sin(ang);
                double x1 = y[i * ncols + h0 + j], x2 = y[i * ncols + h0 + half + j];
                y[i * ncols + h0 + j] = x1 * c - x2 * sn;
                y[i * ncols + h0 + half + j] = x2 * c + x1 * sn;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------ backward of the MLP input ---- */

/*
 * Input gradient of the block  y = SwiGLU( RMSNorm(hb) . W_or^T )  (kucoin page, section
 * "CODA: El epilogo esconde un tesoro", last paragraph: the reparameterisation also holds
 * for the backward pass, whose structure the forward's blockwise-local final stage
 * passes on; section "Resultados del experimento": the backward of this chain).  For
 * each listed row m, given the upstream gradient dy[m, 0..F) of y, the unfused chain
 * rule in the forward's order, reversed:
 *   forward:   r = 1/sqrt(mean(hb^2) + eps),  n = hb r gamma,  z = n . W_or^T,
 *              g = z[0..F), u = z[F..2F),  y = silu(g) u
 *   SwiGLU:    dg = dy u sigma(g) (1 + g (1 - sigma(g))),   du = dy silu(g)
 *   GEMM:      dn[k] = sum_j dz[j] W_or[j, k]                 (dz = [dg, du])
 *   RMSNorm:   dhb[k] = r gamma[k] dn[k] - (r^3 / d) hb[k] sum_k' gamma[k'] dn[k'] hb[k']
 * W_or = Wp * wp_scale / gamma as in orc_chain (Wp the prepared, gamma-folded weight).
 * hb, dy are bf16 codes; outputs fp64: dh [R, d], r [R], dz [R, 2F].
 */
int orc_mlpin_bwd(int64_t R, const int64_t* rows, int64_t d, int64_t F,
                  const uint16_t* hb_in, const float* gamma, const void* Wp, int wp_dt, double wp_scale,
                  const uint16_t* dy_in, double eps, double* dh_out, double* r_out, double* dz_out) {
    int64_t F2 = 2 * F;
    double* wor = (double*)malloc(sizeof(double) * (size_t)(F2 * d));
    if (!wor) return 2;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < F2; ++n)
        for (int64_t k = 0; k < d; ++k)
            wor[n * d + k] = decode(Wp, wp_dt, n * d + k) * wp_scale / (double)gamma[k];
    int fail = 0;
#pragma omp parallel
    {
        double* hb = (double*)malloc(sizeof(double) * (size_t)d);
        double* nrm = (double*)malloc(sizeof(double) * (size_t)d);
        double* dn = (double*)malloc(sizeof(double) * (size_t)d);
        double* dz = (double*)malloc(sizeof(double) * (size_t)F2);
        if (!hb || !nrm || !dn || !dz) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < R; ++i) {
                int64_t m = rows ? rows[i] : i;
                double S = 0.0;
                for (int64_t k = 0; k < d; ++k) {
                    hb[k] = orc_bf16_decode(hb_in[m * d + k]);
                    S += hb[k] * hb[k];
                }
                double r = 1.0 / sqrt(S / (double)d + eps);
                r_out[i] = r;
                for (int64_t k = 0; k < d; ++k) nrm[k] = hb[k] * r * (double)gamma[k];
                for (int64_t j = 0; j < F; ++j) {
                    double g = 0.0, u = 0.0;
                    for (int64_t k = 0; k < d; ++k) {
                        g += nrm[k] * wor[j * d + k];
                        u += nrm[k] * wor[(F + j) * d + k];
                    }
                    double dyj = orc_bf16_decode(dy_in[m * F + j]);
                    double sg = 1.0 / (1.0 + exp(-g));
                    dz[j] = dyj * u * sg * (1.0 + g * (1.0 - sg));
                    dz[F + j] = dyj * g * sg;
                }
                for (int64_t k = 0; k < d; ++k) {
                    double t = 0.0;
                    for (int64_t j = 0; j < F2; ++j) t += dz[j] * wor[j * d + k];
                    dn[k] = t;
                }
                double c = 0.0;
                for (int64_t k = 0; k < d; ++k) c += (double)gamma[k] * dn[k] * hb[k];
                for (int64_t k = 0; k < d; ++k)
                    dh_out[i * d + k] = r * (double)gamma[k] * dn[k] - r * r * r / (double)d * hb[k] * c;
                for (int64_t j = 0; j < F2; ++j) dz_out[i * F2 + j] = dz[j];
            }
        }
        free(hb); free(nrm); free(dn); free(dz);
    }
    free(wor);
    return fail ? 2 : 0;
}

/*
 * Weight gradients of the same block, sampled: for the listed gate/up rows j of the
 * second weight (j in [0, 2F)) and columns k, summed over ALL M tokens,
 *   dW[j, k]   = sum_m dz[m, j] * n[m, k]       (n = hb r gamma, the RMSNorm output;
 *                                                 the gradient of the raw weight W)
 * and, when every j in [0, 2F) is listed (small problems), the RMSNorm weight gradient
 *   dgamma[k]  = sum_m sum_j dz[m, j] * W[j, k] * hb[m, k] * r[m].
 * dz[m, j] needs only the gate and up products of (m, j mod F), so a sampled column of
 * dW costs M * 2d operations.  Inputs as orc_mlpin_bwd plus the raw weight W (bf16).
 *
 * Optional (NULL to skip), for error bounds of an implementation that rounds the summed
 * terms: the root-sum-square over the tokens of the terms of each sum,
 *   rss[j, k]       = sqrt( sum_m (dz[m, j] r[m] hb[m, k])^2 )          (gamma left out)
 *   rss_gamma[k]    = sqrt( sum_m sum_j (dz[m, j] W[j, k] r[m] hb[m, k])^2 )   (full j only)
 */
int orc_mlpin_wgrad(int64_t M, int64_t d, int64_t F, const uint16_t* hb_in, const float* gamma,
                    const void* Wp, int wp_dt, double wp_scale, const uint16_t* W_raw,
                    const uint16_t* dy_in, double eps, int64_t nj, const int64_t* js,
                    int64_t nk, const int64_t* ks, double* dW_out, double* dgamma_out,
                    double* rss_out, double* rss_gamma_out) {
    int64_t F2 = 2 * F;
    double* r = (double*)malloc(sizeof(double) * (size_t)M);
    double* dzc = (double*)malloc(sizeof(double) * (size_t)M);
    if (!r || !dzc) { free(r); free(dzc); return 2; }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double S = 0.0;
        for (int64_t k = 0; k < d; ++k) { double v = orc_bf16_decode(hb_in[m * d + k]); S += v * v; }
        r[m] = 1.0 / sqrt(S / (double)d + eps);
    }
    if (dgamma_out) for (int64_t k = 0; k < nk; ++k) dgamma_out[k] = 0.0;
    if (rss_gamma_out) for (int64_t k = 0; k < nk; ++k) rss_gamma_out[k] = 0.0;
    for (int64_t a = 0; a < nj; ++a) {
        int64_t j = js[a], jg = j < F ? j : j - F;       /* the gate / up pair of column j */
        /* dz[:, j] over all tokens */
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            double g = 0.0, u = 0.0;
            for (int64_t k = 0; k < d; ++k) {
                double nk_ = orc_bf16_decode(hb_in[m * d + k]) * r[m] * (double)gamma[k];
                g += nk_ * decode(Wp, wp_dt, jg * d + k) * wp_scale / (double)gamma[k];
                u += nk_ * decode(Wp, wp_dt, (F + jg) * d + k) * wp_scale / (double)gamma[k];
            }
            double dyv = orc_bf16_decode(dy_in[m * F + jg]);
            double sg = 1.0 / (1.0 + exp(-g));
            dzc[m] = j < F ? dyv * u * sg * (1.0 + g * (1.0 - sg)) : dyv * g * sg;
        }
        for (int64_t b = 0; b < nk; ++b) {
            int64_t k = ks[b];
            double acc = 0.0, accg = 0.0, sq = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double hv = orc_bf16_decode(hb_in[m * d + k]);
                acc += dzc[m] * hv * r[m] * (double)gamma[k];
                accg += dzc[m] * hv * r[m];
                sq += (dzc[m] * hv * r[m]) * (dzc[m] * hv * r[m]);
            }
            dW_out[a * nk + b] = acc;
            double wv = orc_bf16_decode(W_raw[j * d + k]);
            if (dgamma_out) dgamma_out[b] += accg * wv;
            if (rss_out) rss_out[a * nk + b] = sqrt(sq);
            if (rss_gamma_out) rss_gamma_out[b] += sq * wv * wv;
        }
    }
    if (rss_gamma_out) for (int64_t k = 0; k < nk; ++k) rss_gamma_out[k] = sqrt(rss_gamma_out[k]);
    (void)F2;
    free(r); free(dzc);
    return 0;
}

/* -------------------------------------------------------- cross-entropy ---- */

/*
 * Cross-entropy of the LM-head product's logits (kucoin page, section "CODA: El
 * epilogo esconde un tesoro", last paragraph: the reparameterisation covers the
 * cross-entropy loss; section "Cinco bloques y un lenguaje LEGO": block log-sum-exp
 * and the max / sum-exp statistics of online normalisation).  Per row of z [R, V]
 * (fp64, the unrounded chain output, i.e. r * (h . W'^T)):
 *   lse  = log( sum_v exp(z[v]) )          (evaluated as m + log(sum exp(z - m)),
 *                                            m = max z: the same number, no overflow)
 *   loss = lse - z[t]  for a target t in [0, V);  0 for any other t (an ignored row).
 */
int orc_cross_entropy(int64_t R, int64_t V, const double* z, const int32_t* targets,
                      double* lse_out, double* loss_out) {
    if (V < 1) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i) {
        const double* zi = z + i * V;
        double m = zi[0];
        for (int64_t v = 1; v < V; ++v) m = zi[v] > m ? zi[v] : m;
        double s = 0.0;
        for (int64_t v = 0; v < V; ++v) s += exp(zi[v] - m);
        double lse = m + log(s);
        int64_t t = targets[i];
        lse_out[i] = lse;
        loss_out[i] = (t >= 0 && t < V) ? lse - zi[t] : 0.0;
    }
    return 0;
}

/* ------------------------------------------------- array helpers (tests) ---- */

void orc_bf16_decode_n(int64_t n, const uint16_t* c, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_decode(c[i]);
}
void orc_bf16_encode_n(int64_t n, const double* x, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_encode_rne(x[i]);
}
void orc_e4m3_decode_n(int64_t n, const uint8_t* c, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}
void orc_e4m3_encode_n(int64_t n, const double* x, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode_sat_rne(x[i]);
}

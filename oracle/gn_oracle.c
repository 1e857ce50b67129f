/*
 * gn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of GroupNorm with optional SiLU over
 * dense channels-last activations.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code with the HIP library.
 *
 * What it computes (source: "FLUX.2 VAE decoder fast path behind
 * quality=high", Modifications section 1 "Kernel": channels-last GroupNorm
 * over (N, L, C) rows with C innermost, per-(batch, group) mean/rstd, the
 * affine transform, then an optional SiLU; the Motivation section names the
 * op pair as the GroupNorm -> SiLU chains of the diffusers VAE decoder).
 * The plain definition, written out:
 *
 *   x  has N samples of L rows of C channels, element (n, l, c) at offset
 *      (n*L + l)*C + c; C is split into G contiguous groups of Cg = C/G
 *      channels, channel c belongs to group c / Cg.
 *   For each (n, g), over the M = L*Cg elements of the group:
 *      mu    = (1/M) * sum x                      (first pass)
 *      var   = (1/M) * sum (x - mu)^2             (second pass, biased)
 *      rstd  = 1 / sqrt(var + eps)
 *   For each element:
 *      t = gamma[c] * (x - mu) * rstd + beta[c]
 *      y = apply_silu ? t / (1 + exp(-t)) : t      (SiLU(t) = t * sigmoid(t))
 *
 * Readings where the pages are silent (each also listed in the design notes):
 * the variance is the biased (divide by M) one; eps sits inside the square
 * root; groups are contiguous channel blocks; SiLU comes after the affine;
 * a NULL gamma means all ones and a NULL beta all zeros.
 *
 * Inputs may be bf16, IEEE binary16 or binary32 (the page's kernel tests
 * cover fp32 and bf16 activations); every one widens exactly to fp64, so the
 * arithmetic below is the same for all three.
 *
 * All arithmetic is IEEE fp64 in the order written above: no blocking, no
 * fused passes, no reassociation.  OpenMP only splits independent groups
 * (statistics) and independent rows (elementwise output) across threads; the
 * order of every sum is the plain sequential one.
 *
 * The neighbouring convolution (for the fused GroupNorm -> SiLU -> conv of
 * the decoder's ResnetBlock2D, named in the same page's Modifications
 * section 2: "ResnetBlock2D norm1/norm2 + SiLU chains", and its
 * "Conv2d(3x3, p1)"): a 3x3 cross-correlation with zero padding 1 and
 * stride 1 over NHWC activations, the plain definition
 *
 *   out[n,h,w,co] = bias[co] + res[n,h,w,co]
 *                 + sum_{kh,kw in 0..2} sum_{ci} wt[co,kh,kw,ci] * in[n,h+kh-1,w+kw-1,ci]
 *
 * with in = 0 outside the image, weights stored [Co][3][3][Ci] (the
 * channels-last layout of a [Co, Ci, 3, 3] weight), bias and res optional.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16 from its definition: 1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; exponent 0 is zero/subnormal (f * 2^-24), 31 is inf/NaN. */
static double f16_bits_to_double(uint16_t bits) {
    const int sign = (bits >> 15) & 1;
    const int e = (bits >> 10) & 0x1f;
    const int f = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);
    return sign ? -v : v;
}

enum { GNO_BF16 = 0, GNO_F16 = 1, GNO_F32 = 2, GNO_F64 = 3 };

/* Element i of x, widened to fp64. */
static double load(const void *x, int dtype, int64_t i) {
    if (dtype == GNO_BF16) return bf16_bits_to_double(((const uint16_t *)x)[i]);
    if (dtype == GNO_F16) return f16_bits_to_double(((const uint16_t *)x)[i]);
    if (dtype == GNO_F64) return ((const double *)x)[i];
    return (double)((const float *)x)[i];
}

/* Widening of n elements (for pinning the decoders against libraries). */
int gno_widen(const void *x, int dtype, int64_t n, double *out) {
    if (dtype < GNO_BF16 || dtype > GNO_F32) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = load(x, dtype, i);
    return 0;
}

static int check_shape(int64_t N, int64_t L, int64_t C, int64_t G) {
    if (N < 0 || L < 0 || C <= 0 || G <= 0 || C % G != 0) return -1;
    return 0;
}

int gno_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void gno_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Per-(n, g) mean and biased variance, two passes in fp64.
 * mean_out, var_out: N*G doubles, index n*G + g.  Returns 0, or -1 on a bad
 * shape or dtype. */
int gno_group_stats_dt(const void *x, int dtype, int64_t N, int64_t L, int64_t C, int64_t G,
                       double *mean_out, double *var_out) {
    if (check_shape(N, L, C, G) || dtype < GNO_BF16 || dtype > GNO_F64) return -1;
    const int64_t Cg = C / G;
    const int64_t M = L * Cg;
    int64_t ng;
#pragma omp parallel for schedule(dynamic, 1)
    for (ng = 0; ng < N * G; ++ng) {
        const int64_t n = ng / G, g = ng % G;
        const int64_t base = n * L * C + g * Cg;
        double sum = 0.0;
        for (int64_t l = 0; l < L; ++l)
            for (int64_t j = 0; j < Cg; ++j) sum += load(x, dtype, base + l * C + j);
        const double mu = (M > 0) ? sum / (double)M : 0.0;
        double ss = 0.0;
        for (int64_t l = 0; l < L; ++l)
            for (int64_t j = 0; j < Cg; ++j) {
                const double d = load(x, dtype, base + l * C + j) - mu;
                ss += d * d;
            }
        mean_out[ng] = mu;
        var_out[ng] = (M > 0) ? ss / (double)M : 0.0;
    }
    return 0;
}

int gno_group_stats(const uint16_t *x, int64_t N, int64_t L, int64_t C, int64_t G,
                    double *mean_out, double *var_out) {
    return gno_group_stats_dt(x, GNO_BF16, N, L, C, G, mean_out, var_out);
}

/* y = SiLU(t) = t * sigmoid(t), written as t / (1 + exp(-t)).  For t far
 * below zero exp(-t) overflows to +inf and the quotient is -0, the limit. */
static double silu(double t) { return t / (1.0 + exp(-t)); }

/* Full GroupNorm(+SiLU).  Exactly one of out64 / out32 is non-NULL; out32
 * receives the fp64 result rounded once to fp32 (storage for the large
 * shapes only).  mean_out/var_out (may be NULL) receive the statistics.
 * Returns 0, or -1 on a bad argument. */
int gno_gn_silu_dt(const void *x, int dtype, const float *gamma, const float *beta, int64_t N,
                   int64_t L, int64_t C, int64_t G, double eps, int apply_silu,
                   double *out64, float *out32, double *mean_out, double *var_out) {
    if (check_shape(N, L, C, G) || dtype < GNO_BF16 || dtype > GNO_F32) return -1;
    if ((out64 == NULL) == (out32 == NULL)) return -1;
    if (!(eps >= 0.0)) return -1;
    const int64_t Cg = C / G;
    double *mean = mean_out, *var = var_out;
    /* statistics storage: caller-provided or a small heap block */
    double *heap = NULL;
    if (mean == NULL || var == NULL) {
        const size_t ng = (size_t)(N * G > 0 ? N * G : 1);
        heap = (double *)malloc(sizeof(double) * 2 * ng);
        if (heap == NULL) return -1;
        mean = heap;
        var = heap + ng;
    }
    gno_group_stats_dt(x, dtype, N, L, C, G, mean, var);
    int64_t row;
#pragma omp parallel for schedule(static)
    for (row = 0; row < N * L; ++row) {
        const int64_t n = row / L;
        for (int64_t c = 0; c < C; ++c) {
            const int64_t g = c / Cg;
            const double mu = mean[n * G + g];
            const double rstd = 1.0 / sqrt(var[n * G + g] + eps);
            const double ga = gamma ? (double)gamma[c] : 1.0;
            const double be = beta ? (double)beta[c] : 0.0;
            const double xv = load(x, dtype, row * C + c);
            const double t = ga * ((xv - mu) * rstd) + be;
            const double yv = apply_silu ? silu(t) : t;
            if (out64)
                out64[row * C + c] = yv;
            else
                out32[row * C + c] = (float)yv;
        }
    }
    free(heap);
    return 0;
}

int gno_gn_silu(const uint16_t *x, const float *gamma, const float *beta, int64_t N,
                int64_t L, int64_t C, int64_t G, double eps, int apply_silu,
                double *out64, float *out32, double *mean_out, double *var_out) {
    return gno_gn_silu_dt(x, GNO_BF16, gamma, beta, N, L, C, G, eps, apply_silu, out64, out32,
                          mean_out, var_out);
}

/* One output pixel (n, h, w) of the convolution below, all Co channels. */
static void conv_pixel(const double *in, const double *wt, const double *bias, const double *res,
                       int64_t H, int64_t W, int64_t Ci, int64_t Co, int64_t pix, double *out,
                       double *abs_out) {
    const int64_t n = pix / (H * W);
    const int64_t h = (pix / W) % H;
    const int64_t w = pix % W;
    for (int64_t co = 0; co < Co; ++co) {
        double acc = bias ? bias[co] : 0.0;
        double mag = bias ? fabs(bias[co]) : 0.0;
        if (res) {
            acc += res[pix * Co + co];
            mag += fabs(res[pix * Co + co]);
        }
        for (int64_t kh = 0; kh < 3; ++kh) {
            const int64_t ih = h + kh - 1;
            if (ih < 0 || ih >= H) continue;
            for (int64_t kw = 0; kw < 3; ++kw) {
                const int64_t iw = w + kw - 1;
                if (iw < 0 || iw >= W) continue;
                const double *ip = in + ((n * H + ih) * W + iw) * Ci;
                const double *wp = wt + ((co * 3 + kh) * 3 + kw) * Ci;
                for (int64_t ci = 0; ci < Ci; ++ci) {
                    const double term = wp[ci] * ip[ci];
                    acc += term;
                    mag += fabs(term);
                }
            }
        }
        out[co] = acc;
        if (abs_out) abs_out[co] = mag;
    }
}

/* The 3x3 convolution above, in fp64.  in: [N][H][W][Ci]; wt: [Co][3][3][Ci];
 * bias: [Co] or NULL; res: [N][H][W][Co] or NULL; out: [N][H][W][Co].
 * abs_out (may be NULL) receives, per output, the same sum taken over the
 * absolute values of every term (|bias| + |res| + sum |wt * in|): the scale
 * against which rounding errors of the operands are bounded.  Every output
 * sums its terms in the order bias, res, then kh, kw, ci ascending.
 * Returns 0, or -1 on a bad shape. */
int gno_conv3x3_nhwc(const double *in, const double *wt, const double *bias, const double *res,
                     int64_t N, int64_t H, int64_t W, int64_t Ci, int64_t Co, double *out,
                     double *abs_out) {
    if (N < 0 || H < 0 || W < 0 || Ci <= 0 || Co <= 0) return -1;
    int64_t pix;
#pragma omp parallel for schedule(static)
    for (pix = 0; pix < N * H * W; ++pix)
        conv_pixel(in, wt, bias, res, H, W, Ci, Co, pix, out + pix * Co,
                   abs_out ? abs_out + pix * Co : NULL);
    return 0;
}

/* The same convolution at npix selected output pixels only (linear pixel
 * indices (n*H + h)*W + w in pix[]): out and abs_out are [npix][Co].  For
 * checking sampled outputs of tensors too large for the full sum. */
int gno_conv3x3_nhwc_at(const double *in, const double *wt, const double *bias,
                        const double *res, int64_t N, int64_t H, int64_t W, int64_t Ci,
                        int64_t Co, const int64_t *pix, int64_t npix, double *out,
                        double *abs_out) {
    if (N < 0 || H < 0 || W < 0 || Ci <= 0 || Co <= 0 || npix < 0) return -1;
    for (int64_t i = 0; i < npix; ++i)
        if (pix[i] < 0 || pix[i] >= N * H * W) return -1;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < npix; ++i)
        conv_pixel(in, wt, bias, res, H, W, Ci, Co, pix[i], out + i * Co,
                   abs_out ? abs_out + i * Co : NULL);
    return 0;
}

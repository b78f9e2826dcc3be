/*
 * Oracle: plain CPU direct 2-D convolution in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links or calls this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 *
 * What it computes (forward convolution as on the page
 * "dispatch_amd_4wave_conv2d", summary and Args sections; the filter layouts
 * are those named on the page "dispatch_fused_im2col_conv2d_apple",
 * Parameters section, filter_is_fcrs):
 *
 *   y[n,oh,ow,co] = sum_{r<R} sum_{s<S} sum_{ci<C}
 *                     X(n, oh*sh - ph + r, ow*sw - pw + s, ci) * Wt(r, s, ci, co)
 *
 *   X(n,ih,iw,ci) = x[((n*H + ih)*W + iw)*C + ci] when 0 <= ih < H and
 *                   0 <= iw < W, else 0 (zero padding on both sides);
 *   Wt(r,s,ci,co) = w[((r*S + s)*C + ci)*F + co]   RSCF, [R, S, C_in, C_out]
 *                 = w[((co*C + ci)*R + r)*S + s]   FCRS, [C_out, C_in, R, S]
 *   Ho = floor((H + 2*ph - R) / sh) + 1,  Wo = floor((W + 2*pw - S) / sw) + 1.
 *
 * With a residual source (page 1, summary: D = Conv(A, B) + beta * source,
 * source NHWC with the output's shape):  D = y + beta * src.
 *
 * No flip of the filter (cross-correlation, as every deep-learning framework
 * defines "convolution"); the pages never mention a flip.
 *
 * Each output element is one straight loop over (r, s, ci) accumulating in
 * double, in that fixed order; there is no blocking or reordering.  The only
 * parallelism is OpenMP over whole output rows (n, oh), which does not change
 * any element's summation order.  Build without -ffast-math.
 */
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double filter_tap(const double* w, int fcrs, int64_t R, int64_t S,
                         int64_t C, int64_t F, int64_t r, int64_t s,
                         int64_t ci, int64_t co) {
    if (fcrs) return w[((co * C + ci) * R + r) * S + s];
    return w[((r * S + s) * C + ci) * F + co];
}

/* One output element y[n, oh, ow, co] straight from the definition above. */
static double conv_point(const double* x, int64_t H, int64_t W, int64_t C,
                         const double* w, int fcrs, int64_t R, int64_t S,
                         int64_t F, int64_t sh, int64_t sw, int64_t ph,
                         int64_t pw, int64_t n, int64_t oh, int64_t ow,
                         int64_t co) {
    double acc = 0.0;
    for (int64_t r = 0; r < R; ++r) {
        const int64_t ih = oh * sh - ph + r;
        for (int64_t s = 0; s < S; ++s) {
            const int64_t iw = ow * sw - pw + s;
            for (int64_t ci = 0; ci < C; ++ci) {
                double xv = 0.0;
                if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                    xv = x[((n * H + ih) * W + iw) * C + ci];
                acc += xv * filter_tap(w, fcrs, R, S, C, F, r, s, ci, co);
            }
        }
    }
    return acc;
}

int64_t oracle_out_size(int64_t in, int64_t k, int64_t stride, int64_t pad) {
    if (stride <= 0) return -1;
    const int64_t span = in + 2 * pad - k;
    if (span < 0) return 0;
    return span / stride + 1;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Full forward convolution.  x: [N,H,W,C]; w: RSCF or FCRS; y: [N,Ho,Wo,F];
 * src: NULL or [N,Ho,Wo,F].  All arrays are float64, caller-owned.
 * Returns 0, or -1 when the arguments do not describe a valid convolution.
 */
int oracle_conv2d_f64(const double* x, int64_t N, int64_t H, int64_t W,
                      int64_t C, const double* w, int fcrs, int64_t R,
                      int64_t S, int64_t F, int64_t sh, int64_t sw,
                      int64_t ph, int64_t pw, const double* src, double beta,
                      double* y, int64_t Ho, int64_t Wo) {
    if (N < 0 || H < 0 || W < 0 || C < 0 || R <= 0 || S <= 0 || F < 0 ||
        ph < 0 || pw < 0)
        return -1;
    if (Ho != oracle_out_size(H, R, sh, ph) || Wo != oracle_out_size(W, S, sw, pw))
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t oh = 0; oh < Ho; ++oh) {
            for (int64_t ow = 0; ow < Wo; ++ow) {
                for (int64_t co = 0; co < F; ++co) {
                    const int64_t o = ((n * Ho + oh) * Wo + ow) * F + co;
                    double v = conv_point(x, H, W, C, w, fcrs, R, S, F, sh, sw,
                                          ph, pw, n, oh, ow, co);
                    if (src) v = v + beta * src[o];
                    y[o] = v;
                }
            }
        }
    }
    return 0;
}

/*
 * The same definition evaluated only at chosen output pixels.  pix[i] is a
 * flattened output pixel index m = (n*Ho + oh)*Wo + ow; y receives, row by
 * row, all F channels of each chosen pixel: y[i*F + co].  src, when not
 * NULL, is the full [N,Ho,Wo,F] residual source.
 */
int oracle_conv2d_points_f64(const double* x, int64_t N, int64_t H, int64_t W,
                             int64_t C, const double* w, int fcrs, int64_t R,
                             int64_t S, int64_t F, int64_t sh, int64_t sw,
                             int64_t ph, int64_t pw, const double* src,
                             double beta, const int64_t* pix, int64_t npix,
                             double* y, int64_t Ho, int64_t Wo) {
    if (N < 0 || H < 0 || W < 0 || C < 0 || R <= 0 || S <= 0 || F < 0 ||
        ph < 0 || pw < 0)
        return -1;
    if (Ho != oracle_out_size(H, R, sh, ph) || Wo != oracle_out_size(W, S, sw, pw))
        return -1;
    for (int64_t i = 0; i < npix; ++i)
        if (pix[i] < 0 || pix[i] >= N * Ho * Wo) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npix; ++i) {
        const int64_t m = pix[i];
        const int64_t ow = m % Wo;
        const int64_t oh = (m / Wo) % Ho;
        const int64_t n = m / (Wo * Ho);
        for (int64_t co = 0; co < F; ++co) {
            double v = conv_point(x, H, W, C, w, fcrs, R, S, F, sh, sw, ph, pw,
                                  n, oh, ow, co);
            if (src) v = v + beta * src[m * F + co];
            y[i * F + co] = v;
        }
    }
    return 0;
}

/*
 * The general forward convolution: per-axis stride (sh, sw), dilation
 * (dh, dw), padding before (pt, pl) and after (pb, pr) each spatial axis,
 * and `groups` channel groups.  The parameters are the ones page
 * "dispatch_amd_4wave_conv2d" (Args: stride, dilation, symmetric_padding,
 * num_groups) lists and its dispatcher restricts; their meaning is the
 * standard one (this oracle's reading, as in every deep-learning framework):
 *
 *   y[n,oh,ow,co] = sum_{r<R} sum_{s<S} sum_{c<Cg}
 *                     X(n, oh*sh - pt + r*dh, ow*sw - pl + s*dw, g*Cg + c)
 *                     * Wt(r, s, c, co),     g = co / (F / groups)
 *
 *   Cg = C / groups input channels per group (the filter's C_in), F output
 *   channels in all, F / groups per group; X as in oracle_conv2d_f64 (zero
 *   outside the image); Wt(r,s,c,co) = w[((r*S + s)*Cg + c)*F + co] (RSCF)
 *   or w[((co*Cg + c)*R + r)*S + s] (FCRS);
 *   Ho = floor((H + pt + pb - dh*(R - 1) - 1) / sh) + 1, likewise Wo.
 *
 * With pt = pb = ph, pl = pr = pw, unit dilation and one group this is
 * exactly oracle_conv2d_f64.  Each element is one straight (r, s, c) loop
 * accumulating in double; OpenMP over (n, oh) rows only.
 * Returns 0, or -1 for arguments that describe no convolution.
 */
int64_t oracle_out_size_general(int64_t in, int64_t k, int64_t stride, int64_t dil,
                                int64_t pad_before, int64_t pad_after) {
    if (stride <= 0 || dil <= 0 || k <= 0) return -1;
    const int64_t span = in + pad_before + pad_after - dil * (k - 1) - 1;
    if (span < 0) return 0;
    return span / stride + 1;
}

int oracle_conv2d_general_f64(const double* x, int64_t N, int64_t H, int64_t W,
                              int64_t C, const double* w, int fcrs, int64_t R,
                              int64_t S, int64_t Cg, int64_t F, int64_t sh,
                              int64_t sw, int64_t dh, int64_t dw, int64_t pt,
                              int64_t pb, int64_t pl, int64_t pr, int64_t groups,
                              const double* src, double beta, double* y,
                              int64_t Ho, int64_t Wo) {
    if (N < 0 || H < 0 || W < 0 || C < 0 || R <= 0 || S <= 0 || F < 0 ||
        pt < 0 || pb < 0 || pl < 0 || pr < 0 || groups <= 0)
        return -1;
    if (C != Cg * groups || F % groups != 0) return -1;
    if (Ho != oracle_out_size_general(H, R, sh, dh, pt, pb) ||
        Wo != oracle_out_size_general(W, S, sw, dw, pl, pr))
        return -1;
    const int64_t Fg = groups ? F / groups : 0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t oh = 0; oh < Ho; ++oh) {
            for (int64_t ow = 0; ow < Wo; ++ow) {
                for (int64_t co = 0; co < F; ++co) {
                    const int64_t g = co / Fg;
                    double acc = 0.0;
                    for (int64_t r = 0; r < R; ++r) {
                        const int64_t ih = oh * sh - pt + r * dh;
                        for (int64_t s = 0; s < S; ++s) {
                            const int64_t iw = ow * sw - pl + s * dw;
                            for (int64_t c = 0; c < Cg; ++c) {
                                double xv = 0.0;
                                if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                                    xv = x[((n * H + ih) * W + iw) * C + g * Cg + c];
                                acc += xv * filter_tap(w, fcrs, R, S, Cg, F, r, s, c, co);
                            }
                        }
                    }
                    const int64_t o = ((n * Ho + oh) * Wo + ow) * F + co;
                    if (src) acc = acc + beta * src[o];
                    y[o] = acc;
                }
            }
        }
    }
    return 0;
}


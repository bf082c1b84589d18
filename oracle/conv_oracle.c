/*
 * CPU oracle for the fused 2-D convolution layer and its two pools.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct reference
 * that the GPU library is checked against. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it. It shares no code,
 * header, table or constant with the GPU library and includes none of its
 * files.
 *
 * What it computes (all in one canonical layout: x [N][Cin][H][W],
 * w [Cout][Cin][kh][kw], y [N][Cout][OH][OW]; the Python wrapper permutes
 * channel-last tensors into it and back):
 *
 *   Convolution. The layer of the inferencelayer page (src/rtdetr_gpu.rs,
 *   `conv()` with the `IM2COL_SRC` gather and the bias+activation GEMM
 *   epilogue) and of the framecast page (package/rt.js, `wgslConv`) is a
 *   cross-correlation with zero padding: each output sums, over input channel
 *   ci and kernel tap (ky, kx), the product of the weight with the input pixel
 *   at row oh*stride+ky-pad and column ow*stride+kx-pad, taking the input as
 *   0 outside the image. No kernel flip. The output size is
 *   floor((H + 2*pad - kh)/stride) + 1 (inferencelayer `conv()`).
 *   Lowering this sum to im2col + GEMM, as the pages do, reorders the
 *   additions only, so the oracle is the definition itself, evaluated in fp64
 *   with a fixed loop order (ci, then ky, then kx).
 *
 *   Epilogue. bias[co] is added (absent bias = 0). The activation is one of
 *   none, ReLU max(v,0), SiLU v/(1+exp(-v)) (rlx-wgpu `apply_activation_host`;
 *   inferencelayer `ADDACT_SRC`), or per-channel PReLU v>=0 ? v : alpha[co]*v
 *   (framecast `wgslConv`). A residual r is added either before the
 *   activation (inferencelayer `encoder_maps`: the block sum goes through
 *   `addact(..., relu)`) or after it (framecast `wgslConv`: the residual joins
 *   the PReLU output), chosen by the RES_BEFORE_ACT flag.
 *
 *   Max pool 3x3, stride 2, pad 1 (inferencelayer `MAXPOOL_SRC`): the largest
 *   of the in-range taps; out-of-range taps are skipped, which is the same as
 *   padding with -infinity. Output size floor((H - 1)/2) + 1.
 *
 *   Transposed convolution 4x4, stride 2, pad 1 (framecast `wgslDeconv`): see
 *   oracle_conv_transpose4x4s2_nchw at the end of this file.
 *
 *   Average pool 2x2, stride 2, pad 0 (inferencelayer `AVGPOOL_SRC`): the sum
 *   ((x00 + x01) + x10) + x11 in single precision, in exactly that order, then
 *   times 0.25 in single precision. Output size floor(H/2); an odd last row or
 *   column is dropped.
 *
 * Built with -O2 -ffp-contract=off and no fast-math, so no multiply-add is
 * contracted and every operation rounds as written. Each output is computed by
 * one thread in a fixed order, so the result does not depend on the thread
 * count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_SILU 2
#define ORACLE_ACT_PRELU 3
#define ORACLE_RES_BEFORE_ACT 0x100

static int threads_to_use(int requested) {
#ifdef _OPENMP
    return requested > 0 ? requested : omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}

/* Number of threads a call with nthreads = 0 uses. */
int oracle_threads(void) { return threads_to_use(0); }

int oracle_out_dim(int in, int k, int stride, int pad) {
    if (in <= 0 || k <= 0 || stride <= 0 || pad < 0) return -1;
    int span = in + 2 * pad - k;
    if (span < 0) return -1;
    return span / stride + 1;
}

/* ReLU / SiLU / PReLU, in double precision. */
static double oracle_activation(int act, double v, double alpha) {
    switch (act) {
    case ORACLE_ACT_RELU:
        return v > 0.0 ? v : 0.0;
    case ORACLE_ACT_SILU:
        return v / (1.0 + exp(-v));
    case ORACLE_ACT_PRELU:
        return v >= 0.0 ? v : alpha * v;
    default:
        return v;
    }
}

/* One output of the layer: the tap sum, then bias, residual and activation. */
static double oracle_conv_point(const double *x, const double *w, const double *bias,
                                const double *alpha, const double *res, int H, int W,
                                int Cin, int Cout, int kh, int kw, int stride, int pad,
                                int OH, int OW, int act_flags, int n, int co, int oh,
                                int ow) {
    double acc = 0.0;
    for (int ci = 0; ci < Cin; ++ci) {
        const double *xc = x + ((size_t)n * Cin + ci) * (size_t)H * W;
        const double *wc = w + ((size_t)co * Cin + ci) * (size_t)kh * kw;
        for (int ky = 0; ky < kh; ++ky) {
            int iy = oh * stride + ky - pad;
            if (iy < 0 || iy >= H) continue;
            for (int kx = 0; kx < kw; ++kx) {
                int ix = ow * stride + kx - pad;
                if (ix < 0 || ix >= W) continue;
                acc += xc[(size_t)iy * W + ix] * wc[ky * kw + kx];
            }
        }
    }
    double v = acc + (bias ? bias[co] : 0.0);
    int act = act_flags & 0xff;
    double a = alpha ? alpha[co] : 0.0;
    if (res) {
        double r = res[(((size_t)n * Cout + co) * OH + oh) * OW + ow];
        if (act_flags & ORACLE_RES_BEFORE_ACT) {
            v = oracle_activation(act, v + r, a);
        } else {
            v = oracle_activation(act, v, a) + r;
        }
    } else {
        v = oracle_activation(act, v, a);
    }
    return v;
}

static int oracle_conv_check(int N, int H, int W, int Cin, int Cout, int kh, int kw,
                             int stride, int pad, int act_flags, const double *alpha,
                             int *OH, int *OW) {
    if (N <= 0 || H <= 0 || W <= 0 || Cin <= 0 || Cout <= 0) return -1;
    if (kh <= 0 || kw <= 0 || stride <= 0 || pad < 0) return -1;
    int act = act_flags & 0xff;
    if (act > ORACLE_ACT_PRELU || (act_flags & ~(0xff | ORACLE_RES_BEFORE_ACT))) return -1;
    if (act == ORACLE_ACT_PRELU && !alpha) return -1;
    *OH = oracle_out_dim(H, kh, stride, pad);
    *OW = oracle_out_dim(W, kw, stride, pad);
    if (*OH < 1 || *OW < 1) return -1;
    return 0;
}

/*
 * Full layer. x [N][Cin][H][W], w [Cout][Cin][kh][kw], bias/alpha [Cout] or
 * NULL, res [N][Cout][OH][OW] or NULL, y [N][Cout][OH][OW]. Returns 0, or -1
 * on invalid arguments.
 */
int oracle_conv2d_nchw(const double *x, const double *w, const double *bias,
                       const double *alpha, const double *res, double *y, int N, int H,
                       int W, int Cin, int Cout, int kh, int kw, int stride, int pad,
                       int act_flags, int nthreads) {
    int OH, OW;
    if (oracle_conv_check(N, H, W, Cin, Cout, kh, kw, stride, pad, act_flags, alpha, &OH,
                          &OW))
        return -1;
    long rows = (long)N * Cout * OH;
#pragma omp parallel for schedule(dynamic, 4) num_threads(threads_to_use(nthreads))
    for (long r = 0; r < rows; ++r) {
        int oh = (int)(r % OH);
        int co = (int)((r / OH) % Cout);
        int n = (int)(r / ((long)OH * Cout));
        double *yrow = y + (size_t)r * OW;
        for (int ow = 0; ow < OW; ++ow)
            yrow[ow] = oracle_conv_point(x, w, bias, alpha, res, H, W, Cin, Cout, kh, kw,
                                         stride, pad, OH, OW, act_flags, n, co, oh, ow);
    }
    return 0;
}

/*
 * Selected outputs only: idx holds npts quadruples (n, co, oh, ow); out[i]
 * receives the layer's value there. For checking full-size layers on samples.
 */
int oracle_conv2d_points_nchw(const double *x, const double *w, const double *bias,
                              const double *alpha, const double *res, const int64_t *idx,
                              int64_t npts, double *out, int N, int H, int W, int Cin,
                              int Cout, int kh, int kw, int stride, int pad, int act_flags,
                              int nthreads) {
    int OH, OW;
    if (oracle_conv_check(N, H, W, Cin, Cout, kh, kw, stride, pad, act_flags, alpha, &OH,
                          &OW))
        return -1;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t *q = idx + 4 * i;
        if (q[0] < 0 || q[0] >= N || q[1] < 0 || q[1] >= Cout || q[2] < 0 || q[2] >= OH ||
            q[3] < 0 || q[3] >= OW)
            return -1;
    }
#pragma omp parallel for schedule(dynamic, 16) num_threads(threads_to_use(nthreads))
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t *q = idx + 4 * i;
        out[i] = oracle_conv_point(x, w, bias, alpha, res, H, W, Cin, Cout, kh, kw, stride,
                                   pad, OH, OW, act_flags, (int)q[0], (int)q[1], (int)q[2],
                                   (int)q[3]);
    }
    return 0;
}

/* Max pool 3x3 s2 p1 over [N][C][H][W]; y [N][C][OH][OW], OH = (H-1)/2 + 1. */
int oracle_maxpool3x3s2_nchw(const double *x, double *y, int N, int C, int H, int W,
                             int nthreads) {
    if (N <= 0 || C <= 0 || H <= 0 || W <= 0) return -1;
    int OH = oracle_out_dim(H, 3, 2, 1), OW = oracle_out_dim(W, 3, 2, 1);
    long planes = (long)N * C;
#pragma omp parallel for schedule(static) num_threads(threads_to_use(nthreads))
    for (long p = 0; p < planes; ++p) {
        const double *xp = x + (size_t)p * H * W;
        double *yp = y + (size_t)p * OH * OW;
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow) {
                double best = -INFINITY;
                for (int dy = 0; dy < 3; ++dy) {
                    int iy = 2 * oh + dy - 1;
                    if (iy < 0 || iy >= H) continue;
                    for (int dx = 0; dx < 3; ++dx) {
                        int ix = 2 * ow + dx - 1;
                        if (ix < 0 || ix >= W) continue;
                        double v = xp[(size_t)iy * W + ix];
                        if (v > best) best = v;
                    }
                }
                yp[(size_t)oh * OW + ow] = best;
            }
    }
    return 0;
}

/*
 * Average pool 2x2 s2 over [N][C][H][W] single-precision values (the storage
 * values, widened exactly); y [N][C][H/2][W/2] in single precision, before the
 * final rounding to the storage type.
 */
int oracle_avgpool2x2_nchw(const float *x, float *y, int N, int C, int H, int W,
                           int nthreads) {
    if (N <= 0 || C <= 0 || H < 2 || W < 2) return -1;
    int OH = H / 2, OW = W / 2;
    long planes = (long)N * C;
#pragma omp parallel for schedule(static) num_threads(threads_to_use(nthreads))
    for (long p = 0; p < planes; ++p) {
        const float *xp = x + (size_t)p * H * W;
        float *yp = y + (size_t)p * OH * OW;
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow) {
                const float *t = xp + (size_t)(2 * oh) * W + 2 * ow;
                float s = t[0] + t[1];
                s = s + t[W];
                s = s + t[W + 1];
                yp[(size_t)oh * OW + ow] = s * 0.25f;
            }
    }
    return 0;
}

/*
 * Transposed convolution, 4x4 kernel, stride 2, pad 1 (framecast `wgslDeconv`,
 * the ConvTranspose2d that ends an IFNet block): x [N][Cin][H][W], weight
 * [Cin][Cout][4][4] (the transposed conv's own layout), y [N][Cout][2H][2W].
 * Input pixel (iy, ix) with tap (ky, kx) lands on output row 2*iy - 1 + ky and
 * column 2*ix - 1 + kx; written as a gather, output (oy, ox) takes the taps whose
 * oy + 1 - ky and ox + 1 - kx are even and halve to an in-range input pixel. The
 * sum runs over ci, then ky, then kx in fp64; then bias and the activation.
 */
int oracle_conv_transpose4x4s2_nchw(const double *x, const double *w, const double *bias,
                                    const double *alpha, double *y, int N, int H, int W,
                                    int Cin, int Cout, int act, int nthreads) {
    if (N <= 0 || H <= 0 || W <= 0 || Cin <= 0 || Cout <= 0) return -1;
    const int OH = 2 * H, OW = 2 * W;
    long rows = (long)N * Cout * OH;
#pragma omp parallel for schedule(static) num_threads(threads_to_use(nthreads))
    for (long r = 0; r < rows; ++r) {
        const int oy = (int)(r % OH);
        const int co = (int)((r / OH) % Cout);
        const int n = (int)(r / ((long)OH * Cout));
        for (int ox = 0; ox < OW; ++ox) {
            double acc = 0.0;
            for (int ci = 0; ci < Cin; ++ci) {
                const double *xc = x + ((size_t)n * Cin + ci) * (size_t)H * W;
                const double *wc = w + ((size_t)ci * Cout + co) * 16;
                for (int ky = 0; ky < 4; ++ky) {
                    const int ty = oy + 1 - ky;
                    if (ty < 0 || (ty % 2) != 0 || ty / 2 >= H) continue;
                    for (int kx = 0; kx < 4; ++kx) {
                        const int tx = ox + 1 - kx;
                        if (tx < 0 || (tx % 2) != 0 || tx / 2 >= W) continue;
                        acc += xc[(size_t)(ty / 2) * W + tx / 2] * wc[ky * 4 + kx];
                    }
                }
            }
            const double v = acc + (bias ? bias[co] : 0.0);
            y[(((size_t)n * Cout + co) * OH + oy) * OW + ox] =
                oracle_activation(act & 0xff, v, alpha ? alpha[co] : 0.0);
        }
    }
    return 0;
}

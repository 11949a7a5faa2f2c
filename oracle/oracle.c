/*
 * CPU oracle for the pool_stencil operations -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (the HIP library) never calls it and
 * shares no code with it.
 *
 * Every function computes the plain definition of its operation, in the
 * order the problem statement writes it, in double precision, with no
 * blocking, reordering or fusion:
 *
 *   - Conv2d is the cross-correlation sum over input channels and kernel taps
 *     plus the conv bias, with zero padding.
 *   - The fused conv op applies tanh, then the scale, then the per-channel
 *     bias to EVERY conv output, and only then takes the max-pool.  (The GPU
 *     kernel pools first; this oracle deliberately does not.)
 *   - MaxPool2d takes the max over each window, positions outside the image
 *     count as -infinity, floor mode.
 *   - ConvTranspose2d is written in scatter form: every input pixel adds
 *     x * w into the output position  o = i*stride - pad + k*dil.
 *   - The convT epilogue is softmax over channels (max subtracted), then
 *     + bias2, then * scale, then sigmoid 1/(1+exp(-v)).
 *
 * Sources (three POPCORNBENCH transcripts, cited by their page name):
 *   page Kimi-K2.6 l2_p82  -- Conv2d 8->64 k3 -> tanh -> *2 -> +bias -> MaxPool2d(4)
 *   page Kimi-K2.6 l1_p42  -- MaxPool2d k4 s1 p1 d1
 *   page Kimi-K2.6 l2_p91  -- ConvTranspose2d 64->128 k4 s2 p1 op1 -> softmax(dim 1)
 *                             -> +bias -> *2 -> sigmoid
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared oracle.c -lm
 * (-ffp-contract=off keeps every multiply and add separately rounded.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(a, b, c, d, B, C, D) ((((int64_t)(a) * (B) + (b)) * (C) + (c)) * (D) + (d))

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Output extent of a sliding window (Conv2d / MaxPool2d, floor mode):
 * floor((in + 2p - d(k-1) - 1)/s) + 1.  The l2_p82 page derives 256 -> 254
 * for the k3 conv and 254 -> 63 for the k4 pool; the l1_p42 page derives
 * 512 -> 511 for k4 s1 p1 d1 (problem analysis at the top of each page).
 * Returns <= 0 when the window does not fit. */
int or_window_out_dim(int in, int k, int s, int p, int d) {
    int64_t num = (int64_t)in + 2 * (int64_t)p - (int64_t)d * (k - 1) - 1;
    if (num < 0) return 0;
    return (int)(num / s + 1);
}

/* ConvTranspose2d output extent: (in-1)s - 2p + d(k-1) + op + 1.
 * The l2_p91 page derives 64 -> 129 for k4 s2 p1 op1 (shape analysis). */
int or_convT_out_dim(int in, int k, int s, int p, int op, int d) {
    return (int)(((int64_t)in - 1) * s - 2 * (int64_t)p + (int64_t)d * (k - 1) + op + 1);
}

/* Conv2d, cross-correlation (no kernel flip), zero padding, optional bias.
 * x [N,Cin,H,W], w [Cout,Cin,kH,kW], bias [Cout] or NULL -> y [N,Cout,OH,OW] (double).
 * l2_p82 page: the model is nn.Conv2d(8, 64, 3) with default stride 1,
 * padding 0 and bias on (problem analysis). */
void or_conv2d(const float *x, const float *w, const float *bias, double *y,
               int N, int Cin, int H, int W, int Cout, int kH, int kW,
               int s, int p, int d) {
    int OH = or_window_out_dim(H, kH, s, p, d);
    int OW = or_window_out_dim(W, kW, s, p, d);
    if (OH <= 0 || OW <= 0) return;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; n++)
        for (int co = 0; co < Cout; co++)
            for (int oh = 0; oh < OH; oh++)
                for (int ow = 0; ow < OW; ow++) {
                    double acc = 0.0;
                    for (int ci = 0; ci < Cin; ci++)
                        for (int kh = 0; kh < kH; kh++)
                            for (int kw = 0; kw < kW; kw++) {
                                int ih = oh * s - p + kh * d;
                                int iw = ow * s - p + kw * d;
                                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                                acc += (double)x[IDX4(n, ci, ih, iw, Cin, H, W)] *
                                       (double)w[IDX4(co, ci, kh, kw, Cin, kH, kW)];
                            }
                    if (bias) acc += (double)bias[co];
                    y[IDX4(n, co, oh, ow, Cout, OH, OW)] = acc;
                }
}

/* MaxPool2d on double data: out = max over the k x k window (stride s,
 * dilation d), positions outside the image act as -infinity, floor mode.
 * l1_p42 page: PyTorch's padding for max pooling is implicit negative
 * infinity (the passage quoting the documentation), so a window that lies
 * entirely in the padding yields -inf. */
void or_maxpool2d_f64(const double *x, double *y, int N, int C, int H, int W,
                      int k, int s, int p, int d) {
    int OH = or_window_out_dim(H, k, s, p, d);
    int OW = or_window_out_dim(W, k, s, p, d);
    if (OH <= 0 || OW <= 0) return;
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; n++)
        for (int c = 0; c < C; c++)
            for (int oh = 0; oh < OH; oh++)
                for (int ow = 0; ow < OW; ow++) {
                    double m = -INFINITY;
                    for (int kh = 0; kh < k; kh++)
                        for (int kw = 0; kw < k; kw++) {
                            int ih = oh * s - p + kh * d;
                            int iw = ow * s - p + kw * d;
                            double v = (ih < 0 || ih >= H || iw < 0 || iw >= W)
                                           ? -INFINITY
                                           : x[IDX4(n, c, ih, iw, C, H, W)];
                            if (v > m) m = v;
                        }
                    y[IDX4(n, c, oh, ow, C, OH, OW)] = m;
                }
}

/* The same definition on float data (the max of floats is exact, so the
 * result is a float of the input).  Used for the standalone pool. */
void or_maxpool2d_f32(const float *x, float *y, int N, int C, int H, int W,
                      int k, int s, int p, int d) {
    int OH = or_window_out_dim(H, k, s, p, d);
    int OW = or_window_out_dim(W, k, s, p, d);
    if (OH <= 0 || OW <= 0) return;
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; n++)
        for (int c = 0; c < C; c++)
            for (int oh = 0; oh < OH; oh++)
                for (int ow = 0; ow < OW; ow++) {
                    float m = -INFINITY;
                    for (int kh = 0; kh < k; kh++)
                        for (int kw = 0; kw < k; kw++) {
                            int ih = oh * s - p + kh * d;
                            int iw = ow * s - p + kw * d;
                            float v = (ih < 0 || ih >= H || iw < 0 || iw >= W)
                                          ? -INFINITY
                                          : x[IDX4(n, c, ih, iw, C, H, W)];
                            if (v > m) m = v;
                        }
                    y[IDX4(n, c, oh, ow, C, OH, OW)] = m;
                }
}

/* Fused op, in the written order of the l2_p82 page's model:
 *   y = conv2d(x) + conv_bias;  z = tanh(y) * scale + bias2[c];  out = maxpool(z).
 * Every conv output is transformed before the pool; no reordering. */
void or_conv_tanh_scale_bias_maxpool(const float *x, const float *w, const float *conv_bias,
                                     const float *bias2, double *out,
                                     int N, int Cin, int H, int W, int Cout, int kH, int kW,
                                     int cs, int cp, int cd, double scale,
                                     int pk, int ps, int pp, int pd) {
    int OH = or_window_out_dim(H, kH, cs, cp, cd);
    int OW = or_window_out_dim(W, kW, cs, cp, cd);
    if (OH <= 0 || OW <= 0) return;
    double *z = (double *)malloc(sizeof(double) * (size_t)N * Cout * OH * OW);
    if (!z) return;
    or_conv2d(x, w, conv_bias, z, N, Cin, H, W, Cout, kH, kW, cs, cp, cd);
    int64_t total = (int64_t)N * Cout * OH * OW;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; i++) {
        int c = (int)((i / ((int64_t)OH * OW)) % Cout);
        double t = tanh(z[i]);
        t = t * scale;
        t = t + (double)bias2[c];
        z[i] = t;
    }
    or_maxpool2d_f64(z, out, N, Cout, OH, OW, pk, ps, pp, pd);
    free(z);
}

/* The same fused definition evaluated at selected pooled outputs only.
 * idx[i] is the flat NCHW index into the pooled output [N,Cout,PH,PW].
 * For each, every conv output of its window is computed from the conv sum,
 * transformed (tanh, scale, bias2) and the max taken -- the same arithmetic
 * as or_conv_tanh_scale_bias_maxpool, restricted to one output. */
void or_conv_tanh_scale_bias_maxpool_points(const float *x, const float *w,
                                            const float *conv_bias, const float *bias2,
                                            int N, int Cin, int H, int W, int Cout, int kH,
                                            int kW, int cs, int cp, int cd, double scale,
                                            int pk, int ps, int pp, int pd,
                                            int64_t npts, const int64_t *idx, double *out) {
    int OH = or_window_out_dim(H, kH, cs, cp, cd);
    int OW = or_window_out_dim(W, kW, cs, cp, cd);
    int PH = or_window_out_dim(OH, pk, ps, pp, pd);
    int PW = or_window_out_dim(OW, pk, ps, pp, pd);
    (void)N;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < npts; t++) {
        int64_t q = idx[t];
        int pw = (int)(q % PW);
        int ph = (int)((q / PW) % PH);
        int co = (int)((q / ((int64_t)PW * PH)) % Cout);
        int n = (int)(q / ((int64_t)PW * PH * Cout));
        double m = -INFINITY;
        for (int a = 0; a < pk; a++)
            for (int b = 0; b < pk; b++) {
                int oh = ph * ps - pp + a * pd;
                int ow = pw * ps - pp + b * pd;
                double v;
                if (oh < 0 || oh >= OH || ow < 0 || ow >= OW) {
                    v = -INFINITY;
                } else {
                    double acc = 0.0;
                    for (int ci = 0; ci < Cin; ci++)
                        for (int kh = 0; kh < kH; kh++)
                            for (int kw = 0; kw < kW; kw++) {
                                int ih = oh * cs - cp + kh * cd;
                                int iw = ow * cs - cp + kw * cd;
                                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                                acc += (double)x[IDX4(n, ci, ih, iw, Cin, H, W)] *
                                       (double)w[IDX4(co, ci, kh, kw, Cin, kH, kW)];
                            }
                    if (conv_bias) acc += (double)conv_bias[co];
                    v = tanh(acc) * scale + (double)bias2[co];
                }
                if (v > m) m = v;
            }
        out[t] = m;
    }
}

/* Second stage of the l2_p82 page's unfused pipeline, on a stored conv output
 * y [N,C,H,W] (float): z = tanh(y) * scale + bias2[c] for every element, then
 * the max-pool (floor mode, -inf padding).  Written order, no reordering. */
void or_tanh_scale_bias_maxpool(const float *y, const float *bias2, double *out,
                                int N, int C, int H, int W, double scale,
                                int k, int s, int p, int d) {
    int64_t total = (int64_t)N * C * H * W;
    double *z = (double *)malloc(sizeof(double) * (size_t)total);
    if (!z) return;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; i++) {
        int c = (int)((i / ((int64_t)H * W)) % C);
        double t = tanh((double)y[i]);
        t = t * scale;
        t = t + (double)bias2[c];
        z[i] = t;
    }
    or_maxpool2d_f64(z, out, N, C, H, W, k, s, p, d);
    free(z);
}

/* ConvTranspose2d in scatter form: for every input pixel (n, ci, ih, iw) and
 * every tap (kh, kw), the product x[n,ci,ih,iw] * w[ci,co,kh,kw] is added to
 * out[n,co,oh,ow] with oh = ih*s - p + kh*d, ow = iw*s - p + kw*d, when that
 * position lies inside the output.  Then the convT bias is added.
 * w is laid out [Cin, Cout, k, k] (l2_p91 page: the weight of
 * nn.ConvTranspose2d(64,128,4) is (64,128,4,4); the index relation
 * o = i*stride + k - padding is the page's straightforward scatter loop).
 * Parallel over (n, co) so no two threads add into the same output. */
void or_conv_transpose2d(const float *x, const float *w, const float *bias, double *y,
                         int N, int Cin, int H, int W, int Cout, int k, int s, int p,
                         int op, int d) {
    int OH = or_convT_out_dim(H, k, s, p, op, d);
    int OW = or_convT_out_dim(W, k, s, p, op, d);
    if (OH <= 0 || OW <= 0) return;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; n++)
        for (int co = 0; co < Cout; co++) {
            double *yo = y + IDX4(n, co, 0, 0, Cout, OH, OW);
            for (int64_t i = 0; i < (int64_t)OH * OW; i++) yo[i] = 0.0;
            for (int ci = 0; ci < Cin; ci++)
                for (int ih = 0; ih < H; ih++)
                    for (int iw = 0; iw < W; iw++) {
                        double xv = (double)x[IDX4(n, ci, ih, iw, Cin, H, W)];
                        for (int kh = 0; kh < k; kh++)
                            for (int kw = 0; kw < k; kw++) {
                                int oh = ih * s - p + kh * d;
                                int ow = iw * s - p + kw * d;
                                if (oh < 0 || oh >= OH || ow < 0 || ow >= OW) continue;
                                yo[(int64_t)oh * OW + ow] +=
                                    xv * (double)w[IDX4(ci, co, kh, kw, Cout, k, k)];
                            }
                    }
            if (bias)
                for (int64_t i = 0; i < (int64_t)OH * OW; i++) yo[i] += (double)bias[co];
        }
}

/* Channel softmax followed by the l2_p91 page's epilogue, in the model's
 * written order: softmax over dim 1 (the max over channels subtracted before
 * exp, the page's underflow discussion), + bias2[c], * scale, sigmoid
 * 1/(1+exp(-v)).  Operates in place on y [N,C,HW]. */
static void softmax_bias_scale_sigmoid_inplace(double *y, const float *bias2, double scale,
                                               int N, int C, int64_t HW) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; n++)
        for (int64_t q = 0; q < HW; q++) {
            double *v = y + (int64_t)n * C * HW + q;
            double m = -INFINITY;
            for (int c = 0; c < C; c++)
                if (v[c * HW] > m) m = v[c * HW];
            double sum = 0.0;
            for (int c = 0; c < C; c++) sum += exp(v[c * HW] - m);
            for (int c = 0; c < C; c++) {
                double sm = exp(v[c * HW] - m) / sum;
                double t = sm + (double)bias2[c];
                t = t * scale;
                v[c * HW] = 1.0 / (1.0 + exp(-t));
            }
        }
}

/* Second stage of the l2_p91 page's unfused pipeline, on a stored convT
 * output y [N,C,H,W] (float): the channel softmax and epilogue above. */
void or_softmax_bias_scale_sigmoid(const float *y, const float *bias2, double *out,
                                   int N, int C, int H, int W, double scale) {
    int64_t total = (int64_t)N * C * H * W;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; i++) out[i] = (double)y[i];
    softmax_bias_scale_sigmoid_inplace(out, bias2, scale, N, C, (int64_t)H * W);
}

void or_convT_softmax_bias_scale_sigmoid(const float *x, const float *w, const float *convT_bias,
                                         const float *bias2, double *out,
                                         int N, int Cin, int H, int W, int Cout, int k, int s,
                                         int p, int op, int d, double scale) {
    int OH = or_convT_out_dim(H, k, s, p, op, d);
    int OW = or_convT_out_dim(W, k, s, p, op, d);
    if (OH <= 0 || OW <= 0) return;
    or_conv_transpose2d(x, w, convT_bias, out, N, Cin, H, W, Cout, k, s, p, op, d);
    softmax_bias_scale_sigmoid_inplace(out, bias2, scale, N, Cout, (int64_t)OH * OW);
}

/* The same definition at selected output pixels.  pix[i] is the flat index
 * n*OH*OW + oh*OW + ow; out receives Cout values per pixel (channel-major
 * within the pixel: out[i*Cout + c]).  The convT value of each channel is
 * the scatter sum restricted to this output position: every (ih, kh) with
 * ih*s - p + kh*d == oh and every (iw, kw) likewise contribute. */
void or_convT_softmax_bias_scale_sigmoid_pixels(const float *x, const float *w,
                                                const float *convT_bias, const float *bias2,
                                                int N, int Cin, int H, int W, int Cout, int k,
                                                int s, int p, int op, int d, double scale,
                                                int64_t npix, const int64_t *pix, double *out) {
    int OH = or_convT_out_dim(H, k, s, p, op, d);
    int OW = or_convT_out_dim(W, k, s, p, op, d);
    (void)N;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < npix; t++) {
        int64_t q = pix[t];
        int ow = (int)(q % OW);
        int oh = (int)((q / OW) % OH);
        int n = (int)(q / ((int64_t)OW * OH));
        double *v = out + t * Cout;
        /* the (ih, kh) and (iw, kw) pairs that land on this output position */
        int rows_i[64], rows_k[64], cols_i[64], cols_k[64];
        int nr = 0, nc = 0;
        for (int ih = 0; ih < H; ih++)
            for (int kh = 0; kh < k; kh++)
                if (ih * s - p + kh * d == oh && nr < 64) { rows_i[nr] = ih; rows_k[nr] = kh; nr++; }
        for (int iw = 0; iw < W; iw++)
            for (int kw = 0; kw < k; kw++)
                if (iw * s - p + kw * d == ow && nc < 64) { cols_i[nc] = iw; cols_k[nc] = kw; nc++; }
        for (int co = 0; co < Cout; co++) {
            double acc = 0.0;
            for (int ci = 0; ci < Cin; ci++)
                for (int a = 0; a < nr; a++)
                    for (int b = 0; b < nc; b++)
                        acc += (double)x[IDX4(n, ci, rows_i[a], cols_i[b], Cin, H, W)] *
                               (double)w[IDX4(ci, co, rows_k[a], cols_k[b], Cout, k, k)];
            if (convT_bias) acc += (double)convT_bias[co];
            v[co] = acc;
        }
        double m = -INFINITY;
        for (int c = 0; c < Cout; c++)
            if (v[c] > m) m = v[c];
        double sum = 0.0;
        for (int c = 0; c < Cout; c++) sum += exp(v[c] - m);
        for (int c = 0; c < Cout; c++) {
            double sm = exp(v[c] - m) / sum;
            double u = (sm + (double)bias2[c]) * scale;
            v[c] = 1.0 / (1.0 + exp(-u));
        }
    }
}

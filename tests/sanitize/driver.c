/* Host-sanitizer driver (AddressSanitizer + UndefinedBehaviorSanitizer build):
 *  - the C ABI's shape queries over a grid of arguments, extremes included, checked
 *    against the oracle's extent functions;
 *  - every entry point's validation: NULL pointers, bad shapes and parameters,
 *    tensors past the size limits, misaligned pointers and the accepted arguments
 *    (which must reach the launcher stand-in; no pointer is ever dereferenced);
 *  - the oracle's loops on small tensors with padding, stride and dilation, so
 *    every index it forms is checked against its buffers.
 * Prints "sanitize ok" and exits 0 when every check holds. */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "pool_stencil.h"

extern int ps_stub_calls;
int or_window_out_dim(int in, int k, int s, int p, int d);
int or_convT_out_dim(int in, int k, int s, int p, int op, int d);
void or_conv2d(const float *x, const float *w, const float *bias, double *y, int N, int Cin, int H,
               int W, int Cout, int kH, int kW, int s, int p, int d);
void or_maxpool2d_f32(const float *x, float *y, int N, int C, int H, int W, int k, int s, int p,
                      int d);
void or_conv_tanh_scale_bias_maxpool(const float *x, const float *w, const float *conv_bias,
                                     const float *bias2, double *out, int N, int Cin, int H, int W,
                                     int Cout, int kH, int kW, int cs, int cp, int cd, double scale,
                                     int pk, int ps, int pp, int pd);
void or_conv_transpose2d(const float *x, const float *w, const float *bias, double *y, int N,
                         int Cin, int H, int W, int Cout, int k, int s, int p, int op, int d);
void or_convT_softmax_bias_scale_sigmoid(const float *x, const float *w, const float *convT_bias,
                                         const float *bias2, double *out, int N, int Cin, int H,
                                         int W, int Cout, int k, int s, int p, int op, int d,
                                         double scale);

static int failures = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            ++failures;                           \
            if (failures < 20) {                  \
                fprintf(stderr, "FAIL: " __VA_ARGS__); \
                fprintf(stderr, "\n");            \
            }                                     \
        }                                         \
    } while (0)

static float *rnd(size_t n, unsigned seed) {
    float *p = (float *)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) {
        seed = seed * 1664525u + 1013904223u;
        p[i] = (float)((seed >> 8) & 0xffff) / 32768.f - 1.f;
    }
    return p;
}

static void shape_queries(void) {
    const int ins[] = {1, 2, 3, 7, 31, 64, 255, 512, 100000, INT_MAX};
    for (unsigned a = 0; a < sizeof ins / sizeof ins[0]; ++a)
        for (int k = 1; k <= 6; ++k)
            for (int s = 1; s <= 4; ++s)
                for (int p = 0; p <= 4; ++p)
                    for (int d = 1; d <= 3; ++d) {
                        const int in = ins[a];
                        int o = -1;
                        const int st = ps_conv2d_out_dim(in, k, s, p, d, &o);
                        /* the extent in 64 bits; the oracle's int result where it fits */
                        const int64_t num = (int64_t)in + 2 * (int64_t)p - (int64_t)d * (k - 1) - 1;
                        const int64_t r64 = num < 0 ? 0 : num / s + 1;
                        if (r64 >= 1 && r64 <= INT_MAX) {
                            const int ref = or_window_out_dim(in, k, s, p, d);
                            CHECK(st == PS_OK && o == ref && ref == (int)r64, "conv dim %d %d %d %d %d", in, k, s, p, d);
                        } else {
                            CHECK(st == PS_ERR_SHAPE, "conv dim reject %d %d %d %d %d", in, k, s, p, d);
                        }
                        const int ref = (int)(r64 >= 1 && r64 <= INT_MAX ? r64 : 0);
                        o = -1;
                        const int sp = ps_pool2d_out_dim(in, k, s, p, d, &o);
                        if (sp == PS_OK) CHECK(o == ref, "pool dim %d %d %d %d %d", in, k, s, p, d);
                        for (int op = 0; op < 4; ++op) {
                            o = -1;
                            const int sc = ps_convT2d_out_dim(in, k, s, p, op, d, &o);
                            const int64_t r64 = ((int64_t)in - 1) * s - 2 * (int64_t)p +
                                                (int64_t)d * (k - 1) + op + 1;
                            if (sc == PS_OK) {
                                CHECK(r64 >= 1 && r64 <= INT_MAX && o == (int)r64,
                                      "convT dim %d %d %d %d %d %d", in, k, s, p, op, d);
                                CHECK(o == or_convT_out_dim(in, k, s, p, op, d), "convT oracle %d", in);
                            }
                            if (op >= (s > d ? s : d)) CHECK(sc != PS_OK, "convT op rule %d %d %d", op, s, d);
                        }
                    }
    /* extremes: no overflow, a status and no write on error */
    const int ext[] = {0, 1, -1, INT_MAX, INT_MIN, INT_MAX / 2};
    for (unsigned a = 0; a < 6; ++a)
        for (unsigned b = 0; b < 6; ++b)
            for (unsigned c = 0; c < 6; ++c) {
                int o = 12345;
                const int st = ps_conv2d_out_dim(ext[a], ext[b] == 0 ? 3 : ext[b], 1, ext[c] < 0 ? 0 : ext[c], 1, &o);
                if (st != PS_OK) CHECK(o == 12345, "conv dim wrote on error");
                o = 12345;
                const int st2 = ps_convT2d_out_dim(ext[a], 4, 2, ext[b] < 0 ? 0 : ext[b], 1, ext[c] < 1 ? 1 : ext[c] % 1000, &o);
                if (st2 != PS_OK) CHECK(o == 12345, "convT dim wrote on error");
            }
    CHECK(ps_conv2d_out_dim(5, 3, 1, 0, 1, NULL) == PS_ERR_NULL, "NULL out");
}

static void entry_points(void) {
    void *A = (void *)(uintptr_t)0x10000, *M = (void *)(uintptr_t)0x10002;
    const float *fA = (const float *)A;
    float *fy = (float *)A;
    int calls = ps_stub_calls;
#define EXPECT(expr, want) CHECK((expr) == (want), #expr " != " #want)
    /* fused conv */
    EXPECT(ps_conv_tanh_scale_bias_maxpool(NULL, A, NULL, fA, A, PS_F32, 2, 8, 32, 32, 16, 3, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), PS_ERR_NULL);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(A, A, NULL, fA, A, 7, 2, 8, 32, 32, 16, 3, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), PS_ERR_PARAM);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(A, A, NULL, fA, A, PS_F32, 0, 8, 32, 32, 16, 3, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), PS_ERR_SHAPE);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(A, A, NULL, fA, A, PS_F32, 2, 8, 32, 32, 16, 0, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), PS_ERR_PARAM);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(A, A, NULL, fA, A, PS_F32, 2, 8, 2, 2, 16, 3, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), PS_ERR_SHAPE);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(A, A, NULL, fA, A, PS_F32, INT_MAX, INT_MAX, 32, 32, 16, 3, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), PS_ERR_SHAPE);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(M, A, NULL, fA, A, PS_F32, 2, 8, 32, 32, 16, 3, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), PS_ERR_ALIGN);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(A, A, NULL, fA, A, PS_F32, 2, 8, 32, 32, 16, 3, 3, 1, 0, 1, 2.f, 4, 0, 0, 1, NULL), 77);
    EXPECT(ps_conv_tanh_scale_bias_maxpool(A, A, fA, fA, A, PS_BF16, 2, 70, 33, 41, 130, 5, 3, 2, 2, 2, -1.f, 3, 2, 1, 2, NULL), 77);
    /* conv2d */
    EXPECT(ps_conv2d(A, A, NULL, A, PS_F32, 2, 8, 32, 32, 16, 3, 3, 0, 0, 1, NULL), PS_ERR_PARAM);
    EXPECT(ps_conv2d(A, A, NULL, A, PS_F32, 2, 8, 32, 32, 16, 3, 3, 1, -1, 1, NULL), PS_ERR_PARAM);
    EXPECT(ps_conv2d(A, A, NULL, A, PS_F32, 2, 8, 32, 32, 16, 3, 3, 1, 0, 1, NULL), 77);
    /* max-pool */
    EXPECT(ps_maxpool2d(NULL, fy, 2, 3, 40, 50, 4, 1, 1, 1, NULL), PS_ERR_NULL);
    EXPECT(ps_maxpool2d(fA, fy, 2, 3, 40, 50, 0, 1, 1, 1, NULL), PS_ERR_PARAM);
    EXPECT(ps_maxpool2d(fA, fy, 2, 3, 40, 50, 4, 1, -1, 1, NULL), PS_ERR_PARAM);
    EXPECT(ps_maxpool2d(fA, fy, 2, 3, 2, 2, 4, 1, 0, 1, NULL), PS_ERR_SHAPE);
    EXPECT(ps_maxpool2d(fA, (float *)M, 2, 3, 40, 50, 4, 1, 1, 1, NULL), PS_ERR_ALIGN);
    EXPECT(ps_maxpool2d(fA, fy, 2, 3, 40, 50, 4, 1, 1, 1, NULL), 77);
    EXPECT(ps_maxpool2d(fA, fy, 2, 3, 40, 50, 3, -1, 1, 2, NULL), 77);
    EXPECT(ps_maxpool2d(fA, fy, 2, 3, 40, 50, 20, 3, 5, 1, NULL), 77);
    EXPECT(ps_maxpool2d(fA, fy, 1, 1, 8, 8, 3, 1 << 20, 1 << 30, 1, NULL), PS_ERR_UNSUPPORTED);
    /* transposed conv */
    EXPECT(ps_convT_softmax_bias_scale_sigmoid(fA, fA, NULL, NULL, fy, 2, 64, 8, 8, 128, 4, 2, 1, 1, 1, 2.f, NULL), PS_ERR_NULL);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid(fA, fA, NULL, fA, fy, 2, 64, 8, 8, 128, 3, 2, 1, 1, 1, 2.f, NULL), PS_ERR_UNSUPPORTED);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid(fA, fA, NULL, fA, fy, 2, 64, 8, 8, 128, 4, 2, 1, 2, 1, 2.f, NULL), PS_ERR_PARAM);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid(fA, fA, NULL, fA, fy, 2, 64, 8, 8, 272, 4, 2, 1, 1, 1, 2.f, NULL), PS_ERR_UNSUPPORTED);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid(fA, fA, NULL, fA, fy, 2, 64, 8, 8, 120, 4, 2, 1, 1, 1, 2.f, NULL), 77);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid(fA, fA, NULL, fA, fy, 2, 64, 8, 8, 128, 4, 2, 1, 1, 1, 2.f, NULL), 77);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid(fA, fA, NULL, fA, fy, 1, 4, 3, 3, 16, 4, 2, 3, 0, 1, 2.f, NULL), 77);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid_bf16(A, A, NULL, fA, A, 2, 64, 8, 8, 128, 4, 2, 1, 1, 1, 2.f, NULL), 77);
    EXPECT(ps_convT_softmax_bias_scale_sigmoid_bf16(A, A, NULL, fA, A, 2, 64, 8, 8, 96, 4, 2, 1, 1, 2, 2.f, NULL), PS_ERR_UNSUPPORTED);
    EXPECT(ps_convT2d(fA, fA, NULL, fy, 2, 64, 8, 8, 128, 4, 2, 1, 1, 1, NULL), 77);
    EXPECT(ps_convT2d(fA, fA, NULL, (float *)M, 2, 64, 8, 8, 128, 4, 2, 1, 1, 1, NULL), PS_ERR_ALIGN);
    /* post-processing stages */
    EXPECT(ps_tanh_scale_bias_maxpool(A, fA, A, PS_F32, 2, 64, 30, 30, 2.f, 4, 0, 0, 1, NULL), 77);
    EXPECT(ps_tanh_scale_bias_maxpool(A, fA, A, PS_F32, 2, 64, 30, 30, 2.f, 0, 0, 0, 1, NULL), PS_ERR_PARAM);
    EXPECT(ps_softmax_bias_scale_sigmoid(fA, fA, fy, 2, 128, 9, 9, 2.f, NULL), 77);
    EXPECT(ps_softmax_bias_scale_sigmoid(fA, NULL, fy, 2, 128, 9, 9, 2.f, NULL), PS_ERR_NULL);
#undef EXPECT
    CHECK(ps_stub_calls - calls == 13, "accepted calls reaching a launcher: %d", ps_stub_calls - calls);
    for (int st = -1; st <= 8; ++st) CHECK(ps_status_string(st) != NULL, "status string %d", st);
}

static int all_finite(const double *v, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(v[i]) && !isinf(v[i])) return 0;
    return 1;
}

static void oracle_loops(void) {
    const int cfg[][9] = {/* N Cin H W Cout kH kW s p ... d */
                          {2, 3, 9, 11, 5, 3, 3, 1, 0},
                          {1, 4, 12, 7, 3, 3, 2, 2, 1},
                          {2, 2, 10, 10, 4, 5, 3, 3, 2},
                          {1, 1, 1, 1, 1, 1, 1, 1, 0}};
    for (int c = 0; c < 4; ++c)
        for (int d = 1; d <= 2; ++d) {
            const int N = cfg[c][0], Cin = cfg[c][1], H = cfg[c][2], W = cfg[c][3], Co = cfg[c][4];
            const int kH = cfg[c][5], kW = cfg[c][6], s = cfg[c][7], p = cfg[c][8];
            const int OH = or_window_out_dim(H, kH, s, p, d), OW = or_window_out_dim(W, kW, s, p, d);
            if (OH < 1 || OW < 1) continue;
            float *x = rnd((size_t)N * Cin * H * W, 1u + c), *w = rnd((size_t)Co * Cin * kH * kW, 2u + c);
            float *b = rnd(Co, 3u + c);
            double *y = (double *)malloc(sizeof(double) * N * Co * OH * OW);
            or_conv2d(x, w, b, y, N, Cin, H, W, Co, kH, kW, s, p, d);
            CHECK(all_finite(y, (size_t)N * Co * OH * OW), "conv finite");
            for (int pk = 1; pk <= 3; ++pk)
                for (int pp = 0; pp <= pk / 2; ++pp) {
                    const int PH = or_window_out_dim(OH, pk, 2, pp, 1), PW = or_window_out_dim(OW, pk, 2, pp, 1);
                    if (PH < 1 || PW < 1) continue;
                    double *o = (double *)malloc(sizeof(double) * N * Co * PH * PW);
                    or_conv_tanh_scale_bias_maxpool(x, w, b, b, o, N, Cin, H, W, Co, kH, kW, s, p, d,
                                                    pk == 2 ? -1.5 : 2.0, pk, 2, pp, 1);
                    free(o);
                    float *mp = (float *)malloc(sizeof(float) * N * Cin * PH * PW);
                    const int MH = or_window_out_dim(H, pk, 2, pp, d), MW = or_window_out_dim(W, pk, 2, pp, d);
                    if (MH >= 1 && MW >= 1) {
                        float *m2 = (float *)malloc(sizeof(float) * N * Cin * MH * MW);
                        or_maxpool2d_f32(x, m2, N, Cin, H, W, pk, 2, pp, d);
                        free(m2);
                    }
                    free(mp);
                }
            free(x);
            free(w);
            free(b);
            free(y);
        }
    for (int p = 0; p <= 3; ++p)
        for (int op = 0; op <= 1; ++op) {
            const int N = 2, Cin = 3, H = 4, W = 5, Co = 6;
            const int OH = or_convT_out_dim(H, 4, 2, p, op, 1), OW = or_convT_out_dim(W, 4, 2, p, op, 1);
            if (OH < 1 || OW < 1) continue;
            float *x = rnd((size_t)N * Cin * H * W, 7u), *w = rnd((size_t)Cin * Co * 16, 8u), *b = rnd(Co, 9u);
            double *y = (double *)malloc(sizeof(double) * N * Co * OH * OW);
            or_conv_transpose2d(x, w, b, y, N, Cin, H, W, Co, 4, 2, p, op, 1);
            CHECK(all_finite(y, (size_t)N * Co * OH * OW), "convT finite");
            or_convT_softmax_bias_scale_sigmoid(x, w, b, b, y, N, Cin, H, W, Co, 4, 2, p, op, 1, 2.0);
            free(x);
            free(w);
            free(b);
            free(y);
        }
}

int main(void) {
    shape_queries();
    entry_points();
    oracle_loops();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitize ok\n");
    return 0;
}

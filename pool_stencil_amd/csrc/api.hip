// C-ABI entry points of libpool_stencil: argument validation, output extents
// and dispatch to the kernels.  Validation is pure host code and runs before
// any HIP call, so every error path works without a device.
#include <stdint.h>

#include "ps_internal.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;

// floor((in + 2p - d(k-1) - 1)/s) + 1, or <= 0 when the window does not fit.
int64_t window_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d) {
    const int64_t num = in + 2 * p - d * (k - 1) - 1;
    if (num < 0) return 0;
    return num / s + 1;
}

// (in-1)s - 2p + d(k-1) + op + 1
int64_t transposed_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t op, int64_t d) {
    return (in - 1) * s - 2 * p + d * (k - 1) + op + 1;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool too_big(int64_t a, int64_t b, int64_t c, int64_t d) {
    // a*b*c*d >= 2^40 without overflow (all factors >= 1 and < 2^31)
    int64_t v = a * b;
    if (v >= kMaxElems) return true;
    v *= c;
    if (v >= kMaxElems) return true;
    return v * d >= kMaxElems;
}

}  // namespace

extern "C" {

const char *ps_status_string(int status) {
    switch (status) {
        case PS_OK: return "ok";
        case PS_ERR_NULL: return "a required pointer is NULL";
        case PS_ERR_SHAPE: return "a dimension or an output extent is < 1, or a tensor is too large";
        case PS_ERR_PARAM: return "invalid kernel/stride/padding/dilation/output_padding";
        case PS_ERR_UNSUPPORTED: return "valid arguments outside the combinations the kernels cover";
        case PS_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case PS_ERR_HIP: return "the HIP runtime reported an error";
        default: return "unknown status";
    }
}

int ps_version(void) { return 100; }

int ps_conv2d_out_dim(int in, int k, int stride, int pad, int dil, int *out) {
    if (!out) return PS_ERR_NULL;
    if (k < 1 || stride < 1 || dil < 1 || pad < 0) return PS_ERR_PARAM;
    if (in < 1) return PS_ERR_SHAPE;
    const int64_t o = window_extent(in, k, stride, pad, dil);
    if (o < 1 || o > 0x7fffffff) return PS_ERR_SHAPE;  // (an extent past INT_MAX: no int)
    *out = (int)o;
    return PS_OK;
}

int ps_pool2d_out_dim(int in, int k, int stride, int pad, int dil, int *out) {
    if (stride <= 0) stride = k;
    return ps_conv2d_out_dim(in, k, stride, pad, dil, out);
}

int ps_convT2d_out_dim(int in, int k, int stride, int pad, int output_padding, int dil,
                       int *out) {
    if (!out) return PS_ERR_NULL;
    if (k < 1 || stride < 1 || dil < 1 || pad < 0 || output_padding < 0) return PS_ERR_PARAM;
    if (output_padding >= (stride > dil ? stride : dil)) return PS_ERR_PARAM;
    if (in < 1) return PS_ERR_SHAPE;
    const int64_t o = transposed_extent(in, k, stride, pad, output_padding, dil);
    if (o < 1 || o > 0x7fffffff) return PS_ERR_SHAPE;
    *out = (int)o;
    return PS_OK;
}

int ps_maxpool2d(const float *x, float *y, int N, int C, int H, int W, int k, int stride,
                 int pad, int dil, void *stream) {
    if (!x || !y) return PS_ERR_NULL;
    if (N < 1 || C < 1 || H < 1 || W < 1) return PS_ERR_SHAPE;
    if (k < 1 || dil < 1 || pad < 0) return PS_ERR_PARAM;
    if (stride <= 0) stride = k;
    int OH, OW;
    int st = ps_pool2d_out_dim(H, k, stride, pad, dil, &OH);
    if (st != PS_OK) return st;
    st = ps_pool2d_out_dim(W, k, stride, pad, dil, &OW);
    if (st != PS_OK) return st;
    if (too_big(N, C, H, W) || too_big(N, C, OH, OW)) return PS_ERR_SHAPE;
    // window rows and columns are 32-bit indices in -pad .. H + pad - 1
    if ((int64_t)H + 2 * (int64_t)pad > 0x7fffffff || (int64_t)W + 2 * (int64_t)pad > 0x7fffffff)
        return PS_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(y)) return PS_ERR_ALIGN;
    return ps::launch_maxpool2d(x, y, N, C, H, W, OH, OW, k, stride, pad, dil,
                                (hipStream_t)stream);
}

int ps_conv_tanh_scale_bias_maxpool(const void *x, const void *w, const float *conv_bias,
                                    const float *bias2, void *y, int dtype, int N, int Cin,
                                    int H, int W, int Cout, int kH, int kW, int conv_stride,
                                    int conv_pad, int conv_dil, float scale, int pool_k,
                                    int pool_stride, int pool_pad, int pool_dil,
                                    void *stream) {
    if (!x || !w || !bias2 || !y) return PS_ERR_NULL;
    if (dtype != PS_F32 && dtype != PS_BF16) return PS_ERR_PARAM;
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1) return PS_ERR_SHAPE;
    if (kH < 1 || kW < 1 || conv_stride < 1 || conv_dil < 1 || conv_pad < 0) return PS_ERR_PARAM;
    if (pool_k < 1 || pool_dil < 1 || pool_pad < 0) return PS_ERR_PARAM;
    if (pool_stride <= 0) pool_stride = pool_k;
    int OH, OW, PH, PW;
    int st = ps_conv2d_out_dim(H, kH, conv_stride, conv_pad, conv_dil, &OH);
    if (st != PS_OK) return st;
    st = ps_conv2d_out_dim(W, kW, conv_stride, conv_pad, conv_dil, &OW);
    if (st != PS_OK) return st;
    st = ps_pool2d_out_dim(OH, pool_k, pool_stride, pool_pad, pool_dil, &PH);
    if (st != PS_OK) return st;
    st = ps_pool2d_out_dim(OW, pool_k, pool_stride, pool_pad, pool_dil, &PW);
    if (st != PS_OK) return st;
    if (too_big(N, Cin, H, W) || too_big(N, Cout, PH, PW) || too_big(Cout, Cin, kH, kW))
        return PS_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return PS_ERR_ALIGN;
    // The 3x3 / stride-1 / few-channel / disjoint-window case has its own kernel with
    // the weights resident in registers; everything else takes the general kernel.
    const bool small_k3 = kH == 3 && kW == 3 && conv_stride == 1 && conv_dil == 1 &&
                          conv_pad <= 2 && Cin <= 8 && pool_stride == pool_k && pool_k >= 2 &&
                          pool_k <= 8 && pool_pad == 0 && pool_dil == 1 &&
                          (int64_t)Cin * H * W * (dtype == PS_F32 ? 4 : 2) < ((int64_t)1 << 31) &&
                          ((int64_t)Cout + 64) * PH * PW * (dtype == PS_F32 ? 4 : 2) <
                              ((int64_t)1 << 31);
    if (small_k3)
        return ps::launch_conv_pool(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout,
                                    conv_pad, OH, OW, scale, pool_k, PH, PW, (hipStream_t)stream);
    return ps::launch_conv_general(x, w, conv_bias, bias2, y, dtype, 0, N, Cin, H, W, Cout, kH,
                                   kW, conv_stride, conv_pad, conv_dil, OH, OW, scale, pool_k,
                                   pool_stride, pool_pad, pool_dil, PH, PW, (hipStream_t)stream);
}

int ps_conv2d(const void *x, const void *w, const float *bias, void *y, int dtype, int N,
              int Cin, int H, int W, int Cout, int kH, int kW, int stride, int pad, int dil,
              void *stream) {
    if (!x || !w || !y) return PS_ERR_NULL;
    if (dtype != PS_F32 && dtype != PS_BF16) return PS_ERR_PARAM;
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1) return PS_ERR_SHAPE;
    if (kH < 1 || kW < 1 || stride < 1 || dil < 1 || pad < 0) return PS_ERR_PARAM;
    int OH, OW;
    int st = ps_conv2d_out_dim(H, kH, stride, pad, dil, &OH);
    if (st != PS_OK) return st;
    st = ps_conv2d_out_dim(W, kW, stride, pad, dil, &OW);
    if (st != PS_OK) return st;
    if (too_big(N, Cin, H, W) || too_big(N, Cout, OH, OW) || too_big(Cout, Cin, kH, kW))
        return PS_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return PS_ERR_ALIGN;
    return ps::launch_conv_general(x, w, bias, nullptr, y, dtype, 1, N, Cin, H, W, Cout, kH, kW,
                                   stride, pad, dil, OH, OW, 1.f, 1, 1, 0, 1, OH, OW,
                                   (hipStream_t)stream);
}

int ps_convT_softmax_bias_scale_sigmoid(const float *x, const float *w, const float *convT_bias,
                                        const float *bias2, float *y, int N, int Cin, int H,
                                        int W, int Cout, int k, int stride, int pad,
                                        int output_padding, int dil, float scale,
                                        void *stream) {
    if (!x || !w || !bias2 || !y) return PS_ERR_NULL;
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1) return PS_ERR_SHAPE;
    int OH, OW;
    int st = ps_convT2d_out_dim(H, k, stride, pad, output_padding, dil, &OH);
    if (st != PS_OK) return st;
    st = ps_convT2d_out_dim(W, k, stride, pad, output_padding, dil, &OW);
    if (st != PS_OK) return st;
    if (too_big(N, Cin, H, W) || too_big(N, Cout, OH, OW) || too_big(Cin, Cout, k, k))
        return PS_ERR_SHAPE;
    if (k != 4 || stride != 2 || dil != 1) return PS_ERR_UNSUPPORTED;
    if (Cout > 256 || Cin > 256) return PS_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return PS_ERR_ALIGN;
    return ps::launch_convT_softmax(x, w, convT_bias, bias2, y, N, Cin, H, W, Cout, OH, OW, pad,
                                    scale, (hipStream_t)stream);
}

int ps_convT_softmax_bias_scale_sigmoid_bf16(const void *x, const void *w,
                                             const float *convT_bias, const float *bias2,
                                             void *y, int N, int Cin, int H, int W, int Cout,
                                             int k, int stride, int pad, int output_padding,
                                             int dil, float scale, void *stream) {
    if (!x || !w || !bias2 || !y) return PS_ERR_NULL;
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1) return PS_ERR_SHAPE;
    int OH, OW;
    int st = ps_convT2d_out_dim(H, k, stride, pad, output_padding, dil, &OH);
    if (st != PS_OK) return st;
    st = ps_convT2d_out_dim(W, k, stride, pad, output_padding, dil, &OW);
    if (st != PS_OK) return st;
    if (too_big(N, Cin, H, W) || too_big(N, Cout, OH, OW) || too_big(Cin, Cout, k, k))
        return PS_ERR_SHAPE;
    if (k != 4 || stride != 2 || dil != 1) return PS_ERR_UNSUPPORTED;
    // both column classes' bf16 weights (2 x Cout x 4*Cin) must fit the LDS of a CU
    if (Cout % 32 != 0 || Cout > 128 ||
        (int64_t)2 * Cout * (4 * (Cout == 128 ? (Cin + 7) / 8 * 8 : (Cin + 15) / 16 * 16) + 8) *
                    2 + 8 * Cout > 160 * 1024)
        return PS_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return PS_ERR_ALIGN;
    return ps::launch_convT_softmax_bf16((const uint16_t *)x, (const uint16_t *)w, convT_bias,
                                         bias2, (uint16_t *)y, N, Cin, H, W, Cout, OH, OW, pad,
                                         scale, (hipStream_t)stream);
}

int ps_convT2d(const float *x, const float *w, const float *bias, float *y, int N, int Cin, int H,
               int W, int Cout, int k, int stride, int pad, int output_padding, int dil,
               void *stream) {
    if (!x || !w || !y) return PS_ERR_NULL;
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1) return PS_ERR_SHAPE;
    int OH, OW;
    int st = ps_convT2d_out_dim(H, k, stride, pad, output_padding, dil, &OH);
    if (st != PS_OK) return st;
    st = ps_convT2d_out_dim(W, k, stride, pad, output_padding, dil, &OW);
    if (st != PS_OK) return st;
    if (too_big(N, Cin, H, W) || too_big(N, Cout, OH, OW) || too_big(Cin, Cout, k, k))
        return PS_ERR_SHAPE;
    if (k != 4 || stride != 2 || dil != 1) return PS_ERR_UNSUPPORTED;
    if (Cout > 256 || Cin > 256) return PS_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return PS_ERR_ALIGN;
    return ps::launch_convT(x, w, bias, y, N, Cin, H, W, Cout, OH, OW, pad, (hipStream_t)stream);
}

int ps_tanh_scale_bias_maxpool(const void *y, const float *bias2, void *out, int dtype, int N,
                               int C, int H, int W, float scale, int k, int stride, int pad,
                               int dil, void *stream) {
    if (!y || !bias2 || !out) return PS_ERR_NULL;
    if (dtype != PS_F32 && dtype != PS_BF16) return PS_ERR_PARAM;
    if (N < 1 || C < 1 || H < 1 || W < 1) return PS_ERR_SHAPE;
    if (k < 1 || dil < 1 || pad < 0) return PS_ERR_PARAM;
    if (stride <= 0) stride = k;
    int OH, OW;
    int st = ps_pool2d_out_dim(H, k, stride, pad, dil, &OH);
    if (st != PS_OK) return st;
    st = ps_pool2d_out_dim(W, k, stride, pad, dil, &OW);
    if (st != PS_OK) return st;
    if (too_big(N, C, H, W) || too_big(N, C, OH, OW)) return PS_ERR_SHAPE;
    if (!aligned16(y) || !aligned16(out)) return PS_ERR_ALIGN;
    return ps::launch_tanh_scale_bias_maxpool(y, bias2, out, dtype, N, C, H, W, OH, OW, scale, k,
                                              stride, pad, dil, (hipStream_t)stream);
}

int ps_softmax_bias_scale_sigmoid(const float *y, const float *bias2, float *out, int N, int C,
                                  int H, int W, float scale, void *stream) {
    if (!y || !bias2 || !out) return PS_ERR_NULL;
    if (N < 1 || C < 1 || H < 1 || W < 1) return PS_ERR_SHAPE;
    if (too_big(N, C, H, W)) return PS_ERR_SHAPE;
    if (!aligned16(y) || !aligned16(out)) return PS_ERR_ALIGN;
    return ps::launch_softmax_bias_scale_sigmoid(y, bias2, out, N, C, H, W, scale,
                                                 (hipStream_t)stream);
}

}  // extern "C"

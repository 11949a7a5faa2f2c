/*
 * pool_stencil -- fused sliding-window stencils for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpool_stencil.so.  Operations:
 *
 *   ps_conv_tanh_scale_bias_maxpool     Conv2d -> tanh -> *scale -> +bias2[c] -> MaxPool2d,
 *                                       fused: the conv output never reaches memory
 *   ps_conv2d                           Conv2d + bias (the unfused pipeline's first stage)
 *   ps_maxpool2d                        MaxPool2d (stride-1 overlapping windows included)
 *   ps_convT_softmax_bias_scale_sigmoid ConvTranspose2d -> softmax over channels
 *                                       -> +bias2[c] -> *scale -> sigmoid, fused
 *   ps_convT_softmax_bias_scale_sigmoid_bf16   the same with bf16 tensors
 *   ps_convT2d                          ConvTranspose2d + bias (unfused first stage)
 *   ps_tanh_scale_bias_maxpool          tanh/scale/bias + MaxPool2d of a stored conv output
 *   ps_softmax_bias_scale_sigmoid       channel softmax post-process of a stored convT output
 *
 * The operations and their arguments follow the problem statements of three
 * POPCORNBENCH transcripts (cited by page name):
 *   Kimi-K2.6 l2_p82  Conv2d(8->64, k3) + tanh + scale + bias + MaxPool2d(4)
 *   Kimi-K2.6 l1_p42  MaxPool2d(k4, s1, p1, d1)
 *   Kimi-K2.6 l2_p91  ConvTranspose2d(64->128, k4, s2, p1, op1) + softmax(dim 1)
 *                     + bias + scale + sigmoid
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout     All tensors are dense, contiguous, row-major NCHW (PyTorch's default
 *            memory format).  Conv2d weights are [Cout, Cin, kH, kW];
 *            ConvTranspose2d weights are [Cin, Cout, k, k] (PyTorch's layouts).
 *            Bias vectors are [C] float32.
 * Pointers   Tensor pointers are DEVICE pointers on the current HIP device.  The
 *            caller owns every buffer; the library allocates nothing, keeps no
 *            state between calls and never frees.  Inputs and outputs must not
 *            overlap.  Tensor pointers must be 16-byte aligned (PS_ERR_ALIGN).
 * Streams    `stream` is a hipStream_t (NULL = the default stream).  Every call
 *            only enqueues work on that stream and returns; it never synchronises.
 * Errors     Arguments are validated on the host before anything is enqueued; on
 *            any error nothing is launched and the status says why.  A failed
 *            kernel launch returns PS_ERR_HIP.  Faults during execution surface on
 *            the caller's next synchronisation, as for any HIP kernel.
 * Extents    Output sizes use the floor-mode window formula
 *            out = floor((in + 2p - d(k-1) - 1)/s) + 1 and, for the transposed
 *            conv, out = (in-1)s - 2p + d(k-1) + op + 1 (the pages derive
 *            256 -> 254 -> 63, 512 -> 511 and 64 -> 129 from them).
 * Sizes      Every dimension must be >= 1; each tensor must hold < 2^40 elements.
 * Threads    Entry points are reentrant; concurrent calls on different streams
 *            are independent.
 */
#ifndef POOL_STENCIL_H
#define POOL_STENCIL_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PS_OK = 0,
    PS_ERR_NULL = 1,        /* a required pointer is NULL                              */
    PS_ERR_SHAPE = 2,       /* a dimension < 1 or an output extent < 1                 */
    PS_ERR_PARAM = 3,       /* a kernel/stride/pad/dil/output_padding value is invalid */
    PS_ERR_UNSUPPORTED = 4, /* valid, but outside the combinations the kernels cover   */
    PS_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned                 */
    PS_ERR_HIP = 6          /* the HIP runtime reported an error at launch             */
} ps_status;

typedef enum {
    PS_F32 = 0,  /* IEEE binary32                                   */
    PS_BF16 = 1  /* bfloat16 storage (uint16 bit patterns), fp32 math */
} ps_dtype;

/* Short, static, human-readable text for a status code.  Never NULL. */
const char *ps_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int ps_version(void);

/* ---------------------------------------------------------------- shapes --- */
/* Pure host arithmetic; no device needed.  Writes *out and returns PS_OK, or
 * returns PS_ERR_PARAM (k,s,d < 1 or p < 0) / PS_ERR_SHAPE (in < 1, or the
 * result < 1 or above INT_MAX) and leaves *out untouched. */
int ps_conv2d_out_dim(int in, int k, int stride, int pad, int dil, int *out);
/* MaxPool2d, floor mode; stride <= 0 means stride = k (nn.MaxPool2d's default). */
int ps_pool2d_out_dim(int in, int k, int stride, int pad, int dil, int *out);
/* ConvTranspose2d; additionally PS_ERR_PARAM when output_padding >= max(stride, dil)
 * or output_padding < 0 (PyTorch's rule). */
int ps_convT2d_out_dim(int in, int k, int stride, int pad, int output_padding, int dil,
                       int *out);

/* ------------------------------------------------ fused conv + max-pool --- */
/* l2_p82 page (problem statement and the fused-kernel discussion):
 *   y[n,co,oh,ow] = conv_bias[co] + sum_{ci,kh,kw} x[n,ci,oh*s-p+kh*d, ow*s-p+kw*d]
 *                                                   * w[co,ci,kh,kw]   (zero padding)
 *   z = tanh(y) * scale + bias2[co]
 *   out[n,co,ph,pw] = max over the pool window of z   (floor mode, -inf padding)
 * The conv output is never written to memory.  Because tanh and z -> z*scale+b
 * are monotone, the kernel pools the conv value first and applies the epilogue
 * once per pooled output (the page's reordering argument); for scale < 0 the
 * window minimum is taken instead, for scale == 0 the result is bias2[co].
 *
 * x         [N,Cin,H,W]       dtype (PS_F32: float, PS_BF16: uint16 bf16 bits)
 * w         [Cout,Cin,kH,kW]  dtype
 * conv_bias [Cout] float32, or NULL for a conv without bias
 * bias2     [Cout] float32 (the [C,1,1] bias parameter after the conv)
 * y         [N,Cout,PH,PW]    dtype; bf16 output is rounded to nearest even
 * pool_stride <= 0 means pool_stride = pool_k.  A pool window lying wholly in
 * the pool's padding gives -inf (the plain definition's max over -inf values).
 * Any conv kernel size, stride, padding and dilation, any Cin and Cout, and any
 * pool window / stride / padding / dilation are accepted, with two limits of
 * the tiling: the pool window's extent (pool_k-1)*pool_dil+1 must be <= 16, and
 * the conv input patch of one pooled output plus 64 x 4 x kH*kW weights must fit
 * the 160 KB of LDS of a compute unit (kH*kW <= 144 always does); and one image
 * and the weight tensor must each be below 2^31 bytes (32-bit byte offsets).
 * Beyond them the call returns PS_ERR_UNSUPPORTED.  The 3x3, stride-1, dilation-1,
 * conv_pad <= 2, Cin <= 8, disjoint-window (pool_stride = pool_k <= 8, no pool
 * padding or dilation) case runs a kernel of its own with the weights held in
 * registers; every other case runs the general tiled kernel. */
int ps_conv_tanh_scale_bias_maxpool(
    const void *x, const void *w, const float *conv_bias, const float *bias2, void *y,
    int dtype, int N, int Cin, int H, int W, int Cout, int kH, int kW, int conv_stride,
    int conv_pad, int conv_dil, float scale, int pool_k, int pool_stride, int pool_pad,
    int pool_dil, void *stream);

/* ------------------------------------------------------------ conv 2d --- */
/* The first stage of the l2_p82 page's unfused pipeline (its first kernel
 * writes the full conv output, a second kernel applies the epilogue and the
 * pool); also a plain nn.Conv2d forward:
 *   y[n,co,oh,ow] = bias[co] + sum_{ci,kh,kw} x[n,ci,oh*s-p+kh*d, ow*s-p+kw*d] * w[co,ci,kh,kw]
 * (cross-correlation, zero padding).
 * x [N,Cin,H,W] dtype, w [Cout,Cin,kH,kW] dtype, bias [Cout] float32 or NULL,
 * y [N,Cout,OH,OW] dtype (bf16: fp32 accumulation, output rounded to nearest even).
 * Any kernel size, stride, padding, dilation and channel counts, within the
 * same LDS limit as the fused call (kH*kW <= 144 always fits). */
int ps_conv2d(const void *x, const void *w, const float *bias, void *y, int dtype, int N,
              int Cin, int H, int W, int Cout, int kH, int kW, int stride, int pad, int dil,
              void *stream);

/* ---------------------------------------------------------- max-pool 2d --- */
/* l1_p42 page (problem statement; PyTorch's implicit -inf padding):
 *   y[n,c,oh,ow] = max_{kh,kw < k} x[n,c,oh*s-p+kh*d, ow*s-p+kw*d], -inf outside,
 *   floor mode.  The result is bit-exact (a max of the inputs).
 * x [N,C,H,W] float32, y [N,C,OH,OW] float32.  stride <= 0 means stride = k.
 * NaN inputs are outside the contract (the result may or may not carry them).
 * Supported: any k >= 1, 1 <= dil, 0 <= pad with H + 2*pad and W + 2*pad below
 * 2^31, any stride >= 1, OH <= 65535 for stride > 1 (524280 for stride 1),
 * H*W < 2^31. */
int ps_maxpool2d(const float *x, float *y, int N, int C, int H, int W, int k, int stride,
                 int pad, int dil, void *stream);

/* ------------------------------------ transposed conv + channel softmax --- */
/* l2_p91 page (problem statement, scatter definition and epilogue order):
 *   t[n,co,oh,ow] = convT_bias[co] + sum over (ci, ih, iw, kh, kw) with
 *                   oh = ih*s - p + kh*d, ow = iw*s - p + kw*d of x[n,ci,ih,iw]*w[ci,co,kh,kw]
 *   sm = softmax over co of t (max subtracted)
 *   y  = 1 / (1 + exp(-(sm + bias2[co]) * scale))
 * x [N,Cin,H,W] float32, w [Cin,Cout,k,k] float32, convT_bias [Cout] float32 or NULL,
 * bias2 [Cout] float32, y [N,Cout,OH,OW] float32.
 * Supported: k = 4, stride = 2, dil = 1, any pad >= 0 with OH, OW >= 1,
 * output_padding in {0, 1}, 1 <= Cout <= 256, and 1 <= Cin <= 256 where one parity
 * class's fp32 weights stay resident in the LDS of a compute unit:
 * (Cp*(16*Cq + 4) + 2*Cp)*4 <= 160 KB with Cp = Cout rounded up to a multiple of 16
 * and Cq = ceil(Cin/4) (Cin <= 76 at Cp = 128, <= 68 at 144, <= 36 at 256); x with
 * its channels rounded up to 4*Cq, and y with Cp channels, below 2^29 elements each.
 * Beyond these PS_ERR_UNSUPPORTED. */
int ps_convT_softmax_bias_scale_sigmoid(
    const float *x, const float *w, const float *convT_bias, const float *bias2, float *y,
    int N, int Cin, int H, int W, int Cout, int k, int stride, int pad, int output_padding,
    int dil, float scale, void *stream);

/* The same fused operation with bfloat16 x, w and y (uint16 bit patterns), fp32
 * products and accumulation, fp32 softmax and epilogue, y rounded to nearest even.
 * (The l2_p91 page considers reduced precision for this problem and keeps fp32;
 * this variant runs the GEMM on the bf16 matrix cores.)  convT_bias and bias2 are
 * float32.  Supported: k = 4, stride = 2, dil = 1, any pad >= 0 with OH, OW >= 1,
 * output_padding in {0, 1}, Cout in {32, 64, 96, 128} (the bf16 kernels hold a
 * pixel's channels for both column classes in one wave's registers), and
 * 2*Cout*(4*Cp + 8)*2 + 8*Cout <= 160 KB with Cp = Cin rounded up to a multiple
 * of 8 (Cout = 128) or 16 (else), i.e. Cin <= 72 at Cout = 128, <= 144 at
 * Cout = 64; and x below 2^30 elements. */
int ps_convT_softmax_bias_scale_sigmoid_bf16(
    const void *x, const void *w, const float *convT_bias, const float *bias2, void *y,
    int N, int Cin, int H, int W, int Cout, int k, int stride, int pad, int output_padding,
    int dil, float scale, void *stream);

/* ------------------------------------------------ plain transposed conv --- */
/* The first stage of the l2_p91 page's unfused pipeline (the transposed conv
 * writes its full output, then a post-processing kernel runs in place on it);
 * also a plain nn.ConvTranspose2d forward:
 *   y[n,co,oh,ow] = bias[co] + sum over (ci, ih, iw, kh, kw) with
 *                   oh = ih*s - p + kh*d, ow = iw*s - p + kw*d of x[n,ci,ih,iw]*w[ci,co,kh,kw]
 * x [N,Cin,H,W] float32, w [Cin,Cout,k,k] float32, bias [Cout] float32 or NULL,
 * y [N,Cout,OH,OW] float32.  Supported: the same set as the fp32 fused call above. */
int ps_convT2d(const float *x, const float *w, const float *bias, float *y, int N, int Cin, int H,
               int W, int Cout, int k, int stride, int pad, int output_padding, int dil,
               void *stream);

/* -------------------------------------- post-processing of stored outputs --- */
/* The l2_p82 page's second kernel of the unfused pipeline, on a stored conv output:
 *   out[n,c,ph,pw] = max over the pool window of tanh(y)*scale + bias2[c]
 * (floor mode, -inf padding; a window wholly in the padding gives -inf; the window
 * is reduced before tanh, by the same monotonicity argument as the fused call).
 * y [N,C,H,W] dtype, bias2 [C] float32, out [N,C,OH,OW] dtype (bf16 rounded to
 * nearest even).  stride <= 0 means stride = k.  Any window, stride, padding and
 * dilation.  y and out must not overlap. */
int ps_tanh_scale_bias_maxpool(const void *y, const float *bias2, void *out, int dtype, int N,
                               int C, int H, int W, float scale, int k, int stride, int pad,
                               int dil, void *stream);

/* The l2_p91 page's post-processing kernel of the unfused pipeline, on a stored
 * transposed-conv output:
 *   out[n,c,h,w] = 1 / (1 + exp(-(softmax over c of y[n,:,h,w] + bias2[c]) * scale))
 * y, out [N,C,H,W] float32, bias2 [C] float32.  Any C (up to 128 channels one read
 * of y, more channels two).  out == y (in place, as on the page) is allowed; any
 * other overlap is not. */
int ps_softmax_bias_scale_sigmoid(const float *y, const float *bias2, float *out, int N, int C,
                                  int H, int W, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* POOL_STENCIL_H */

// Second stages of the unfused pipelines the pages measure their fused kernels
// against, usable on their own as post-processing ops.
//
// tanh_scale_bias_maxpool (POPCORNBENCH page Kimi-K2.6 l2_p82: the unfused
// version writes the full conv output to memory and a second kernel applies
// tanh, the scale, the channel bias and the max-pool):
//   out[n,c,ph,pw] = max over the window of tanh(y)*scale + bias2[c]
//   (floor mode, -inf padding; a window wholly in the padding gives -inf).
//   As in the fused kernels, the window is reduced first (max of y for
//   scale >= 0, min for scale < 0) and tanh is evaluated once per output: tanh
//   and v -> v*scale + b are monotone.  fp32 windows with k 2..5 and stride /
//   dilation (2,1), (3,1), (4,1), (1,2), (2,2) run on the row-streaming max-pool
//   kernel with this map applied at its stores (each stored value read once).
//   Other windows and bf16: one thread per output, the window read through the
//   cache hierarchy.
//
// softmax_bias_scale_sigmoid (page Kimi-K2.6 l2_p91: the post-processing
// kernel that runs in place on the stored transposed-conv output):
//   out[n,c,h,w] = sigmoid((softmax over c of y[n,:,h,w] + bias2[c]) * scale)
//   One thread per pixel; consecutive threads take consecutive pixels, so each
//   channel plane is read and written with coalesced accesses.  Up to 128
//   channels are held in registers (one read, one write per element); more
//   channels take a second read (online max / rescaled sum, then the output
//   pass).  In place is allowed: a thread reads all of its pixel's channels
//   before writing any.
#include "ps_internal.h"

#include <math.h>

namespace ps {
namespace {

__device__ __forceinline__ float ld(const float *p) { return *p; }
__device__ __forceinline__ float ld(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st(float *p, float v) { *p = v; }
__device__ __forceinline__ void st(uint16_t *p, float v) { *p = f32_to_bf16_rne(v); }

// grid.x covers the OH*OW outputs of a plane, grid.y strides over the N*C planes.
template <typename TI>
__global__ __launch_bounds__(256) void tanh_scale_bias_maxpool_k(
    const TI *__restrict__ y, const float *__restrict__ b2, TI *__restrict__ out, int C, int H,
    int W, int OH, int OW, int k, int s, int p, int d, float scale, int planes) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= OH * OW) return;
    const int oh = q / OW, ow = q - (q / OW) * OW;
    const float sgn = scale < 0.f ? -1.f : 1.f;
    for (int pl = blockIdx.y; pl < planes; pl += gridDim.y) {
        const TI *yp = y + (size_t)pl * H * W;
        float best = -INFINITY;
        for (int kh = 0; kh < k; ++kh) {
            const int ih = oh * s - p + kh * d;
            if (ih < 0 || ih >= H) continue;
            for (int kw = 0; kw < k; ++kw) {
                const int iw = ow * s - p + kw * d;
                if (iw < 0 || iw >= W) continue;
                best = fmaxf(best, sgn * ld(yp + (size_t)ih * W + iw));
            }
        }
        const float o = best == -INFINITY ? -INFINITY : tanh_exp(sgn * best) * scale + b2[pl % C];
        st(out + (size_t)pl * OH * OW + q, o);
    }
}

// sigmoid((e*inv + b) * scale) with the hardware reciprocal (the fused kernels use it
// too; 1 ulp), not the IEEE division sequence.
__device__ __forceinline__ float epilogue(float e, float inv, float b, float scale) {
    const float v = (e * inv + b) * scale;
    return __builtin_amdgcn_rcpf(1.f + __expf(-v));
}

// grid.x covers the HW pixels of an image, grid.y strides over the N images.
// CMAX > 0: all C <= CMAX channel values of a pixel in registers.  CMAX == 0:
// any C, two reads.
template <int CMAX>
__global__ __launch_bounds__(256) void softmax_bias_scale_sigmoid_k(const float *y,
                                                                   const float *__restrict__ b2,
                                                                   float *out, int N, int C,
                                                                   int HW, float scale) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= HW) return;
    for (int n = blockIdx.y; n < N; n += gridDim.y) {
        const size_t base = (size_t)n * C * HW + q;
        if constexpr (CMAX > 0) {
            float v[CMAX];
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < CMAX; ++c) {
                v[c] = c < C ? y[base + (size_t)c * HW] : -INFINITY;
                mx = fmaxf(mx, v[c]);
            }
            float sum = 0.f;
#pragma unroll
            for (int c = 0; c < CMAX; ++c) {
                v[c] = c < C ? __expf(v[c] - mx) : 0.f;
                sum += v[c];
            }
            const float inv = __builtin_amdgcn_rcpf(sum);
#pragma unroll
            for (int c = 0; c < CMAX; ++c)
                if (c < C) out[base + (size_t)c * HW] = epilogue(v[c], inv, b2[c], scale);
        } else {
            float mx = -INFINITY, sum = 0.f;
            for (int c = 0; c < C; ++c) {
                const float t = y[base + (size_t)c * HW];
                if (t > mx) {
                    sum = sum * __expf(mx - t) + 1.f;
                    mx = t;
                } else {
                    sum += __expf(t - mx);
                }
            }
            const float inv = __builtin_amdgcn_rcpf(sum);
            for (int c = 0; c < C; ++c) {
                const size_t i = base + (size_t)c * HW;
                out[i] = epilogue(__expf(y[i] - mx), inv, b2[c], scale);
            }
        }
    }
}

}  // namespace

int launch_tanh_scale_bias_maxpool(const void *y, const float *bias2, void *out, int dtype, int N,
                                   int C, int H, int W, int OH, int OW, float scale, int k, int s,
                                   int p, int d, hipStream_t stream) {
    const int64_t planes = (int64_t)N * C;
    if ((int64_t)OH * OW > 0x7fffffff - 256 || planes > 0x7fffffff) return PS_ERR_UNSUPPORTED;
    if (dtype != PS_BF16) {  // fp32 windows the row-streaming kernel covers
        const int rc = launch_tanh_scale_bias_maxpool_rows((const float *)y, bias2, (float *)out,
                                                           N, C, H, W, OH, OW, scale, k, s, p, d,
                                                           stream);
        if (rc >= 0) return rc;
    }
    const dim3 grid((unsigned)((OH * OW + 255) / 256), (unsigned)(planes < 65535 ? planes : 65535));
    if (dtype == PS_BF16)
        return launch(tanh_scale_bias_maxpool_k<uint16_t>, grid, dim3(256), 0, stream,
                      (const uint16_t *)y, bias2, (uint16_t *)out, C, H, W, OH, OW, k, s, p, d,
                      scale, (int)planes);
    return launch(tanh_scale_bias_maxpool_k<float>, grid, dim3(256), 0, stream, (const float *)y,
                  bias2, (float *)out, C, H, W, OH, OW, k, s, p, d, scale, (int)planes);
}

int launch_softmax_bias_scale_sigmoid(const float *y, const float *bias2, float *out, int N,
                                      int C, int H, int W, float scale, hipStream_t stream) {
    const int64_t hw = (int64_t)H * W;
    if (hw > 0x7fffffff - 256) return PS_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((hw + 255) / 256), (unsigned)(N < 65535 ? N : 65535));
    if (C <= 32)
        return launch(softmax_bias_scale_sigmoid_k<32>, grid, dim3(256), 0, stream, y, bias2, out,
                      N, C, (int)hw, scale);
    if (C <= 64)
        return launch(softmax_bias_scale_sigmoid_k<64>, grid, dim3(256), 0, stream, y, bias2, out,
                      N, C, (int)hw, scale);
    if (C <= 128)
        return launch(softmax_bias_scale_sigmoid_k<128>, grid, dim3(256), 0, stream, y, bias2,
                      out, N, C, (int)hw, scale);
    return launch(softmax_bias_scale_sigmoid_k<0>, grid, dim3(256), 0, stream, y, bias2, out, N,
                  C, (int)hw, scale);
}

}  // namespace ps

// Internal declarations shared by the HIP translation units of libpool_stencil.
// Not part of the public C ABI (that is include/pool_stencil.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "pool_stencil.h"

namespace ps {

// Enqueue a kernel and return the status of THIS launch: hipLaunchKernel reports
// the launch's own error, so an earlier, unrelated sticky error on the calling
// thread is neither taken for this call's failure nor cleared.  The arguments are
// converted to the kernel's parameter types first (as a <<<>>> launch would).
template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
           Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> params(static_cast<KArgs>(args)...);
    const hipError_t st = std::apply(
        [&](auto &...p) {
            void *ptrs[] = {(void *)&p...};
            return hipLaunchKernel((const void *)kernel, grid, block, ptrs, shmem, stream);
        },
        params);
    return st == hipSuccess ? PS_OK : PS_ERR_HIP;
}

// Launchers.  Arguments have already been validated by the entry points in
// api.hip; each returns PS_OK or PS_ERR_HIP.
int launch_maxpool2d(const float *x, float *y, int N, int C, int H, int W, int OH, int OW,
                     int k, int s, int p, int d, hipStream_t stream);

int launch_conv_pool(const void *x, const void *w, const float *conv_bias, const float *bias2,
                     void *y, int dtype, int N, int Cin, int H, int W, int Cout, int conv_pad,
                     int OH, int OW, float scale, int pool_k, int PH, int PW,
                     hipStream_t stream);

// General fused conv + pool (epi = 0) or plain conv + bias (epi = 1; pool
// arguments ignored, output [N,Cout,OH,OW]).  Any kernel size, stride,
// padding, dilation and channel counts; returns PS_ERR_UNSUPPORTED (before any
// HIP call) when no tile of the kernel fits the arguments.
int launch_conv_general(const void *x, const void *w, const float *conv_bias, const float *bias2,
                        void *y, int dtype, int epi, int N, int Cin, int H, int W, int Cout,
                        int kH, int kW, int cs, int cp, int cd, int OH, int OW, float scale,
                        int pk, int ps, int pp, int pd, int PH, int PW, hipStream_t stream);

// Transposed conv k4 s2 d1, any padding `pad` (OH, OW already include it and the
// output_padding), Cout a multiple of 16 up to 256.
int launch_convT_softmax(const float *x, const float *w, const float *convT_bias,
                         const float *bias2, float *y, int N, int Cin, int H, int W, int Cout,
                         int OH, int OW, int pad, float scale, hipStream_t stream);

// The row-class transposed conv (softmax epilogue or plain + bias): Cout = 128,
// Cin <= 64, W a multiple of 4, at least 64 column positions per output row.
// PS_ERR_UNSUPPORTED (before any HIP call) outside that envelope.
int launch_convT_rows(const float *x, const float *w, const float *cb, const float *b2, float *y,
                      int N, int Cin, int H, int W, int Cout, int OH, int OW, int pad,
                      float scale, bool softmax, hipStream_t stream);

// Its bf16 version (fp32 accumulation and epilogue): Cout = 128, Cin <= 64, W a
// multiple of 8, at least 64 column positions per output row.
int launch_convT_rows_bf16(const uint16_t *x, const uint16_t *w, const float *cb,
                           const float *b2, uint16_t *y, int N, int Cin, int H, int W, int Cout,
                           int OH, int OW, int pad, float scale, hipStream_t stream);

// bf16 x, w and y (uint16 bit patterns), fp32 accumulation; Cout a multiple of 32.
int launch_convT_softmax_bf16(const uint16_t *x, const uint16_t *w, const float *convT_bias,
                              const float *bias2, uint16_t *y, int N, int Cin, int H, int W,
                              int Cout, int OH, int OW, int pad, float scale, hipStream_t stream);

// The same transposed conv without the softmax epilogue (y = convT + bias).
int launch_convT(const float *x, const float *w, const float *convT_bias, float *y, int N,
                 int Cin, int H, int W, int Cout, int OH, int OW, int pad, hipStream_t stream);

// Post-processing stages of the unfused pipelines.
int launch_tanh_scale_bias_maxpool(const void *y, const float *bias2, void *out, int dtype, int N,
                                   int C, int H, int W, int OH, int OW, float scale, int k, int s,
                                   int p, int d, hipStream_t stream);
// The same stage for fp32 through the strided row-streaming max-pool kernel (k 2..5
// with stride / dilation (2,1), (3,1), (4,1), (1,2), (2,2)); -1 for other windows.
int launch_tanh_scale_bias_maxpool_rows(const float *y, const float *bias2, float *out, int N,
                                        int C, int H, int W, int OH, int OW, float scale, int k,
                                        int s, int p, int d, hipStream_t stream);
int launch_softmax_bias_scale_sigmoid(const float *y, const float *bias2, float *out, int N,
                                      int C, int H, int W, float scale, hipStream_t stream);

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN): the hardware
// conversion (v_cvt_pk_bf16_f32 on gfx950), one instruction per pair of values.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// tanh from the identity tanh(v) = 1 - 2 / (exp(2v) + 1), with the hardware
// exponential and reciprocal: about 10 instructions instead of the library
// tanhf's 40.  Absolute error below 7e-7 over the whole range (checked in fp32
// with exp and reciprocal perturbed by 2 ulp; exp overflow gives +1, underflow
// -1), against the 1e-4 absolute bar of the fp32 outputs.
__device__ __forceinline__ float tanh_exp(float v) {
    const float e = __expf(2.f * v);
    return 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
}

// Raw buffer resource over [base, base + bytes): loads through it are range-checked
// by the hardware, and an offset at or past `bytes` reads as zero (used to express
// zero padding without branches).  The fourth word is the gfx9-family setting for
// untyped buffer access, as the ROCm libraries use it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_range_checked(const void *base,
                                                                     uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes,
                                             0x00020000);
}

// Blocks of one launch are handed to the 8 XCDs of an MI355X round-robin
// (block b runs on XCD b % 8).  This remaps the hardware block index so that
// consecutive LOGICAL blocks (which share halo rows and weights) run on the
// same XCD and therefore share its L2.  A bijection on [0, nblocks).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nblocks) {
    constexpr uint32_t kXcd = 8;
    const uint32_t per = nblocks / kXcd;          // full rounds
    const uint32_t tail = nblocks - per * kXcd;   // blocks of the last partial round
    const uint32_t xcd = b % kXcd;
    const uint32_t pos = b / kXcd;
    // XCD x owns per (+1 if x < tail) logical blocks, in order.
    const uint32_t start = xcd * per + (xcd < tail ? xcd : tail);
    return start + pos;
}

}  // namespace ps

// Fused ConvTranspose2d(k4, s2, p1) -> softmax over channels -> +bias2 -> *scale -> sigmoid
// for gfx950.
//
// Definition (POPCORNBENCH page Kimi-K2.6 l2_p91, problem statement and its
// scatter loop):
//   t[n,co,oh,ow] = bias[co] + sum over (ci, ih, iw, kh, kw) with oh = 2*ih - 1 + kh,
//                   ow = 2*iw - 1 + kw of x[n,ci,ih,iw] * w[ci,co,kh,kw]
//   y = sigmoid((softmax_co(t) + bias2[co]) * scale)
//
// Parity decomposition (the page's phase table): output row oh = 2m + a only
// receives kernel rows kh = 1 - a + 2u (u = 0, 1), from input rows
// ih = m + a - u; columns likewise with (b, v).  Each of the four classes
// (a, b) is therefore a dense GEMM
//   D[co][pixel] = sum_{k = (ci, u, v)} A_ab[co][k] * B_ab[k][pixel],  K = 4*Cin,
// with a class-specific weight matrix A_ab (a 2x2 sub-kernel per (ci, co)).
//
// Kernel layout (weights stationary):
//   - a workgroup serves ONE class; its whole A_ab (Cout x 4*Cin fp32, 128 KB
//     for 64 -> 128 channels) is staged into LDS once and reused for every
//     pixel tile the workgroup processes;
//   - each wave owns tiles of 16*NQ pixels x all Cout channels, so the channel
//     softmax never leaves the wave: D tiles are 16 channels x 16 pixels
//     (v_mfma_f32_16x16x4_f32), a lane holds 4*MT channels of one pixel, and
//     the cross-channel max / sum finish with two lane exchanges (xor 16, 32);
//   - the B operand (input pixels) is read straight from global memory / L2:
//     each lane needs the 2x2 input neighbourhood of its pixel for one input
//     channel per four K-steps;
//   - A is read from LDS as 16-byte vectors covering four K-steps.
//   - The page's online max/sum recurrence is not needed: all channel values
//     of a pixel sit in registers, so the max is taken first and the sum of
//     exp(t - max) second, both in registers.
//   - Workgroups of the column classes b = 0 and b = 1 of the same row class
//     run on the same XCD and walk the pixels in the same order, so the two
//     interleaved halves of every output row meet in that XCD's L2.
#include "ps_internal.h"

#include <math.h>

namespace ps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves: two per SIMD

// SOFTMAX = false: the same transposed conv with the epilogue left out (the
// stored intermediate of the page's unfused pipeline, or a plain
// ConvTranspose2d + bias).
template <int MT, int NQ, bool SOFTMAX>
__global__ __launch_bounds__(kThreads) void convT_softmax_f32(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cbias,
    const float *__restrict__ b2, float *__restrict__ y, int N, int Cin, int H, int W, int OH,
    int OW, float scale, int Cq, int wg_per_class) {
    constexpr int COUT = 16 * MT;
    extern __shared__ float lds[];
    const int KS = 4 * Cq;          // K-steps per lane group
    const int CS = 4 * KS + 4;      // words per output channel row (padded)
    float *lw = lds;                // [COUT][4 lane groups][KS]
    float *lcb = lds + COUT * CS;   // [COUT] conv-transpose bias
    float *lb2 = lcb + COUT;        // [COUT] bias2

    // Block b runs on XCD b % 8.  Class = (b / 8) % 4, so blocks b and b + 8
    // (same XCD) serve the column classes (a, 0) and (a, 1).
    const int blk = blockIdx.x;
    const int cls = (blk >> 3) & 3;
    const int a = cls >> 1, b = cls & 1;
    const int rank = (blk & 7) + 8 * (blk >> 5);  // rank among the blocks of this class
    const int Mc = (OH - a + 1) >> 1;            // rows of this class
    const int Qc = (OW - b + 1) >> 1;            // columns of this class
    const int Cin4 = 4 * Cq;

    // ---- stage A_ab: lw[co][G][s] = w[ci][co][1-a+2u][1-b+2v],
    //      ci = G*Cq + s/4, (u, v) = ((s%4)/2, (s%4)%2); zero for ci >= Cin
    for (int e = threadIdx.x; e < COUT * 4 * KS; e += kThreads) {
        const int s = e % KS;
        const int G = (e / KS) & 3;
        const int co = e / (4 * KS);
        const int ci = G * Cq + (s >> 2);
        const int u = (s >> 1) & 1, v = s & 1;
        const int kh = 1 - a + 2 * u, kw = 1 - b + 2 * v;
        float val = 0.f;
        if (ci < Cin) val = w[(((size_t)ci * COUT + co) * 4 + kh) * 4 + kw];
        lw[co * CS + G * KS + s] = val;
    }
    for (int e = threadIdx.x; e < COUT; e += kThreads) {
        lcb[e] = cbias ? cbias[e] : 0.f;
        if constexpr (SOFTMAX) lb2[e] = b2[e];  // b2 is NULL without the softmax epilogue
    }
    __syncthreads();
    (void)Cin4;

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int j = lane & 15;
    const int G = lane >> 4;
    const int64_t cls_pix = (int64_t)N * Mc * Qc;
    const int64_t ntiles = (cls_pix + 16 * NQ - 1) / (16 * NQ);
    const int64_t wstride = (int64_t)wg_per_class * (kThreads / 64);
    const float *aw = lw + j * CS + G * KS;  // + mt*16*CS + s
    const size_t plane = (size_t)H * W;
    const uint32_t xbytes = 4u * (uint32_t)((size_t)N * Cin * plane);  // < 2^32 (host check)
    const __amdgpu_buffer_rsrc_t xr = make_range_checked(x, xbytes);
    const size_t oplane = (size_t)OH * OW;

    for (int64_t tile = (int64_t)rank * (kThreads / 64) + wv; tile < ntiles; tile += wstride) {
        // per-lane pixel geometry for each of the NQ pixel groups
        uint32_t xb[NQ];   // byte offset of (n, G*Cq, ih0, iw0) in x
        bool r0[NQ], r1[NQ], c0[NQ], c1[NQ], pok[NQ];
        size_t obase[NQ];
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) {
            const int64_t P = tile * (16 * NQ) + 16 * nq + j;
            pok[nq] = P < cls_pix;
            const int64_t Pc = pok[nq] ? P : 0;
            const int q = (int)(Pc % Qc);
            const int m = (int)((Pc / Qc) % Mc);
            const int n = (int)(Pc / ((int64_t)Qc * Mc));
            const int ih0 = m + a, iw0 = q + b;  // u = 0 / v = 0 input position
            r0[nq] = ih0 < H;
            r1[nq] = ih0 - 1 >= 0 && ih0 - 1 < H;
            c0[nq] = iw0 < W;
            c1[nq] = iw0 - 1 >= 0 && iw0 - 1 < W;
            xb[nq] = 4u * (uint32_t)(((size_t)n * Cin + (size_t)G * Cq) * plane + (size_t)ih0 * W + iw0);
            obase[nq] = (size_t)n * COUT * oplane + (size_t)(2 * m + a) * OW + (2 * q + b);
        }

        f32x4 acc[MT][NQ];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq) acc[mt][nq] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // B operands of input channel cl of this lane group: the 2x2 input
        // neighbourhood of each pixel, (u,v) = (0,0) (0,1) (1,0) (1,1).  Range-checked
        // buffer loads: a tap outside the image (or a channel >= Cin) gets the offset
        // xbytes, past the end of x, and reads zero.  The loads are unconditional, so
        // the next channel's stay in flight while the current channel's MFMAs run
        // (masked loads in branches made the compiler wait for all of them).
        auto load_b = [&](int cl, float (&bv)[NQ][4]) {
            const bool ciok = G * Cq + cl < Cin;
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq) {
                const uint32_t o = xb[nq] + 4u * (uint32_t)cl * (uint32_t)plane;
                const bool ok = ciok && pok[nq];
                bv[nq][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    xr, (ok && r0[nq] && c0[nq]) ? o : xbytes, 0, 0));
                bv[nq][1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    xr, (ok && r0[nq] && c1[nq]) ? o - 4u : xbytes, 0, 0));
                bv[nq][2] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    xr, (ok && r1[nq] && c0[nq]) ? o - 4u * (uint32_t)W : xbytes, 0, 0));
                bv[nq][3] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    xr, (ok && r1[nq] && c1[nq]) ? o - 4u * (uint32_t)(W + 1) : xbytes, 0, 0));
            }
        };
        auto compute = [&](int cl, const float (&bv)[NQ][4]) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 av = *(const f32x4 *)(aw + mt * 16 * CS + 4 * cl);
#pragma unroll
                for (int tp = 0; tp < 4; ++tp)
#pragma unroll
                    for (int nq = 0; nq < NQ; ++nq)
                        acc[mt][nq] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[tp], bv[nq][tp],
                                                                           acc[mt][nq], 0, 0, 0);
            }
        };
        // three channel buffers: the loads of the next two channels are in flight while
        // the current one feeds the matrix cores.  Loads are unconditional (those past
        // the last channel are unused), so the waits on them stay partial.
        float bA[NQ][4], bB[NQ][4], bC[NQ][4];
        load_b(0, bA);
        load_b(1, bB);
        for (int cl = 0; cl < Cq; cl += 3) {
            load_b(cl + 2, bC);
            compute(cl, bA);
            load_b(cl + 3, bA);
            if (cl + 1 < Cq) compute(cl + 1, bB);
            load_b(cl + 4, bB);
            if (cl + 2 < Cq) compute(cl + 2, bC);
        }

        // ---- epilogue: D row 4G + r of tile mt = channel 16mt + 4G + r ----
        if constexpr (!SOFTMAX) {
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq)
                if (pok[nq]) {
                    float *yo = y + obase[nq];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int co = 16 * mt + 4 * G + r;
                            yo[(size_t)co * oplane] = acc[mt][nq][r] + lcb[co];
                        }
                }
            continue;
        }
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[mt][nq][r] += lcb[16 * mt + 4 * G + r];
                    mx = fmaxf(mx, acc[mt][nq][r]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            float sum = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = __expf(acc[mt][nq][r] - mx);
                    acc[mt][nq][r] = e;
                    sum += e;
                }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            const float inv = 1.f / sum;
            if (pok[nq]) {
                float *yo = y + obase[nq];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int co = 16 * mt + 4 * G + r;
                        const float v = (acc[mt][nq][r] * inv + lb2[co]) * scale;
                        yo[(size_t)co * oplane] = 1.f / (1.f + __expf(-v));
                    }
            }
        }
    }
}

template <int MT, bool SOFTMAX>
int launch_mt(const float *x, const float *w, const float *cb, const float *b2, float *y, int N,
              int Cin, int H, int W, int OH, int OW, float scale, hipStream_t stream) {
    constexpr int NQ = 2;
    const int Cq = (Cin + 3) / 4;
    const int KS = 4 * Cq;
    const size_t lds_bytes = ((size_t)16 * MT * (4 * KS + 4) + 2 * 16 * MT) * sizeof(float);
    if (lds_bytes > 160 * 1024) return PS_ERR_UNSUPPORTED;
    // byte offsets into x are 32-bit (range-checked buffer loads)
    if ((int64_t)N * Cin * H * W >= (1ll << 30)) return PS_ERR_UNSUPPORTED;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PS_ERR_HIP;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PS_ERR_HIP;
    // one workgroup per CU (the weight tile fills most of the LDS), a multiple
    // of 32 so every XCD holds whole (class pair) groups
    int wg_per_class = (ncu + 3) / 4;
    wg_per_class = ((wg_per_class + 7) / 8) * 8;
    const int nblocks = 4 * wg_per_class;
    // a per-device function attribute, so it is set on every launch
    if (lds_bytes > 65536 &&
        hipFuncSetAttribute((const void *)convT_softmax_f32<MT, NQ, SOFTMAX>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes) !=
            hipSuccess)
        return PS_ERR_HIP;
    hipLaunchKernelGGL((convT_softmax_f32<MT, NQ, SOFTMAX>), dim3(nblocks), dim3(kThreads),
                       lds_bytes, stream, x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, Cq,
                       wg_per_class);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_HIP;
}

template <bool SOFTMAX>
int launch_cout(const float *x, const float *w, const float *cb, const float *b2, float *y, int N,
                int Cin, int H, int W, int Cout, int OH, int OW, float scale,
                hipStream_t stream) {
    switch (Cout / 16) {
        case 1: return launch_mt<1, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
        case 2: return launch_mt<2, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
        case 3: return launch_mt<3, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
        case 4: return launch_mt<4, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
        case 5: return launch_mt<5, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
        case 6: return launch_mt<6, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
        case 7: return launch_mt<7, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
        case 8: return launch_mt<8, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, OH, OW, scale, stream);
    }
    return PS_ERR_UNSUPPORTED;
}

}  // namespace

int launch_convT_softmax(const float *x, const float *w, const float *convT_bias,
                         const float *bias2, float *y, int N, int Cin, int H, int W, int Cout,
                         int OH, int OW, float scale, hipStream_t stream) {
    return launch_cout<true>(x, w, convT_bias, bias2, y, N, Cin, H, W, Cout, OH, OW, scale,
                             stream);
}

int launch_convT(const float *x, const float *w, const float *convT_bias, float *y, int N,
                 int Cin, int H, int W, int Cout, int OH, int OW, hipStream_t stream) {
    return launch_cout<false>(x, w, convT_bias, nullptr, y, N, Cin, H, W, Cout, OH, OW, 1.f,
                              stream);
}

}  // namespace ps

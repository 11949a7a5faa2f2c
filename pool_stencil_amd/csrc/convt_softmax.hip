// Fused ConvTranspose2d(k4, s2, any padding p) -> softmax over channels -> +bias2 -> *scale
// -> sigmoid for gfx950.
//
// Definition (POPCORNBENCH page Kimi-K2.6 l2_p91, problem statement and its
// scatter loop):
//   t[n,co,oh,ow] = bias[co] + sum over (ci, ih, iw, kh, kw) with oh = 2*ih - p + kh,
//                   ow = 2*iw - p + kw of x[n,ci,ih,iw] * w[ci,co,kh,kw]
//   y = sigmoid((softmax_co(t) + bias2[co]) * scale)
//
// Parity decomposition (the page's phase table, written there for p = 1): output
// row oh = 2m + a only receives the kernel rows of one parity, kh = ka + 2u
// (u = 0, 1) with ka = (a + p) mod 2, from input rows ih = m + ra - u with
// ra = floor((a + p) / 2) (2*ih + kh = oh + p); for p = 1 that is kh = 1 - a + 2u
// from ih = m + a - u.  Columns likewise with (b, v).  Each of the four classes
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
//     channel per four K-steps, as range-checked buffer loads whose offsets are
//     fixed per tile (the channel advances the buffer resource, a scalar);
//   - A is read from LDS as 16-byte vectors covering four K-steps, one channel
//     ahead of the MFMAs that use it;
//   - the page's online max/sum recurrence is not needed: all channel values
//     of a pixel sit in registers, so the max is taken first and the sum of
//     exp(t - max) second, both in registers;
//   - the output stores are buffer stores: a per-lane offset for the pixel plus
//     a wave-uniform one for the channel, so they cost no address arithmetic;
//   - the four classes get workgroups in proportion to their pixel counts.
#include "ps_internal.h"

#include <math.h>

namespace ps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves: two per SIMD (12 measured slower)
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kMasked = 0x80000000u;  // an offset past the end of every tensor here

// floor(n / d) for n * d < 2^32, with m = ceil(2^32 / d) (m = 0 encodes d = 1).
__device__ __forceinline__ uint32_t fdiv(uint32_t n, uint32_t m) {
    return m ? __umulhi(n, m) : n;
}

// Divisors of the pixel decomposition, per row class a and column class b, and the
// blocks of each class (a, b) = (c / 2, c % 2): blocks [start[c], start[c + 1]).
struct ClassGeom {
    uint32_t Qc[2], mQ[2];  // columns of column class b, and ceil(2^32 / Qc[b])
    uint32_t Mc[2], mM[2];  // rows of row class a, and ceil(2^32 / Mc[a])
    int start[5];
};

// SOFTMAX = false: the same transposed conv with the epilogue left out (the
// stored intermediate of the page's unfused pipeline, or a plain
// ConvTranspose2d + bias).
template <int MT, int NQ, bool SOFTMAX>
__global__ __launch_bounds__(kThreads) void convT_softmax_f32(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cbias,
    const float *__restrict__ b2, float *__restrict__ y, int N, int Cin, int H, int W, int OH,
    int OW, int pad, float scale, int Cq, int Cout, ClassGeom geo) {
    // Cout output channels padded to COUT = 16*MT: the padded channels get zero weights,
    // a convT bias of -inf with the softmax (so they add nothing to the channel max and
    // sum) and no stores
    constexpr int COUT = 16 * MT;
    extern __shared__ float lds[];
    const int KS = 4 * Cq;          // K-steps per lane group
    const int CS = 4 * KS + 4;      // words per output channel row (padded)
    float *lw = lds;                // [COUT][4 lane groups][KS]
    float *lcb = lds + COUT * CS;   // [COUT] conv-transpose bias (times log2 e with the softmax)
    float *lb2 = lcb + COUT;        // [COUT] -bias2 * scale * log2 e

    // The classes get blocks in proportion to their pixel tiles (their row and column
    // counts differ by one), so every wave ends with about the same number of tiles.
    const int blk = blockIdx.x;
    const int cls = (blk >= geo.start[1]) + (blk >= geo.start[2]) + (blk >= geo.start[3]);
    const int a = cls >> 1, b = cls & 1;
    const int rank = blk - geo.start[cls];  // rank among the blocks of this class
    const int wg_per_class = geo.start[cls + 1] - geo.start[cls];
    const uint32_t Mc = geo.Mc[a], mM = geo.mM[a];  // rows of this class
    const uint32_t Qc = geo.Qc[b], mQ = geo.mQ[b];  // columns of this class
    // kernel row / column of tap u = 0 / v = 0, and the input row / column offsets
    const int ka = (a + pad) & 1, ra = (a + pad) >> 1;
    const int kb = (b + pad) & 1, rb = (b + pad) >> 1;

    // ---- stage A_ab: lw[co][G][s] = w[ci][co][ka+2u][kb+2v],
    //      ci = G*Cq + s/4, (u, v) = ((s%4)/2, (s%4)%2); zero for ci >= Cin or co >= Cout
    for (int e = threadIdx.x; e < COUT * 4 * KS; e += kThreads) {
        const int s = e % KS;
        const int G = (e / KS) & 3;
        const int co = e / (4 * KS);
        const int ci = G * Cq + (s >> 2);
        const int u = (s >> 1) & 1, v = s & 1;
        const int kh = ka + 2 * u, kw = kb + 2 * v;
        float val = 0.f;
        if (ci < Cin && co < Cout) val = w[(((size_t)ci * Cout + co) * 4 + kh) * 4 + kw];
        lw[co * CS + G * KS + s] = val;
    }
    for (int e = threadIdx.x; e < COUT; e += kThreads) {
        if (e < Cout) {
            const float cb = cbias ? cbias[e] : 0.f;
            lcb[e] = SOFTMAX ? cb * kLog2e : cb;
            if constexpr (SOFTMAX) lb2[e] = -b2[e] * scale * kLog2e;  // b2 is NULL without it
        } else {
            lcb[e] = SOFTMAX ? -INFINITY : 0.f;
            if constexpr (SOFTMAX) lb2[e] = 0.f;
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    // wave index, made visibly wave-uniform: the tile index and everything derived
    // from it (the per-channel buffer resources) then stay in scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;
    const int G = lane >> 4;
    const uint32_t cls_pix = (uint32_t)N * Mc * Qc;  // < 2^31 (host check)
    const uint32_t ntiles = (cls_pix + 16 * NQ - 1) / (16 * NQ);
    const uint32_t wstride = (uint32_t)wg_per_class * (kThreads / 64);
    const float *aw = lw + j * CS + G * KS;  // + mt*16*CS + s
    const uint32_t plane = (uint32_t)H * W;
    const uint32_t xbytes = 4u * (uint32_t)N * Cin * plane;   // < 2^31 (host check)
    const uint32_t oplane = (uint32_t)OH * OW;
    const uint32_t ybytes = 4u * (uint32_t)N * Cout * oplane;  // < 2^31 (host check)
    // channels 16*mt + 4G + r of the last channel tile at or past Cout are not stored
    const int ylim = Cout - 16 * (MT - 1) - 4 * G;
    const __amdgpu_buffer_rsrc_t yr = make_range_checked(y, ybytes);

    // Waves wv and wv + 4 share a SIMD and have the same work per tile; started
    // together they reach their (matrix-core-free) epilogues together and the matrix
    // core idles.  The second wave starts about half a tile later (2 x 8128 clocks).
    if (wv >= 4) {
        __builtin_amdgcn_s_sleep(127);
        __builtin_amdgcn_s_sleep(127);
    }
    for (uint32_t tile = (uint32_t)rank * (kThreads / 64) + wv; tile < ntiles; tile += wstride) {
        // Per-lane geometry of each of the NQ pixel groups: the byte offsets of the
        // 2x2 input neighbourhood (u,v) = (0,0) (0,1) (1,0) (1,1) in input channel
        // G*Cq, masked (kMasked) where the tap lies outside the image, and the byte
        // offset of output channel 4G of the pixel (kMasked past the last pixel).
        uint32_t xo[NQ][4], yo[NQ];
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) {
            const uint32_t P = tile * (16 * NQ) + 16 * nq + j;
            const bool pok = P < cls_pix;
            const uint32_t Pc = pok ? P : 0;
            const uint32_t t = fdiv(Pc, mQ);
            const uint32_t q = Pc - t * Qc;
            const uint32_t n = fdiv(t, mM);
            const uint32_t m = t - n * Mc;
            const int ih0 = (int)m + ra, iw0 = (int)q + rb;  // u = 0 / v = 0 input position
            const bool r0 = ih0 < H, r1 = ih0 >= 1 && ih0 - 1 < H;
            const bool c0 = iw0 < W, c1 = iw0 >= 1 && iw0 - 1 < W;
            const uint32_t o = 4u * ((n * Cin + G * Cq) * plane + (uint32_t)ih0 * W + iw0);
            xo[nq][0] = r0 && c0 ? o : kMasked;
            xo[nq][1] = r0 && c1 ? o - 4u : kMasked;
            xo[nq][2] = r1 && c0 ? o - 4u * W : kMasked;
            xo[nq][3] = r1 && c1 ? o - 4u * (W + 1) : kMasked;
            yo[nq] = pok ? 4u * ((n * Cout + 4 * G) * oplane + (2 * m + a) * OW + (2 * q + b))
                         : kMasked;
        }

        f32x4 acc[MT][NQ];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq) acc[mt][nq] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // B operands of input channel G*Cq + cl: range-checked buffer loads through a
        // resource that starts at channel cl of image 0, so the per-lane offsets stay
        // fixed for the whole tile and the loads need no vector arithmetic.  A masked
        // tap reads zero.  A channel >= Cin (only when Cin % 4 != 0) reads the next
        // image's data or zero; its weights are zero, and the input is finite.
        auto load_b = [&](int cl, float (&bv)[NQ][4]) {
            // (the resource words go through readfirstlane so that the compiler keeps
            // them in scalar registers instead of wrapping each load in a loop)
            const uint32_t sh = 4u * (uint32_t)cl * plane;
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)x + sh);
            const uint32_t hi = __builtin_amdgcn_readfirstlane(
                (uint32_t)(((uintptr_t)x + sh) >> 32));
            const uint32_t nrec = __builtin_amdgcn_readfirstlane(xbytes > sh ? xbytes - sh : 0u);
            const __amdgpu_buffer_rsrc_t xr = make_range_checked(
                (const void *)(((uint64_t)hi << 32) | lo), nrec);
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
                for (int tp = 0; tp < 4; ++tp)
                    bv[nq][tp] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(xr, xo[nq][tp], 0, 0));
        };
        // A operands of channel cl: 16-byte LDS reads covering its four K-steps.  The
        // first one (tile mt = 0) is read one channel ahead (a0), the others at the
        // start of the channel, where the MFMAs of tile 0 cover their latency.
        auto read_a = [&](int cl, int mt) { return *(const f32x4 *)(aw + mt * 16 * CS + 4 * cl); };
        auto compute = [&](int cl, const float (&bv)[NQ][4], const f32x4 &a0) {
            f32x4 av[MT];
            av[0] = a0;
#pragma unroll
            for (int mt = 1; mt < MT; ++mt) av[mt] = read_a(cl, mt);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int tp = 0; tp < 4; ++tp)
#pragma unroll
                    for (int nq = 0; nq < NQ; ++nq)
                        acc[mt][nq] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            av[mt][tp], bv[nq][tp], acc[mt][nq], 0, 0, 0);
        };
        // Three channel buffers for B: the loads of the next two channels are in flight
        // while the current one feeds the matrix cores.  Scheduling barriers keep the
        // compiler from sinking the loads down to their first use (it does so to save
        // registers, which exposes the whole memory latency).  B loads past the last
        // channel are issued and unused.
        float bA[NQ][4], bB[NQ][4], bC[NQ][4];
        f32x4 aX = read_a(0, 0), aY;
        load_b(0, bA);
        load_b(1, bB);
        __builtin_amdgcn_sched_barrier(0);
        // one channel: read A tile 0 of the next channel, then this channel's MFMAs
#define PS_CONVT_STEP(k, BCUR, ACUR, ANEXT)                                   \
    if (cl + (k) < Cq) {                                                     \
        if (cl + (k) + 1 < Cq) ANEXT = read_a(cl + (k) + 1, 0);              \
        compute(cl + (k), BCUR, ACUR);                                       \
    }                                                                        \
    __builtin_amdgcn_sched_barrier(0);
#define PS_CONVT_LOADB(k, BDST)     \
    load_b(cl + (k), BDST);         \
    __builtin_amdgcn_sched_barrier(0);
        for (int cl = 0; cl < Cq; cl += 6) {
            PS_CONVT_LOADB(2, bC)
            PS_CONVT_STEP(0, bA, aX, aY)
            PS_CONVT_LOADB(3, bA)
            PS_CONVT_STEP(1, bB, aY, aX)
            PS_CONVT_LOADB(4, bB)
            PS_CONVT_STEP(2, bC, aX, aY)
            PS_CONVT_LOADB(5, bC)
            PS_CONVT_STEP(3, bA, aY, aX)
            PS_CONVT_LOADB(6, bA)
            PS_CONVT_STEP(4, bB, aX, aY)
            PS_CONVT_LOADB(7, bB)
            PS_CONVT_STEP(5, bC, aY, aX)
        }
#undef PS_CONVT_STEP
#undef PS_CONVT_LOADB

        // ---- epilogue: D row 4G + r of tile mt = channel 16mt + 4G + r.  Stores go
        // through the output resource: the lane's offset (channel 4G of its pixel) plus
        // a wave-uniform offset for channel 16mt + r.
        if constexpr (!SOFTMAX) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float4 cb4 = *(const float4 *)(lcb + 16 * mt + 4 * G);
                const float cbv[4] = {cb4.x, cb4.y, cb4.z, cb4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int nq = 0; nq < NQ; ++nq)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __float_as_uint(acc[mt][nq][r] + cbv[r]), yr,
                            mt < MT - 1 || r < ylim ? yo[nq] : kMasked,
                            (int)(4u * (uint32_t)(16 * mt + r) * oplane), 0);
            }
            continue;
        }
        // exp2 form with the constants folded: t_c = y_c*log2e, e_c = 2^(t_c - max),
        // out_c = 1 / (1 + 2^(e_c * inv + b2'_c)), inv = -scale*log2e / sum_c e_c,
        // b2'_c = -bias2_c * scale * log2e (the written order: softmax, +bias2, *scale,
        // sigmoid).
        float inv[NQ];
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float4 cb4 = *(const float4 *)(lcb + 16 * mt + 4 * G);
                const float cbv[4] = {cb4.x, cb4.y, cb4.z, cb4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[mt][nq][r] = fmaf(acc[mt][nq][r], kLog2e, cbv[r]);
                    mx = fmaxf(mx, acc[mt][nq][r]);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            float sum = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[mt][nq][r] = __builtin_amdgcn_exp2f(acc[mt][nq][r] - mx);
                    sum += acc[mt][nq][r];
                }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            inv[nq] = -scale * kLog2e * __builtin_amdgcn_rcpf(sum);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float4 b4 = *(const float4 *)(lb2 + 16 * mt + 4 * G);
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int nq = 0; nq < NQ; ++nq) {
                    const float t = __builtin_amdgcn_exp2f(fmaf(acc[mt][nq][r], inv[nq], bv[r]));
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(__builtin_amdgcn_rcpf(1.f + t)), yr,
                        mt < MT - 1 || r < ylim ? yo[nq] : kMasked,
                        (int)(4u * (uint32_t)(16 * mt + r) * oplane), 0);
                }
        }
    }
}

template <int MT, bool SOFTMAX>
int launch_mt(const float *x, const float *w, const float *cb, const float *b2, float *y, int N,
              int Cin, int H, int W, int Cout, int OH, int OW, int pad, float scale,
              hipStream_t stream) {
    // pixel groups per wave tile: two (32 pixels) up to 128 channels; one beyond, so
    // that accumulators (4*MT*NQ) and A operands (4*MT) stay within the registers of
    // two waves per SIMD
    constexpr int NQ = MT > 8 ? 1 : 2;
    const int Cq = (Cin + 3) / 4;
    const int KS = 4 * Cq;
    const size_t lds_bytes = ((size_t)16 * MT * (4 * KS + 4) + 2 * 16 * MT) * sizeof(float);
    if (lds_bytes > 160 * 1024) return PS_ERR_UNSUPPORTED;
    // 32-bit byte offsets with a masked offset of 2^31: x (including the channels
    // that round Cin up to a multiple of 4) and y below 2^29 elements
    if ((int64_t)N * 4 * Cq * H * W >= (1ll << 29) ||
        (int64_t)N * 16 * MT * OH * OW >= (1ll << 29))
        return PS_ERR_UNSUPPORTED;
    ClassGeom geo;
    auto magic = [](int64_t d) -> uint32_t {
        return d <= 1 ? 0u : (uint32_t)(((1ll << 32) + d - 1) / d);
    };
    for (int c = 0; c < 2; ++c) {
        geo.Mc[c] = (uint32_t)((OH - c + 1) >> 1);
        geo.Qc[c] = (uint32_t)((OW - c + 1) >> 1);
        geo.mM[c] = magic(geo.Mc[c]);
        geo.mQ[c] = magic(geo.Qc[c]);
        // exactness of the multiply-shift divisions: dividend * divisor < 2^32
        const int64_t pix = (int64_t)N * geo.Mc[c] * ((OW + 1) >> 1);
        if (pix * ((OW + 1) >> 1) >= (1ll << 32) || pix >= (1ll << 31) ||
            (int64_t)N * geo.Mc[c] * geo.Mc[c] >= (1ll << 32))
            return PS_ERR_UNSUPPORTED;
    }
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PS_ERR_HIP;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PS_ERR_HIP;
    // one workgroup per CU (the weight tile fills most of the LDS), shared among the
    // four classes in proportion to their tiles (largest remainders), at least one each
    const int nblocks = ncu < 4 ? 4 : ncu;
    {
        int64_t tiles[4], total = 0;
        for (int c = 0; c < 4; ++c) {
            tiles[c] = ((int64_t)N * geo.Mc[c >> 1] * geo.Qc[c & 1] + 16 * NQ - 1) / (16 * NQ);
            total += tiles[c];
        }
        int share[4], used = 0;
        int64_t rem[4];
        for (int c = 0; c < 4; ++c) {
            const int64_t num = tiles[c] * (nblocks - 4);
            share[c] = 1 + (int)(num / total);
            rem[c] = num % total;
            used += share[c];
        }
        while (used < nblocks) {  // hand the rest out by largest remainder
            int best = 0;
            for (int c = 1; c < 4; ++c)
                if (rem[c] > rem[best]) best = c;
            ++share[best];
            rem[best] = -1;
            ++used;
        }
        geo.start[0] = 0;
        for (int c = 0; c < 4; ++c) geo.start[c + 1] = geo.start[c] + share[c];
    }
    // a per-device function attribute, so it is set on every launch
    if (lds_bytes > 65536 &&
        hipFuncSetAttribute((const void *)convT_softmax_f32<MT, NQ, SOFTMAX>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes) !=
            hipSuccess)
        return PS_ERR_HIP;
    return launch(convT_softmax_f32<MT, NQ, SOFTMAX>, dim3(nblocks), dim3(kThreads), lds_bytes,
                  stream, x, w, cb, b2, y, N, Cin, H, W, OH, OW, pad, scale, Cq, Cout, geo);
}

template <bool SOFTMAX>
int launch_cout(const float *x, const float *w, const float *cb, const float *b2, float *y, int N,
                int Cin, int H, int W, int Cout, int OH, int OW, int pad, float scale,
                hipStream_t stream) {
#define PS_CONVT_MT(M) \
    case M:                                                                                  \
        return launch_mt<M, SOFTMAX>(x, w, cb, b2, y, N, Cin, H, W, Cout, OH, OW, pad, scale,  \
                                     stream)
    // Cout rounded up to 16-channel tiles (the last one masked)
    switch ((Cout + 15) / 16) {
        PS_CONVT_MT(1); PS_CONVT_MT(2); PS_CONVT_MT(3); PS_CONVT_MT(4);
        PS_CONVT_MT(5); PS_CONVT_MT(6); PS_CONVT_MT(7); PS_CONVT_MT(8);
        PS_CONVT_MT(9); PS_CONVT_MT(10); PS_CONVT_MT(11); PS_CONVT_MT(12);
        PS_CONVT_MT(13); PS_CONVT_MT(14); PS_CONVT_MT(15); PS_CONVT_MT(16);
    }
#undef PS_CONVT_MT
    return PS_ERR_UNSUPPORTED;
}

}  // namespace

// The row-class kernel (convt_rows.hip: whole output lines per workgroup) where its
// envelope allows; the class-per-workgroup kernel above otherwise.
int launch_convT_softmax(const float *x, const float *w, const float *convT_bias,
                         const float *bias2, float *y, int N, int Cin, int H, int W, int Cout,
                         int OH, int OW, int pad, float scale, hipStream_t stream) {
    const int st = launch_convT_rows(x, w, convT_bias, bias2, y, N, Cin, H, W, Cout, OH, OW, pad,
                                     scale, true, stream);
    if (st != PS_ERR_UNSUPPORTED) return st;
    return launch_cout<true>(x, w, convT_bias, bias2, y, N, Cin, H, W, Cout, OH, OW, pad, scale,
                             stream);
}

int launch_convT(const float *x, const float *w, const float *convT_bias, float *y, int N,
                 int Cin, int H, int W, int Cout, int OH, int OW, int pad, hipStream_t stream) {
    const int st = launch_convT_rows(x, w, convT_bias, nullptr, y, N, Cin, H, W, Cout, OH, OW,
                                     pad, 1.f, false, stream);
    if (st != PS_ERR_UNSUPPORTED) return st;
    return launch_cout<false>(x, w, convT_bias, nullptr, y, N, Cin, H, W, Cout, OH, OW, pad, 1.f,
                              stream);
}

}  // namespace ps

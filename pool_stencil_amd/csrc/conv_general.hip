// General Conv2d (any kernel, stride, padding, dilation, channel counts) with
// either the fused tanh -> *scale -> +bias2 -> MaxPool2d epilogue (overlapping,
// padded or dilated pools included) or no epilogue at all (plain Conv2d + bias).
//
// Definitions (POPCORNBENCH page Kimi-K2.6 l2_p82: problem statement; the
// output-size formula of its analysis for any stride/padding/dilation; page
// Kimi-K2.6 l1_p42: the generic pooling index form with -inf padding):
//   y[n,co,oh,ow] = conv_bias[co] + sum_{ci,kh,kw} x[n,ci,oh*cs-cp+kh*cd, ow*cs-cp+kw*cd]
//                                                  * w[co,ci,kh,kw]          (zero padding)
//   z = tanh(y) * scale + bias2[co]
//   out[n,co,ph,pw] = max_{a,b<pk} z[n,co,ph*ps-pp+a*pd, pw*ps-pp+b*pd]     (-inf outside)
//
// Tiling.  A workgroup (4 waves) owns 64 output channels and a rectangle of
// PTH x PTW pooled outputs of one image.  The conv outputs those windows read
// form a CR x CC "region" (at most 256 pixels); the workgroup computes the
// whole region as an implicit GEMM on the matrix cores,
//   D[co][pixel] += A[co][k] * B[k][pixel],  k = (ci, kh, kw),
// with v_mfma_f32_16x16x4_f32 (one K-step = one tap x 4 input channels).
// Each wave holds 4 x 4 D tiles: all 64 channels x 4 blocks of 16 pixels.
//
// K is consumed in chunks of CK input channels.  Per chunk the input patch
// the region needs ((CR-1)*cs + (kH-1)*cd + 1 rows, likewise columns; zero
// outside the image) and the chunk's 64 x CK x kH*kW weights are staged in
// LDS:
//   - patch: [ci][row][col], channel stride padded to 16 (mod 64) words, so
//     the four lane groups of a wave (one input channel each) use disjoint
//     banks;
//   - weights: [tap][ci][co], the co position XOR-swizzled by (ci mod 4) in
//     16-channel blocks, so the four lane groups read four different
//     16-bank blocks.
//
// Epilogue (fused): the region is written to LDS as sgn*(y) (sgn = -1 when
// scale < 0) with -inf where the pool's padding lies, each thread takes the
// max over its pooled windows, and tanh is evaluated once per pooled output:
// tanh and v -> v*scale + b are monotone, so the max (scale >= 0) or the min
// (scale < 0) of y over a window gives the max of z.  A window holding only
// padding gives -inf, as the plain definition does.
// Epilogue (plain conv): D registers + bias go straight to global memory.
#include "ps_internal.h"

#include <math.h>

#include <initializer_list>

namespace ps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kCoTile = 64;     // output channels per workgroup
constexpr int kPix = 256;       // region pixels per workgroup (4 waves x 4 x 16)
constexpr int kYS = 260;        // LDS row stride of the staged region (4 mod 64 words)
constexpr int kFillBatch = 8;   // global loads in flight per thread during a fill

struct GenGeom {
    int Cin, H, W, Cout, kH, kW, cs, cp, cd, OH, OW;
    int pk, ps, pp, pd, PH, PW;        // pool (plain conv: 1, 1, 0, 1, OH, OW)
    int PTH, PTW, CR, CC, IR, IC, CK, PSZ;
    int tiles_h, tiles_w, co_tiles;
    float scale;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t *p, float v) { *p = f32_to_bf16_rne(v); }

template <typename TI, int EPI>
__global__ __launch_bounds__(kThreads, 2) void conv_general(
    const TI *__restrict__ x, const TI *__restrict__ w, const float *__restrict__ cbias,
    const float *__restrict__ b2, TI *__restrict__ y, const GenGeom g) {
    extern __shared__ float smem[];

    // ---- work item: channel tile fastest (those blocks share the input patch) ----
    uint32_t q = xcd_remap(blockIdx.x, gridDim.x);
    const int ct = kCoTile * (int)(q % (uint32_t)g.co_tiles);
    q /= (uint32_t)g.co_tiles;
    const int tw = (int)(q % (uint32_t)g.tiles_w);
    q /= (uint32_t)g.tiles_w;
    const int th = (int)(q % (uint32_t)g.tiles_h);
    const int n = (int)(q / (uint32_t)g.tiles_h);

    const int pr0 = th * g.PTH, pc0 = tw * g.PTW;      // first pooled row / column
    const int oh0 = pr0 * g.ps - g.pp;                 // conv row of region row 0
    const int ow0 = pc0 * g.ps - g.pp;
    const int ih0 = oh0 * g.cs - g.cp;                 // input row of patch row 0
    const int iw0 = ow0 * g.cs - g.cp;

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int c = lane & 15;    // B/D column: pixel within a 16-pixel block
    const int grp = lane >> 4;  // lane group: input channel of a K-step; D row block
    const int T = g.kH * g.kW;
    const int npix = g.CR * g.CC;

    // Region pixels of this lane: block jb = wv + 4*tt, pixel 16*jb + c.
    int off[4], orow[4], ocol[4];
    unsigned inside = 0;  // bit tt: the pixel is a real conv output
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int p = 16 * (wv + 4 * tt) + c;
        const int r = p / g.CC, cc = p - (p / g.CC) * g.CC;
        off[tt] = p < npix ? r * g.cs * g.IC + cc * g.cs : 0;
        orow[tt] = oh0 + r;
        ocol[tt] = ow0 + cc;
        if (p < npix && orow[tt] >= 0 && orow[tt] < g.OH && ocol[tt] >= 0 && ocol[tt] < g.OW)
            inside |= 1u << tt;
    }
    int aoff[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) aoff[cb] = grp * kCoTile + (((cb ^ grp) << 4) | c);

    f32x4 acc[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[cb][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    float *xs = smem;                    // [CK][PSZ]
    float *ws = smem + g.CK * g.PSZ;     // [T][CK][64] (swizzled)
    const TI *xn = x + (size_t)n * g.Cin * g.H * g.W;
    const size_t plane = (size_t)g.H * g.W;
    const int irc = g.IR * g.IC;
    const int pe = g.CK * irc;           // patch elements per chunk
    const int ckt = g.CK * T;
    const int we = kCoTile * ckt;        // weight elements per chunk

    for (int c0 = 0; c0 < g.Cin; c0 += g.CK) {
        if (c0 > 0) __syncthreads();     // every wave is done with the previous chunk
        // ---- input patch: all loads of a batch in flight, then the LDS writes ----
        for (int e0 = threadIdx.x; e0 < pe; e0 += kThreads * kFillBatch) {
            float v[kFillBatch];
            int dst[kFillBatch];
#pragma unroll
            for (int i = 0; i < kFillBatch; ++i) {
                const int e = e0 + i * kThreads;
                const int ci = e / irc;
                const int rem = e - ci * irc;
                const int r = rem / g.IC;
                const int col = rem - r * g.IC;
                const int ih = ih0 + r, iw = iw0 + col;
                const bool ok = e < pe && c0 + ci < g.Cin && ih >= 0 && ih < g.H && iw >= 0 &&
                                iw < g.W;
                v[i] = ok ? to_f32(xn[(size_t)(c0 + ci) * plane + (size_t)ih * g.W + iw]) : 0.f;
                dst[i] = e < pe ? ci * g.PSZ + rem : -1;
            }
#pragma unroll
            for (int i = 0; i < kFillBatch; ++i)
                if (dst[i] >= 0) xs[dst[i]] = v[i];
        }
        // ---- weights of the chunk: w[ct+co][c0+ci][tap] -> ws[tap][ci][co ^ swz] ----
        for (int e0 = threadIdx.x; e0 < we; e0 += kThreads * kFillBatch) {
            float v[kFillBatch];
            int dst[kFillBatch];
#pragma unroll
            for (int i = 0; i < kFillBatch; ++i) {
                const int e = e0 + i * kThreads;
                const int co = e / ckt;
                const int rem = e - co * ckt;
                const int ci = rem / T;
                const int t = rem - ci * T;
                const bool ok = e < we && ct + co < g.Cout && c0 + ci < g.Cin;
                v[i] = ok ? to_f32(w[((size_t)(ct + co) * g.Cin + c0 + ci) * T + t]) : 0.f;
                dst[i] = e < we ? (t * g.CK + ci) * kCoTile + (co ^ ((ci & 3) << 4)) : -1;
            }
#pragma unroll
            for (int i = 0; i < kFillBatch; ++i)
                if (dst[i] >= 0) ws[dst[i]] = v[i];
        }
        __syncthreads();

        // ---- MFMA over the chunk: taps outer, 4-channel groups inner ----
        for (int t = 0; t < T; ++t) {
            const int kh = t / g.kW, kw = t - (t / g.kW) * g.kW;
            const float *xa = xs + grp * g.PSZ + kh * g.cd * g.IC + kw * g.cd;
            const float *wa = ws + t * g.CK * kCoTile;
#pragma unroll 2
            for (int cq = 0; cq < g.CK; cq += 4) {
                float b[4], a[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) b[tt] = xa[cq * g.PSZ + off[tt]];
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) a[cb] = wa[cq * kCoTile + aoff[cb]];
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        acc[cb][tt] =
                            __builtin_amdgcn_mfma_f32_16x16x4f32(a[cb], b[tt], acc[cb][tt], 0, 0, 0);
            }
        }
    }

    if constexpr (EPI == 1) {
        // ---- plain conv: D row 4*grp + r of block cb is channel ct + 16cb + 4grp + r ----
        const size_t oplane = (size_t)g.OH * g.OW;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = ct + 16 * cb + 4 * grp + r;
                if (co >= g.Cout) continue;
                const float bias = cbias ? cbias[co] : 0.f;
                TI *yp = y + ((size_t)n * g.Cout + co) * oplane;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    if (inside & (1u << tt))
                        store_out(yp + (size_t)orow[tt] * g.OW + ocol[tt], acc[cb][tt][r] + bias);
            }
    } else {
        // ---- fused: stage sgn*y of the region (-inf on the pool's padding) ----
        const float sgn = g.scale < 0.f ? -1.f : 1.f;
        __syncthreads();                 // the region overwrites the chunk buffers
        float *ys = smem;                // [64][kYS]
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = 16 * cb + 4 * grp + r;
                const int co = ct + col;
                const float bias = (cbias && co < g.Cout) ? cbias[co] : 0.f;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int p = 16 * (wv + 4 * tt) + c;
                    if (p < npix)
                        ys[col * kYS + p] =
                            (inside & (1u << tt)) ? sgn * (acc[cb][tt][r] + bias) : -INFINITY;
                }
            }
        __syncthreads();
        const int ptile = g.PTH * g.PTW;
        for (int e = threadIdx.x; e < kCoTile * ptile; e += kThreads) {
            const int col = e / ptile;
            const int rem = e - col * ptile;
            const int pr = rem / g.PTW;
            const int pc = rem - pr * g.PTW;
            const int co = ct + col, ph = pr0 + pr, pw = pc0 + pc;
            if (co >= g.Cout || ph >= g.PH || pw >= g.PW) continue;
            const float *yr = ys + col * kYS + pr * g.ps * g.CC + pc * g.ps;
            float best = -INFINITY;
            for (int a = 0; a < g.pk; ++a)
                for (int bb = 0; bb < g.pk; ++bb) best = fmaxf(best, yr[a * g.pd * g.CC + bb * g.pd]);
            const float o = best == -INFINITY ? -INFINITY : tanhf(sgn * best) * g.scale + b2[co];
            store_out(y + (((size_t)n * g.Cout + co) * g.PH + ph) * g.PW + pw, o);
        }
    }
}

constexpr int pad_words_16mod64(int v) { return v + ((16 - (v % 64)) + 64) % 64; }

// Chooses the pooled tile, the region and the channel chunk.  Pure host
// arithmetic; false when no tile fits the LDS limits.
bool plan(GenGeom &g, int epi, int &lds_bytes) {
    const int T = g.kH * g.kW;
    const int cinp = (g.Cin + 3) / 4 * 4;
    int64_t best_cost = -1;
    GenGeom bestg = g;
    int best_lds = 0;
    const int maxh = g.PH < 64 ? g.PH : 64, maxw = g.PW < 256 ? g.PW : 256;
    for (int pth = 1; pth <= maxh; ++pth) {
        const int64_t cr = (int64_t)(pth - 1) * g.ps + (int64_t)(g.pk - 1) * g.pd + 1;
        if (cr > kPix) break;
        for (int ptw = 1; ptw <= maxw; ++ptw) {
            const int64_t cc = (int64_t)(ptw - 1) * g.ps + (int64_t)(g.pk - 1) * g.pd + 1;
            if (cr * cc > kPix) break;
            const int64_t ir = (cr - 1) * g.cs + (int64_t)(g.kH - 1) * g.cd + 1;
            const int64_t ic = (cc - 1) * g.cs + (int64_t)(g.kW - 1) * g.cd + 1;
            if (ir * ic > (1 << 20)) continue;
            const int psz = pad_words_16mod64((int)(ir * ic));
            // channel chunk: the largest of 16, 12, 8, 4 (<= Cin rounded up) that fits;
            // up to 80 KB (two workgroups per CU), else up to 160 KB
            int ck = 0, lds = 0;
            for (int lim : {80 * 1024, 160 * 1024}) {
                for (int k = 16; k >= 4; k -= 4) {
                    if (k > cinp && k > 4) continue;
                    const int64_t fill = ((int64_t)k * psz + (int64_t)T * k * kCoTile) * 4;
                    const int64_t need = epi == 0 && fill < kCoTile * kYS * 4 ? kCoTile * kYS * 4 : fill;
                    if (need <= lim) { ck = k; lds = (int)need; break; }
                }
                if (ck) break;
            }
            if (!ck) continue;
            const int64_t tiles = (int64_t)((g.PH + pth - 1) / pth) * ((g.PW + ptw - 1) / ptw);
            const int64_t nchunks = (g.Cin + ck - 1) / ck;
            // MFMA work is the same per tile; patch re-reads and LDS pressure break ties
            const int64_t cost = tiles * (1 << 20) * (lds > 80 * 1024 ? 2 : 1) +
                                 (tiles * nchunks * ck * ir * ic) / 64 - cc;
            if (best_cost < 0 || cost < best_cost) {
                best_cost = cost;
                bestg = g;
                bestg.PTH = pth; bestg.PTW = ptw; bestg.CR = (int)cr; bestg.CC = (int)cc;
                bestg.IR = (int)ir; bestg.IC = (int)ic; bestg.CK = ck; bestg.PSZ = psz;
                bestg.tiles_h = (g.PH + pth - 1) / pth;
                bestg.tiles_w = (g.PW + ptw - 1) / ptw;
                best_lds = lds;
            }
        }
    }
    if (best_cost < 0) return false;
    g = bestg;
    lds_bytes = best_lds;
    return true;
}

template <typename TI, int EPI>
int launch_t(const void *x, const void *w, const float *cb, const float *b2, void *y, int N,
             const GenGeom &g, int lds, hipStream_t stream) {
    const uint64_t nblocks = (uint64_t)N * g.tiles_h * g.tiles_w * g.co_tiles;
    if (nblocks > 0x7fffffffull) return PS_ERR_UNSUPPORTED;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute((const void *)conv_general<TI, EPI>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return PS_ERR_HIP;
    hipLaunchKernelGGL((conv_general<TI, EPI>), dim3((unsigned)nblocks), dim3(kThreads),
                       (size_t)lds, stream, (const TI *)x, (const TI *)w, cb, b2, (TI *)y, g);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_HIP;
}

}  // namespace

int launch_conv_general(const void *x, const void *w, const float *conv_bias, const float *bias2,
                        void *y, int dtype, int epi, int N, int Cin, int H, int W, int Cout,
                        int kH, int kW, int cs, int cp, int cd, int OH, int OW, float scale,
                        int pk, int ps_, int pp, int pd, int PH, int PW, hipStream_t stream) {
    GenGeom g{};
    g.Cin = Cin; g.H = H; g.W = W; g.Cout = Cout; g.kH = kH; g.kW = kW;
    g.cs = cs; g.cp = cp; g.cd = cd; g.OH = OH; g.OW = OW;
    if (epi == 1) {
        g.pk = 1; g.ps = 1; g.pp = 0; g.pd = 1; g.PH = OH; g.PW = OW; g.scale = 1.f;
    } else {
        g.pk = pk; g.ps = ps_; g.pp = pp; g.pd = pd; g.PH = PH; g.PW = PW; g.scale = scale;
    }
    g.co_tiles = (Cout + kCoTile - 1) / kCoTile;
    int lds = 0;
    if (!plan(g, epi, lds)) return PS_ERR_UNSUPPORTED;
    if (dtype == PS_BF16)
        return epi == 1 ? launch_t<uint16_t, 1>(x, w, conv_bias, bias2, y, N, g, lds, stream)
                        : launch_t<uint16_t, 0>(x, w, conv_bias, bias2, y, N, g, lds, stream);
    return epi == 1 ? launch_t<float, 1>(x, w, conv_bias, bias2, y, N, g, lds, stream)
                    : launch_t<float, 0>(x, w, conv_bias, bias2, y, N, g, lds, stream);
}

}  // namespace ps

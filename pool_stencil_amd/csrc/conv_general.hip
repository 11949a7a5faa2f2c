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
//   - weights: one 68-word row per k = ci*T + tap of the chunk, channel
//     co = 16*cb + c at word 4*c + cb, so one 16-byte LDS read gives a lane the
//     A operands of all four 16-channel blocks (and the fill's writes, 16
//     consecutive k of 4 channels per instruction, hit distinct banks).
// When a chunk's fill fits in registers, the next chunk's loads are issued
// before the current chunk's MFMA work and written to LDS after it.
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
#include <type_traits>

namespace ps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kCoTile = 64;     // output channels per workgroup
constexpr int kPix = 256;       // region pixels per workgroup (4 waves x 4 x 16)
constexpr int kYS = 260;        // LDS row stride of the staged region (4 mod 64 words)
constexpr int kMaxPR = 28;      // patch values per thread per fill pass
constexpr int kKB = 9;          // 16-wide weight k blocks per channel group per fill pass
constexpr int kMaxWR = 4 * kKB; // weights per thread per fill pass

struct GenGeom {
    int Cin, H, W, Cout, kH, kW, cs, cp, cd, OH, OW;
    int pk, ps, pp, pd, PH, PW;        // pool (plain conv: 1, 1, 0, 1, OH, OW)
    int PTH, PTW, CR, CC, IR, IC, CK, PSZ;
    int SW, lgSW, CPL, npass;          // patch fill: segment width, log2, segments per row
    int tiles_h, tiles_w, co_tiles;
    float scale;
    // ceil(2^32 / d) for the divisions by IR, CPL, CC, PTW and PTH*PTW (0 when d == 1);
    // the host checks n * d < 2^32 for every dividend n, which makes them exact.
    uint32_t mIR, mCPL, mCC, mPTW, mPT;
};

// floor(n / d) for 0 <= n, n * d < 2^32, with m = ceil(2^32 / d) (m = 0 encodes d = 1).
// Branch-free: with m = 0 the high product is 0 and n passes through the mask.
__device__ __forceinline__ int fdiv(int n, uint32_t m) {
    const uint32_t keep = 0u - (uint32_t)(m == 0u);
    return (int)(__umulhi((uint32_t)n, m) + ((uint32_t)n & keep));
}

constexpr int kWRS = 68;        // LDS words per weight row (64 channels + 4: conflict-free fill)

// Range-checked element loads: an offset at or past the resource's end reads zero.
__device__ __forceinline__ float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, const float *) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, const uint16_t *) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0));
}
constexpr uint32_t kMaskedOff = 0x80000000u;  // past the end of every tensor here
__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t *p, float v) { *p = f32_to_bf16_rne(v); }

template <typename TI, int EPI, bool PF>
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
        const int r = fdiv(p, g.mCC), cc = p - r * g.CC;
        off[tt] = p < npix ? r * g.cs * g.IC + cc * g.cs : 0;
        orow[tt] = oh0 + r;
        ocol[tt] = ow0 + cc;
        if (p < npix && orow[tt] >= 0 && orow[tt] < g.OH && ocol[tt] >= 0 && ocol[tt] < g.OW)
            inside |= 1u << tt;
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[cb][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    float *xs = smem;                    // [CK][PSZ]
    float *ws = smem + g.CK * g.PSZ;     // [CK*T][kWRS]: row k = ci*T + tap of the chunk
    // Loads are range-checked buffer loads with 32-bit byte offsets from
    // workgroup-uniform bases (the host keeps one image and the weight tensor below
    // 2^31 bytes), so each in-flight load holds one VGPR of address, and a value
    // outside the image (the conv's zero padding) or past the weights is an
    // unconditional load at a masked offset that reads zero: no branches.
    const TI *xn = x + (size_t)n * g.Cin * g.H * g.W;
    const uint32_t plane = (uint32_t)g.H * (uint32_t)g.W;
    constexpr uint32_t esz = sizeof(TI);
    const __amdgpu_buffer_rsrc_t xr = make_range_checked(xn, esz * (uint32_t)g.Cin * plane);
    const __amdgpu_buffer_rsrc_t wrs =
        make_range_checked(w, esz * (uint32_t)g.Cout * (uint32_t)g.Cin * (uint32_t)(g.kH * g.kW));
    const int ckt = g.CK * T;
    // Patch fill: the rows (ci, r) of a chunk are cut into segments of SW columns
    // (SW a power of two <= 64); one wave instruction covers 64/SW segments, lane ->
    // (segment, column), so loads are coalesced along a row and LDS writes are
    // consecutive.  Segment s of the chunk goes to instruction s / (4*spi) of wave
    // (s / spi) % 4.
    const int spi = 64 >> g.lgSW;
    const int sub = lane >> g.lgSW;
    const int scol = lane & (g.SW - 1);
    const int nseg = g.CK * g.IR * g.CPL;
    // Weight fill: a wave instruction covers 16 consecutive k (= ci*T + tap) of the
    // chunk for 4 channels co = cg + 16*cb (lane = 16*cb + kk).  Wave wv takes the
    // channel groups cg = wv + 4q (q < 4) and walks their k blocks in order, so the
    // addresses of one group differ by immediates.  The channel sits at word
    // 4*cg + cb of row k: one 16-byte LDS read gives a lane the A operands of its
    // four 16-channel blocks, and the 68-word row stride makes the fill's writes
    // conflict-free.
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int wcb = lane >> 4, wkk = lane & 15;
    const uint32_t wcs = (uint32_t)g.Cin * (uint32_t)T;   // weight elements per channel

    // One pass moves up to kMaxPR patch values and kMaxWR weights per thread through
    // registers.  With PF (the chunk takes one pass) the next chunk's loads are issued
    // before the current chunk's MFMA work and stored to LDS after it.
    float pr[kMaxPR], wr[kMaxWR];
    // The segment decode is the same for every chunk; an opaque zero keeps the
    // compiler from hoisting all of it out of the chunk loop (which would hold
    // several registers per segment for the whole kernel).
    auto lane_sub = [&]() {
        int z = 0;
        asm volatile("" : "+v"(z));
        return sub + z;
    };
    auto load = [&](int c0, int p) {
        const int kvalid = (g.Cin - c0 < g.CK ? g.Cin - c0 : g.CK) * T;
        const int sb = lane_sub();
#pragma unroll
        for (int j = 0; j < kMaxPR; ++j) {
            const int s = (wvu + 4 * (p * kMaxPR + j)) * spi + sb;
            const int row = fdiv(s < nseg ? s : 0, g.mCPL);
            const int col = ((s < nseg ? s : 0) - row * g.CPL) * g.SW + scol;
            const int ci = fdiv(row, g.mIR);
            const int ih = ih0 + row - ci * g.IR, iw = iw0 + col;
            // (bitwise: a short-circuit chain compiles to a branch per load)
            const bool ok = (s < nseg) & (col < g.IC) & (c0 + ci < g.Cin) & (ih >= 0) &
                            (ih < g.H) & (iw >= 0) & (iw < g.W);
            const uint32_t o = esz * ((uint32_t)(c0 + ci) * plane + (uint32_t)(ih * g.W + iw));
            pr[j] = load_elem(xr, ok ? o : kMaskedOff, x);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int co = ct + wvu + 4 * q + 16 * wcb;
            const uint32_t wq = esz * ((uint32_t)co * wcs + (uint32_t)(c0 * T + wkk));
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) {
                const int k = 16 * (p * kKB + kb) + wkk;
                const bool ok = (co < g.Cout) & (k < kvalid);
                wr[q * kKB + kb] =
                    load_elem(wrs, ok ? wq + esz * (uint32_t)(16 * (p * kKB + kb)) : kMaskedOff, w);
            }
        }
    };
    auto store = [&](int p) {
        const int sb = lane_sub();
#pragma unroll
        for (int j = 0; j < kMaxPR; ++j) {
            const int s = (wvu + 4 * (p * kMaxPR + j)) * spi + sb;
            if (s < nseg) {
                const int row = fdiv(s, g.mCPL);
                const int col = (s - row * g.CPL) * g.SW + scol;
                const int ci = fdiv(row, g.mIR);
                if (col < g.IC) xs[ci * g.PSZ + (row - ci * g.IR) * g.IC + col] = pr[j];
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) {
                const int k = 16 * (p * kKB + kb) + wkk;
                if (k < ckt) ws[k * kWRS + (((wvu + 4 * q) << 2) | wcb)] = wr[q * kKB + kb];
            }
    };

    // One-pass fill (PF): the lane's patch segments decode the same way for every
    // chunk, so the decode runs once.  xoff: byte offset of the value in the chunk's
    // first channel frame (masked outside the image); lidx: its LDS word, two 16-bit
    // indices per register, or a per-lane dummy word after the weights when the value
    // has no place.  Per chunk only scalar state changes: the resources start at
    // channel c0 (input) and tap row c0*T (weights).  Channels past Cin then read zero
    // (past the image's resource), and weight rows past Cin meet those zero patches.
    uint32_t xoff[PF ? kMaxPR : 1], lidx[PF ? (kMaxPR + 1) / 2 : 1], woff[4];
    const int dummy = g.CK * g.PSZ + ckt * kWRS + lane;
    if constexpr (PF) {
#pragma unroll
        for (int j = 0; j < kMaxPR; ++j) {
            const int s = (wvu + 4 * j) * spi + sub;
            const int sc = s < nseg ? s : 0;
            const int row = fdiv(sc, g.mCPL);
            const int col = (sc - row * g.CPL) * g.SW + scol;
            const int ci = fdiv(row, g.mIR);
            const int ih = ih0 + row - ci * g.IR, iw = iw0 + col;
            const bool placed = (s < nseg) & (col < g.IC);
            const bool inimg = placed & (ih >= 0) & (ih < g.H) & (iw >= 0) & (iw < g.W);
            xoff[j] = inimg ? esz * ((uint32_t)ci * plane + (uint32_t)(ih * g.W + iw)) : kMaskedOff;
            const uint32_t li = (uint32_t)(placed ? ci * g.PSZ + (row - ci * g.IR) * g.IC + col : dummy);
            if (j & 1) lidx[j >> 1] |= li << 16;
            else lidx[j >> 1] = li;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int co = ct + wvu + 4 * q + 16 * wcb;
            woff[q] = co < g.Cout ? esz * ((uint32_t)co * wcs + (uint32_t)wkk) : kMaskedOff;
        }
    }
    auto load_pf = [&](int c0) {
        const uint32_t xsh = esz * (uint32_t)c0 * plane;
        const uint32_t xlo = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)xn + xsh);
        const uint32_t xhi = __builtin_amdgcn_readfirstlane((uint32_t)(((uintptr_t)xn + xsh) >> 32));
        const uint32_t xnr = __builtin_amdgcn_readfirstlane(esz * (uint32_t)(g.Cin - c0) * plane);
        const __amdgpu_buffer_rsrc_t xrc =
            make_range_checked((const void *)(((uint64_t)xhi << 32) | xlo), xnr);
#pragma unroll
        for (int j = 0; j < kMaxPR; ++j) pr[j] = load_elem(xrc, xoff[j], x);
        const uint32_t wsh = esz * (uint32_t)(c0 * T);
        const uint32_t wlo = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)w + wsh);
        const uint32_t whi = __builtin_amdgcn_readfirstlane((uint32_t)(((uintptr_t)w + wsh) >> 32));
        const uint32_t wnr = __builtin_amdgcn_readfirstlane(
            esz * (uint32_t)g.Cout * wcs - wsh);
        const __amdgpu_buffer_rsrc_t wrc =
            make_range_checked((const void *)(((uint64_t)whi << 32) | wlo), wnr);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
                wr[q * kKB + kb] = load_elem(wrc, woff[q] + esz * (uint32_t)(16 * kb), w);
    };
    auto store_pf = [&]() {
#pragma unroll
        for (int j = 0; j < kMaxPR; ++j)
            smem[(j & 1) ? (lidx[j >> 1] >> 16) : (lidx[j >> 1] & 0xffffu)] = pr[j];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) {
                const int k = 16 * kb + wkk;
                const int wi = g.CK * g.PSZ + k * kWRS + (((wvu + 4 * q) << 2) | wcb);
                smem[k < ckt ? wi : dummy] = wr[q * kKB + kb];
            }
    };

    if constexpr (PF) load_pf(0);
    for (int c0 = 0; c0 < g.Cin; c0 += g.CK) {
        if (c0 > 0) __syncthreads();     // every wave is done with the previous chunk
        if constexpr (PF) {
            store_pf();
        } else {
            for (int p = 0; p < g.npass; ++p) {
                load(c0, p);
                store(p);
            }
        }
        __syncthreads();
        if constexpr (PF) {
            if (c0 + g.CK < g.Cin) load_pf(c0 + g.CK);
        }

        // ---- MFMA over the chunk: step = (tap, 4-channel group cq), taps outer ----
        // Operands of the next step are read from LDS while the 16 MFMAs of the
        // current one run, into two operand sets used in turn (fp32: the loop is unrolled
        // by two): rotating one set through the other had cost 8 register moves per step,
        // and on this chip VALU time adds to the matrix cores' time (1.08 -> 0.94 ms on
        // the 64 -> 128-channel workload).  A is weight row (cq + grp)*T + tap; B is the
        // patch at the tap's offset (the scalar state cq, tap, kw, tapoff advances with
        // the step).
        {
            const float4 *wa4 = (const float4 *)ws + grp * T * (kWRS / 4) + c;
            const float *xb = xs + grp * g.PSZ;
            const int nsteps = T * (g.CK >> 2);
            const int dstep_row = g.cd * g.IC - g.kW * g.cd;   // tapoff change at a new tap row
            int cq = 0, kw = 0, tapoff = 0, tap = 0;
            auto next = [&]() {
                cq += 4;
                if (cq == g.CK) {
                    cq = 0;
                    ++tap;
                    ++kw;
                    tapoff += g.cd;
                    if (kw == g.kW) {
                        kw = 0;
                        tapoff += dstep_row;
                    }
                }
            };
            auto read_ops = [&](float4 &a, float (&b)[4]) {
                a = wa4[(cq * T + tap) * (kWRS / 4)];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) b[tt] = xb[cq * g.PSZ + tapoff + off[tt]];
            };
            auto mfma_step = [&](const float4 &a, const float (&b)[4]) {
                const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        acc[cb][tt] =
                            __builtin_amdgcn_mfma_f32_16x16x4f32(av[cb], b[tt], acc[cb][tt], 0, 0, 0);
            };
            if constexpr (sizeof(TI) == 4) {
                float4 a0, a1;
                float b0[4], b1[4];
                read_ops(a0, b0);
                for (int st = 0; st < nsteps; st += 2) {
                    next();
                    if (st + 1 < nsteps) read_ops(a1, b1);
                    mfma_step(a0, b0);
                    if (st + 1 >= nsteps) break;
                    next();
                    if (st + 2 < nsteps) read_ops(a0, b0);
                    mfma_step(a1, b1);
                }
            } else {
                // bf16 inputs: the one-pass fill's prefetch registers leave no room for a
                // second operand set, so the next step's operands rotate through one
                (void)next;
                (void)read_ops;
                (void)mfma_step;
                int tap_c = 0;
                cq = 0;
                kw = 0;
                tapoff = 0;
                float4 a_c = wa4[0];
                float b_c[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) b_c[tt] = xb[off[tt]];
                for (int st = 0;; ++st) {
                    int cq_n = cq + 4, kw_n = kw, tap_n = tapoff;
                    if (cq_n == g.CK) {
                        cq_n = 0;
                        ++kw_n;
                        tap_n += g.cd;
                        if (kw_n == g.kW) {
                            kw_n = 0;
                            tap_n += dstep_row;
                        }
                    }
                    const int tap_i = cq_n == 0 ? tap_c + 1 : tap_c;
                    const bool more = st + 1 < nsteps;
                    float4 a_n = a_c;
                    float b_n[4] = {b_c[0], b_c[1], b_c[2], b_c[3]};
                    if (more) {
                        a_n = wa4[(cq_n * T + tap_i) * (kWRS / 4)];
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) b_n[tt] = xb[cq_n * g.PSZ + tap_n + off[tt]];
                    }
                    const float av[4] = {a_c.x, a_c.y, a_c.z, a_c.w};
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt)
                            acc[cb][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[cb], b_c[tt],
                                                                               acc[cb][tt], 0, 0, 0);
                    if (!more) break;
                    a_c = a_n;
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) b_c[tt] = b_n[tt];
                    cq = cq_n;
                    kw = kw_n;
                    tapoff = tap_n;
                    tap_c = tap_i;
                }
            }
        }
    }

    // conv bias of D row 4*grp + r of block cb (channel ct + 16cb + 4grp + r): the 16
    // loads at clamped indices, all in flight together (a conditional load per channel
    // had compiled to a branch and a wait each)
    float cbv[4][4];
    if (cbias) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = ct + 16 * cb + 4 * grp + r;
                cbv[cb][r] = cbias[co < g.Cout ? co : 0];
            }
    } else {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) cbv[cb][r] = 0.f;
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
                const float bias = cbv[cb][r];
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
        float *lb2 = smem + kCoTile * kYS;  // [64] bias2 of the channel tile
        if (threadIdx.x < kCoTile)
            lb2[threadIdx.x] = ct + (int)threadIdx.x < g.Cout ? b2[ct + threadIdx.x] : 0.f;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = 16 * cb + 4 * grp + r;
                const float bias = cbv[cb][r];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int p = 16 * (wv + 4 * tt) + c;
                    if (p < npix)
                        ys[col * kYS + p] =
                            (inside & (1u << tt)) ? sgn * (acc[cb][tt][r] + bias) : -INFINITY;
                }
            }
        __syncthreads();
        // ---- pool: thread (pooled pixel q, channel group gi) takes the pixel's window
        // in channels [c_lo, c_hi): the window's LDS addresses are computed once and step
        // by one region row per channel, and windows of 2-4 with dilation 1 are unrolled
        // with immediate offsets (a per-output index decode and runtime window loops had
        // cost about 50 VALU instructions per pooled output)
        const int ptile = g.PTH * g.PTW;  // <= kPix: the region holds every window
        const int ngrp = kThreads / ptile;
        const int gi = fdiv(threadIdx.x, g.mPT);
        const int q = threadIdx.x - gi * ptile;
        const int pr = fdiv(q, g.mPTW), pc = q - pr * g.PTW;
        const int ph = pr0 + pr, pw = pc0 + pc;
        const int cpg = (kCoTile + ngrp - 1) / ngrp;
        const int c_lo = gi * cpg;
        const int c_hi = min(min(kCoTile, c_lo + cpg), g.Cout - ct);
        if (gi < ngrp && ph < g.PH && pw < g.PW && c_lo < c_hi) {
            const float *yb = ys + c_lo * kYS + pr * g.ps * g.CC + pc * g.ps;
            TI *yp = y + (((size_t)n * g.Cout + ct + c_lo) * g.PH + ph) * g.PW + pw;
            const size_t cstride = (size_t)g.PH * g.PW;
            const float scale = g.scale;
            auto finish = [&](int col, float best) {
                const float o =
                    best == -INFINITY ? -INFINITY : tanh_exp(sgn * best) * scale + lb2[col];
                store_out(yp, o);
                yp += cstride;
            };
            auto unrolled = [&](auto KC) {
                constexpr int K = decltype(KC)::value;
                for (int col = c_lo; col < c_hi; ++col, yb += kYS) {
                    float best = -INFINITY;
#pragma unroll
                    for (int a = 0; a < K; ++a) {
                        const float *row = yb + a * g.CC;
#pragma unroll
                        for (int bb = 0; bb < K; ++bb) best = fmaxf(best, row[bb]);
                    }
                    finish(col, best);
                }
            };
            if (g.pd == 1 && g.pk == 3) {
                unrolled(std::integral_constant<int, 3>{});
            } else if (g.pd == 1 && g.pk == 2) {
                unrolled(std::integral_constant<int, 2>{});
            } else if (g.pd == 1 && g.pk == 4) {
                unrolled(std::integral_constant<int, 4>{});
            } else {
                for (int col = c_lo; col < c_hi; ++col, yb += kYS) {
                    float best = -INFINITY;
                    for (int a = 0; a < g.pk; ++a)
                        for (int bb = 0; bb < g.pk; ++bb)
                            best = fmaxf(best, yb[a * g.pd * g.CC + bb * g.pd]);
                    finish(col, best);
                }
            }
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
            int sw = 1, lg = 0;
            while (sw < ic && sw < 64) { sw *= 2; ++lg; }
            const int cpl = (int)((ic + sw - 1) / sw);
            const int spi = 64 / sw;
            // channel chunk: prefer the largest of 16, 12, 8, 4 (<= Cin rounded up) whose
            // fill takes one register pass (prefetch) within 80 KB of LDS (two workgroups
            // per CU); else the largest that fits 80 KB, else 160 KB.
            int ck = 0, lds = 0, npass = 0;
            for (int mode = 0; mode < 3 && !ck; ++mode) {
                const int64_t lim = mode < 2 ? 80 * 1024 : 160 * 1024;
                for (int k = 16; k >= 4; k -= 4) {
                    if (k > cinp && k > 4) continue;
                    // patch + weights + a 64-word dummy area for the one-pass fill's stores
                    const int64_t fill = ((int64_t)k * psz + (int64_t)T * k * kWRS + 64) * 4;
                    // (the fused epilogue's region + bias2 reuse the chunk buffers)
                    const int64_t epi_lds = (int64_t)kCoTile * (kYS + 1) * 4;
                    const int64_t need = epi == 0 && fill < epi_lds ? epi_lds : fill;
                    const int64_t npr = ((int64_t)k * ir * cpl + 4 * spi - 1) / (4 * spi);
                    const int64_t nkb = ((int64_t)k * T + 15) / 16;
                    const int64_t np1 = (npr + kMaxPR - 1) / kMaxPR, np2 = (nkb + kKB - 1) / kKB;
                    const int64_t np = np1 > np2 ? np1 : np2;
                    if (need > lim || (mode == 0 && np > 1)) continue;
                    ck = k; lds = (int)need; npass = (int)np;
                    break;
                }
            }
            if (!ck) continue;
            const int64_t tiles = (int64_t)((g.PH + pth - 1) / pth) * ((g.PW + ptw - 1) / ptw);
            const int64_t nchunks = (g.Cin + ck - 1) / ck;
            // MFMA work is the same per tile; exposed fill latency (no prefetch), one
            // workgroup per CU, and patch re-reads break ties
            const int64_t cost = tiles * (1 << 20) * (lds > 80 * 1024 ? 2 : 1) * (npass > 1 ? 3 : 2) +
                                 (tiles * nchunks * ck * ir * ic) / 64 - cc;
            if (best_cost < 0 || cost < best_cost) {
                best_cost = cost;
                bestg = g;
                bestg.PTH = pth; bestg.PTW = ptw; bestg.CR = (int)cr; bestg.CC = (int)cc;
                bestg.IR = (int)ir; bestg.IC = (int)ic; bestg.CK = ck; bestg.PSZ = psz;
                bestg.SW = sw; bestg.lgSW = lg; bestg.CPL = cpl; bestg.npass = npass;
                bestg.tiles_h = (g.PH + pth - 1) / pth;
                bestg.tiles_w = (g.PW + ptw - 1) / ptw;
                best_lds = lds;
            }
        }
    }
    if (best_cost < 0) return false;
    // exactness of the multiply-shift divisions: every dividend n has n * d < 2^32
    const int64_t nseg = (int64_t)bestg.CK * bestg.IR * bestg.CPL;
    const int64_t ptile = (int64_t)bestg.PTH * bestg.PTW;
    if (nseg * bestg.CPL >= (1ll << 32) || nseg * bestg.IR >= (1ll << 32) ||
        (int64_t)kPix * bestg.CC >= (1ll << 32) || kCoTile * ptile * ptile >= (1ll << 32))
        return false;
    auto magic = [](int64_t d) -> uint32_t {
        return d <= 1 ? 0u : (uint32_t)(((1ll << 32) + d - 1) / d);
    };
    bestg.mIR = magic(bestg.IR);
    bestg.mCPL = magic(bestg.CPL);
    bestg.mCC = magic(bestg.CC);
    bestg.mPTW = magic(bestg.PTW);
    bestg.mPT = magic(ptile);
    g = bestg;
    lds_bytes = best_lds;
    return true;
}

template <typename TI, int EPI, bool PF>
int launch_t(const void *x, const void *w, const float *cb, const float *b2, void *y, int N,
             const GenGeom &g, int lds, hipStream_t stream) {
    const uint64_t nblocks = (uint64_t)N * g.tiles_h * g.tiles_w * g.co_tiles;
    if (nblocks > 0x7fffffffull) return PS_ERR_UNSUPPORTED;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute((const void *)conv_general<TI, EPI, PF>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return PS_ERR_HIP;
    return launch(conv_general<TI, EPI, PF>, dim3((unsigned)nblocks), dim3(kThreads),
                  (size_t)lds, stream, (const TI *)x, (const TI *)w, cb, b2, (TI *)y, g);
}

template <typename TI, int EPI>
int launch_e(const void *x, const void *w, const float *cb, const float *b2, void *y, int N,
             const GenGeom &g, int lds, hipStream_t stream) {
    return g.npass == 1 ? launch_t<TI, EPI, true>(x, w, cb, b2, y, N, g, lds, stream)
                        : launch_t<TI, EPI, false>(x, w, cb, b2, y, N, g, lds, stream);
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
    // 32-bit byte offsets with a masked offset of 2^31: one image and the weights
    // below 2^31 bytes
    const int64_t esz = dtype == PS_BF16 ? 2 : 4;
    if ((int64_t)Cin * H * W * esz >= (1ll << 31) || (int64_t)Cout * Cin * kH * kW * esz >= (1ll << 31))
        return PS_ERR_UNSUPPORTED;
    int lds = 0;
    if (!plan(g, epi, lds)) return PS_ERR_UNSUPPORTED;
    if (dtype == PS_BF16)
        return epi == 1 ? launch_e<uint16_t, 1>(x, w, conv_bias, bias2, y, N, g, lds, stream)
                        : launch_e<uint16_t, 0>(x, w, conv_bias, bias2, y, N, g, lds, stream);
    return epi == 1 ? launch_e<float, 1>(x, w, conv_bias, bias2, y, N, g, lds, stream)
                    : launch_e<float, 0>(x, w, conv_bias, bias2, y, N, g, lds, stream);
}

}  // namespace ps

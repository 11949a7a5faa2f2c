// bf16 ConvTranspose2d(k4, s2, any padding p) -> softmax over channels -> +bias2
// -> *scale -> sigmoid for gfx950: bf16 x, w and output, fp32 accumulation.
//
// Same definition and parity decomposition as the fp32 kernel (POPCORNBENCH
// page Kimi-K2.6 l2_p91: problem statement, scatter loop and phase table):
// output row oh = 2m + a, column ow = 2q + b receives kernel taps
// kh = ka + 2u, kw = kb + 2v from input (m + ra - u, q + rb - v), with
// ka = (a + p) mod 2, ra = floor((a + p) / 2) and likewise kb, rb (for p = 1:
// kh = 1 - a + 2u from row m + a - u), so each parity class (a, b) is a dense
// GEMM with K = 4*Cin, k = 4*ci + (2u + v).
// The page weighs reduced precision for this problem and keeps fp32; this
// variant takes bf16 operands (products exact in fp32) for the bf16 matrix
// cores.
//
// Kernel layout:
//   - a workgroup (8 waves) serves one ROW class a and holds the bf16 weight
//     matrices of both column classes (a, 0) and (a, 1) in LDS (2 x Cout x 4*Cin);
//   - a wave owns 32 consecutive pixels (n, m, q) of the row class (flattened,
//     so no lanes idle at row ends) and computes them for b = 0 and then b = 1,
//     so the two interleaved halves of those output rows are written back to
//     back by the same wave and meet in L2;
//   - v_mfma_f32_32x32x16_bf16: D tiles of 32 channels x 32 pixels; a lane
//     holds 16 channels of one pixel per tile and its partner lane (xor 32)
//     the other 16, so the channel softmax needs one lane exchange;
//   - A (weights) is a 16-byte LDS read per MFMA; B (input) is the 2x2 input
//     neighbourhood of the lane's pixel for 2 channels, read with range-checked
//     buffer loads (taps outside the image read as zero); both are fetched one
//     K-step ahead;
//   - epilogue in exp2 form with the constants folded:
//       e_c = exp2(t_c*log2e - max), out_c = 1 / (1 + exp2(e_c*inv' + b2'_c))
//     with inv' = -scale*log2e/sum and b2'_c = -bias2_c*scale*log2e.
#include "ps_internal.h"

#include <math.h>

namespace ps {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
// K-steps of input loads in flight: 4, or 2 for 128 channels (register budget)
template <int MT>
constexpr int ring_steps() { return MT >= 4 ? 2 : 4; }

constexpr int kThreads = 512;  // 8 waves: two per SIMD
constexpr float kLog2e = 1.4426950408889634f;


template <int MT>  // Cout = 32 * MT
__global__ __launch_bounds__(kThreads, 1) void convT_softmax_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const float *__restrict__ cbias, const float *__restrict__ b2, uint16_t *__restrict__ y,
    int N, int Cin, int H, int W, int OH, int OW, int pad, float scale, int C4,
    int wg_per_class) {
    constexpr int COUT = 32 * MT;
    constexpr int kRing = ring_steps<MT>();
    extern __shared__ float lds[];
    const int K = 4 * C4;                    // k = 4*ci + tap, tap = 2u + v
    const int KP = K + 8;                    // bf16 per LDS row (16-byte pad)
    uint16_t *la = (uint16_t *)lds;          // [b][COUT][KP]
    float *lcb = lds + COUT * KP;            // conv-transpose bias * log2e
    float *lb2 = lcb + COUT;                 // -bias2 * scale * log2e

    // Block b runs on XCD b % 8; blocks b and b + 8 (same XCD) take the two row
    // classes, so an XCD's L2 sees both halves of the input rows it reads.
    const int blk = blockIdx.x;
    const int a = (blk >> 3) & 1;
    const int rank = (blk & 7) + 8 * (blk >> 4);
    const int Mc = (OH - a + 1) >> 1;        // output rows of this row class
    const int ka = (a + pad) & 1, ra = (a + pad) >> 1;

    for (int e = threadIdx.x; e < 2 * COUT * K; e += kThreads) {
        const int k = e % K;
        const int rest = e / K;
        const int co = rest % COUT, b = rest / COUT;
        const int ci = k >> 2, u = (k >> 1) & 1, v = k & 1;
        const int kh = ka + 2 * u, kw = ((b + pad) & 1) + 2 * v;
        la[(b * COUT + co) * KP + k] = ci < Cin ? w[(((size_t)ci * COUT + co) * 4 + kh) * 4 + kw] : 0;
    }
    for (int e = threadIdx.x; e < COUT; e += kThreads) {
        lcb[e] = (cbias ? cbias[e] : 0.f) * kLog2e;
        lb2[e] = -b2[e] * scale * kLog2e;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int j = lane & 31;  // pixel (B/D column) and A row within a 32-channel tile
    const int h = lane >> 5;  // K half of a step; D row half
    const int Qmax = (OW + 1) >> 1;          // columns q of the wider column class
    // pixels of this row class, flattened as P = (n*Mc + m)*Qmax + q; a wave tile is 32
    // consecutive P (it may span two output rows)
    const int npix = N * Mc * Qmax;
    const int ntiles = (npix + 31) / 32;
    const int wstride = wg_per_class * (kThreads / 64);
    const int plane = H * W;
    const int oplane = OH * OW;
    const int nsteps = C4 / 4;               // K-steps of 16 (4 channels x 4 taps)
    const float ninv_s = -scale * kLog2e;
    // range-checked view of x (raw buffer, byte offsets; the host keeps its size
    // below 2^31 bytes)
    const uint32_t xbytes = 2u * (uint32_t)(N * Cin * plane);
    const __amdgpu_buffer_rsrc_t xr = make_range_checked(x, xbytes);

    for (int tile = rank * (kThreads / 64) + wv; tile < ntiles; tile += wstride) {
        // element offsets from the tensor bases (the host keeps N*Cin*H*W, N*Cout*OH*OW
        // and the pixel count below 2^31)
        const int P = 32 * tile + j;
        const bool inr = P < npix;
        const int Pc = inr ? P : 0;
        const int q = Pc % Qmax;
        const int m = (Pc / Qmax) % Mc;
        const int n = Pc / (Qmax * Mc);
        const int ih0 = m + ra;               // input row of tap u = 0
        const bool r0 = ih0 < H, r1 = ih0 >= 1 && ih0 - 1 < H;
        const uint32_t xrow = (uint32_t)((n * Cin + 2 * h) * plane + ih0 * W);
        const uint32_t yrow = (uint32_t)(n * COUT * oplane + (2 * m + a) * OW);

#pragma unroll 1
        for (int b = 0; b < 2; ++b) {
            const int Qc = (OW - b + 1) >> 1;
            const bool pok = inr && q < Qc;
            const int iw0 = q + ((b + pad) >> 1);  // input column of tap v = 0
            const bool c0 = iw0 < W, c1 = iw0 >= 1 && iw0 - 1 < W;
            const bool m00 = pok && r0 && c0, m01 = pok && r0 && c1;
            const bool m10 = pok && r1 && c0, m11 = pok && r1 && c1;
            const uint32_t xb = xrow + (uint32_t)iw0;

            // B of step s: channels 4s + 2h + {0, 1}, taps (u,v) = 00 01 10 11, read with
            // range-checked buffer loads: a tap outside the image (or a channel >= Cin) is
            // given the byte offset xbytes, one past the end of x, which the hardware
            // range check turns into a zero read (no branches, no selects).
            auto load_b = [&](int s, uint32_t (&r)[8]) {
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    const bool ok = 4 * s + 2 * h + ch < Cin;
                    const uint32_t o = 2u * (xb + (uint32_t)((4 * s + ch) * plane));
                    r[4 * ch + 0] = __builtin_amdgcn_raw_buffer_load_b16(
                        xr, (ok && m00) ? o : xbytes, 0, 0);
                    r[4 * ch + 1] = __builtin_amdgcn_raw_buffer_load_b16(
                        xr, (ok && m01) ? o - 2u : xbytes, 0, 0);
                    r[4 * ch + 2] = __builtin_amdgcn_raw_buffer_load_b16(
                        xr, (ok && m10) ? o - 2u * (uint32_t)W : xbytes, 0, 0);
                    r[4 * ch + 3] = __builtin_amdgcn_raw_buffer_load_b16(
                        xr, (ok && m11) ? o - 2u * (uint32_t)(W + 1) : xbytes, 0, 0);
                }
            };
            const uint16_t *ab = la + (b * COUT + j) * KP + 8 * h;
            auto load_a = [&](int s, uint4 (&av)[MT]) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = *(const uint4 *)(ab + mt * 32 * KP + 16 * s);
            };

            f32x16 acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;

            // The 16-bit input values of the next kRing K-steps are held unpacked in a
            // ring carried from trip to trip; a step packs its values (the first use of
            // the loaded data, so the only wait on them) kRing steps after they were
            // requested, then refills its ring slot.  The step count is a multiple of
            // kRing; refills past the last step read channels >= Cin (zeros).  A is read
            // from LDS one step ahead.
            uint32_t raw[kRing][8];
#pragma unroll
            for (int d = 0; d < kRing; ++d) load_b(d, raw[d]);
            uint4 acur[MT], anxt[MT];
            load_a(0, acur);
            for (int s0 = 0; s0 < nsteps; s0 += kRing) {
#pragma unroll
                for (int d = 0; d < kRing; ++d) {
                    const int s = s0 + d;
                    const u16x8 bv = (u16x8){(unsigned short)raw[d][0], (unsigned short)raw[d][1],
                                             (unsigned short)raw[d][2], (unsigned short)raw[d][3],
                                             (unsigned short)raw[d][4], (unsigned short)raw[d][5],
                                             (unsigned short)raw[d][6], (unsigned short)raw[d][7]};
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, bv);
                    load_b(s + kRing, raw[d]);
                    load_a(s + 1 < nsteps ? s + 1 : s, anxt);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, acur[mt]), bop, acc[mt], 0, 0, 0);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acur[mt] = anxt[mt];
                }
            }

            // ---- epilogue: D element i of tile mt = channel 32mt + 8(i/4) + 4h + i%4 ----
            float mx = -INFINITY;
            // the 4 channels of a D quad are consecutive: one 16-byte read of the biases
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const float4 cb4 = *(const float4 *)(lcb + 32 * mt + 8 * i4 + 4 * h);
                    const float cbv[4] = {cb4.x, cb4.y, cb4.z, cb4.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * i4 + r;
                        acc[mt][i] = fmaf(acc[mt][i], kLog2e, cbv[r]);
                        mx = fmaxf(mx, acc[mt][i]);
                    }
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            float sum = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc[mt][i] = __builtin_amdgcn_exp2f(acc[mt][i] - mx);
                    sum += acc[mt][i];
                }
            sum += __shfl_xor(sum, 32);
            const float inv = ninv_s * __builtin_amdgcn_rcpf(sum);
            if (pok) {
                const uint32_t yo = yrow + (uint32_t)(2 * q + b);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        const int co0 = 32 * mt + 8 * i4 + 4 * h;
                        const float4 b4 = *(const float4 *)(lb2 + co0);
                        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float t =
                                __builtin_amdgcn_exp2f(fmaf(acc[mt][4 * i4 + r], inv, bv[r]));
                            y[yo + (uint32_t)(co0 + r) * (uint32_t)oplane] =
                                f32_to_bf16_rne(__builtin_amdgcn_rcpf(1.f + t));
                        }
                    }
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// Staged variant, taken when W % 8 == 0 and its buffers fit the LDS.
//
// Indexing the pixels of a row class by input position instead: output row 2m + a
// takes input rows r - u with r = m + ra, and output column 2c - p + (b ^ (p mod 2))
// takes input columns c - v (u, v in {0, 1}) with kernel taps kh = ka + 2u,
// kw = kb + 2v, so the B operand of position (r, c) is the same for both column
// classes b and one B fragment feeds the MFMAs of both (positions c = floor(p/2) ..
// floor((OW - 1 + p)/2) cover every output column; ow outside [0, OW) is masked).
//
// Input channels are staged 8 at a time in LDS, channel-last: [slot][col + 1][8
// channels], 16 bytes per entry, with zero entries at columns -1, W and W + 1, so a lane's B
// fragment (8 channels of one tap) is one 16-byte LDS read.  The global reads that
// fill a chunk are 16 bytes wide (8 columns of one channel) and are issued one chunk
// ahead; a thread transposes two channels x 8 columns with byte permutes into 8
// 4-byte LDS writes.  K order: k = 32*(ci/8) + 8*(2u + v) + ci%8; K-step s = (chunk
// ci/8, u), lane half h holding tap v = h.
//
// Work item: 256 consecutive positions m*Wc + (c - cmin) of one image and row class
// (8 waves x 32, Wc positions per row), which touch at most `slots` input rows.
constexpr int kStagedPix = 256;
constexpr int kStageRow = 66;  // bf16 per row of a wave's output staging (64 + pad)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int MT>  // Cout = 32 * MT
__global__ __launch_bounds__(kThreads, 1) void convT_softmax_bf16_staged(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const float *__restrict__ cbias, const float *__restrict__ b2, uint16_t *__restrict__ y,
    int N, int Cin, int H, int W, int OH, int OW, int pad, float scale, int C8, int slots,
    int wg_per_class) {
    constexpr int COUT = 32 * MT;
    extern __shared__ float lds[];
    const int K = 4 * C8;
    const int KP = K + 8;                         // bf16 per weight row (16-byte pad)
    uint16_t *la = (uint16_t *)lds;               // [b][COUT][KP]
    float *lcb = lds + COUT * KP;                 // conv-transpose bias * log2e
    float *lb2 = lcb + COUT;                      // -bias2 * scale * log2e
    uint4 *lx = (uint4 *)(lb2 + COUT);            // [2][slots][W + 3] input entries
    const int WE = W + 3;                         // input columns -1 .. W + 1
    const int bufsz = slots * WE;
    // per wave: 8 channels x 64 output columns of bf16 outputs on their way to memory
    uint16_t *lo = (uint16_t *)(lx + 2 * bufsz) + (threadIdx.x >> 6) * 8 * kStageRow;

    const int blk = blockIdx.x;
    const int a = (blk >> 3) & 1;
    const int rank = (blk & 7) + 8 * (blk >> 4);
    const int Mc = (OH - a + 1) >> 1;             // output rows 2m + a of this row class
    const int ka = (a + pad) & 1, ra = (a + pad) >> 1;  // input row m + ra - u, tap ka + 2u
    // Positions: input columns c = cmin .. cmax (tap v = 0); class b writes output column
    // 2c - pad + (b ^ (pad & 1)), so these positions cover every output column.
    const int cmin = pad >> 1;
    const int Wc = ((OW - 1 + pad) >> 1) - cmin + 1;
    const int npix = Mc * Wc;
    const int ipi = (npix + kStagedPix - 1) / kStagedPix;  // items per image
    const int nitems = N * ipi;
    if (rank >= nitems) return;                   // whole block: before any barrier

    for (int e = threadIdx.x; e < 2 * COUT * K; e += kThreads) {
        const int k = e % K;
        const int rest = e / K;
        const int co = rest % COUT, b = rest / COUT;
        const int ci = 8 * (k >> 5) + (k & 7);
        const int t = (k >> 3) & 3;
        const int kh = ka + 2 * (t >> 1), kw = ((b + pad) & 1) + 2 * (t & 1);
        la[(b * COUT + co) * KP + k] = ci < Cin ? w[(((size_t)ci * COUT + co) * 4 + kh) * 4 + kw] : 0;
    }
    for (int e = threadIdx.x; e < COUT; e += kThreads) {
        lcb[e] = (cbias ? cbias[e] : 0.f) * kLog2e;
        lb2[e] = -b2[e] * scale * kLog2e;
    }
    for (int e = threadIdx.x; e < 2 * slots; e += kThreads) {
        lx[e * WE] = make_uint4(0u, 0u, 0u, 0u);
        lx[e * WE + W + 1] = make_uint4(0u, 0u, 0u, 0u);
        lx[e * WE + W + 2] = make_uint4(0u, 0u, 0u, 0u);
    }

    // ---- chunk fill: thread -> (slot, 8-column group g, channel pair cp) ----
    const int W8 = W >> 3;
    const int f_cp = threadIdx.x & 3;
    const int f_g = (threadIdx.x >> 2) % W8;
    const int f_slot = (threadIdx.x >> 2) / W8;
    const bool f_on = f_slot < slots;
    const uint32_t plane = (uint32_t)(H * W);
    const uint32_t xbytes = 2u * (uint32_t)(N * Cin) * plane;
    const __amdgpu_buffer_rsrc_t xr = make_range_checked(x, xbytes);
    auto fill_load = [&](int it, int k, uint32_t (&v)[8]) {
        const int n = it / ipi;
        const int m0 = ((it - n * ipi) * kStagedPix) / Wc;
        const int ir = m0 + ra - 1 + f_slot;
        const int ch = 8 * k + 2 * f_cp;
        const bool rok = f_on && ir >= 0 && ir < H;
        const uint32_t o = 2u * (((uint32_t)(n * Cin + ch) * (uint32_t)H + (uint32_t)ir) * (uint32_t)W +
                                 8u * (uint32_t)f_g);
        const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(xr, (rok && ch < Cin) ? o : xbytes, 0, 0);
        const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(
            xr, (rok && ch + 1 < Cin) ? o + 2u * plane : xbytes, 0, 0);
        v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
        v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    };
    auto fill_store = [&](int buf, const uint32_t (&v)[8]) {
        if (f_on) {
            uint32_t *dst = (uint32_t *)(lx + buf * bufsz + f_slot * WE + 8 * f_g + 1) + f_cp;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dst[4 * e] = __builtin_amdgcn_perm(v[4 + (e >> 1)], v[e >> 1],
                                                   (e & 1) ? 0x07060302u : 0x05040100u);
        }
    };

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int j = lane & 31;  // position (B/D column) and A row within a 32-channel tile
    const int h = lane >> 5;  // K half of a step (tap v = h); D row half
    const int nchunks = C8 / 8;
    const int oplane = OH * OW;
    const float ninv_s = -scale * kLog2e;
    const uint32_t ybytes = 2u * (uint32_t)COUT * (uint32_t)oplane;

    uint32_t pre[8];
    int it = rank;
    fill_load(it, 0, pre);
    fill_store(0, pre);
    __syncthreads();
    int buf = 0;

    for (; it < nitems; it += wg_per_class) {
        const int n = it / ipi;
        const int p0 = (it - n * ipi) * kStagedPix;
        const int m0 = p0 / Wc;
        const int p = p0 + 32 * wv + j;
        const bool pv = p < npix;
        const int pc = pv ? p : p0;
        const int m = pc / Wc;
        const int c = pc - m * Wc;
        // B entries of taps (u, v = h), u = 0, 1: input (m + ra - u, cmin + c - h)
        const int eo0 = (m - m0 + 1) * WE + (cmin + c - h + 1);
        const int eo1 = eo0 - WE;
        const uint16_t *ab = la + j * KP + 8 * h;

        f32x16 acc[2][MT];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[b][mt][i] = 0.f;

        for (int k = 0; k < nchunks; ++k) {
            const bool last = k + 1 == nchunks;
            const bool more = !last || it + wg_per_class < nitems;
            if (more) fill_load(last ? it + wg_per_class : it, last ? 0 : k + 1, pre);
            const uint4 *xb = lx + buf * bufsz;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8 bop = __builtin_bit_cast(bf16x8, xb[u ? eo1 : eo0]);
                const int s = 2 * k + u;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const uint4 av = *(const uint4 *)(ab + (b * COUT + 32 * mt) * KP + 16 * s);
                        acc[b][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, av), bop, acc[b][mt], 0, 0, 0);
                    }
            }
            if (more) fill_store(buf ^ 1, pre);
            __syncthreads();
            buf ^= 1;
        }

        // ---- epilogue: D element i of tile mt = channel 32mt + 8(i/4) + 4h + i%4; the
        // partner lane (xor 32) holds the other half of each 8-channel group ----
        float inv[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const float4 cb4 = *(const float4 *)(lcb + 32 * mt + 8 * i4 + 4 * h);
                    const float cbv[4] = {cb4.x, cb4.y, cb4.z, cb4.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * i4 + r;
                        acc[b][mt][i] = fmaf(acc[b][mt][i], kLog2e, cbv[r]);
                        mx = fmaxf(mx, acc[b][mt][i]);
                    }
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            float sum = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc[b][mt][i] = __builtin_amdgcn_exp2f(acc[b][mt][i] - mx);
                    sum += acc[b][mt][i];
                }
            sum += __shfl_xor(sum, 32);
            inv[b] = ninv_s * __builtin_amdgcn_rcpf(sum);
        }
        // The 32 positions x 2 column classes of the wave are 64 output columns
        // ow = 2c - pad + (b ^ podd), ascending within an output row: slot 2j + (b ^ podd).
        // Each 8-channel group goes through LDS so that a store writes one channel's 64
        // columns (128 contiguous bytes, or two runs where the positions wrap to the next
        // row).  Store lane L takes slot L: position L/2, output column 2c - pad + L%2; a
        // masked store gets an offset past the end of the range (dropped).
        const int podd = pad & 1;
        const __amdgpu_buffer_rsrc_t yr =
            make_range_checked(y + (size_t)n * COUT * oplane, ybytes);
        const int ps = p0 + 32 * wv + (lane >> 1);
        const bool psv = ps < npix;
        const int msx = psv ? ps / Wc : 0;
        const int ows = 2 * (cmin + (psv ? ps - msx * Wc : 0)) - pad + (lane & 1);
        const uint32_t so = (psv && ows >= 0 && ows < OW)
                                ? 2u * (uint32_t)((2 * msx + a) * OW + ows)
                                : 0x80000000u;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int co0 = 32 * mt + 8 * i4;
                const float4 b4 = *(const float4 *)(lb2 + co0 + 4 * h);
                const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float t =
                            __builtin_amdgcn_exp2f(fmaf(acc[b][mt][4 * i4 + r], inv[b], bv[r]));
                        lo[(4 * h + r) * kStageRow + 2 * j + (b ^ podd)] =
                            f32_to_bf16_rne(__builtin_amdgcn_rcpf(1.f + t));
                    }
#pragma unroll
                for (int ch = 0; ch < 8; ++ch)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        lo[ch * kStageRow + lane], yr,
                        (int)(so + 2u * (uint32_t)(co0 + ch) * (uint32_t)oplane), 0, 0);
            }
    }
}

template <int MT>
int launch_mt(const uint16_t *x, const uint16_t *w, const float *cb, const float *b2, uint16_t *y,
              int N, int Cin, int H, int W, int OH, int OW, int pad, float scale,
              hipStream_t stream) {
    constexpr int kRing = ring_steps<MT>();
    const int C4 = (Cin + 4 * kRing - 1) / (4 * kRing) * (4 * kRing);  // whole rings of K-steps
    const int KP = 4 * C4 + 8;
    if ((int64_t)N * Cin * H * W >= (1ll << 30) || (int64_t)N * 32 * MT * OH * OW >= (1ll << 31))
        return PS_ERR_UNSUPPORTED;
    const size_t lds_bytes = (size_t)2 * 32 * MT * KP * 2 + 2 * 32 * MT * sizeof(float);
    if (lds_bytes > 160 * 1024) return PS_ERR_UNSUPPORTED;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PS_ERR_HIP;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PS_ERR_HIP;
    // one workgroup per CU (the two weight matrices fill most of the LDS), a multiple
    // of 16 blocks so every XCD holds whole row-class pairs
    int wg_per_class = (ncu + 1) / 2;
    wg_per_class = ((wg_per_class + 7) / 8) * 8;
    const int nblocks = 2 * wg_per_class;

    // staged variant: 16-byte input rows, every fill unit one thread, buffers in LDS,
    // and masked output offsets (2^31 + image bytes) that cannot wrap
    {
        const int C8 = (Cin + 7) / 8 * 8;
        const int Wc = ((OW - 1 + pad) >> 1) - (pad >> 1) + 1;   // positions per row
        const int slots = (Wc + kStagedPix - 2) / Wc + 2;
        const size_t lds_staged = (size_t)2 * 32 * MT * (4 * C8 + 8) * 2 +
                                  2 * 32 * MT * sizeof(float) + (size_t)2 * slots * (W + 3) * 16 +
                                  (size_t)(kThreads / 64) * 8 * kStageRow * 2;
        if (W % 8 == 0 && (int64_t)slots * (W / 8) * 4 <= kThreads &&
            lds_staged <= 160 * 1024 && (int64_t)2 * 32 * MT * OH * OW < (1ll << 31)) {
            if (lds_staged > 65536 &&
                hipFuncSetAttribute((const void *)convT_softmax_bf16_staged<MT>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)lds_staged) != hipSuccess)
                return PS_ERR_HIP;
            return launch(convT_softmax_bf16_staged<MT>, dim3(nblocks), dim3(kThreads),
                          lds_staged, stream, x, w, cb, b2, y, N, Cin, H, W, OH, OW, pad, scale,
                          C8, slots, wg_per_class);
        }
    }

    if (lds_bytes > 65536 &&
        hipFuncSetAttribute((const void *)convT_softmax_bf16<MT>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes) !=
            hipSuccess)
        return PS_ERR_HIP;
    return launch(convT_softmax_bf16<MT>, dim3(nblocks), dim3(kThreads), lds_bytes, stream, x, w,
                  cb, b2, y, N, Cin, H, W, OH, OW, pad, scale, C4, wg_per_class);
}

}  // namespace

int launch_convT_softmax_bf16(const uint16_t *x, const uint16_t *w, const float *convT_bias,
                              const float *bias2, uint16_t *y, int N, int Cin, int H, int W,
                              int Cout, int OH, int OW, int pad, float scale, hipStream_t stream) {
    // the row-class kernel (convt_rows.hip: whole output lines per workgroup) where its
    // envelope allows
    const int st = launch_convT_rows_bf16(x, w, convT_bias, bias2, y, N, Cin, H, W, Cout, OH, OW,
                                          pad, scale, stream);
    if (st != PS_ERR_UNSUPPORTED) return st;
    switch (Cout / 32) {
        case 1: return launch_mt<1>(x, w, convT_bias, bias2, y, N, Cin, H, W, OH, OW, pad, scale, stream);
        case 2: return launch_mt<2>(x, w, convT_bias, bias2, y, N, Cin, H, W, OH, OW, pad, scale, stream);
        case 3: return launch_mt<3>(x, w, convT_bias, bias2, y, N, Cin, H, W, OH, OW, pad, scale, stream);
        case 4: return launch_mt<4>(x, w, convT_bias, bias2, y, N, Cin, H, W, OH, OW, pad, scale, stream);
    }
    return PS_ERR_UNSUPPORTED;
}

}  // namespace ps

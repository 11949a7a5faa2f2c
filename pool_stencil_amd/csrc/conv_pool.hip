// Fused Conv2d(k3, s1, d1) -> tanh -> *scale -> +bias2 -> MaxPool2d(k = s = PK) for gfx950.
//
// Definition (POPCORNBENCH page Kimi-K2.6 l2_p82, problem statement):
//   y  = conv_bias[co] + sum_{ci,kh,kw} x[n,ci,oh-p+kh,ow-p+kw] * w[co,ci,kh,kw]
//   z  = tanh(y) * scale + bias2[co]
//   out[n,co,ph,pw] = max_{dy,dx<PK} z[n,co,PK*ph+dy,PK*pw+dx]
//
// The pool windows are disjoint (stride = kernel), so every conv output the
// pool reads is computed exactly once and the conv output never leaves
// registers.  tanh and z -> z*scale + b are monotone (nondecreasing when
// scale >= 0), so max_window(z) = tanh(max_window(y))*scale + b: the kernel
// pools the raw conv sums and evaluates tanh once per pooled output (the
// page's reordering argument).  For scale < 0 the map is nonincreasing and
// the window minimum of y is taken instead (kept as max of -y).
//
// The conv is an implicit GEMM on the matrix cores:
//   D[co][pixel] += A[co][k] * B[k][pixel],  k = (ci, kh, kw)
// with one 16x16 D tile = 16 output channels x 16 pooled columns for one
// pool-window position (dy, dx).  The 16 (dy,dx) positions of a window are 16
// separate D tiles of the same pooled pixels, so the pool max is an
// elementwise max across D tiles held by the same lane -- no cross-lane work.
//
// Data movement per workgroup (one image n, one pooled row ph, 16*NPW pooled
// columns, all output channels):
//   - the input halo tile (PK+2 rows x PK*16*NPW+2 columns x Cin) is staged
//     once in LDS, zero-filled outside the image (the conv's zero padding);
//   - LDS columns are stored de-interleaved by (column mod PK), so the 16
//     lanes that feed one MFMA read 16 consecutive words, and the channel
//     stride is padded to 16 (mod 64) words so the four lane groups of a wave
//     hit disjoint banks;
//   - all weights of a 64-channel output tile live in VGPRs for the whole
//     workgroup (fp32: 9*Cin_pad*64/64 registers per lane).
//
// fp32: v_mfma_f32_16x16x4_f32 (fp32 products and accumulation), one K-step
//       = one kernel tap x 4 input channels.
// bf16: v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 accumulation), one
//       K-step = 4 kernel taps x 8 input channels; the LDS tile is channel-last
//       so one 16-byte LDS read gives a lane its 8 channels.  Output rounded to
//       nearest even.
#include "ps_internal.h"

#include <math.h>

namespace ps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int pad_words_16mod64(int n) { return n + ((16 - (n % 64)) + 64) % 64; }

template <int PK, int NPW>
struct TileGeom {
    static constexpr int T = 16 * NPW;       // pooled columns per workgroup
    static constexpr int ROWS = PK + 2;      // input rows per pooled row (kH = 3)
    static constexpr int COLS = PK * T + 2;  // input columns per tile (kW = 3)
    static constexpr int Q = T + 1;          // entries per column-residue plane
    static constexpr int RS = PK * Q;        // entries per tile row
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ---------------------------------------------------------------- fp32 ---
template <int PK, int NPW, int CING>
__global__ __launch_bounds__(64 * NPW) void conv_pool_f32(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cb,
    const float *__restrict__ b2, float *__restrict__ y, int Cin, int H, int W, int Cout,
    int pad, int PH, int PW, float scale, int npwt) {
    using G = TileGeom<PK, NPW>;
    constexpr int PS = pad_words_16mod64(G::ROWS * G::RS);  // words per input channel
    constexpr int CINP = 4 * CING;
    __shared__ float tile[CINP * PS];

    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int pwt = (int)(L % (uint32_t)npwt);
    const int ph = (int)((L / (uint32_t)npwt) % (uint32_t)PH);
    const int n = (int)(L / ((uint32_t)npwt * (uint32_t)PH));

    // ---- stage the zero-padded halo tile ----
    const int ir0 = PK * ph - pad;
    const int ic0 = PK * pwt * G::T - pad;
    const float *xn = x + (size_t)n * Cin * H * W;
    for (int e = threadIdx.x; e < CINP * G::ROWS * G::COLS; e += 64 * NPW) {
        const int c = e % G::COLS;
        const int t = e / G::COLS;
        const int r = t % G::ROWS;
        const int ci = t / G::ROWS;
        const int ir = ir0 + r, ic = ic0 + c;
        float v = 0.f;
        if (ci < Cin && ir >= 0 && ir < H && ic >= 0 && ic < W)
            v = xn[((size_t)ci * H + ir) * W + ic];
        tile[ci * PS + r * G::RS + (c % PK) * G::Q + c / PK] = v;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int j = lane & 15;  // pooled column within the 16-wide group (B/D column)
    const int g4 = lane >> 4; // lane group: input channel within a K-step; D row block
    const int pw = pwt * G::T + 16 * wv + j;
    const float *tb = tile + g4 * PS + 16 * wv + j;
    const float sgn = scale < 0.f ? -1.f : 1.f;

    for (int ct = 0; ct < Cout; ct += 64) {
        // A operands: w[co = ct + 16*nt + j][ci = 4*g + g4][tap]
        float wr[4][9][CING];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int co = ct + 16 * nt + j;
#pragma unroll
            for (int g = 0; g < CING; ++g) {
                const int ci = 4 * g + g4;
                const bool ok = co < Cout && ci < Cin;
                const float *wp = w + ((size_t)co * Cin + ci) * 9;
#pragma unroll
                for (int tap = 0; tap < 9; ++tap) wr[nt][tap][g] = ok ? wp[tap] : 0.f;
            }
        }

        f32x4 best[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) best[nt] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};

#pragma unroll 1
        for (int dy = 0; dy < PK; ++dy) {
            const float *tr = tb + dy * G::RS;
#pragma unroll
            for (int dx = 0; dx < PK; ++dx) {
                f32x4 acc[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < CING; ++g)
#pragma unroll
                    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                        for (int kw = 0; kw < 3; ++kw) {
                            const int t = dx + kw;
                            const float b = tr[g * 4 * PS + kh * G::RS + (t % PK) * G::Q + t / PK];
#pragma unroll
                            for (int nt = 0; nt < 4; ++nt)
                                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    wr[nt][kh * 3 + kw][g], b, acc[nt], 0, 0, 0);
                        }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) best[nt][r] = fmaxf(best[nt][r], sgn * acc[nt][r]);
            }
        }

        // ---- epilogue: conv bias, tanh, scale, bias2; D row 4*g4 + r = channel ----
        if (pw < PW) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int co = ct + 16 * nt + 4 * g4 + r;
                    if (co < Cout) {
                        const float v = sgn * best[nt][r] + (cb ? cb[co] : 0.f);
                        y[(((size_t)n * Cout + co) * PH + ph) * PW + pw] = tanhf(v) * scale + b2[co];
                    }
                }
        }
    }
}

// ---------------------------------------------------------------- bf16 ---
template <int PK, int NPW>
__global__ __launch_bounds__(64 * NPW) void conv_pool_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ cb,
    const float *__restrict__ b2, uint16_t *__restrict__ y, int Cin, int H, int W, int Cout,
    int pad, int PH, int PW, float scale, int npwt) {
    using G = TileGeom<PK, NPW>;
    // channel-last tile: entry (row, plane, q) = 8 input channels as 8 bf16
    __shared__ uint4 tile[G::ROWS * G::RS];

    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int pwt = (int)(L % (uint32_t)npwt);
    const int ph = (int)((L / (uint32_t)npwt) % (uint32_t)PH);
    const int n = (int)(L / ((uint32_t)npwt * (uint32_t)PH));

    const int ir0 = PK * ph - pad;
    const int ic0 = PK * pwt * G::T - pad;
    const uint16_t *xn = x + (size_t)n * Cin * H * W;
    const size_t cstride = (size_t)H * W;
    for (int e = threadIdx.x; e < G::ROWS * G::COLS; e += 64 * NPW) {
        const int c = e % G::COLS;
        const int r = e / G::COLS;
        const int ir = ir0 + r, ic = ic0 + c;
        uint32_t h[8];
#pragma unroll
        for (int ci = 0; ci < 8; ++ci) h[ci] = 0;
        if (ir >= 0 && ir < H && ic >= 0 && ic < W) {
            const uint16_t *p = xn + (size_t)ir * W + ic;
#pragma unroll
            for (int ci = 0; ci < 8; ++ci)
                if (ci < Cin) h[ci] = p[ci * cstride];
        }
        uint4 v;
        v.x = h[0] | (h[1] << 16);
        v.y = h[2] | (h[3] << 16);
        v.z = h[4] | (h[5] << 16);
        v.w = h[6] | (h[7] << 16);
        tile[r * G::RS + (c % PK) * G::Q + c / PK] = v;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int j = lane & 15;
    const int g4 = lane >> 4;
    const int pw = pwt * G::T + 16 * wv + j;
    const float sgn = scale < 0.f ? -1.f : 1.f;

    // Per lane, K-step s covers kernel tap 4*s + g4 (taps >= 9 carry zero weights
    // and read a valid in-tile entry).  LDS entry offsets for each (s, dx).
    int off[3][PK];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int tap = min(4 * s + g4, 8);
        const int kh = tap / 3, kw = tap % 3;
#pragma unroll
        for (int dx = 0; dx < PK; ++dx) {
            const int t = dx + kw;
            off[s][dx] = kh * G::RS + (t % PK) * G::Q + 16 * wv + j + t / PK;
        }
    }

    for (int ct = 0; ct < Cout; ct += 64) {
        // A operands: lane holds w[co = ct + 16*nt + j][ci = 0..7][tap = 4*s + g4]
        bf16x8 wa[4][3];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int co = ct + 16 * nt + j;
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                const int tap = 4 * s + g4;
                uint32_t hv[8];
#pragma unroll
                for (int ci = 0; ci < 8; ++ci)
                    hv[ci] = (co < Cout && ci < Cin && tap < 9) ? (uint32_t)w[((size_t)co * Cin + ci) * 9 + tap]
                                                                : 0u;
                uint4 pk;
                pk.x = hv[0] | (hv[1] << 16);
                pk.y = hv[2] | (hv[3] << 16);
                pk.z = hv[4] | (hv[5] << 16);
                pk.w = hv[6] | (hv[7] << 16);
                wa[nt][s] = __builtin_bit_cast(bf16x8, pk);
            }
        }

        f32x4 best[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) best[nt] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};

#pragma unroll 1
        for (int dy = 0; dy < PK; ++dy) {
            const uint4 *tr = tile + dy * G::RS;
#pragma unroll
            for (int dx = 0; dx < PK; ++dx) {
                f32x4 acc[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    const uint4 bv = tr[off[s][dx]];
                    const bf16x8 b = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[nt][s], b, acc[nt], 0, 0, 0);
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) best[nt][r] = fmaxf(best[nt][r], sgn * acc[nt][r]);
            }
        }

        if (pw < PW) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int co = ct + 16 * nt + 4 * g4 + r;
                    if (co < Cout) {
                        const float v = sgn * best[nt][r] + (cb ? cb[co] : 0.f);
                        y[(((size_t)n * Cout + co) * PH + ph) * PW + pw] =
                            f32_to_bf16_rne(tanhf(v) * scale + b2[co]);
                    }
                }
        }
    }
}

template <int PK, int NPW>
int launch_pk_npw(const void *x, const void *w, const float *cb, const float *b2, void *y,
                  int dtype, int N, int Cin, int H, int W, int Cout, int pad, float scale, int PH,
                  int PW, hipStream_t stream) {
    const int npwt = (PW + 16 * NPW - 1) / (16 * NPW);
    const uint64_t nblocks = (uint64_t)N * PH * npwt;
    if (nblocks > 0x7fffffffull) return PS_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)nblocks), block(64 * NPW);
    if (dtype == PS_BF16) {
        hipLaunchKernelGGL((conv_pool_bf16<PK, NPW>), grid, block, 0, stream,
                           (const uint16_t *)x, (const uint16_t *)w, cb, b2, (uint16_t *)y, Cin, H,
                           W, Cout, pad, PH, PW, scale, npwt);
    } else if (Cin <= 4) {
        hipLaunchKernelGGL((conv_pool_f32<PK, NPW, 1>), grid, block, 0, stream, (const float *)x,
                           (const float *)w, cb, b2, (float *)y, Cin, H, W, Cout, pad, PH, PW,
                           scale, npwt);
    } else {
        hipLaunchKernelGGL((conv_pool_f32<PK, NPW, 2>), grid, block, 0, stream, (const float *)x,
                           (const float *)w, cb, b2, (float *)y, Cin, H, W, Cout, pad, PH, PW,
                           scale, npwt);
    }
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_HIP;
}

template <int PK>
int launch_pk(const void *x, const void *w, const float *cb, const float *b2, void *y, int dtype,
              int N, int Cin, int H, int W, int Cout, int pad, float scale, int PH, int PW,
              hipStream_t stream) {
    constexpr bool wide_ok = PK <= 4;  // 64-column tiles keep the fp32 tile under 64 KB
    if (wide_ok && PW > 32)
        return launch_pk_npw<PK, (wide_ok ? 4 : 2)>(x, w, cb, b2, y, dtype, N, Cin, H, W, Cout,
                                                    pad, scale, PH, PW, stream);
    if (PW > 16)
        return launch_pk_npw<PK, 2>(x, w, cb, b2, y, dtype, N, Cin, H, W, Cout, pad, scale, PH,
                                    PW, stream);
    return launch_pk_npw<PK, 1>(x, w, cb, b2, y, dtype, N, Cin, H, W, Cout, pad, scale, PH, PW,
                                stream);
}

}  // namespace

int launch_conv_pool(const void *x, const void *w, const float *conv_bias, const float *bias2,
                     void *y, int dtype, int N, int Cin, int H, int W, int Cout, int conv_pad,
                     int OH, int OW, float scale, int pool_k, int PH, int PW,
                     hipStream_t stream) {
    (void)OH;
    (void)OW;
    switch (pool_k) {
        case 2: return launch_pk<2>(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout, conv_pad, scale, PH, PW, stream);
        case 3: return launch_pk<3>(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout, conv_pad, scale, PH, PW, stream);
        case 4: return launch_pk<4>(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout, conv_pad, scale, PH, PW, stream);
        case 5: return launch_pk<5>(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout, conv_pad, scale, PH, PW, stream);
        case 6: return launch_pk<6>(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout, conv_pad, scale, PH, PW, stream);
        case 7: return launch_pk<7>(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout, conv_pad, scale, PH, PW, stream);
        case 8: return launch_pk<8>(x, w, conv_bias, bias2, y, dtype, N, Cin, H, W, Cout, conv_pad, scale, PH, PW, stream);
    }
    return PS_ERR_UNSUPPORTED;
}

}  // namespace ps

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
// bf16: exact bf16 products, fp32 accumulation; the LDS tile is channel-last so
//       one 16-byte LDS read gives a lane its 8 channels.  One channel tile with
//       pool <= 4: v_mfma_f32_32x32x16_bf16, one K-step = 2 kernel taps x 8 input
//       channels (9 taps in 5 steps); otherwise v_mfma_f32_16x16x32_bf16, one K-step
//       = 4 taps x 8 channels (9 taps in 3 steps).  Output rounded to nearest even.
#include "ps_internal.h"

#include <math.h>

#include <type_traits>

namespace ps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int pad_words_16mod64(int n) { return n + ((16 - (n % 64)) + 64) % 64; }

template <int PK, int NPW>
struct TileGeom {
    static constexpr int T = 16 * NPW;       // pooled columns per workgroup
    static constexpr int ROWS = PK + 2;      // input rows per pooled row (kH = 3)
    static constexpr int COLS = PK * T + 2;  // input columns per tile (kW = 3)
    static constexpr int Q = T + 1;          // entries per column-residue plane
    static constexpr int RS = PK * Q;        // entries per tile row
    // fp32 tile: one more entry per plane, so the (masked) columns of a row's last
    // 16-byte group, up to column 4 * ceil(COLS / 4) - 1 <= PK*T + PK - 1 for PK >= 5
    // and <= PK*T + 3 otherwise, land on unused entries of their own row
    static constexpr int QF = T + 2;
    static constexpr int RSF = PK * QF;
};

// ---------------------------------------------------------------- fp32 ---
// fp32 conv tuning: tile rows a wave loads per batch (bounds the registers the fill
// holds next to the resident weights; 12 is every row of a wave at 8 input channels
// and pool 4), window columns per unrolled group (0 = all), and the minimum resident
// waves per SIMD asked of the register allocator for pool windows up to 4 (three
// 52 KB workgroups then share a CU's LDS).  On MI355X, 3 waves/SIMD took the 8->64 k3
// + pool-4 workload from 0.745 to 0.68 ms; one batch of 12 rows instead of 7 + 5 was
// about 4% faster again.
#ifndef PS_CONV_FILL_BATCH
#define PS_CONV_FILL_BATCH 12
#endif
#ifndef PS_CONV_DXG
#define PS_CONV_DXG 0
#endif
#ifndef PS_BF16_MAX_STEP
#define PS_BF16_MAX_STEP 1
#endif
#ifndef PS_BF16_LDS_AHEAD
#define PS_BF16_LDS_AHEAD 3
#endif
// B fragments read ahead of their MFMAs in the 32x32x16 form (5 and 8 measured no faster)
#ifndef PS_BF16_W32_AHEAD
#define PS_BF16_W32_AHEAD 3
#endif
#ifndef PS_CONV_MIN_WAVES
#define PS_CONV_MIN_WAVES 3
#endif

// NCT: 16-channel tiles per workgroup pass (4, or 1 when Cout <= 16)
template <int PK, int NPW, int CING, int NCT>
__global__ __launch_bounds__(64 * NPW, (PK <= 4 ? PS_CONV_MIN_WAVES : 1)) void conv_pool_f32(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cb,
    const float *__restrict__ b2, float *__restrict__ y, int Cin, int H, int W, int Cout,
    int pad, int PH, int PW, float scale, int npwt) {
    using G = TileGeom<PK, NPW>;
    constexpr int PS = pad_words_16mod64(G::ROWS * G::RSF);  // words per input channel
    constexpr int CINP = 4 * CING;
    // the halo tile
    __shared__ float tile[CINP * PS];
    __shared__ float s_bias[2][64];  // conv bias, bias2 of the current 64-channel tile

    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int pwt = (int)(L % (uint32_t)npwt);
    const int ph = (int)((L / (uint32_t)npwt) % (uint32_t)PH);
    const int n = (int)(L / ((uint32_t)npwt * (uint32_t)PH));

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int j = lane & 15;  // pooled column within the 16-wide group (B/D column)
    const int g4 = lane >> 4; // lane group: input channel within a K-step; D row block

    // A operands of channel tile ct: sgn * w[co = ct + 16*nt + j][ci = 4*g + g4][tap].
    // sgn = -1 for scale < 0 makes the window max of the products the negated window
    // minimum of the conv sums, so the pool loop is a plain max (no multiply per value).
    const float sgn = scale < 0.f ? -1.f : 1.f;
    const uint32_t sgn_bit = scale < 0.f ? 0x80000000u : 0u;
    float wr[NCT][9][CING];
    auto load_weights = [&](int ct) {
        // Every weight of the tile present and scale >= 0 (a uniform test): plain loads,
        // without the per-weight select and sign flip (144 VALU instructions per wave,
        // which the matrix cores would wait for).
        if (sgn_bit == 0u && Cin == CINP && ct + 16 * NCT <= Cout) {
#pragma unroll
            for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
                for (int g = 0; g < CING; ++g) {
                    const float *wp = w + ((size_t)(ct + 16 * nt + j) * Cin + 4 * g + g4) * 9;
#pragma unroll
                    for (int tap = 0; tap < 9; ++tap) wr[nt][tap][g] = wp[tap];
                }
            return;
        }
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) {
            const int co = ct + 16 * nt + j;
#pragma unroll
            for (int g = 0; g < CING; ++g) {
                const int ci = 4 * g + g4;
                const bool ok = co < Cout && ci < Cin;
                const float *wp = w + ((size_t)(ok ? co : 0) * Cin + (ok ? ci : 0)) * 9;
#pragma unroll
                for (int tap = 0; tap < 9; ++tap) {
                    // (the sign as a bit flip after the select: multiplying inside it
                    // turned the unconditional loads into one branch and wait per load)
                    const float v = wp[tap];
                    wr[nt][tap][g] = __uint_as_float(__float_as_uint(ok ? v : 0.f) ^ sgn_bit);
                }
            }
        }
    };
    // Epilogue constants: with u = sgn*best + cb, tanh(u) = 1 - 2/(2^(2u log2e) + 1), so
    // out = (scale + b2) - 2 scale / (2^(best*k2 + cb*2log2e) + 1), k2 = 2 log2e sgn:
    // s_bias holds cb*2log2e and scale + b2.
    constexpr float kTwoLog2e = 2.8853900817779268f;
    const float k2 = sgn * kTwoLog2e;
    const float m2 = -2.f * scale;
    auto stage_bias = [&](int ct) {
        if (threadIdx.x < 64) {
            const int co = ct + threadIdx.x;
            s_bias[0][threadIdx.x] = (co < Cout && cb) ? cb[co] * kTwoLog2e : 0.f;
            s_bias[1][threadIdx.x] = co < Cout ? scale + b2[co] : 0.f;
        }
    };
    // first tile's weights and biases: in flight together with the halo loads
    load_weights(0);
    stage_bias(0);

    // ---- stage the zero-padded halo tile ----
    // Tile rows (input channel, input row) are streamed by whole waves: lane l of a wave
    // loads the l-th 4-column group of the row, so the per-lane column offsets, their
    // validity and the lane's LDS words are computed once and a row costs one load, one
    // select and four LDS writes (per-vector index arithmetic had cost about 35 VALU
    // instructions per 16-byte load, and on this chip VALU time adds to the matrix
    // cores' time).  Groups past the last whole 64 of a row go through a short flat loop
    // over all threads.  Every load is issued before any LDS write of its batch.
    // Range-checked buffer loads over image n (below 2^31 bytes, host check): a value
    // outside the image -- the conv's zero padding -- gets a masked offset and reads zero.
    const int ir0 = PK * ph - pad;
    const int ic0 = PK * pwt * G::T - pad;
    const float *xn = x + (size_t)n * Cin * H * W;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);  // (wave-uniform: rows in scalars)
    constexpr uint32_t kMasked = 0x80000000u;
    const __amdgpu_buffer_rsrc_t xr =
        make_range_checked(xn, 4u * (uint32_t)Cin * (uint32_t)H * (uint32_t)W);
    constexpr int NROWS = CINP * G::ROWS;     // tile rows
    constexpr int NV = (G::COLS + 3) / 4;     // 4-column groups per tile row
    constexpr int NFULL = NV / 64;            // groups covered by whole waves
    constexpr int NTAIL = NV - 64 * NFULL;    // the rest of each row
    constexpr int RPW = (NROWS + NPW - 1) / NPW;  // rows per wave
    // image byte offset of tile row rr, and whether it lies in the image (and below Cin)
    auto row_in = [&](int rr, uint32_t &off) {
        const int ci = rr / G::ROWS, ir = ir0 + rr % G::ROWS;
        off = 4u * ((uint32_t)(ci * H + ir) * (uint32_t)W);
        return ci < Cin && ir >= 0 && ir < H;
    };
    auto row_lds = [&](int rr) { return (rr / G::ROWS) * PS + (rr % G::ROWS) * G::RSF; };
    // LDS word of tile column c within its row (de-interleaved by c mod PK)
    auto col_lds = [](int c) { return (c % PK) * G::QF + c / PK; };
    // (instantiated once per load width: a uniform test per element split the fill
    // into one branch per load)
    auto fill = [&](auto VEC) {
        constexpr bool vec = decltype(VEC)::value;
        if constexpr (NFULL > 0) {
            // per-lane column offsets (kMasked outside the image) and LDS words
            uint32_t co[NFULL][vec ? 1 : 4];
            int lw[NFULL][4];
#pragma unroll
            for (int ch = 0; ch < NFULL; ++ch) {
                const int v = 64 * ch + lane;
                const int ic = ic0 + 4 * v;
                if constexpr (vec) {
                    co[ch][0] = ((ic >= 0) & (ic < W)) ? 4u * (uint32_t)ic : kMasked;
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        co[ch][k] = ((ic + k >= 0) & (ic + k < W)) ? 4u * (uint32_t)(ic + k) : kMasked;
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) lw[ch][k] = col_lds(4 * v + k);
            }
            constexpr int FB = PS_CONV_FILL_BATCH > 0 && PS_CONV_FILL_BATCH < RPW ? PS_CONV_FILL_BATCH : RPW;
#pragma unroll
            for (int i0 = 0; i0 < RPW; i0 += FB) {
                float4 buf[FB][NFULL];
                // (no branch around the loads: a row past the last one reads zeros through
                // masked offsets; branches here made the compiler wait before each load)
#pragma unroll
                for (int ii = 0; ii < FB; ++ii) {
                    if (i0 + ii >= RPW) continue;  // compile-time after unrolling
                    const int rr = wvu + NPW * (i0 + ii);
                    uint32_t ro;
                    const bool rok = (rr < NROWS) & row_in(rr < NROWS ? rr : 0, ro);
#pragma unroll
                    for (int ch = 0; ch < NFULL; ++ch) {
                        if constexpr (vec) {
                            const uint4 q = __builtin_bit_cast(
                                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           xr, rok ? co[ch][0] : kMasked, rok ? ro : 0u, 0));
                            buf[ii][ch] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y),
                                                      __uint_as_float(q.z), __uint_as_float(q.w));
                        } else {
                            float vv[4];
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                vv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                    xr, rok ? co[ch][k] : kMasked, rok ? ro : 0u, 0));
                            buf[ii][ch] = make_float4(vv[0], vv[1], vv[2], vv[3]);
                        }
                    }
                }
#pragma unroll
                for (int ii = 0; ii < FB; ++ii) {
                    const int rr = wvu + NPW * (i0 + ii);
                    if (i0 + ii < RPW && rr < NROWS) {
                        float *trow = tile + row_lds(rr);
#pragma unroll
                        for (int ch = 0; ch < NFULL; ++ch) {
                            trow[lw[ch][0]] = buf[ii][ch].x;
                            trow[lw[ch][1]] = buf[ii][ch].y;
                            trow[lw[ch][2]] = buf[ii][ch].z;
                            trow[lw[ch][3]] = buf[ii][ch].w;
                        }
                    }
                }
            }
        }
        if constexpr (NTAIL > 0) {
            // the last NTAIL groups of every row: item e = (row, group) over all threads
            constexpr int NT = 64 * NPW;
            constexpr int TOTAL = NROWS * NTAIL;
            constexpr int PER = (TOTAL + NT - 1) / NT;
            // in batches of 7 loads (the narrow tiles run their whole fill here)
            constexpr int TB = PER < 7 ? PER : 7;
#pragma unroll
            for (int i0 = 0; i0 < PER; i0 += TB) {
            float4 buf[TB];
#pragma unroll
            for (int ii = 0; ii < TB; ++ii) {
                const int i = i0 + ii;
                const int e = threadIdx.x + i * NT;
                const int rr = e / NTAIL, v = 64 * NFULL + e % NTAIL;
                const int ic = ic0 + 4 * v;
                uint32_t ro;
                const bool rok = (i < PER) & (e < TOTAL) & row_in(rr, ro);
                if constexpr (vec) {
                    const bool ok = rok & (ic >= 0) & (ic < W);
                    const uint4 q = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? ro + 4u * ic : kMasked, 0, 0));
                    buf[ii] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y),
                                         __uint_as_float(q.z), __uint_as_float(q.w));
                } else {
                    float vv[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const bool ok = rok & (ic + k >= 0) & (ic + k < W);
                        vv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                            xr, ok ? ro + 4u * (ic + k) : kMasked, 0, 0));
                    }
                    buf[ii] = make_float4(vv[0], vv[1], vv[2], vv[3]);
                }
            }
#pragma unroll
            for (int ii = 0; ii < TB; ++ii) {
                const int i = i0 + ii;
                const int e = threadIdx.x + i * NT;
                if (i < PER && e < TOTAL) {
                    const int rr = e / NTAIL, v = 64 * NFULL + e % NTAIL;
                    float *trow = tile + row_lds(rr);
                    trow[col_lds(4 * v)] = buf[ii].x;
                    trow[col_lds(4 * v + 1)] = buf[ii].y;
                    trow[col_lds(4 * v + 2)] = buf[ii].z;
                    trow[col_lds(4 * v + 3)] = buf[ii].w;
                }
            }
            }
        }
    };
    if (((ic0 & 3) == 0) && ((W & 3) == 0))
        fill(std::true_type{});
    else
        fill(std::false_type{});
    __syncthreads();

    const int pw = pwt * G::T + 16 * wv + j;
    const float *tb = tile + g4 * PS + 16 * wv + j;
    const uint32_t cplane = (uint32_t)(PH * PW);
    const __amdgpu_buffer_rsrc_t yr =
        make_range_checked(y + (size_t)n * Cout * cplane, 4u * (uint32_t)Cout * cplane);
    const uint32_t lane_off =
        pw < PW ? 4u * ((uint32_t)(4 * g4) * cplane + (uint32_t)(ph * PW + pw)) : 0x80000000u;

    for (int ct = 0; ct < Cout; ct += 16 * NCT) {
        if (ct > 0) {
            __syncthreads();  // every wave is done with the previous tile's biases
            stage_bias(ct);
            load_weights(ct);
            __syncthreads();
        }
        f32x4 best[NCT];
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) best[nt] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};

#pragma unroll 1
        for (int dy = 0; dy < PK; ++dy) {
            const float *tr = tb + dy * G::RSF;
            // window columns in groups of DXG: fewer live accumulators when DXG < PK
            constexpr int DXG = PS_CONV_DXG > 0 && PS_CONV_DXG < PK ? PS_CONV_DXG : PK;
#pragma unroll 1
            for (int dx0 = 0; dx0 < PK; dx0 += DXG)
#pragma unroll
            for (int dk = 0; dk < DXG; ++dk) {
                const int dx = dx0 + dk;
                if (DXG < PK && dx >= PK) break;
                f32x4 acc[NCT];
#pragma unroll
                for (int nt = 0; nt < NCT; ++nt) acc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < CING; ++g)
#pragma unroll
                    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                        for (int kw = 0; kw < 3; ++kw) {
                            const int t = dx + kw;
                            const float b = tr[g * 4 * PS + kh * G::RSF + (t % PK) * G::QF + t / PK];
#pragma unroll
                            for (int nt = 0; nt < NCT; ++nt)
                                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    wr[nt][kh * 3 + kw][g], b, acc[nt], 0, 0, 0);
                        }
#pragma unroll
                for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) best[nt][r] = fmaxf(best[nt][r], acc[nt][r]);
            }
        }

        // ---- epilogue: conv bias, tanh, scale, bias2; D row 4*g4 + r = channel ----
        // Range-checked buffer stores over image n's Cout planes: a column pw >= PW
        // takes an offset past the end, and so does a channel >= Cout, so the stores
        // are dropped without branches (the host keeps (Cout + 64) planes below 2^31
        // bytes, so no offset wraps).
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cl = 16 * nt + 4 * g4 + r;
                const float e = __builtin_amdgcn_exp2f(fmaf(best[nt][r], k2, s_bias[0][cl]));
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(fmaf(m2, __builtin_amdgcn_rcpf(e + 1.f), s_bias[1][cl])), yr,
                    lane_off + 4u * (uint32_t)(ct + 16 * nt + r) * cplane, 0, 0);
            }
    }
}

// ---------------------------------------------------------------- bf16 ---
// Persistent, software-pipelined: a workgroup owns a run of consecutive pooled
// rows [p0, p1) of one image and one 16*NPW-column strip.  Its weights are loaded
// once.  Input rows live in an LDS ring of 2*PK + 2 rows (channel-last entries of
// 8 bf16): pooled row ph reads ring rows PK*ph - pad ... + PK + 1, while the PK
// rows that pooled row ph+1 adds are loaded from HBM during the MFMA work of row ph
// (into an LDS staging area when rows are 16-byte aligned, else into registers) and
// transposed into the ring afterwards.  One barrier per row.
template <int PK, int NPW, bool VEC, bool MULTI>
__global__ __launch_bounds__(64 * NPW, (PK <= 4 ? 2 : 1)) void conv_pool_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ cb,
    const float *__restrict__ b2, uint16_t *__restrict__ y, int Cin, int H, int W, int Cout,
    int pad, int PH, int PW, float scale, int npwt, int nseg) {
    using G = TileGeom<PK, NPW>;
    constexpr int NT = 64 * NPW;
    constexpr int RING = 2 * PK + 2;        // input rows held in LDS
    constexpr int NG = (G::COLS + 7) / 8;   // 8-column groups per tile row
    __shared__ uint4 ring[RING * G::RS];
    __shared__ float s_bias[2][64];
    constexpr int NTOT = PK * NG;           // 8-column groups of the PK rows a pooled row adds
    constexpr int NPER = (NTOT + NT - 1) / NT;
    // VEC: the rows of the next pooled row are loaded straight into LDS (buffer loads
    // with the LDS flag, range-checked like the register loads).  A lane's 16 bytes
    // land in its own slot, stage[i][wave][ci][lane], so each thread reads back only
    // what it loaded itself, after its own loads have completed: no barrier, and no
    // registers held across the MFMA stream.
    __shared__ uint4 stage[VEC ? NPER : 1][VEC ? NPW : 1][8][VEC ? 64 : 1];
    const int wvu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- work item: (image n, column strip pwt, pooled rows [p0, p1)) ----
    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int seg = (int)(L % (uint32_t)nseg);
    const int pwt = (int)((L / (uint32_t)nseg) % (uint32_t)npwt);
    const int n = (int)(L / ((uint32_t)nseg * (uint32_t)npwt));
    const int p0 = (int)(((int64_t)PH * seg) / nseg);
    const int p1 = (int)(((int64_t)PH * (seg + 1)) / nseg);

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int j = lane & 15;
    const int g4 = lane >> 4;
    const int ic0 = PK * pwt * G::T - pad;
    const uint16_t *xn = x + (size_t)n * Cin * H * W;
    const size_t cstride = (size_t)H * W;
    // VEC: the strip's columns are 16-byte aligned (ic0 % 8 == 0, W % 8 == 0), so a
    // group of 8 columns is one 16-byte load per channel and lies wholly inside or
    // wholly outside the image; otherwise columns are loaded one by one.

    // Load input row ir, columns [ic0 + 8u, ic0 + 8u + 8), all 8 channels.  VEC: one
    // range-checked 16-byte buffer load per channel over image n (below 2^31 bytes,
    // host check); a group outside the image or a channel >= Cin gets a masked offset
    // and reads zero, so the loads are unconditional (no branch per load).
    const __amdgpu_buffer_rsrc_t xr =
        make_range_checked(xn, 2u * (uint32_t)Cin * (uint32_t)cstride);
    auto load_group = [&](int ir, int u, uint4 (&v)[8]) {
        const int ic = ic0 + 8 * u;
        const bool rok = ir >= 0 && ir < H;
#pragma unroll
        for (int ci = 0; ci < 8; ++ci) {
            v[ci] = make_uint4(0u, 0u, 0u, 0u);
            const uint16_t *src = xn + ci * cstride + (size_t)ir * W + ic;
            if constexpr (VEC) {
                const bool ok = rok & (ci < Cin) & (ic >= 0) & (ic < W);
                const uint32_t o = 2u * ((uint32_t)ci * (uint32_t)cstride + (uint32_t)(ir * W + ic));
                v[ci] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? o : 0x80000000u, 0, 0));
            } else if (rok && ci < Cin) {
                uint32_t hv[8];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    hv[k] = (ic + k >= 0 && ic + k < W) ? (uint32_t)src[k] : 0u;
                v[ci] = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16),
                                   hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16));
            }
        }
    };
    // Transpose the 8x8 block (channel x column) and write 8 channel-last entries.
    auto store_group = [&](int ir, int u, const uint4 (&v)[8]) {
        uint4 *rrow = ring + (((ir % RING) + RING) % RING) * G::RS;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = 8 * u + k;
            // column k sits in word k/2 of each channel's vector, low half for even k;
            // one byte permute packs that half of two channels into one word
            const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
            uint32_t wd[8];
#pragma unroll
            for (int ci = 0; ci < 8; ++ci)
                wd[ci] = (k >> 1) == 0 ? v[ci].x : (k >> 1) == 1 ? v[ci].y
                       : (k >> 1) == 2 ? v[ci].z : v[ci].w;
            if (c < G::COLS)
                rrow[(c % PK) * G::Q + c / PK] =
                    make_uint4(__builtin_amdgcn_perm(wd[1], wd[0], sel), __builtin_amdgcn_perm(wd[3], wd[2], sel),
                               __builtin_amdgcn_perm(wd[5], wd[4], sel), __builtin_amdgcn_perm(wd[7], wd[6], sel));
        }
    };

    // A operands: lane holds w[co = ct + 16*nt + j][ci = 0..7][tap = 4*s + g4]
    const uint32_t wsign = scale < 0.f ? 0x80008000u : 0u;
    bf16x8 wa[4][3];
    auto load_weights = [&](int ct) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int co = ct + 16 * nt + j;
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                const int tap = 4 * s + g4;
                uint32_t hv[8];
#pragma unroll
                for (int ci = 0; ci < 8; ++ci) {
                    const bool ok = co < Cout && ci < Cin && tap < 9;
                    const uint32_t v = w[ok ? ((size_t)co * Cin + ci) * 9 + tap : 0];
                    hv[ci] = ok ? v : 0u;
                }
                // negative scale: negate the weights (exact), so the window max of the
                // negated sums is minus the window min of the sums
                uint4 pk;
                pk.x = (hv[0] | (hv[1] << 16)) ^ wsign;
                pk.y = (hv[2] | (hv[3] << 16)) ^ wsign;
                pk.z = (hv[4] | (hv[5] << 16)) ^ wsign;
                pk.w = (hv[6] | (hv[7] << 16)) ^ wsign;
                wa[nt][s] = __builtin_bit_cast(bf16x8, pk);
            }
        }
    };
    // Epilogue constants: with u = sgn*best + cb, tanh(u) = 1 - 2/(2^(2u log2e) + 1), so
    // out = (scale + b2) - 2 scale / (2^(best*k2 + cb*2log2e) + 1), k2 = 2 log2e sgn.
    constexpr float kTwoLog2e = 2.8853900817779268f;
    auto stage_bias = [&](int ct) {
        if (threadIdx.x < 64) {
            const int co = ct + threadIdx.x;
            s_bias[0][threadIdx.x] = (co < Cout && cb) ? cb[co] * kTwoLog2e : 0.f;
            s_bias[1][threadIdx.x] = co < Cout ? scale + b2[co] : 0.f;
        }
    };

    // ---- prologue: the PK + 2 input rows of pooled row p0 ----
    if (p0 < p1) {
        constexpr int TOTAL = (PK + 2) * NG;
        constexpr int PER = (TOTAL + NT - 1) / NT;
        const int ir0 = PK * p0 - pad;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = threadIdx.x + i * NT;
            if (e < TOTAL) {
                uint4 v[8];
                load_group(ir0 + e / NG, e % NG, v);
                store_group(ir0 + e / NG, e % NG, v);
            }
        }
    }

    // Per lane, K-step s covers kernel tap 4*s + g4; taps >= 9 carry
    // zero weights and read a valid in-ring entry.  Column part of the ring offset per
    // (s, dx), and the lane's pooled column within the strip.
    constexpr int NS = 3;
    const int pwl = 16 * wv + j;
    int coff[NS][PK];
    int khs[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int tap = min(4 * s + g4, 8);
        const int kh = tap / 3, kw = tap % 3;
        khs[s] = kh;
#pragma unroll
        for (int dx = 0; dx < PK; ++dx) {
            const int t = dx + kw;
            coff[s][dx] = (t % PK) * G::Q + pwl + t / PK;
        }
    }
    const int pw = pwt * G::T + pwl;
    const float k2 = scale < 0.f ? -kTwoLog2e : kTwoLog2e;
    const float m2 = -2.f * scale;
    // Output stores go through a range-checked resource over image n's Cout planes:
    // a store at or past its end is dropped, which masks channels >= Cout without
    // branches; columns pw >= PW take an offset far past the end (the host keeps
    // (Cout + 64) planes under 2^31 bytes, so no offset wraps).
    const uint32_t cplane = (uint32_t)(PH * PW);
    const __amdgpu_buffer_rsrc_t yr =
        make_range_checked(y + (size_t)n * Cout * cplane, 2u * (uint32_t)Cout * cplane);
    const uint32_t lane_c0 = 4 * g4;  // the lane's first channel
    const uint32_t lane_off = pw < PW ? 2u * (lane_c0 * cplane + (uint32_t)pw) : 0x80000000u;
    // MULTI: Cout > 64, the weights and biases of each 64-channel tile are reloaded per row
    constexpr bool single_tile = !MULTI;
    if constexpr (single_tile) {
        load_weights(0);
        stage_bias(0);
    }
    __syncthreads();

    for (int ph = p0; ph < p1; ++ph) {
        // issue the loads of the PK rows that pooled row ph + 1 adds
        uint4 pre[VEC ? 1 : NPER][8];  // unaligned rows: loaded into registers
        const int nr0 = PK * (ph + 1) - pad + 2;
        const bool more = ph + 1 < p1;
        if (more) {
#pragma unroll
            for (int i = 0; i < NPER; ++i) {
                const int e = threadIdx.x + i * NT;
                if (e < NTOT) {
                    if constexpr (VEC) {
                        const int ir = nr0 + e / NG, ic = ic0 + 8 * (e % NG);
                        const bool rok = ir >= 0 && ir < H;
#pragma unroll
                        for (int ci = 0; ci < 8; ++ci) {
                            const bool ok = rok & (ci < Cin) & (ic >= 0) & (ic < W);
                            const uint32_t o = 2u * ((uint32_t)ci * (uint32_t)cstride + (uint32_t)(ir * W + ic));
                            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                                xr, (__attribute__((address_space(3))) void *)&stage[i][wvu][ci][0], 16,
                                ok ? o : 0x80000000u, 0, 0, 0);
                        }
                    } else {
                        load_group(nr0 + e / NG, e % NG, pre[i]);
                    }
                }
            }
        }

        // write the prefetched rows of pooled row ph + 1 into the ring
        auto refill = [&]() {
#pragma unroll
            for (int i = 0; i < NPER; ++i) {
                const int e = threadIdx.x + i * NT;
                if (e < NTOT) {
                    if constexpr (VEC) {
                        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's loads have landed
                        uint4 v[8];
#pragma unroll
                        for (int ci = 0; ci < 8; ++ci) v[ci] = stage[i][wvu][ci][lane];
                        store_group(nr0 + e / NG, e % NG, v);
                    } else {
                        store_group(nr0 + e / NG, e % NG, pre[i]);
                    }
                }
            }
        };
        const int rbase = PK * ph - pad;
        for (int ct = 0; ct < Cout; ct += 64) {
            if constexpr (!single_tile) {
                __syncthreads();
                load_weights(ct);
                stage_bias(ct);
                __syncthreads();
            }
            // The pooled row's B fragments stream from the ring in (dy, dx, s) order, each
            // read AHEAD fragments before its four MFMAs, so the matrix cores do not wait
            // on LDS latency.  Position p = dy*PK + dx accumulates into acc[p % 3]; the
            // pool max of positions p-2 and p-1 (one v_max3 per value) is taken after
            // position p's first MFMAs, when their results are long complete.
            constexpr int NPOS = PK * PK;
            constexpr int NFR = NS * NPOS;
            constexpr int AHEAD_REQ = (MULTI || !VEC) && PS_BF16_LDS_AHEAD > 2 ? 2 : PS_BF16_LDS_AHEAD;
            constexpr int AHEAD = AHEAD_REQ < NFR ? AHEAD_REQ : NFR;
            // the variants with more live registers (row loads held in registers, or
            // several channel tiles) take the pool max at the first K-step
            constexpr int MAX_STEP = (MULTI || !VEC) ? 0 : PS_BF16_MAX_STEP;
            int ridx[NS][PK];  // ring entry index of kernel row khs[s] for window row dy
            {
                const int rb = ((rbase % RING) + RING) % RING;
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                    for (int dy = 0; dy < PK; ++dy) {
                        const int r = rb + dy + khs[s];
                        ridx[s][dy] = (r >= RING ? r - RING : r) * G::RS;
                    }
            }
            auto frag = [&](int f) {
                const int pp = f / NS, s = f % NS;
                return __builtin_bit_cast(bf16x8, ring[ridx[s][pp / PK] + coff[s][pp % PK]]);
            };
            bf16x8 bq[AHEAD];
#pragma unroll
            for (int f = 0; f < AHEAD; ++f) bq[f] = frag(f);
            f32x4 best[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) best[nt] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            f32x4 acc[3][4];
#pragma unroll
            for (int f = 0; f < NFR; ++f) {
                const int pp = f / NS, s = f % NS;
                const bf16x8 b = bq[f % AHEAD];
                if (f + AHEAD < NFR) bq[f % AHEAD] = frag(f + AHEAD);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[pp % 3][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        wa[nt][s], b, s == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : acc[pp % 3][nt], 0, 0, 0);
                if (s == MAX_STEP && pp >= 2 && pp % 2 == 0) {
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            best[nt][r] = fmaxf(fmaxf(best[nt][r], acc[(pp - 2) % 3][nt][r]),
                                                acc[(pp - 1) % 3][nt][r]);
                    // an empty volatile asm that takes the maxima as operands keeps them
                    // in this step (pure arithmetic would otherwise sink to the epilogue
                    // and hold every position's sums live)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        asm volatile("" : "+v"(best[nt]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (NPOS % 2 == 0)
                        best[nt][r] = fmaxf(fmaxf(best[nt][r], acc[(NPOS - 2) % 3][nt][r]),
                                            acc[(NPOS - 1) % 3][nt][r]);
                    else
                        best[nt][r] = fmaxf(best[nt][r], acc[(NPOS - 1) % 3][nt][r]);
                }
            // One channel tile: write the prefetched rows to the ring before the output
            // stores (their ring slots are not read by row ph), so that waiting for the
            // loads does not also wait for the output stores (on this chip a wait on a
            // load issued before pending stores waits for those stores too).
            if (single_tile && more) refill();
            // output (n, co = ct + 16 nt + 4 g4 + r, ph, pw)
            const uint32_t row_off = lane_off + 2u * ((uint32_t)ct * cplane + (uint32_t)(ph * PW));
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float4 cbv = *(const float4 *)&s_bias[0][16 * nt + 4 * g4];
                const float4 c2v = *(const float4 *)&s_bias[1][16 * nt + 4 * g4];
                const float cbr[4] = {cbv.x, cbv.y, cbv.z, cbv.w};
                const float c2r[4] = {c2v.x, c2v.y, c2v.z, c2v.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = __builtin_amdgcn_exp2f(fmaf(best[nt][r], k2, cbr[r]));
                    const float o = fmaf(m2, __builtin_amdgcn_rcpf(e + 1.f), c2r[r]);
                    __builtin_amdgcn_raw_buffer_store_b16(
                        f32_to_bf16_rne(o), yr, (int)(row_off + 2u * (uint32_t)(16 * nt + r) * cplane),
                        0, 0);
                }
            }
        }
        if (!single_tile && more) refill();
        __syncthreads();
    }
}

// bf16, one 64-channel tile, pool <= 4, rows 16-byte aligned: v_mfma_f32_32x32x16_bf16.
// Persistent like the kernel above (a run of pooled rows of one strip per workgroup,
// weights loaded once), with:
//   - a ring of 2*PK input rows: after each pooled row's matrix work a barrier, then the
//     next row's PK new rows (already in the LDS staging area) overwrite the two oldest
//     rows of the current one, then a second barrier;
//   - pooled rows processed in pairs, so the ring slot of every B fragment is known at
//     compile time: a fragment address is one of a few per-lane bases plus an immediate
//     offset, with no per-row address arithmetic;
//   - a staging area that holds only the 8-column groups in use (stage[wave][channel]
//     [group of the wave]).
// At pool 4 and 64 columns: 141 VGPRs and 50.7 KB of LDS (with a 2*PK + 2 row ring and
// per-row addresses: 194 VGPRs, 74 KB).  Three workgroups would fit a CU, but it is
// launched with two: a 63-row plane splits into 4 runs of 15-16 rows, and into 6 runs of
// 10-11 rows the longest run is 5% above the mean, which cost more than the third
// workgroup's latency hiding gained on the conv+pool workload.
template <int PK, int NPW>
__global__ __launch_bounds__(64 * NPW, 3) void conv_pool_bf16_w32(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ cb,
    const float *__restrict__ b2, uint16_t *__restrict__ y, int Cin, int H, int W, int Cout,
    int pad, int PH, int PW, float scale, int npwt, int nseg) {
    using G = TileGeom<PK, NPW>;
    constexpr int NT = 64 * NPW;
    constexpr int RING = 2 * PK;             // input rows held in LDS
    constexpr int NG = (G::COLS + 7) / 8;    // 8-column groups per tile row
    constexpr int NTOT = PK * NG;            // groups of the PK rows a pooled row adds
    constexpr int IPW = (NTOT + NPW - 1) / NPW;  // of them per wave
    static_assert(IPW <= 64, "one group per lane");
    static_assert(RING * G::RS * 16 < 65536, "fragment offsets fit the LDS offset field");
    __shared__ uint4 ring[RING * G::RS];
    __shared__ uint4 stage[NPW][8][IPW];
    __shared__ float s_bias[2][64];
    const int wvu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- work item: (image n, column strip pwt, pooled rows [p0, p1)) ----
    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int seg = (int)(L % (uint32_t)nseg);
    const int pwt = (int)((L / (uint32_t)nseg) % (uint32_t)npwt);
    const int n = (int)(L / ((uint32_t)nseg * (uint32_t)npwt));
    const int p0 = (int)(((int64_t)PH * seg) / nseg);
    const int p1 = (int)(((int64_t)PH * (seg + 1)) / nseg);

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int ic0 = PK * pwt * G::T - pad;
    const int r0 = PK * p0 - pad;  // input row in ring slot 0
    const uint16_t *xn = x + (size_t)n * Cin * H * W;
    const uint32_t cstride = (uint32_t)H * (uint32_t)W;
    const __amdgpu_buffer_rsrc_t xr = make_range_checked(xn, 2u * (uint32_t)Cin * cstride);
    // byte offset of input (row ir, column ic) of channel ci, or a masked offset (reads 0)
    auto in_off = [&](int ir, int ic, int ci) {
        const bool ok = (ir >= 0) & (ir < H) & (ci < Cin) & (ic >= 0) & (ic < W);
        return ok ? 2u * ((uint32_t)ci * cstride + (uint32_t)(ir * W + ic)) : 0x80000000u;
    };
    // Transpose an 8x8 block (channel x column: 8 columns of each channel) and write the
    // 8 channel-last entries of input row ir, group u.
    auto store_group = [&](int ir, int u, const uint4 (&v)[8]) {
        uint4 *rrow = ring + ((ir - r0) % RING) * G::RS;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = 8 * u + k;
            const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
            uint32_t wd[8];
#pragma unroll
            for (int ci = 0; ci < 8; ++ci)
                wd[ci] = (k >> 1) == 0 ? v[ci].x : (k >> 1) == 1 ? v[ci].y
                       : (k >> 1) == 2 ? v[ci].z : v[ci].w;
            if (c < G::COLS)
                rrow[(c % PK) * G::Q + c / PK] =
                    make_uint4(__builtin_amdgcn_perm(wd[1], wd[0], sel), __builtin_amdgcn_perm(wd[3], wd[2], sel),
                               __builtin_amdgcn_perm(wd[5], wd[4], sel), __builtin_amdgcn_perm(wd[7], wd[6], sel));
        }
    };

    // Wave wv owns channels 32*(wv & 1) .. +31 and pooled columns 32*(wv >> 1) .. +31 of
    // the strip; lane l is pixel (B/D column) l & 31 and, as A row, channel
    // 32*(wv & 1) + (l & 31).  K-step s (0..4) = kernel taps 2s, 2s+1 x 8 channels, lane
    // half h = l >> 5 taking tap 2s + h (tap 9 carries zero weights).
    const int h32 = lane >> 5, n32 = lane & 31;
    const int cw32 = wv & 1, px32 = wv >> 1;
    const uint32_t wsign = scale < 0.f ? 0x80008000u : 0u;
    bf16x8 wa32[5];
    {
        const int co = 32 * cw32 + n32;
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            const int tap = 2 * s + h32;
            uint32_t hv[8];
#pragma unroll
            for (int ci = 0; ci < 8; ++ci) {
                const bool ok = co < Cout && ci < Cin && tap < 9;
                const uint32_t v = w[ok ? ((size_t)co * Cin + ci) * 9 + tap : 0];
                hv[ci] = ok ? v : 0u;
            }
            // negative scale: negate the weights (exact), so the window max of the
            // negated sums is minus the window min of the sums
            uint4 pk;
            pk.x = (hv[0] | (hv[1] << 16)) ^ wsign;
            pk.y = (hv[2] | (hv[3] << 16)) ^ wsign;
            pk.z = (hv[4] | (hv[5] << 16)) ^ wsign;
            pk.w = (hv[6] | (hv[7] << 16)) ^ wsign;
            wa32[s] = __builtin_bit_cast(bf16x8, pk);
        }
    }
    // with u = sgn*best + cb, tanh(u) = 1 - 2/(2^(2u log2e) + 1), so
    // out = (scale + b2) - 2 scale / (2^(best*k2 + cb*2log2e) + 1), k2 = 2 log2e sgn
    constexpr float kTwoLog2e = 2.8853900817779268f;
    if (threadIdx.x < 64) {
        const int co = threadIdx.x;
        s_bias[0][threadIdx.x] = (co < Cout && cb) ? cb[co] * kTwoLog2e : 0.f;
        s_bias[1][threadIdx.x] = co < Cout ? scale + b2[co] : 0.f;
    }

    // ---- prologue: the PK + 2 input rows of pooled row p0, into slots 0 .. PK + 1 ----
    if (p0 < p1) {
        constexpr int TOTAL = (PK + 2) * NG;
        constexpr int PER = (TOTAL + NT - 1) / NT;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = threadIdx.x + i * NT;
            if (e < TOTAL) {
                const int ir = r0 + e / NG, ic = ic0 + 8 * (e % NG);
                uint4 v[8];
#pragma unroll
                for (int ci = 0; ci < 8; ++ci)
                    v[ci] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, in_off(ir, ic, ci), 0, 0));
                store_group(ir, e % NG, v);
            }
        }
    }

    const int pwl = 32 * px32 + n32;  // the lane's pooled column within the strip
    const int pw = pwt * G::T + pwl;
    const float k2 = scale < 0.f ? -kTwoLog2e : kTwoLog2e;
    const float m2 = -2.f * scale;
    // Output stores go through a range-checked resource over image n's Cout planes: a
    // store at or past its end is dropped (channels >= Cout); columns pw >= PW take an
    // offset far past the end (the host keeps (Cout + 64) planes under 2^31 bytes).
    const uint32_t cplane = (uint32_t)(PH * PW);
    const __amdgpu_buffer_rsrc_t yr =
        make_range_checked(y + (size_t)n * Cout * cplane, 2u * (uint32_t)Cout * cplane);
    const uint32_t lane_off =
        pw < PW ? 2u * ((uint32_t)(32 * cw32 + 4 * h32) * cplane + (uint32_t)pw) : 0x80000000u;
    // this thread's group of the PK new rows: e = wave * IPW + lane
    const int fe = wvu * IPW + lane;
    const bool f_on = lane < IPW && fe < NTOT;
    const int f_row = fe / NG, f_u = fe % NG;
    const char *ringb = (const char *)ring;
    const int lane16 = 16 * pwl;
    // the wave's staging slots as an LDS pointer (the DMA loads' destination)
    typedef __attribute__((address_space(3))) uint4 lds_uint4;
    lds_uint4 *const stg = (lds_uint4 *)&stage[wvu][0][0];
    __syncthreads();

    // Pooled rows in pairs; phase = (ph - p0) mod 2 is a constant in each unrolled copy,
    // so the row's input rows r0 + PK*(ph - p0) + k sit in known ring slots
    // (phase*PK + k) mod RING.
    for (int ph0 = p0; ph0 < p1; ph0 += 2) {
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
        const int ph = ph0 + phase;
        if (ph >= p1) break;
        const bool more = ph + 1 < p1;
        const int nr0 = PK * (ph + 1) - pad + 2;  // first new row of pooled row ph + 1
        if (more && f_on) {
            const int ir = nr0 + f_row, ic = ic0 + 8 * f_u;
#pragma unroll
            for (int ci = 0; ci < 8; ++ci) {
                const uint32_t o = in_off(ir, ic, ci);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (__attribute__((address_space(3))) void *)(stg + ci * IPW), 16, o, 0, 0, 0);
            }
        }
        // byte offset within the ring of entry (row k of this pooled row, tile column c)
        auto eoff = [&](int k, int c) {
            return ((phase * PK + k) % RING) * G::RS * 16 + ((c % PK) * G::Q + c / PK) * 16;
        };
        // B fragment f = (window position pp, K-step s): lane half h reads tap
        // min(2s + h, 8) at (dy + kh, dx + kw); the half-1 difference is a per-lane
        // constant, the rest an immediate offset
        auto frag = [&](int f) {
            const int pp = f / 5, s = f % 5, dy = pp / PK, dx = pp % PK;
            const int t0 = 2 * s, t1 = 2 * s + 1 < 9 ? 2 * s + 1 : 8;
            const int o0 = eoff(dy + t0 / 3, dx + t0 % 3);
            const int o1 = eoff(dy + t1 / 3, dx + t1 % 3);
            return *(const bf16x8 *)(ringb + (lane16 + (h32 ? o1 - o0 : 0)) + o0);
        };
        constexpr int NPOS = PK * PK;
        constexpr int NFR = 5 * NPOS;
        constexpr int AHEAD = PS_BF16_W32_AHEAD < NFR ? PS_BF16_W32_AHEAD : NFR;
        bf16x8 bq[AHEAD];
#pragma unroll
        for (int f = 0; f < AHEAD; ++f) bq[f] = frag(f);
        // D (32x32): lane l, register r = channel 32*(wv & 1) + 8*(r/4) + 4*h32 + r%4 of
        // the tile, pooled column pwl.  Position p = dy*PK + dx accumulates into
        // acc[p % 3]; the pool max of positions p-2 and p-1 (one v_max3 per value) is
        // taken at position p's third K-step, when their results are long complete.
        f32x16 best;
#pragma unroll
        for (int r = 0; r < 16; ++r) best[r] = -INFINITY;
        f32x16 acc[3];
#pragma unroll
        for (int f = 0; f < NFR; ++f) {
            const int pp = f / 5, s = f % 5;
            const bf16x8 b = bq[f % AHEAD];
            if (f + AHEAD < NFR) bq[f % AHEAD] = frag(f + AHEAD);
            acc[pp % 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                wa32[s], b, s == 0 ? (f32x16){} : acc[pp % 3], 0, 0, 0);
            if (s == 2 && pp >= 2 && pp % 2 == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    best[r] = fmaxf(fmaxf(best[r], acc[(pp - 2) % 3][r]), acc[(pp - 1) % 3][r]);
                // an empty volatile asm that takes the maxima as operands keeps them in
                // this step (sunk to the end they would hold every position's sums live)
                asm volatile("" : "+v"(best));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (NPOS % 2 == 0)
                best[r] = fmaxf(fmaxf(best[r], acc[(NPOS - 2) % 3][r]), acc[(NPOS - 1) % 3][r]);
            else
                best[r] = fmaxf(best[r], acc[(NPOS - 1) % 3][r]);
        }
        __syncthreads();  // every wave is done reading this row's ring slots
        if (more && f_on) {
            // the new rows go to slots ((phase + 1)*PK + 2 + i) mod RING, two of which
            // held this row's first two input rows
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's loads have landed
            uint4 v[8];
#pragma unroll
            for (int ci = 0; ci < 8; ++ci) v[ci] = stage[wvu][ci][lane];
            store_group(nr0 + f_row, f_u, v);
        }
        // output (n, co = 32*(wv & 1) + 8*(r/4) + 4*h32 + r%4, ph, pw)
        const uint32_t row_off = lane_off + 2u * (uint32_t)(ph * PW);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c0 = 32 * cw32 + 8 * q + 4 * h32;
            const float4 cbv = *(const float4 *)&s_bias[0][c0];
            const float4 c2v = *(const float4 *)&s_bias[1][c0];
            const float cbr[4] = {cbv.x, cbv.y, cbv.z, cbv.w};
            const float c2r[4] = {c2v.x, c2v.y, c2v.z, c2v.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = __builtin_amdgcn_exp2f(fmaf(best[4 * q + r], k2, cbr[r]));
                const float o = fmaf(m2, __builtin_amdgcn_rcpf(e + 1.f), c2r[r]);
                __builtin_amdgcn_raw_buffer_store_b16(
                    f32_to_bf16_rne(o), yr, (int)(row_off + 2u * (uint32_t)(8 * q + r) * cplane), 0, 0);
            }
        }
        __syncthreads();  // the ring holds pooled row ph + 1's rows; the stage is free
    }
    }
}

template <int PK, int NPW>
int launch_pk_npw(const void *x, const void *w, const float *cb, const float *b2, void *y,
                  int dtype, int N, int Cin, int H, int W, int Cout, int pad, float scale, int PH,
                  int PW, hipStream_t stream) {
    const int npwt = (PW + 16 * NPW - 1) / (16 * NPW);
    if (dtype == PS_BF16) {
        // persistent workgroups, each a run of pooled rows of one strip, about two per CU
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) != hipSuccess) return PS_ERR_HIP;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return PS_ERR_HIP;
        // every strip starts at a multiple of 16*NPW*PK columns, so alignment is uniform
        const bool vec = (pad % 8 == 0) && (W % 8 == 0);
        const bool multi = Cout > 64;
        // one channel tile, pool <= 4, 32 or 64 columns per strip and rows staged through
        // LDS: the 32x32x16 form (with rows held in registers it would spill)
        constexpr bool w32_ok = PK <= 4 && (NPW == 2 || NPW == 4);
        const bool w32 = w32_ok && vec && !multi;
        const int64_t strips = (int64_t)N * npwt;
        int64_t nseg = (2 * (int64_t)ncu + strips - 1) / strips;
        if (nseg > PH) nseg = PH;
        if (nseg < 1) nseg = 1;
        const uint64_t nblocks = (uint64_t)strips * nseg;
        if (nblocks > 0x7fffffffull) return PS_ERR_UNSUPPORTED;
        const dim3 grid((unsigned)nblocks), block(64 * NPW);
        if constexpr (w32_ok) {
            if (w32)
                return launch(conv_pool_bf16_w32<PK, NPW>, grid, block, 0, stream,
                              (const uint16_t *)x, (const uint16_t *)w, cb, b2, (uint16_t *)y, Cin,
                              H, W, Cout, pad, PH, PW, scale, npwt, (int)nseg);
        }
#define PS_BF16_LAUNCH(V, M)                                                                  \
    launch(conv_pool_bf16<PK, NPW, V, M>, grid, block, 0, stream, (const uint16_t *)x,        \
           (const uint16_t *)w, cb, b2, (uint16_t *)y, Cin, H, W, Cout, pad, PH, PW, scale,   \
           npwt, (int)nseg)
        if (vec && !multi) return PS_BF16_LAUNCH(true, false);
        if (vec) return PS_BF16_LAUNCH(true, true);
        if (!multi) return PS_BF16_LAUNCH(false, false);
        return PS_BF16_LAUNCH(false, true);
#undef PS_BF16_LAUNCH
    }
    const uint64_t nblocks = (uint64_t)N * PH * npwt;
    if (nblocks > 0x7fffffffull) return PS_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)nblocks), block(64 * NPW);
#define PS_F32_LAUNCH(CG, NCT)                                                                 \
    launch(conv_pool_f32<PK, NPW, CG, NCT>, grid, block, 0, stream, (const float *)x,           \
           (const float *)w, cb, b2, (float *)y, Cin, H, W, Cout, pad, PH, PW, scale, npwt)
    // one 16-channel tile when Cout <= 16 (narrow strips only: the small problems), so
    // no matrix work is spent on channels that do not exist
    if constexpr (NPW == 1) {
        if (Cout <= 16) return Cin <= 4 ? PS_F32_LAUNCH(1, 1) : PS_F32_LAUNCH(2, 1);
    }
    if (Cin <= 4) return PS_F32_LAUNCH(1, 4);
    return PS_F32_LAUNCH(2, 4);
#undef PS_F32_LAUNCH
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

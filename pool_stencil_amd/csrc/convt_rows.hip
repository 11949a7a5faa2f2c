// Fused ConvTranspose2d(k4, s2, any padding p) -> softmax over channels -> +bias2 -> *scale
// -> sigmoid for gfx950, with whole output lines written by one workgroup (128 output
// channels).
//
// Definition (POPCORNBENCH page Kimi-K2.6 l2_p91, problem statement and its scatter
// loop):
//   t[n,co,oh,ow] = bias[co] + sum over (ci, ih, iw, kh, kw) with oh = 2*ih - p + kh,
//                   ow = 2*iw - p + kw of x[n,ci,ih,iw] * w[ci,co,kh,kw]
//   y = sigmoid((softmax_co(t) + bias2[co]) * scale)
//
// Parity decomposition (the page's phase table, written there for p = 1).
//   Rows: output row oh = 2m + a (row class a) takes kernel rows kh = ka + 2u (u = 0, 1),
//   ka = (a + p) mod 2, from input rows ih = m + ra - u, ra = floor((a + p) / 2).
//   Columns: a POSITION c covers the output column pair ow = 2c - (p mod 2) + b'
//   (b' = 0, 1).  Both columns of the pair read the same two input columns
//   iw = c + floor(p / 2) - v (v = 0, 1), column b' through kernel column kw = b' + 2v
//   (2*iw - p + kw = ow).  One B operand (input neighbourhood) therefore feeds both
//   column classes.
//
// Kernel layout:
//   - a workgroup owns a run of 64-position tiles of one image and one row class; the
//     positions of the (row class, image) plane are numbered row by row, so a tile
//     spans at most two position rows and rows have no padding to a tile multiple;
//   - wave w owns output channels 16w .. 16w+15 of every position: its weights for
//     both column classes (16 channels x 4*Cin x 2, 128 VGPRs at Cin = 64) stay in
//     registers for the whole launch, so the LDS holds only input rows and the
//     epilogue exchange, and one workgroup writes every column of its output rows;
//   - input rows go through an LDS ring of 4 rows, channel-last ([column][channel],
//     zero columns at both ends), so a lane's B operand for four K-steps (four input
//     channels of one tap) is one 16-byte LDS read; each input row is loaded once per
//     row class, the next tile's new row in flight during the current tile's matrix
//     work;
//   - GEMM on v_mfma_f32_16x16x4_f32: D = 16 channels x 16 positions per column
//     class, K ordered (channel quad, tap, step) with lane group g taking input
//     channel 16q + 4g + step;
//   - epilogue: the D tiles go to LDS ([pair = (position, column class)][channel]); a
//     thread then owns 32 channels of one pair, so max and sum over the 128 channels
//     are in-lane plus two DPP exchanges inside a quad of lanes;
//   - stores are range-checked buffer stores (masked columns and positions past the
//     plane get an offset past the end and are dropped).
#include "ps_internal.h"

#include <math.h>

#include <type_traits>

namespace ps {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves, two per SIMD
constexpr int kCout = 128;     // 8 waves x 16 channels
constexpr int kTP = 64;        // positions per tile: 4 blocks of 16
constexpr int kRing = 4;       // input-row ring slots
constexpr int kES = kCout + 4; // words per pair in the epilogue exchange
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kMasked = 0x80000000u;  // an offset past the end of every tensor here

__device__ __forceinline__ uint32_t fdiv(uint32_t n, uint32_t m) {
    return m ? __umulhi(n, m) : n;
}

// Lane exchanges inside a quad of lanes (DPP quad_perm): lane i takes lane i^1 / i^2.
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

struct RowsGeom {
    int Cpos;        // positions per row
    uint32_t mC;     // ceil(2^32 / Cpos)
    int segs;        // workgroups per (image, row class) plane
    int Mc[2];       // position rows of row class a
    int ntile[2];    // tiles of a plane of row class a
    int items;       // fill items per input row: (channel pairs) x (4-column groups)
    int W4;          // 4-column groups per input row
};

template <int CQ, int NF, bool SOFTMAX>
__global__ __launch_bounds__(kThreads) void convT_rows_f32(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cbias,
    const float *__restrict__ b2, float *__restrict__ y, int N, int Cin, int H, int W, int OH,
    int OW, int pad, float scale, RowsGeom geo) {
    extern __shared__ float lds[];
    const int Cpos = geo.Cpos;
    constexpr int CST = 16 * CQ + 4;  // LDS words per ring column (channels padded)
    const int slot_words = (Cpos + 1) * CST;
    float *ring = lds;                          // [kRing][Cpos + 1][CST]
    float *ex = lds + kRing * slot_words;       // [2 * kTP pairs][kES], swizzled (ex_quad)
    float *lcb = ex + 2 * kTP * kES;            // [kCout] convT bias (times log2 e with the softmax)
    float *lb2 = lcb + kCout;                   // [kCout] -bias2 * scale * log2 e
    float *dummy = lb2 + kCout;                 // [64][2] fill writes with no place in the ring

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;

    // ---- unit: (image n, row class a, segment s); the two row classes of an image
    // are neighbouring logical blocks, which xcd_remap keeps on one XCD (they read
    // the same input rows at about the same time)
    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int a = L & 1;
    const int seg = (int)((L >> 1) % (uint32_t)geo.segs);
    const int n = (int)((L >> 1) / (uint32_t)geo.segs);
    const int Mc = geo.Mc[a];
    const int plane_pos = Mc * Cpos;
    const int ntile = geo.ntile[a];
    const int T0 = (int)((int64_t)seg * ntile / geo.segs);
    const int T1 = (int)((int64_t)(seg + 1) * ntile / geo.segs);
    const int ka = (a + pad) & 1, ra = (a + pad) >> 1;
    const int e = pad >> 1;   // input column of position c, tap v = 0, is c + e
    const int d0 = -(pad & 1);  // output column of position c, b' = 0, is 2c + d0

    // ---- weights: wr[b][q][tap][s] = w[ci][co][ka + 2u][b + 2v] for co = 16*wv + j,
    // ci = 16q + 4g + s, tap = 2u + v; zero for ci >= Cin.  With the softmax they are
    // scaled by log2 e (the epilogue works in base 2), so the MFMAs produce t * log2 e.
    const float wscale = SOFTMAX ? kLog2e : 1.f;
    float wr[2][CQ][4][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < CQ; ++q)
#pragma unroll
            for (int tp = 0; tp < 4; ++tp)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    // (a load at a clamped index and a select: a conditional load compiled
                    // to a branch and a wait per weight)
                    const int ci = 16 * q + 4 * g + s;
                    const bool ok = ci < Cin;
                    const int kh = ka + 2 * (tp >> 1), kw = b + 2 * (tp & 1);
                    const float v =
                        w[(((size_t)(ok ? ci : 0) * kCout + 16 * wv + j) * 4 + kh) * 4 + kw];
                    wr[b][q][tp][s] = ok ? v * wscale : 0.f;
                }
    for (int i = tid; i < kCout; i += kThreads) {
        const float cb = cbias ? cbias[i] : 0.f;
        lcb[i] = SOFTMAX ? cb * kLog2e : cb;
        if constexpr (SOFTMAX) lb2[i] = -b2[i] * scale * kLog2e;
    }
    // zero the ring: columns outside the image stay zero for the whole launch
    for (int i = tid; i < kRing * slot_words; i += kThreads) ring[i] = 0.f;

    // ---- fill items of this thread (the same for every input row): channel pair cp,
    // 4-column group cg (cg fastest, so a wave's loads cover whole row segments)
    const uint32_t plane = (uint32_t)H * W;
    const uint32_t xbytes = 4u * (uint32_t)N * Cin * plane;  // < 2^31 (host check)
    const __amdgpu_buffer_rsrc_t xr = make_range_checked(x, xbytes);
    uint32_t fo[NF][2];   // byte offsets of the item's two channels at row 0 (kMasked if none)
    int fl[NF];           // LDS word of the item's first column and first channel in a slot
    int fm[NF];           // bit r: column 4*cg + r has a place in the slot
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int it = tid + f * kThreads;
        const bool ok = it < geo.items;
        const int cg = ok ? it % geo.W4 : 0, cp = ok ? it / geo.W4 : 0;
        const int ci0 = 2 * cp;
        const uint32_t o = 4u * (((uint32_t)n * Cin + ci0) * plane + 4u * cg);
        fo[f][0] = ok && ci0 < Cin ? o : kMasked;
        fo[f][1] = ok && ci0 + 1 < Cin ? o + 4u * plane : kMasked;
        const int j0 = 4 * cg - e + 1;  // slot column of input column 4*cg
        fl[f] = j0 * CST + ci0;
        int m = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (ok && j0 + r >= 0 && j0 + r <= Cpos) m |= 1 << r;
        fm[f] = m;
    }
    // loads of input row ih (zero outside the image) and their LDS writes.  Both are
    // unconditional and branch-free (a row that is not needed, `on` false, reads zeros
    // through masked offsets and goes to a per-lane dummy area), so the compiler can
    // count the memory operations in flight and waits for these loads only, not for the
    // output stores issued after them.
    float *const dl = dummy + 2 * lane;
    auto fill_load = [&](int ih, bool on, f32x4 (&v)[NF][2]) {
        const bool rin = on && ih >= 0 && ih < H;
        const uint32_t ro = 4u * (uint32_t)(rin ? ih : 0) * W;
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t off = rin ? fo[f][h] + ro : kMasked;
                v[f][h] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            }
    };
    auto fill_store = [&](int ih, bool on, const f32x4 (&v)[NF][2]) {
        float *slot = ring + ((ih + 1) & (kRing - 1)) * slot_words;
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *dst = on && (fm[f] & (1 << r)) ? slot + fl[f] + r * CST : dl;
                *(f32x2 *)dst = (f32x2){v[f][0][r], v[f][1][r]};
            }
    };
    // input rows of tile T: [lo, hi]
    auto tile_rows = [&](int T, int &lo, int &hi) {
        const int t0 = T * kTP;
        const int t1 = min(t0 + kTP, plane_pos) - 1;
        lo = (int)fdiv((uint32_t)t0, geo.mC) + ra - 1;
        hi = (int)fdiv((uint32_t)t1, geo.mC) + ra;
    };

    // (No start stagger: while each tile's ring write waited for all of the tile's
    // output stores, staggered starts kept the chip's stores from arriving in bursts;
    // with the exact wait it no longer pays.)
    __syncthreads();  // ring zeroed before the first fill writes into it
    if (T0 >= T1) return;
    int lo, hi;
    tile_rows(T0, lo, hi);
    for (int ih = lo; ih <= hi; ++ih) {
        f32x4 v[NF][2];
        fill_load(ih, true, v);
        fill_store(ih, true, v);
    }
    __syncthreads();

    const uint32_t oplane = (uint32_t)OH * OW;
    const uint32_t ybytes = 4u * (uint32_t)N * kCout * oplane;  // < 2^31 (host check)
    const __amdgpu_buffer_rsrc_t yr = make_range_checked(y, ybytes);
    const char *ringb = (const char *)ring;

    // Position (row pm, column pc) of this lane in each 16-position block, advanced by
    // one tile (64 <= Cpos positions) per iteration.  Positions past the plane read ring
    // rows that hold finite values; their outputs are dropped.
    int pm[4], pc[4];
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
        const uint32_t t = (uint32_t)(T0 * kTP + 16 * bk + j);
        pm[bk] = (int)fdiv(t, geo.mC);
        pc[bk] = (int)t - pm[bk] * Cpos;
    }
    // epilogue: thread (pair p, channel quarter cq) owns channels 32cq .. 32cq+31 of
    // pair p = 2 * (position in the tile) + b'; its position (em, ec) likewise.  (Eight
    // channels per lane of both column classes, stored as 8-byte column pairs, measured
    // slower: with an odd output width most of those stores are misaligned.)
    const int p = tid >> 2, cq = tid & 3;
    int em, ec;
    {
        const uint32_t t = (uint32_t)(T0 * kTP + (p >> 1));
        em = (int)fdiv(t, geo.mC);
        ec = (int)t - em * Cpos;
    }
    // output row index (n, channel 32cq, row class a) at position row 0; rows below
    // 2^22 (y below 2^29 elements, OW >= 127), so 24-bit multiplies are exact
    const uint32_t yrow0 = __umul24((uint32_t)n * kCout + 32 * cq, (uint32_t)OH) + a;

    // Exchange layout: pair p's slot holds channel quad C (channels 4C .. 4C+3) at quad
    // ex_quad(p, C).  With this swizzle the D-tile writes (16 positions of one column
    // class per 16 lanes) and the epilogue reads (two pairs x four channel quarters per
    // 8 lanes) hit 8 distinct 16-byte bank groups; unswizzled, the writes were 2-way and
    // the reads 4-way bank conflicts.
    auto ex_quad = [](int pair, int C) { return (C ^ ((C >> 2) & 6)) ^ ((pair >> 1) & 15); };
    // this lane's D-tile write: pair 2(16 bk + j) + b, whose (pair >> 1) & 15 is j
    const int ex_w = 2 * j * kES + 4 * ((4 * wv + g) ^ (((4 * wv + g) >> 2) & 6) ^ j);
    // this lane's 8 epilogue reads, channel quads 8 cq + r
    int ex_r[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) ex_r[r] = p * kES + 4 * ex_quad(p, 8 * cq + r);

    // The next tile's new input row (at most one: a tile spans at most two position
    // rows) is loaded one tile ahead, before the current tile's output stores: queued
    // behind those stores, the load held the wave's in-order issue until they drained.
    f32x4 pv[NF][2];
    int nhi = hi;
    if (T0 + 1 < T1) {
        int nlo;
        tile_rows(T0 + 1, nlo, nhi);
    }
    bool has_new = nhi > hi;
    fill_load(nhi, has_new, pv);
    // As many (dropped) stores as a tile's epilogue issues after its prefetch: the
    // compiler counts the memory operations younger than the prefetch over every path
    // into the ring write, and with none on the first tile's path it waited for all of
    // them (every output store of every tile) instead of for the prefetch.
#pragma unroll
    for (int r = 0; r < 32; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(0u, yr, kMasked, (int)(4u * (uint32_t)r * oplane), 0);

    for (int T = T0; T < T1; ++T) {

        // ---- B addresses of block bk, tap row u, at input column v = 1; the v = 0
        // column is CST words further on (an immediate offset, as is the channel quad)
        const char *bp[4][2];
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t slot = (uint32_t)(pm[bk] + ra - u + 1) & (kRing - 1);
                bp[bk][u] = ringb + 4u * (__umul24(slot, (uint32_t)slot_words) +
                                          __umul24((uint32_t)pc[bk], (uint32_t)CST) + 4u * g);
            }
        auto read_b = [&](int bk, int k) {
            const int q = k >> 2, u = (k >> 1) & 1, v = k & 1;
            return *(const f32x4 *)(bp[bk][u] + (v ? 0 : 4 * CST) + 64 * q);
        };

        // accumulators start at the convT bias (times log2 e with the softmax): D row
        // 4g + r is channel 16*wv + 4g + r
        const f32x4 cb4 = *(const f32x4 *)(lcb + 16 * wv + 4 * g);
        f32x4 acc[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int bk = 0; bk < 4; ++bk) acc[b][bk] = cb4;
        // K-step groups k = (q, tap): the B operands of group k + 1 are read from LDS
        // while group k's 32 MFMAs run; inside a group the 8 accumulators alternate, so
        // an MFMA never waits on the one before it.  Scheduling barriers keep that order
        // (left alone, the compiler waited on each read right before its first use and
        // chained dependent MFMAs).  NBK: position blocks computed (a plane's last tile
        // with at most 16 positions computes one; the other blocks keep the bias and
        // their outputs are dropped).
        auto kloop = [&](auto nbk_c) {
            constexpr int NBK = decltype(nbk_c)::value;
            f32x4 bv[2][4];
#pragma unroll
            for (int bk = 0; bk < NBK; ++bk) bv[0][bk] = read_b(bk, 0);
#pragma unroll
            for (int k = 0; k < 4 * CQ; ++k) {
                const int q = k >> 2, tp = k & 3;
                if (k + 1 < 4 * CQ) {
#pragma unroll
                    for (int bk = 0; bk < NBK; ++bk) bv[(k + 1) & 1][bk] = read_b(bk, k + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
                        for (int b = 0; b < 2; ++b)
                            acc[b][bk] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                wr[b][q][tp][s], bv[k & 1][bk][s], acc[b][bk], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // (the class-0 plane of the workload, 65 x 65 positions, ends in a tile of one)
        if (T == ntile - 1 && plane_pos - T * kTP <= 16)
            kloop(std::integral_constant<int, 1>{});
        else
            kloop(std::integral_constant<int, 4>{});

        // the new row goes to a slot that tile T does not read
        fill_store(nhi, has_new, pv);
        hi = nhi;
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
            pc[bk] += kTP;
            if (pc[bk] >= Cpos) {
                pc[bk] -= Cpos;
                ++pm[bk];
            }
        }
        __syncthreads();  // every wave is done with the previous tile's exchange

        // ---- D -> exchange: pair 2*pos + b', channel 16*wv + 4g + r
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int bk = 0; bk < 4; ++bk)
                *(f32x4 *)(ex + (32 * bk + b) * kES + ex_w) = acc[b][bk];
        __syncthreads();  // exchange complete, and the ring holds the next tile's rows

        // ---- epilogue
        uint32_t yo;
        {
            const int ow = 2 * ec + d0 + (p & 1);
            const bool ok = em < Mc && ow >= 0 && ow < OW;
            yo = ok ? 4u * (__umul24(yrow0 + 2u * (uint32_t)em, (uint32_t)OW) + (uint32_t)ow)
                    : kMasked;
            ec += kTP;
            if (ec >= Cpos) {
                ec -= Cpos;
                ++em;
            }
        }
        float v[32];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const f32x4 t = *(const f32x4 *)(ex + ex_r[r]);
            v[4 * r] = t[0];
            v[4 * r + 1] = t[1];
            v[4 * r + 2] = t[2];
            v[4 * r + 3] = t[3];
        }
        if constexpr (SOFTMAX) {
            // exp2 form with the constants folded: v = t * log2 e, e_c = 2^(v_c - max),
            // out_c = 1 / (1 + 2^(e_c * inv + b2'_c)), inv = -scale * log2 e / sum_c e_c,
            // b2'_c = -bias2_c * scale * log2 e (the written order: softmax, +bias2,
            // *scale, sigmoid)
            float mx = v[0];
#pragma unroll
            for (int r = 1; r < 32; ++r) mx = fmaxf(mx, v[r]);
            mx = fmaxf(mx, quad_xor1(mx));
            mx = fmaxf(mx, quad_xor2(mx));
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                v[r] = __builtin_amdgcn_exp2f(v[r] - mx);
                sum += v[r];
            }
            sum += quad_xor1(sum);
            sum += quad_xor2(sum);
            const float inv = -scale * kLog2e * __builtin_amdgcn_rcpf(sum);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const f32x4 bb = *(const f32x4 *)(lb2 + 32 * cq + 4 * r);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float t = __builtin_amdgcn_exp2f(fmaf(v[4 * r + i], inv, bb[i]));
                    v[4 * r + i] = __builtin_amdgcn_rcpf(1.f + t);
                }
            }
        }
        // the row tile T + 2 adds (written into the ring after tile T + 1's matrix work)
        if (T + 2 < T1) {
            int nlo;
            tile_rows(T + 2, nlo, nhi);
        }
        has_new = nhi > hi;
        fill_load(nhi, has_new, pv);
#pragma unroll
        for (int r = 0; r < 32; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), yr, yo,
                                                  (int)(4u * (uint32_t)r * oplane), 0);
    }
}

// bf16 x, w and y (uint16 bit patterns), fp32 accumulation and epilogue: the same
// row-class layout on v_mfma_f32_16x16x32_bf16, with smaller workgroups.
//   - 4 waves per workgroup, two workgroups per CU: wave w keeps 32 channels
//     (32w .. 32w+31, two 16-channel tiles) of both column classes as bf16x8 A operands
//     (128 VGPRs at Cin = 64), so each 16-byte B read from the ring feeds 4 MFMAs (with
//     8 waves of 16 channels every B fragment was read from LDS 8 times, and the matrix
//     phase was bound by LDS bandwidth), and the two workgroups of a CU drift apart so
//     one's softmax arithmetic runs beside the other's matrix work (bf16 MFMA and VALU
//     work overlap on this chip, unlike fp32 MFMA);
//   - tiles of 32 positions (the exchange then fits two workgroups' LDS);
//   - K is ordered (tap, 32-channel block, lane group g), lane group g taking 8
//     consecutive input channels; the ring stores input rows channel-last as bf16
//     channel pairs (16 pad bytes per column), so a lane's B operand is one 16-byte read;
//   - the accumulators start at the convT bias; log2 e is applied inside the softmax's
//     fma (scaling the bf16 weights would round them);
//   - outputs are rounded to bf16 (nearest even) and stored as 2-byte range-checked
//     buffer stores.
constexpr int kThreadsB = 256;  // 4 waves x 32 channels
constexpr int kTPB = 32;        // positions per bf16 tile: 2 blocks of 16

template <int CB>  // input-channel blocks of 32: Cin <= 32 * CB
__global__ __launch_bounds__(kThreadsB, 2) void convT_rows_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const float *__restrict__ cbias, const float *__restrict__ b2, uint16_t *__restrict__ y,
    int N, int Cin, int H, int W, int OH, int OW, int pad, float scale, RowsGeom geo) {
    extern __shared__ float lds[];
    const int Cpos = geo.Cpos;
    constexpr int CSTW = 16 * CB + 4;  // LDS words per ring column: 32*CB channels + 16 bytes
    const int slot_words = (Cpos + 1) * CSTW;
    uint32_t *ring = (uint32_t *)lds;         // [kRing][Cpos + 1][CSTW] channel-pair words
    float *ex = lds + kRing * slot_words;     // [2 * kTPB pairs][kES]
    float *lb2 = ex + 2 * kTPB * kES;         // [kCout] -bias2 * scale * log2 e

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;

    const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int a = L & 1;
    const int seg = (int)((L >> 1) % (uint32_t)geo.segs);
    const int n = (int)((L >> 1) / (uint32_t)geo.segs);
    const int Mc = geo.Mc[a];
    const int plane_pos = Mc * Cpos;
    const int ntile = geo.ntile[a];
    const int T0 = (int)((int64_t)seg * ntile / geo.segs);
    const int T1 = (int)((int64_t)(seg + 1) * ntile / geo.segs);
    const int ka = (a + pad) & 1, ra = (a + pad) >> 1;
    const int e = pad >> 1;
    const int d0 = -(pad & 1);

    // ---- weights: step s = tap * CB + cb (tap = 2u + v), lane (j, g), channel tile ct:
    // wr[ct][b][s][i] = w[ci = 32cb + 8g + i][co = 32*wv + 16ct + j][ka + 2u][b + 2v]
    bf16x8 wr[2][2][4 * CB];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int st = 0; st < 4 * CB; ++st) {
                const int tp = st / CB, cb = st % CB;
                const int kh = ka + 2 * (tp >> 1), kw = b + 2 * (tp & 1);
                uint32_t hv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int ci = 32 * cb + 8 * g + i;
                    const bool ok = ci < Cin;
                    const uint32_t v = w[((size_t)(ok ? ci : 0) * kCout + 32 * wv + 16 * ct + j) *
                                             16 + kh * 4 + kw];
                    hv[i] = ok ? v : 0u;
                }
                const u32x4 pk = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16),
                                  hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
                wr[ct][b][st] = __builtin_bit_cast(bf16x8, pk);
            }
    // accumulator start: the convT bias of D row 4g + r of tile ct
    f32x4 cb4[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            cb4[ct][r] = cbias ? cbias[32 * wv + 16 * ct + 4 * g + r] : 0.f;
    for (int i = tid; i < kCout; i += kThreadsB) lb2[i] = -b2[i] * scale * kLog2e;
    for (int i = tid; i < kRing * slot_words; i += kThreadsB) ring[i] = 0u;

    // ---- fill items (the same for every input row): channel pair cp, 8-column group cg
    // (cg fastest: a wave's loads cover whole row segments)
    const uint32_t plane = (uint32_t)H * W;
    const uint32_t xbytes = 2u * (uint32_t)N * Cin * plane;  // < 2^31 (host check)
    const __amdgpu_buffer_rsrc_t xr = make_range_checked(x, xbytes);
    const int W8 = W >> 3;
    const int items = 16 * CB * W8;
    const bool f_on = tid < items;  // one pass: 16*CB*W/8 <= 256 (host check)
    const int f_cg = f_on ? tid % W8 : 0, f_cp = f_on ? tid / W8 : 0;
    uint32_t fo[2];  // byte offsets of the item's two channels at row 0 (kMasked if none)
    {
        const uint32_t o = 2u * (((uint32_t)n * Cin + 2 * f_cp) * plane + 8u * f_cg);
        fo[0] = f_on && 2 * f_cp < Cin ? o : kMasked;
        fo[1] = f_on && 2 * f_cp + 1 < Cin ? o + 2u * plane : kMasked;
    }
    const int f_j0 = 8 * f_cg - e + 1;  // slot column of input column 8*cg
    int f_m = 0;                         // bit k: column 8*cg + k has a place in the slot
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (f_on && f_j0 + k >= 0 && f_j0 + k <= Cpos) f_m |= 1 << k;
    auto fill_load = [&](int ih, u32x4 (&v)[2]) {
        const bool rin = ih >= 0 && ih < H;
        const uint32_t ro = 2u * (uint32_t)(rin ? ih : 0) * W;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            v[h] = __builtin_amdgcn_raw_buffer_load_b128(xr, rin ? fo[h] + ro : kMasked, 0, 0);
    };
    // word k of the slot column: the bf16 of column k of both channels (byte permute)
    auto fill_store = [&](int ih, const u32x4 (&v)[2]) {
        uint32_t *dst = ring + ((ih + 1) & (kRing - 1)) * slot_words + f_j0 * CSTW + f_cp;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (f_m & (1 << k))
                dst[k * CSTW] = __builtin_amdgcn_perm(v[1][k >> 1], v[0][k >> 1],
                                                      (k & 1) ? 0x07060302u : 0x05040100u);
    };
    auto tile_rows = [&](int T, int &lo, int &hi) {
        const int t0 = T * kTPB;
        const int t1 = min(t0 + kTPB, plane_pos) - 1;
        lo = (int)fdiv((uint32_t)t0, geo.mC) + ra - 1;
        hi = (int)fdiv((uint32_t)t1, geo.mC) + ra;
    };

    // (No start stagger: with the stores spread over the next tile's K-steps, workgroups
    // that start together finish sooner than ones started in eight groups 0.85 us apart.)
    __syncthreads();
    if (T0 >= T1) return;
    int lo, hi;
    tile_rows(T0, lo, hi);
    for (int ih = lo; ih <= hi; ++ih) {
        u32x4 v[2];
        fill_load(ih, v);
        fill_store(ih, v);
    }
    __syncthreads();

    const uint32_t oplane = (uint32_t)OH * OW;
    const uint32_t ybytes = 2u * (uint32_t)N * kCout * oplane;  // < 2^31 (host check)
    const __amdgpu_buffer_rsrc_t yr = make_range_checked(y, ybytes);
    const char *ringb = (const char *)ring;

    int pm[2], pc[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
        const uint32_t t = (uint32_t)(T0 * kTPB + 16 * bk + j);
        pm[bk] = (int)fdiv(t, geo.mC);
        pc[bk] = (int)t - pm[bk] * Cpos;
    }
    // epilogue: thread (pair p, channel quarter cq), pair p = 2 * (position) + b'
    const int p = tid >> 2, cq = tid & 3;
    int em, ec;
    {
        const uint32_t t = (uint32_t)(T0 * kTPB + (p >> 1));
        em = (int)fdiv(t, geo.mC);
        ec = (int)t - em * Cpos;
    }
    // output row index (n, channel 32cq, row class a) at position row 0 (below 2^24)
    const uint32_t yrow0 = __umul24((uint32_t)n * kCout + 32 * cq, (uint32_t)OH) + a;

    // next tile's new row loaded one tile ahead, before the stores (as in the fp32 kernel)
    u32x4 pv[2];
    int nhi = hi;
    if (T0 + 1 < T1) {
        int nlo;
        tile_rows(T0 + 1, nlo, nhi);
    }
    bool has_new = nhi > hi;
    if (has_new) fill_load(nhi, pv);

    // The previous tile's outputs (bf16 pairs: channels 2i, 2i + 1 of the lane's 32) and
    // their offset; stored a few at a time between the next tile's K-steps, so the stores
    // drain beside the matrix work instead of in one burst per tile.
    uint32_t pend[16];
    uint32_t pyo = kMasked;
#pragma unroll
    for (int i = 0; i < 16; ++i) pend[i] = 0u;
    auto store_pend = [&](int i0, int cnt) {
#pragma unroll
        for (int i = i0; i < i0 + cnt; ++i) {
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pend[i], yr, pyo,
                                                  (int)(2u * (uint32_t)(2 * i) * oplane), 0);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pend[i] >> 16), yr, pyo,
                                                  (int)(2u * (uint32_t)(2 * i + 1) * oplane), 0);
        }
    };

    for (int T = T0; T < T1; ++T) {
        // B addresses of block bk, tap row u, at input column v = 1 (+ 16 bytes per lane
        // group); v = 0 is CSTW words further on, channel block cb 64 bytes
        const char *bp[2][2];
#pragma unroll
        for (int bk = 0; bk < 2; ++bk)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t slot = (uint32_t)(pm[bk] + ra - u + 1) & (kRing - 1);
                bp[bk][u] = ringb + 4u * (__umul24(slot, (uint32_t)slot_words) +
                                          __umul24((uint32_t)pc[bk], (uint32_t)CSTW) + 4u * g);
            }
        auto read_b = [&](int bk, int st) {
            const int tp = st / CB, cb = st % CB;
            const int u = tp >> 1, v = tp & 1;
            return *(const bf16x8 *)(bp[bk][u] + (v ? 0 : 4 * CSTW) + 64 * cb);
        };

        f32x4 acc[2][2][2];  // [channel tile][column class][block]
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int bk = 0; bk < 2; ++bk) acc[ct][b][bk] = cb4[ct];
        // K-steps: the B operands of step st + 1 are read while step st's 8 MFMAs run
        bf16x8 bv[2][2];
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) bv[0][bk] = read_b(bk, 0);
#pragma unroll
        for (int st = 0; st < 4 * CB; ++st) {
            if (st + 1 < 4 * CB) {
#pragma unroll
                for (int bk = 0; bk < 2; ++bk) bv[(st + 1) & 1][bk] = read_b(bk, st + 1);
            }
            // the previous tile's stores, 16 / (4 CB) pairs per step (none before the first)
            if (T > T0) store_pend(st * (4 / CB), 4 / CB);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int bk = 0; bk < 2; ++bk)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[ct][b][bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            wr[ct][b][st], bv[st & 1][bk], acc[ct][b][bk], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        if (has_new) fill_store(nhi, pv);
        hi = nhi;
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
            pc[bk] += kTPB;
            if (pc[bk] >= Cpos) {
                pc[bk] -= Cpos;
                ++pm[bk];
            }
        }
        __syncthreads();  // every wave is done with the previous tile's exchange
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int bk = 0; bk < 2; ++bk)
                    *(f32x4 *)(ex + (2 * (16 * bk + j) + b) * kES + 32 * wv + 16 * ct + 4 * g) =
                        acc[ct][b][bk];
        __syncthreads();  // exchange complete, and the ring holds the next tile's rows

        // ---- epilogue: 32 channels of one pair
        uint32_t yo;
        {
            const int ow = 2 * ec + d0 + (p & 1);
            const bool ok = em < Mc && ow >= 0 && ow < OW;
            yo = ok ? 2u * (__umul24(yrow0 + 2u * (uint32_t)em, (uint32_t)OW) + (uint32_t)ow)
                    : kMasked;
            ec += kTPB;
            if (ec >= Cpos) {
                ec -= Cpos;
                ++em;
            }
        }
        float v[32];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const f32x4 t = *(const f32x4 *)(ex + p * kES + 32 * cq + 4 * r);
            v[4 * r] = t[0];
            v[4 * r + 1] = t[1];
            v[4 * r + 2] = t[2];
            v[4 * r + 3] = t[3];
        }
        // e_c = 2^((t_c - max) log2 e), out_c = 1 / (1 + 2^(e_c * inv + b2'_c)),
        // inv = -scale * log2 e / sum_c e_c, b2'_c = -bias2_c * scale * log2 e
        float mx = v[0];
#pragma unroll
        for (int r = 1; r < 32; ++r) mx = fmaxf(mx, v[r]);
        mx = fmaxf(mx, quad_xor1(mx));
        mx = fmaxf(mx, quad_xor2(mx));
        const float nmx = -mx * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            v[r] = __builtin_amdgcn_exp2f(fmaf(v[r], kLog2e, nmx));
            sum += v[r];
        }
        sum += quad_xor1(sum);
        sum += quad_xor2(sum);
        const float inv = -scale * kLog2e * __builtin_amdgcn_rcpf(sum);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const f32x4 bb = *(const f32x4 *)(lb2 + 32 * cq + 4 * r);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float t = __builtin_amdgcn_exp2f(fmaf(v[4 * r + i], inv, bb[i]));
                v[4 * r + i] = __builtin_amdgcn_rcpf(1.f + t);
            }
        }
        if (T + 2 < T1) {
            int nlo;
            tile_rows(T + 2, nlo, nhi);
        }
        has_new = nhi > hi;
        if (has_new) fill_load(nhi, pv);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            pend[i] = (uint32_t)f32_to_bf16_rne(v[2 * i]) |
                      ((uint32_t)f32_to_bf16_rne(v[2 * i + 1]) << 16);
        pyo = yo;
    }
    store_pend(0, 16);  // the last tile's outputs
}

}  // namespace

// Returns PS_ERR_UNSUPPORTED (before any HIP call) outside this kernel's envelope:
// Cout = 128, Cin <= 64, W a multiple of 4, at least 64 positions per row (so a tile
// spans at most two position rows), the ring and exchange within the LDS, x and y
// below 2^31 bytes.
int launch_convT_rows(const float *x, const float *w, const float *cb, const float *b2, float *y,
                      int N, int Cin, int H, int W, int Cout, int OH, int OW, int pad,
                      float scale, bool softmax, hipStream_t stream) {
    if (Cout != kCout || Cin > 64 || W % 4 != 0) return PS_ERR_UNSUPPORTED;
    RowsGeom geo;
    geo.Cpos = (OW + 1 + (pad & 1)) >> 1;
    if (geo.Cpos < kTP) return PS_ERR_UNSUPPORTED;
    const int CQ = (Cin + 15) / 16;
    const size_t lds_words =
        (size_t)kRing * (geo.Cpos + 1) * (16 * CQ + 4) + 2 * kTP * kES + 2 * kCout + 128;
    if (lds_words * 4 > 160 * 1024) return PS_ERR_UNSUPPORTED;
    if ((int64_t)4 * N * Cin * H * W >= (1ll << 31) ||
        (int64_t)4 * N * kCout * OH * OW >= (1ll << 31))
        return PS_ERR_UNSUPPORTED;
    geo.mC = (uint32_t)(((1ll << 32) + geo.Cpos - 1) / geo.Cpos);
    for (int a = 0; a < 2; ++a) {
        geo.Mc[a] = (OH - a + 1) >> 1;
        const int64_t pp = (int64_t)geo.Mc[a] * geo.Cpos;
        // the multiply-shift division by Cpos is exact for dividend * Cpos < 2^32
        if (pp * geo.Cpos >= (1ll << 32)) return PS_ERR_UNSUPPORTED;
        geo.ntile[a] = (int)((pp + kTP - 1) / kTP);
    }
    geo.W4 = W / 4;
    geo.items = 8 * CQ * geo.W4;
    const int nf = (geo.items + kThreads - 1) / kThreads;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PS_ERR_HIP;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PS_ERR_HIP;
    // one workgroup per CU (the ring and exchange fill most of the LDS): split the
    // planes into segments when there are fewer planes than CUs
    const int planes = 2 * N;
    int segs = planes >= ncu ? 1 : (ncu + planes - 1) / planes;
    segs = segs > geo.ntile[1] ? (geo.ntile[1] > 0 ? geo.ntile[1] : 1) : segs;
    geo.segs = segs;
    const int64_t nblocks = (int64_t)planes * segs;
    if (nblocks >= (1ll << 31)) return PS_ERR_UNSUPPORTED;
    const size_t lds_bytes = lds_words * 4;

#define PS_ROWS_LAUNCH(CQv, NFv)                                                           \
    do {                                                                                  \
        auto kern = softmax ? convT_rows_f32<CQv, NFv, true> : convT_rows_f32<CQv, NFv, false>; \
        if (hipFuncSetAttribute((const void *)kern,                                       \
                                hipFuncAttributeMaxDynamicSharedMemorySize,               \
                                (int)lds_bytes) != hipSuccess)                            \
            return PS_ERR_HIP;                                                            \
        return launch(kern, dim3((unsigned)nblocks), dim3(kThreads), lds_bytes, stream, x, w, \
                      cb, b2, y, N, Cin, H, W, OH, OW, pad, scale, geo);                   \
    } while (0)
    if (nf == 1) {
        switch (CQ) {
            case 1: PS_ROWS_LAUNCH(1, 1);
            case 2: PS_ROWS_LAUNCH(2, 1);
            case 3: PS_ROWS_LAUNCH(3, 1);
            case 4: PS_ROWS_LAUNCH(4, 1);
        }
    } else if (nf == 2) {
        switch (CQ) {
            case 1: PS_ROWS_LAUNCH(1, 2);
            case 2: PS_ROWS_LAUNCH(2, 2);
            case 3: PS_ROWS_LAUNCH(3, 2);
            case 4: PS_ROWS_LAUNCH(4, 2);
        }
    }
#undef PS_ROWS_LAUNCH
    return PS_ERR_UNSUPPORTED;
}

// bf16: Cout = 128, Cin <= 64, W a multiple of 8 and at most 128 (one fill pass per
// row), at least 64 positions per row, ring and exchange within the LDS, x and y below
// 2^31 bytes; PS_ERR_UNSUPPORTED otherwise.
int launch_convT_rows_bf16(const uint16_t *x, const uint16_t *w, const float *cb,
                           const float *b2, uint16_t *y, int N, int Cin, int H, int W, int Cout,
                           int OH, int OW, int pad, float scale, hipStream_t stream) {
    if (Cout != kCout || Cin > 64 || W % 8 != 0) return PS_ERR_UNSUPPORTED;
    RowsGeom geo;
    geo.Cpos = (OW + 1 + (pad & 1)) >> 1;
    if (geo.Cpos < kTP) return PS_ERR_UNSUPPORTED;
    const int CB = (Cin + 31) / 32;
    const size_t lds_words =
        (size_t)kRing * (geo.Cpos + 1) * (16 * CB + 4) + 2 * kTPB * kES + kCout;
    if (lds_words * 4 > 160 * 1024) return PS_ERR_UNSUPPORTED;
    if ((int64_t)2 * N * Cin * H * W >= (1ll << 31) ||
        (int64_t)2 * N * kCout * OH * OW >= (1ll << 31) ||
        (int64_t)N * kCout * OH >= (1ll << 24))  // 24-bit output row index
        return PS_ERR_UNSUPPORTED;
    if (16 * CB * (W / 8) > kThreadsB) return PS_ERR_UNSUPPORTED;  // one fill pass per row
    geo.mC = (uint32_t)(((1ll << 32) + geo.Cpos - 1) / geo.Cpos);
    for (int a = 0; a < 2; ++a) {
        geo.Mc[a] = (OH - a + 1) >> 1;
        const int64_t pp = (int64_t)geo.Mc[a] * geo.Cpos;
        if (pp * geo.Cpos >= (1ll << 32)) return PS_ERR_UNSUPPORTED;
        geo.ntile[a] = (int)((pp + kTPB - 1) / kTPB);
    }
    geo.W4 = W / 4;
    geo.items = 0;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PS_ERR_HIP;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PS_ERR_HIP;
    // two workgroups per CU: split the planes into segments so there are at least twice
    // as many workgroups as CUs
    const int planes = 2 * N;
    int segs = planes >= 2 * ncu ? 1 : (2 * ncu + planes - 1) / planes;
    segs = segs > geo.ntile[1] ? (geo.ntile[1] > 0 ? geo.ntile[1] : 1) : segs;
    geo.segs = segs;
    const int64_t nblocks = (int64_t)planes * segs;
    if (nblocks >= (1ll << 31)) return PS_ERR_UNSUPPORTED;
    const size_t lds_bytes = lds_words * 4;
    auto kern = CB == 1 ? convT_rows_bf16<1> : convT_rows_bf16<2>;
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_bytes) != hipSuccess)
        return PS_ERR_HIP;
    return launch(kern, dim3((unsigned)nblocks), dim3(kThreadsB), lds_bytes, stream, x, w, cb,
                  b2, y, N, Cin, H, W, OH, OW, pad, scale, geo);
}

}  // namespace ps

// MaxPool2d kernels for gfx950.
//
// Definition (POPCORNBENCH page Kimi-K2.6 l1_p42, problem statement and the
// passage on PyTorch's implicit negative-infinity padding):
//   y[n,c,oh,ow] = max_{kh,kw<k} x[n,c, oh*s - p + kh*d, ow*s - p + kw*d],
//   positions outside the image count as -inf, floor mode.
//
// Three kernels:
//   maxpool_s1_rows  stride 1, dilation 1, window k <= 8, pad < k.  The case
//                    that is pure HBM streaming (every input is read about once,
//                    every output written once).  One wavefront owns a band of
//                    output rows of one (n,c) plane and a strip of 64*V output
//                    columns.  It walks the input rows of its band top to bottom:
//                      - each input row is loaded once, as V+1 fully coalesced
//                        256-byte wave loads (lane l holds column 64j + l);
//                      - the horizontal k-max is formed in registers by
//                        rotating the row across lanes (ds_bpermute), using
//                        doubling windows (1 -> 2 -> 4 -> 8) so a k=4 window costs
//                        two rotations per chunk instead of three;
//                      - the last k horizontal maxima are kept in a register
//                        ring, and each output row is the max down that ring
//                        (the separable max of the l1_p42 page, done in
//                        registers rather than through a shared-memory tile);
//                      - each output row is written as V coalesced wave stores.
//                    The k-1 input rows shared by neighbouring bands are read
//                    from HBM once: eight consecutive bands of a plane share a
//                    workgroup, and each wave hands the horizontal maxima of
//                    its band's first k-1 rows to the wave of the band above
//                    through LDS (only every eighth band boundary re-reads).
//   maxpool_rows_sd  k 2..5 with stride / dilation (2,1), (3,1), (1,2), (2,2): the
//                    same row streaming, each input row staged in the wave's LDS
//                    buffer and its strided / dilated taps read back from there.
//   maxpool_cols     any k, stride, pad, dilation: a thread owns one output
//                    column of 8 (stride 1) or 1 consecutive output rows; every
//                    window tap is a branch-free load (see the kernel).
#include "ps_internal.h"

#include <math.h>

namespace ps {
namespace {

constexpr int kWave = 64;

// Tuning knobs (compile-time): rows of loads in flight per wave, output rows
// per band, nontemporal hints on the output stores / input loads.
#ifndef PS_MAXPOOL_PREFETCH
#define PS_MAXPOOL_PREFETCH 2
#endif
#ifndef PS_MAXPOOL_BAND_ROWS
#define PS_MAXPOOL_BAND_ROWS 32
#endif
#ifndef PS_MAXPOOL_NT_STORE
#define PS_MAXPOOL_NT_STORE 0
#endif
#ifndef PS_MAXPOOL_NT_LOAD
#define PS_MAXPOOL_NT_LOAD 0
#endif
// Resident workgroups per CU (0 = as many as registers allow).  Fewer concurrent
// row streams keep more DRAM pages open per stream.  The cap is applied by
// reserving a matching share of the CU's LDS for each workgroup.
#ifndef PS_MAXPOOL_WGS_PER_CU
#define PS_MAXPOOL_WGS_PER_CU 1
#endif
// Strided / dilated streaming kernel: output columns per strip (64*V), output rows
// per band at stride 1 and at stride >= 2, rows of loads in flight, resident
// workgroups per CU at stride 1 and at stride >= 2 (0 = as many as registers allow).
// Measured on MI355X over the 32x64x512x512 input: k3 s2 p1 0.546 ms with 32-row
// bands and no cap, 0.470 ms with 8-row bands and 2 workgroups per CU (4-row
// bands, 1 or 3 per CU slower); k3 s1 p2 d2 0.875 ms with 64-row bands, 0.773 ms
// with 16-row bands and 4 per CU (8 or 12 rows, 2, 3 or 6 per CU slower); V = 8
// and 3 prefetched rows slower.
#ifndef PS_MPSD_V
#define PS_MPSD_V 4
#endif
#ifndef PS_MPSD_BAND_S1
#define PS_MPSD_BAND_S1 16
#endif
#ifndef PS_MPSD_BAND_S2
#define PS_MPSD_BAND_S2 8
#endif
#ifndef PS_MPSD_PF
#define PS_MPSD_PF 2
#endif
#ifndef PS_MPSD_WGS_S1
#define PS_MPSD_WGS_S1 4
#endif
#ifndef PS_MPSD_WGS_S2
#define PS_MPSD_WGS_S2 2
#endif
#ifndef PS_MPSD_WGS_V1
#define PS_MPSD_WGS_V1 0
#endif
// Waves (consecutive bands of one plane) per workgroup: all but the last hand their
// halo rows over through LDS.  Measured on MI355X (k4 s1 p1, 32x64x512x512): one
// 8-wave workgroup per CU beats 4 waves at 3 per CU by about 3%, and 16 resident
// waves per CU (either shape) is 8-10% slower than 8.
#ifndef PS_MAXPOOL_WG_WAVES
#define PS_MAXPOOL_WG_WAVES 8
#endif

__device__ __forceinline__ float rot_lanes(float v, int src_lane_x4) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane_x4, __float_as_int(v)));
}

__device__ __forceinline__ float fmax_ordered(float a, float b) { return b > a ? b : a; }

// hw[j] <- max over the window [64j + lane, 64j + lane + span) of the row held in
// chunks v[0..V] (chunk j lane l = element 64j + l), given that v already holds the
// window-`have` maxima.  Shifts by `have` lanes with carry from the next chunk.
template <int V>
__device__ __forceinline__ void widen(float (&v)[V + 1], int lane, int shift) {
    const int src = ((lane + shift) & (kWave - 1)) << 2;
    const bool carry = lane + shift >= kWave;
    float rot[V + 1];
#pragma unroll
    for (int j = 0; j <= V; ++j) rot[j] = rot_lanes(v[j], src);
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = fmax_ordered(v[j], carry ? rot[j + 1] : rot[j]);
    // chunk V only feeds the lanes of chunk V-1 that carry into it; its own
    // widened value is never used as an output.
    v[V] = fmax_ordered(v[V], rot[V]);
}

template <int K, int V, int PF>
__global__ __launch_bounds__(kWave * PS_MAXPOOL_WG_WAVES) void maxpool_s1_rows(
    const float *__restrict__ x, float *__restrict__ y, int H, int W, int OH, int OW, int pad,
    int band_rows, int nbands, int nstrips, uint64_t ntasks) {
    // [wave][K-1][V][64]: the horizontal maxima of each band's first K-1 input rows,
    // which are also the last K-1 input rows of the band above it
    extern __shared__ float halo[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const uint32_t blk = xcd_remap(blockIdx.x, gridDim.x);
    const uint64_t task = (uint64_t)blk * nw + wave;
    // Every wave passes the kernel's one barrier exactly once, idle waves included.
    if (task >= ntasks) {
        __syncthreads();
        return;
    }
    const int band = (int)(task % (uint64_t)nbands);
    const uint64_t t2 = task / (uint64_t)nbands;
    const int strip = (int)(t2 % (uint64_t)nstrips);
    const uint64_t plane = t2 / (uint64_t)nstrips;

    const float *xp = x + plane * (uint64_t)H * W;
    float *yp = y + plane * (uint64_t)OH * OW;
    const int c0 = strip * (kWave * V);  // first output column of the strip
    const int ic0 = c0 - pad;            // input column under lane 0 of chunk 0
    const int oh0 = band * band_rows;
    const int oh1 = min(OH, oh0 + band_rows);
    const int ih_first = oh0 - pad;
    const int ih_last = oh1 - 1 - pad + K - 1;
    const int nrows = ih_last - ih_first + 1;
    // The next wave of the workgroup holds the band below in the same plane and strip
    // (task + 1): its first K-1 input rows are this band's last K-1, so their
    // horizontal maxima come from the LDS instead of a second HBM read.  Such a band
    // is not the plane's last, so it has band_rows >= K - 1 rows of its own to load.
    const bool from_below = wave + 1 < nw && band + 1 < nbands;
    const int nload = nrows - (from_below ? K - 1 : 0);  // >= K - 1

    // Column validity is fixed for the whole band.
    bool colok[V + 1];
#pragma unroll
    for (int j = 0; j <= V; ++j) {
        const int c = ic0 + kWave * j + lane;
        colok[j] = (c >= 0) && (c < W);
    }

    auto load_row = [&](int ih, float (&v)[V + 1]) {
        const bool rowok = (ih >= 0) && (ih < H);
        const float *rp = xp + (int64_t)ih * W + ic0 + lane;
#pragma unroll
        for (int j = 0; j <= V; ++j)
#if PS_MAXPOOL_NT_LOAD
            v[j] = (rowok && colok[j]) ? __builtin_nontemporal_load(rp + kWave * j) : -INFINITY;
#else
            v[j] = (rowok && colok[j]) ? rp[kWave * j] : -INFINITY;
#endif
    };

    // Append input row r's horizontal maxima to the vertical ring of the last K and,
    // once K rows are in, write output row r - (K-1) of the band.
    float ring[K][V];
    auto consume = [&](int r, const float (&v)[V + 1]) {
#pragma unroll
        for (int i = 0; i < K - 1; ++i)
#pragma unroll
            for (int j = 0; j < V; ++j) ring[i][j] = ring[i + 1][j];
#pragma unroll
        for (int j = 0; j < V; ++j) ring[K - 1][j] = v[j];

        if (r >= K - 1) {
            const int oh = oh0 + r - (K - 1);
            float *orow = yp + (int64_t)oh * OW + c0 + lane;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                float m = ring[0][j];
#pragma unroll
                for (int i = 1; i < K; ++i) m = fmax_ordered(m, ring[i][j]);
                if (c0 + kWave * j + lane < OW) {
#if PS_MAXPOOL_NT_STORE
                    __builtin_nontemporal_store(m, orow + kWave * j);
#else
                    orow[kWave * j] = m;
#endif
                }
            }
        }
    };

    // PF input rows are in flight at any time: slot s of `pf` holds row
    // ih_first + base + s; after a row is consumed its slot is refilled with the
    // row PF further down.  The slot loop is unrolled, so every register index is
    // static and no pending load is ever copied.
    float pf[PF][V + 1];
#pragma unroll
    for (int s = 0; s < PF; ++s)
        if (s < nload) load_row(ih_first + s, pf[s]);

    for (int base = 0; base < nload; base += PF) {
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            const int r = base + s;
            if (r >= nload) break;
            const int ih = ih_first + r;
            float v[V + 1];
#pragma unroll
            for (int j = 0; j <= V; ++j) v[j] = pf[s][j];
            if (r + PF < nload) load_row(ih + PF, pf[s]);

            // horizontal window-K max by doubling: window 1 -> 2 -> 4 (-> 8)
            constexpr int P = K >= 8 ? 8 : K >= 4 ? 4 : K >= 2 ? 2 : 1;  // largest power of 2 <= K
            if constexpr (P >= 2) widen<V>(v, lane, 1);
            if constexpr (P >= 4) widen<V>(v, lane, 2);
            if constexpr (P >= 8) widen<V>(v, lane, 4);
            if constexpr (K != P) {
                // window K = window P at c  combined with window P at c + (K - P)
                const int sh = K - P;
                const int src = ((lane + sh) & (kWave - 1)) << 2;
                const bool carry = lane + sh >= kWave;
                float rot[V + 1];
#pragma unroll
                for (int j = 0; j <= V; ++j) rot[j] = rot_lanes(v[j], src);
#pragma unroll
                for (int j = 0; j < V; ++j) v[j] = fmax_ordered(v[j], carry ? rot[j + 1] : rot[j]);
            }

            // hand the first K-1 rows to the band above (the previous wave)
            if (r < K - 1 && wave > 0) {
#pragma unroll
                for (int j = 0; j < V; ++j) halo[((wave * (K - 1) + r) * V + j) * kWave + lane] = v[j];
            }
            if (r == K - 2) __syncthreads();
            consume(r, v);
        }
    }
    if (from_below) {
        for (int i = 0; i < K - 1; ++i) {
            float v[V + 1];
#pragma unroll
            for (int j = 0; j < V; ++j) v[j] = halo[(((wave + 1) * (K - 1) + i) * V + j) * kWave + lane];
            consume(nload + i, v);
        }
    }
}

// Strided and dilated windows (compile-time K, S, D), streamed by rows like
// maxpool_s1_rows: one wavefront owns a band of output rows of one (n,c) plane and a
// strip of 64*V output columns, and reads each input row of its band once:
//   - the row's span of input columns (64*V*S + (K-1)*D of them) is loaded as
//     coalesced 256-byte wave loads (-inf outside the image) and written to the
//     wave's own LDS row buffer;
//   - lane l's horizontal window max for output column 64j + l is read back from
//     LDS at the K fixed addresses (64j + l)*S + kw*D;
//   - a register ring keeps the horizontal maxima of the last (K-1)*D + 1 input
//     rows; whenever an input row completes output row oh (row oh*S - p + (K-1)*D),
//     the vertical max over the ring's taps 0, D, .., (K-1)*D is written.
// Neighbouring bands share (K-1)*D + 1 - S input rows, which both read.
// EPI: the second stage of the page's unfused conv pipeline (l2_p82) on a stored
// conv output: out = max over the window of tanh(x)*scale + bias2[c].  The window
// reduces sgn*x (sgn = -1 when scale < 0: tanh and v -> v*scale + b are monotone,
// so the max of the map is taken at the max of x for scale >= 0 and at the min for
// scale < 0), and the map is applied once per output; an all-padding window stays
// -inf.  C = channels (the plane's channel is plane % C).
struct PoolEpi {
    float sgn, scale;
    const float *b2;
    int C;
};

template <int K, int S, int D, int V, int PF, bool EPI>
__global__ __launch_bounds__(256) void maxpool_rows_sd(
    const float *__restrict__ x, float *__restrict__ y, int H, int W, int OH, int OW, int pad,
    int band_rows, int nbands, int nstrips, uint64_t ntasks, PoolEpi epi) {
    constexpr int R = (K - 1) * D + 1;                        // input rows per window
    constexpr int SPAN = (kWave * V - 1) * S + (K - 1) * D + 1;  // input columns per strip
    constexpr int NCH = (SPAN + kWave - 1) / kWave;           // 64-column load chunks
    constexpr int OV = R > S ? R - S : 0;                     // input rows shared with the band below
    __shared__ float lrow[4][NCH * kWave];                    // one row buffer per wave
    // [wave][OV][V][64]: horizontal maxima of each band's first OV input rows, which
    // are the last OV input rows of the band above it (the previous wave's)
    __shared__ float lhalo[OV > 0 ? 4 * OV * V * kWave : 1];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const uint32_t blk = xcd_remap(blockIdx.x, gridDim.x);
    const uint64_t task = (uint64_t)blk * 4 + wave;
    // With a hand-over, every wave passes the kernel's one barrier exactly once.
    if (task >= ntasks) {
        if constexpr (OV > 0) __syncthreads();
        return;
    }
    const int band = (int)(task % (uint64_t)nbands);
    const uint64_t t2 = task / (uint64_t)nbands;
    const int strip = (int)(t2 % (uint64_t)nstrips);
    const uint64_t plane = t2 / (uint64_t)nstrips;

    const float *xp = x + plane * (uint64_t)H * W;
    float *yp = y + plane * (uint64_t)OH * OW;
    const int c0 = strip * (kWave * V);  // first output column of the strip
    const int ic0 = c0 * S - pad;        // input column of buffer entry 0
    const int oh0 = band * band_rows;
    const int oh1 = min(OH, oh0 + band_rows);
    const int ih_first = oh0 * S - pad;
    const int nrows = (oh1 - 1 - oh0) * S + R;  // input rows of the band
    // The next wave of the workgroup holds the band below in the same plane and strip:
    // its first OV input rows are this band's last OV, whose horizontal maxima then come
    // from the LDS instead of a second read.  Such a band has band_rows*S >= OV rows of
    // its own to load (host check), so every wave reaches the barrier below.
    const bool from_below = OV > 0 && wave + 1 < 4 && band + 1 < nbands;
    const int nload = nrows - (from_below ? OV : 0);
    float *buf = lrow[wave];

    bool colok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ic = ic0 + kWave * c + lane;
        colok[c] = ic >= 0 && ic < W;
    }
    const float sgn = EPI ? epi.sgn : 1.f;
    auto load_row = [&](int ih, float (&v)[NCH]) {
        const bool rowok = ih >= 0 && ih < H;
        const float *rp = xp + (int64_t)ih * W + ic0 + lane;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            v[c] = (rowok && colok[c]) ? rp[kWave * c] : -INFINITY;
            if constexpr (EPI) v[c] = (rowok && colok[c]) ? sgn * v[c] : -INFINITY;
        }
    };
    float b2c = 0.f;
    if constexpr (EPI) b2c = epi.b2[plane % (uint64_t)epi.C];

    // Append input row r's horizontal maxima to the ring of the last R and, when the
    // row completes output row oh (row oh*S - p + (K-1)*D), write it.
    float ring[R][V];
    auto consume = [&](int r, const float (&hm)[V]) {
#pragma unroll
        for (int i = 0; i < R - 1; ++i)
#pragma unroll
            for (int j = 0; j < V; ++j) ring[i][j] = ring[i + 1][j];
#pragma unroll
        for (int j = 0; j < V; ++j) ring[R - 1][j] = hm[j];
        const int q = r - (R - 1);  // = (oh - oh0) * S when row r completes output oh
        if (q >= 0 && q % S == 0) {
            const int oh = oh0 + q / S;
            float *orow = yp + (int64_t)oh * OW + c0 + lane;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                float m = ring[0][j];
#pragma unroll
                for (int kh = 1; kh < K; ++kh) m = fmax_ordered(m, ring[kh * D][j]);
                if constexpr (EPI)
                    m = m == -INFINITY ? -INFINITY : tanh_exp(sgn * m) * epi.scale + b2c;
                if (c0 + kWave * j + lane < OW) orow[kWave * j] = m;
            }
        }
    };

    float pf[PF][NCH];
#pragma unroll
    for (int s = 0; s < PF; ++s)
        if (s < nload) load_row(ih_first + s, pf[s]);

    for (int base = 0; base < nload; base += PF) {
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            const int r = base + s;
            if (r >= nload) break;
            // the row into the wave's LDS buffer, the slot refilled PF rows further down
#pragma unroll
            for (int c = 0; c < NCH; ++c) buf[kWave * c + lane] = pf[s][c];
            if (r + PF < nload) load_row(ih_first + r + PF, pf[s]);
            __builtin_amdgcn_wave_barrier();
            float hm[V];
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const float *bp = buf + (kWave * j + lane) * S;
                float m = bp[0];
#pragma unroll
                for (int kw = 1; kw < K; ++kw) m = fmax_ordered(m, bp[kw * D]);
                hm[j] = m;
            }
            __builtin_amdgcn_wave_barrier();  // the next row's writes come after these reads
            if constexpr (OV > 0) {
                // hand the first OV rows to the band above (the previous wave)
                if (r < OV && wave > 0) {
#pragma unroll
                    for (int j = 0; j < V; ++j)
                        lhalo[((wave * OV + r) * V + j) * kWave + lane] = hm[j];
                }
                if (r == OV - 1) __syncthreads();
            }
            consume(r, hm);
        }
    }
    if constexpr (OV > 0) {
        if (from_below) {
            for (int i = 0; i < OV; ++i) {
                float hm[V];
#pragma unroll
                for (int j = 0; j < V; ++j)
                    hm[j] = lhalo[(((wave + 1) * OV + i) * V + j) * kWave + lane];
                consume(nload + i, hm);
            }
        }
    }
}

// Disjoint windows: stride = k (2 or 4), no padding or dilation, W even.  A thread
// owns one output column of one output row; its window is k consecutive columns of k
// consecutive rows, read as 8-byte vectors (8-byte aligned: k, W and the column
// offset are even), so a wave's load of one window row is 64 contiguous 8k-byte
// pieces and the k rows of an output row are one contiguous block of memory.  No
// LDS and no lane exchange: a read-streaming kernel (the strided row-streaming
// kernel stages rows through LDS and reads them back at stride k, which for these
// windows made the epilogue + pool stage of the unfused conv pipeline run at 3.7 TB/s).
// grid.x: 64-column chunks of the output row, grid.y: groups of 4 output rows (one
// per wave), grid.z: planes (strided).  EPI as in maxpool_rows_sd.
template <int K, bool EPI>
__global__ __launch_bounds__(256) void maxpool_disjoint(const float *__restrict__ x,
                                                        float *__restrict__ y, int H, int W,
                                                        int OH, int OW, int planes,
                                                        PoolEpi epi) {
    static_assert(K % 2 == 0, "8-byte vectors");
    const int ow = blockIdx.x * kWave + (threadIdx.x & (kWave - 1));
    const int oh = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (ow >= OW || oh >= OH) return;
    const float sgn = EPI ? epi.sgn : 1.f;
    for (int pl = blockIdx.z; pl < planes; pl += gridDim.z) {
        const float *xr = x + ((size_t)pl * H + (size_t)oh * K) * W + (size_t)ow * K;
        float2 v[K][K / 2];
#pragma unroll
        for (int kh = 0; kh < K; ++kh)
#pragma unroll
            for (int h = 0; h < K / 2; ++h)
                v[kh][h] = *(const float2 *)(xr + (size_t)kh * W + 2 * h);
        // row-major order over the window, first maximum kept (as the other kernels)
        float m = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < K; ++kh)
#pragma unroll
            for (int h = 0; h < K / 2; ++h) {
                m = fmax_ordered(m, sgn * v[kh][h].x);
                m = fmax_ordered(m, sgn * v[kh][h].y);
            }
        if constexpr (EPI)
            m = tanh_exp(sgn * m) * epi.scale + epi.b2[pl % epi.C];
        y[((size_t)pl * OH + oh) * OW + ow] = m;
    }
}

// stride = k in {2, 4}, d = 1, p = 0, W even; -1 otherwise
template <bool EPI>
int launch_disjoint(const float *x, float *y, int N, int C, int H, int W, int OH, int OW, int k,
                    int s, int p, int d, const PoolEpi &epi, hipStream_t stream) {
    if (s != k || d != 1 || p != 0 || (k != 2 && k != 4) || W % 2 != 0) return -1;
    const int64_t planes = (int64_t)N * C;
    if (planes > 0x7fffffff) return -1;
    const dim3 grid((unsigned)((OW + kWave - 1) / kWave), (unsigned)((OH + 3) / 4),
                    (unsigned)(planes < 65535 ? planes : 65535));
    if (grid.y > 65535u) return -1;
    if (k == 2)
        return launch(maxpool_disjoint<2, EPI>, grid, dim3(256), 0, stream, x, y, H, W, OH, OW,
                      (int)planes, epi);
    return launch(maxpool_disjoint<4, EPI>, grid, dim3(256), 0, stream, x, y, H, W, OH, OW,
                  (int)planes, epi);
}

int occupancy_cap_lds_bytes(int wgs, int static_bytes);

template <int K, int S, int D, int V, bool EPI>
int launch_rows_sd_v(const float *x, float *y, int N, int C, int H, int W, int OH, int OW, int p,
                     const PoolEpi &epi, hipStream_t stream) {
    const int band_rows = S >= 2 ? PS_MPSD_BAND_S2 : PS_MPSD_BAND_S1;
    // the kernel's static LDS (row buffers and the halo hand-over), as declared there
    constexpr int R = (K - 1) * D + 1;
    constexpr int NCH = ((kWave * V - 1) * S + (K - 1) * D + 1 + kWave - 1) / kWave;
    constexpr int OV = R > S ? R - S : 0;
    constexpr int static_bytes = 4 * (4 * NCH * kWave + (OV > 0 ? 4 * OV * V * kWave : 1));
    // a band that hands rows over must load at least OV rows of its own
    if (band_rows * S < OV) return PS_ERR_UNSUPPORTED;
    const int nbands = (OH + band_rows - 1) / band_rows;
    const int nstrips = (OW + kWave * V - 1) / (kWave * V);
    const uint64_t ntasks = (uint64_t)N * C * nstrips * nbands;
    const uint64_t nblocks = (ntasks + 3) / 4;
    if (nblocks > 0x7fffffffull) return PS_ERR_UNSUPPORTED;
    // narrow strips keep little in flight per wave: no cap on resident workgroups
    const int lds_bytes = occupancy_cap_lds_bytes(
        V == 1 ? PS_MPSD_WGS_V1 : S >= 2 ? PS_MPSD_WGS_S2 : PS_MPSD_WGS_S1, static_bytes);
    if (lds_bytes > 65536 &&
        hipFuncSetAttribute((const void *)maxpool_rows_sd<K, S, D, V, PS_MPSD_PF, EPI>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess)
        return PS_ERR_HIP;
    return launch(maxpool_rows_sd<K, S, D, V, PS_MPSD_PF, EPI>, dim3((unsigned)nblocks),
                  dim3(256), lds_bytes, stream, x, y, H, W, OH, OW, p, band_rows, nbands, nstrips,
                  ntasks, epi);
}

// strips of 64 output columns for rows up to 64 wide (no idle chunks), else 256
template <int K, int S, int D, bool EPI>
int launch_rows_sd(const float *x, float *y, int N, int C, int H, int W, int OH, int OW, int p,
                   const PoolEpi &epi, hipStream_t stream) {
    if (OW <= 64) return launch_rows_sd_v<K, S, D, 1, EPI>(x, y, N, C, H, W, OH, OW, p, epi, stream);
    return launch_rows_sd_v<K, S, D, PS_MPSD_V, EPI>(x, y, N, C, H, W, OH, OW, p, epi, stream);
}

// (K, S, D) combinations with a streaming kernel; -1 when there is none.
template <bool EPI>
int launch_rows_sd_any(const float *x, float *y, int N, int C, int H, int W, int OH, int OW,
                       int k, int s, int p, int d, const PoolEpi &epi, hipStream_t stream) {
#define PS_SD(KK, SS, DD)                                                                      \
    if (k == KK && s == SS && d == DD)                                                         \
        return launch_rows_sd<KK, SS, DD, EPI>(x, y, N, C, H, W, OH, OW, p, epi, stream);
#define PS_SD_K(SS, DD) PS_SD(2, SS, DD) PS_SD(3, SS, DD) PS_SD(4, SS, DD) PS_SD(5, SS, DD)
    PS_SD_K(2, 1)
    PS_SD_K(3, 1)
    PS_SD_K(4, 1)
    PS_SD_K(1, 2)
    PS_SD_K(2, 2)
#undef PS_SD_K
#undef PS_SD
    return -1;
}

// Any window, stride, padding and dilation.  A thread owns one output column ow of
// RB consecutive output rows of one plane; the lanes of a wave take consecutive
// columns, so a window tap's load is a coalesced row read (s = 1) or a row read
// spread over s*256 bytes whose remaining words the next taps take from the cache.
// The window's column offsets and column masks are computed once per thread; every
// tap is a branch-free load (clamped address, -inf where the tap lies in the
// padding), all taps of an output in flight together.  Rows shared by neighbouring
// output rows are re-read from the cache rather than tracked.  KC > 0: the window
// size as a compile-time constant (k = KC); KC == 0: any k (runtime loops).
template <int KC, int RB>
__global__ __launch_bounds__(256) void maxpool_cols(const float *__restrict__ x,
                                                    float *__restrict__ y, int H, int W, int OH,
                                                    int OW, int kr, int s, int p, int d,
                                                    int planes) {
    const int ow = blockIdx.x * blockDim.x + threadIdx.x;
    if (ow >= OW) return;
    const int oh0 = blockIdx.y * RB;
    const int iw0 = ow * s - p;
    const uint32_t plane = (uint32_t)H * (uint32_t)W;  // < 2^31 (checked by the host)
    if constexpr (KC > 0) {
        int coff[KC];
        bool cok[KC];
#pragma unroll
        for (int kw = 0; kw < KC; ++kw) {
            const int iw = iw0 + kw * d;
            cok[kw] = iw >= 0 && iw < W;
            coff[kw] = iw < 0 ? 0 : (iw >= W ? W - 1 : iw);
        }
        for (int pl = blockIdx.z; pl < planes; pl += gridDim.z) {
            const float *xp = x + (size_t)pl * plane;
            float *yp = y + (size_t)pl * OH * OW + ow;
#pragma unroll 1
            for (int r = 0; r < RB; ++r) {
                const int oh = oh0 + r;
                if (oh >= OH) break;
                float v[KC][KC];
#pragma unroll
                for (int kh = 0; kh < KC; ++kh) {
                    const int ih = oh * s - p + kh * d;
                    const bool rok = ih >= 0 && ih < H;
                    const uint32_t ro = (uint32_t)(ih < 0 ? 0 : (ih >= H ? H - 1 : ih)) * (uint32_t)W;
#pragma unroll
                    for (int kw = 0; kw < KC; ++kw) {
                        v[kh][kw] = xp[ro + (uint32_t)coff[kw]];
                        v[kh][kw] = (rok && cok[kw]) ? v[kh][kw] : -INFINITY;
                    }
                }
                float m = -INFINITY;
#pragma unroll
                for (int kh = 0; kh < KC; ++kh)
#pragma unroll
                    for (int kw = 0; kw < KC; ++kw) m = fmaxf(m, v[kh][kw]);
                yp[(size_t)oh * OW] = m;
            }
        }
    } else {
        for (int pl = blockIdx.z; pl < planes; pl += gridDim.z) {
            const float *xp = x + (size_t)pl * plane;
            float *yp = y + (size_t)pl * OH * OW + ow;
            for (int r = 0; r < RB; ++r) {
                const int oh = oh0 + r;
                if (oh >= OH) break;
                float m = -INFINITY;
                for (int kh = 0; kh < kr; ++kh) {
                    const int ih = oh * s - p + kh * d;
                    if (ih < 0 || ih >= H) continue;
                    for (int kw = 0; kw < kr; ++kw) {
                        const int iw = iw0 + kw * d;
                        if (iw >= 0 && iw < W) m = fmaxf(m, xp[(uint32_t)ih * W + iw]);
                    }
                }
                yp[(size_t)oh * OW] = m;
            }
        }
    }
}

// Dynamic LDS bytes that, with the kernel's static LDS, leave room for exactly `wgs`
// workgroups per CU (0: no cap).
int occupancy_cap_lds_bytes(int wgs, int static_bytes) {
    if (wgs <= 0) return 0;
    int dev = 0, lds = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
        hipSuccess)
        return 0;
    const int share = lds / wgs - static_bytes - 512;  // 512 B of allocation slack
    return share > 0 ? share : 0;
}

template <int K, int V>
int launch_rows(const float *x, float *y, int N, int C, int H, int W, int OH, int OW, int p,
                hipStream_t stream) {
    const int band_rows = PS_MAXPOOL_BAND_ROWS;
    const int nbands = (OH + band_rows - 1) / band_rows;
    const int nstrips = (OW + kWave * V - 1) / (kWave * V);
    const uint64_t ntasks = (uint64_t)N * C * nstrips * nbands;
    constexpr int nw = PS_MAXPOOL_WG_WAVES;
    const uint64_t nblocks = (ntasks + nw - 1) / nw;
    if (nblocks > 0x7fffffffull) return PS_ERR_UNSUPPORTED;
    // the halo hand-over buffer, at least the occupancy cap's LDS share
    const int halo_bytes = nw * (K - 1) * V * kWave * (int)sizeof(float);
    const int cap_bytes = occupancy_cap_lds_bytes(PS_MAXPOOL_WGS_PER_CU, 0);
    const int lds_bytes = cap_bytes > halo_bytes ? cap_bytes : halo_bytes;
    if (lds_bytes > 65536 &&
        hipFuncSetAttribute((const void *)maxpool_s1_rows<K, V, PS_MAXPOOL_PREFETCH>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess)
        return PS_ERR_HIP;
    return launch(maxpool_s1_rows<K, V, PS_MAXPOOL_PREFETCH>, dim3((unsigned)nblocks),
                  dim3(kWave * nw), lds_bytes, stream, x, y, H, W, OH, OW, p, band_rows, nbands,
                  nstrips, ntasks);
}

template <int K>
int launch_rows_k(const float *x, float *y, int N, int C, int H, int W, int OH, int OW, int p,
                  hipStream_t stream) {
    // strip width 64*V: one strip covers rows up to 512 outputs wide
    if (OW > 256) return launch_rows<K, 8>(x, y, N, C, H, W, OH, OW, p, stream);
    if (OW > 128) return launch_rows<K, 4>(x, y, N, C, H, W, OH, OW, p, stream);
    if (OW > 64) return launch_rows<K, 2>(x, y, N, C, H, W, OH, OW, p, stream);
    return launch_rows<K, 1>(x, y, N, C, H, W, OH, OW, p, stream);
}

}  // namespace

int launch_maxpool2d(const float *x, float *y, int N, int C, int H, int W, int OH, int OW,
                     int k, int s, int p, int d, hipStream_t stream) {
    if (s == 1 && d == 1 && p < k && k >= 2 && k <= 8) {
        switch (k) {
            case 2: return launch_rows_k<2>(x, y, N, C, H, W, OH, OW, p, stream);
            case 3: return launch_rows_k<3>(x, y, N, C, H, W, OH, OW, p, stream);
            case 4: return launch_rows_k<4>(x, y, N, C, H, W, OH, OW, p, stream);
            case 5: return launch_rows_k<5>(x, y, N, C, H, W, OH, OW, p, stream);
            case 6: return launch_rows_k<6>(x, y, N, C, H, W, OH, OW, p, stream);
            case 7: return launch_rows_k<7>(x, y, N, C, H, W, OH, OW, p, stream);
            case 8: return launch_rows_k<8>(x, y, N, C, H, W, OH, OW, p, stream);
        }
    }
    {
        int rc = launch_disjoint<false>(x, y, N, C, H, W, OH, OW, k, s, p, d, PoolEpi{}, stream);
        if (rc >= 0) return rc;
        rc = launch_rows_sd_any<false>(x, y, N, C, H, W, OH, OW, k, s, p, d, PoolEpi{}, stream);
        if (rc >= 0) return rc;
    }
    // output rows per thread: 8 at stride 1 (neighbouring rows share most input rows
    // in the cache), 1 otherwise (MI355X: k3 s1 d2 1.20 ms at 8 vs 1.73 ms at 1;
    // k3 s2 0.77 ms at 1 vs 0.81 ms at 4)
    const int64_t planes = (int64_t)N * C;
    if (planes > 0x7fffffff || (int64_t)H * W >= (1ll << 31)) return PS_ERR_UNSUPPORTED;
    const int rb = s == 1 ? 8 : 1;
    const dim3 grid((unsigned)((OW + 255) / 256), (unsigned)((OH + rb - 1) / rb),
                    (unsigned)(planes < 65535 ? planes : 65535));
    if (grid.y > 65535u) return PS_ERR_UNSUPPORTED;
    const int pl = (int)planes;
#define PS_COLS(KC)                                                                            \
    return rb == 8 ? launch(maxpool_cols<KC, 8>, grid, dim3(256), 0, stream, x, y, H, W, OH, OW, \
                            k, s, p, d, pl)                                                      \
                   : launch(maxpool_cols<KC, 1>, grid, dim3(256), 0, stream, x, y, H, W, OH, OW, \
                            k, s, p, d, pl)
    switch (k) {
        case 1: PS_COLS(1);
        case 2: PS_COLS(2);
        case 3: PS_COLS(3);
        case 4: PS_COLS(4);
        case 5: PS_COLS(5);
        case 6: PS_COLS(6);
        case 7: PS_COLS(7);
        case 8: PS_COLS(8);
        default: PS_COLS(0);
    }
#undef PS_COLS
}

// The fp32 tanh -> *scale -> +bias2 -> max-pool stage through the streaming kernel;
// -1 when the window has no streaming instantiation.
int launch_tanh_scale_bias_maxpool_rows(const float *y, const float *bias2, float *out, int N,
                                        int C, int H, int W, int OH, int OW, float scale, int k,
                                        int s, int p, int d, hipStream_t stream) {
    const PoolEpi epi{scale < 0.f ? -1.f : 1.f, scale, bias2, C};
    const int rc = launch_disjoint<true>(y, out, N, C, H, W, OH, OW, k, s, p, d, epi, stream);
    if (rc >= 0) return rc;
    return launch_rows_sd_any<true>(y, out, N, C, H, W, OH, OW, k, s, p, d, epi, stream);
}

}  // namespace ps

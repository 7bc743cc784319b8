// Row-streaming variant for 2D 3x3 windows (stride 1 or 2, dilation 1).
//
// The box kernel above stages a halo box in LDS and computes only once all of
// it has landed.  This one has no LDS and no barriers: every wave streams its
// own input rows straight into MFMA operand registers, like the depthwise
// kernel.  A wave owns one M tile of 16 output columns and NTW merged-group
// tiles, over R consecutive output rows.  The 16 columns are 16 consecutive
// (row chunk, ow) pairs of one image, so a tile can wrap from one row chunk
// into the next and no MFMA column idles on a ragged image width; each lane
// keeps the rows of its own column.  The wave walks the (R - 1) * SH + 3
// input rows of its chunk in order.  One input row gives 3 * CH8 K slices per
// tile (window column dx, 8-channel chunk c) -- a 16-byte load per lane per
// slice, straight from x in NHWGC order -- and each is folded into the output
// rows it belongs to with the weights of that window row dy (input
// stationary; the weight fragments of all 3 x 3 taps stay in registers).  An
// output row is stored from the accumulators as soon as its last input row
// is in.
#include "smallg_common.h"

namespace gconv {
namespace smallg {
namespace {

struct RowParams {
    Div dCpg, dKpg;
    int H, W, Ho, Wo, C, K, Cpg, Kpg, GN, NT;
    int sw, ph, pw;
    int nchunk, nmt, ntb;         // row chunks per image, M tiles per image, tile blocks
    unsigned in_row, out_row;     // bytes of one row of x / of y
    unsigned img_bytes, oimg_bytes;
};

template <typename T, int SH, int R, int CH8, int NTW, int CPGC, int PF>
__global__ __launch_bounds__(kBlock) void rows_kernel(RowParams q, const T *__restrict__ x,
                                                      const T *__restrict__ w,
                                                      const T *__restrict__ bias, T *__restrict__ y)
{
    typedef typename Mfma<T>::V V;
    constexpr int NSL = 3 * CH8;             // K slices of one input row
    constexpr int NSR = (NSL + 3) / 4;       // MFMAs per (input row, tile, window row)
    constexpr int NI = (R - 1) * SH + 3;     // input rows of R output rows
    constexpr int kStorePolicy = 0;

    // ---- (image, M tile, block of 4 * NTW tiles); the waves of a workgroup
    //      read the same pixels (adjacent channel slices, shared cache lines)
    int tile = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int tb = tile % q.ntb;   tile /= q.ntb;
    const int mt = tile % q.nmt;
    const int n = tile / q.nmt;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    const int nn = lane & 15, kq = lane >> 4;
    const int t0 = (tb * kWaves + wave) * NTW;   // first merged-group tile of the wave
    if (t0 >= q.NT) return;                      // whole wave idle

    // ---- the lane's output column: (row chunk, ow) pair mt * 16 + nn
    const int task = mt * 16 + nn;
    const int chunk = task / q.Wo, ow = task - (task / q.Wo) * q.Wo;
    const bool cok = chunk < q.nchunk;
    const int oh0 = chunk * R;
    const int ih0 = oh0 * SH - q.ph;

    // x offsets of the lane's slices: slice k8 = 4 s + kq of a row is window
    // column dx = k8 / CH8, chunk c = k8 % CH8 of tile t0 + j
    unsigned coff[NTW][NSR];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int s2 = 0; s2 < NSR; ++s2) {
            const int k8 = 4 * s2 + kq;
            const int dx = k8 / CH8, c = k8 - (k8 / CH8) * CH8;
            const int iw = ow * q.sw - q.pw + dx;
            const bool ok = cok && k8 < NSL && t0 + j < q.NT && iw >= 0 && iw < q.W;
            coff[j][s2] = ok ? ((unsigned)iw * (unsigned)q.C + (unsigned)((t0 + j) * CH8 + c) * 8u) * 2u : kOob;
        }

    // ---- weight fragments of all taps: W[j][dy][s2], lane (row nn, slice kq)
    V wfrag[NTW][3][NSR];
    const int gout = fdiv(nn, q.dKpg), kout = nn - gout * q.Kpg;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const bool tile_ok = t0 + j < q.NT;
        const int g0 = (tile_ok ? t0 + j : 0) * q.GN;
        const T *wk = w + ((size_t)(g0 + gout) * q.Kpg + kout) * 9 * q.Cpg;
#pragma unroll
        for (int dy = 0; dy < 3; ++dy)
#pragma unroll
            for (int s2 = 0; s2 < NSR; ++s2) {
                const int k8 = 4 * s2 + kq;
                const bool live = tile_ok && k8 < NSL;
                const int dx = live ? k8 / CH8 : 0, c = live ? k8 - (k8 / CH8) * CH8 : 0;
                const uint4 raw = wslice<T, CPGC>(wk, live ? dy * 3 + dx : 0, c, gout, q.dCpg, live);
                wfrag[j][dy][s2] = *reinterpret_cast<const V *>(&raw);
            }
    }
    // bias of output channels (t0 + j) * 16 + 4 kq + i
    float bias_v[NTW][4];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int chb = (t0 + j < q.NT ? t0 + j : 0) * 16 + 4 * kq;
        uint2 braw = make_uint2(0u, 0u);
        if (bias) braw = *reinterpret_cast<const uint2 *>(bias + chb);
        const T *bel = reinterpret_cast<const T *>(&braw);
#pragma unroll
        for (int i = 0; i < 4; ++i) bias_v[j][i] = bias ? to_f32(bel[i]) : 0.f;
    }

    const auto rx = buf_rsrc(x + (size_t)n * q.H * q.W * q.C, q.img_bytes);
    const auto ry = buf_rsrc(y + (size_t)n * q.Ho * q.Wo * q.K, q.oimg_bytes);
    // the lane's output element offset in the image, row oh0 (channels of tile t0, quad kq)
    const unsigned obase = ((unsigned)(oh0 * q.Wo + ow) * (unsigned)q.K + (unsigned)(t0 * 16 + 4 * kq)) * 2u;

    f32x4 acc[R][NTW];
#pragma unroll
    for (int o = 0; o < R; ++o)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[o][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    V xb[NI][NTW][NSR];
    auto load_row = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int ih = ih0 + i;
        const bool rok = ih >= 0 && ih < q.H;
        const unsigned roff = (unsigned)ih * q.in_row;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int s2 = 0; s2 < NSR; ++s2) {
                const unsigned co = coff[j][s2];
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, (rok && co != kOob) ? roff + co : kOob, 0, 0);
                xb[i][j][s2] = __builtin_bit_cast(V, v);
            }
    };
    static_for(std::make_integer_sequence<int, (PF < NI ? PF : NI)>{}, load_row);
    static_for(std::make_integer_sequence<int, NI>{}, [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + PF < NI) load_row(std::integral_constant<int, i + PF>{});
        __builtin_amdgcn_sched_barrier(0);
        // fold row i into output rows o = (i - dy) / SH
        static_for(std::make_integer_sequence<int, 3>{}, [&](auto dyc) __attribute__((always_inline)) {
            constexpr int dy = decltype(dyc)::value;
            constexpr int d = i - dy;
            if constexpr (d >= 0 && d % SH == 0 && d / SH < R) {
                constexpr int o = d / SH;
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int s2 = 0; s2 < NSR; ++s2)
                        acc[o][j] = Mfma<T>::run(wfrag[j][dy][s2], xb[i][j][s2], acc[o][j]);
            }
        });
        // the output row whose window ends at input row i is complete
        constexpr int dl = i - 2;
        if constexpr (dl >= 0 && dl % SH == 0 && dl / SH < R) {
            constexpr int o = dl / SH;
            const bool ook = cok && oh0 + o < q.Ho;
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                T ov[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = from_f32<T>(acc[o][j][e] + bias_v[j][e]);
                const u32x2 packed = *reinterpret_cast<const u32x2 *>(ov);
                const bool tok = ook && t0 + j < q.NT;
                __builtin_amdgcn_raw_buffer_store_b64(
                    packed, ry, tok ? obase + (unsigned)(o * q.Wo) * (unsigned)q.K * 2u + (unsigned)(j * 32) : kOob,
                    0, kStorePolicy);
            }
        }
    });
}


template <typename T, int SH, int R, int CH8, int CPGC, int NTW = 2, int PF = 2>
hipError_t rows_go(const Problem &p, const RowConfig &c, const Args &a, hipStream_t s)
{
    RowParams q;
    q.H = p.H; q.W = p.W; q.Ho = p.Ho; q.Wo = p.Wo; q.C = p.C(); q.K = p.K();
    q.Cpg = p.Cpg; q.Kpg = p.Kpg; q.GN = c.GN; q.NT = c.NT;
    q.dCpg = make_div(p.Cpg); q.dKpg = make_div(p.Kpg);
    q.sw = p.sw; q.ph = p.ph; q.pw = p.pw;
    q.nchunk = c.nchunk; q.nmt = c.nmt; q.ntb = c.ntb;
    q.in_row = (unsigned)((long long)p.W * p.C() * 2);
    q.out_row = (unsigned)((long long)p.Wo * p.K() * 2);
    q.img_bytes = (unsigned)((long long)p.H * p.W * p.C() * 2);
    q.oimg_bytes = (unsigned)((long long)p.Ho * p.Wo * p.K() * 2);
    const int blocks = c.nmt * c.ntb * p.N;
    return enqueue(rows_kernel<T, SH, R, CH8, NTW, CPGC, PF>, dim3(blocks), dim3(kBlock), 0, s, a, q,
                   (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y);
}

template <typename T, int SH, int R, int CH8>
hipError_t rows_go3(const Problem &p, const RowConfig &c, const Args &a, hipStream_t s)
{
    switch (p.Cpg) {
    case 1: return rows_go<T, SH, R, CH8, 1>(p, c, a, s);
    case 2: return rows_go<T, SH, R, CH8, 2>(p, c, a, s);
    case 4: return rows_go<T, SH, R, CH8, 4>(p, c, a, s);
    default: return rows_go<T, SH, R, CH8, 8>(p, c, a, s);
    }
}

template <typename T, int SH, int R>
hipError_t rows_go2(const Problem &p, const RowConfig &c, const Args &a, hipStream_t s)
{
    return c.CH8 == 1 ? rows_go3<T, SH, R, 1>(p, c, a, s) : rows_go3<T, SH, R, 2>(p, c, a, s);
}

template <typename T>
hipError_t rows_launch_t(const Problem &p, const RowConfig &c, const Args &a, hipStream_t s)
{
    if (p.sh == 1) return c.R == 14 ? rows_go2<T, 1, 14>(p, c, a, s) : rows_go2<T, 1, 7>(p, c, a, s);
    return c.R == 14 ? rows_go2<T, 2, 14>(p, c, a, s) : rows_go2<T, 2, 7>(p, c, a, s);
}

}  // namespace

bool rows_configure(const Problem &p, RowConfig &c)
{
    if (p.ndim != 2 || p.Y != 3 || p.X != 3 || p.dh != 1 || p.dw != 1) return false;
    if (p.sh != 1 && p.sh != 2) return false;
    c.GN = 16 / p.Kpg;
    c.CH8 = c.GN * p.Cpg / 8;
    if (c.CH8 != 1 && c.CH8 != 2) return false;
    c.NT = p.G / c.GN;
    c.NTW = 2;
    c.ntb = (c.NT + kWaves * c.NTW - 1) / (kWaves * c.NTW);
    // rows per wave from {7, 14}: the longer run unless it leaves fewer
    // than two waves per SIMD
    const long long es = 2;
    if ((long long)p.H * p.W * p.C() * es >= (1LL << 31) || (long long)p.Ho * p.Wo * p.K() * es >= (1LL << 31))
        return false;
    c.R = 7;
    for (int r : {14}) {
        const long long chunks = (p.Ho + r - 1) / r;
        const long long mts = (chunks * p.Wo + 15) / 16;
        if (mts * p.N * ((c.NT + c.NTW - 1) / c.NTW) >= 2048) c.R = r;
    }
    c.nchunk = (p.Ho + c.R - 1) / c.R;
    const long long tasks = (long long)c.nchunk * p.Wo;
    c.nmt = (int)((tasks + 15) / 16);
    return tasks < (1LL << 30) && (long long)c.nmt * c.ntb * p.N < (1LL << 31);
}

hipError_t rows_launch(const Problem &p, const RowConfig &c, const Args &a, hipStream_t s)
{
    return p.dtype == GCONV_F16 ? rows_launch_t<_Float16>(p, c, a, s) : rows_launch_t<__bf16>(p, c, a, s);
}

}  // namespace smallg
}  // namespace gconv

// Small-group MFMA direct conv through an LDS ring of input rows (3x3 and
// 3x3x3 windows).
//
// Loading MFMA operand fragments straight from x (k_smallg_rows.hip) moves
// 16 bytes of 16 different pixels per lane group, and every input element is
// fetched three times (once per window column): the texture path, not HBM,
// is then the limit.  Here a workgroup owns one M tile of 16 output columns,
// R output rows and TPB = 4 x NTW consecutive merged-group tiles, whose input
// channels are TPB x CH8 16-byte chunks of every pixel -- 256 contiguous
// bytes for the ResNeXt 8/8 shape.  Each input row segment (IW = 15 S + 3
// pixels x those chunks) is brought into an LDS ring with direct-to-LDS
// loads, PF rows ahead, and each wave reads its operand fragments from LDS (a
// window column is just an address offset).  The accumulators of each output
// row leave as soon as the row is complete, the workgroup's four waves
// together writing TPB x 16 contiguous output channels of each pixel.
//
// fp16/bf16 tiles take 16-byte chunks of 8 channels and 16x16x32 MFMAs; fp32
// tiles take chunks of 4 channels, each fragment read feeding four chained
// 16x16x4 fp32 MFMAs (smallg_common.h); byte offsets follow the element size.
//
// LDS: slot j (16 bytes) of ring pixel p holds channel chunk j ^ f(p),
// f(p) = (p / S) mod 16, so the 16 pixels one fragment read touches (p =
// S nn + dx) fall on 16 different bank groups; the swizzle costs nothing on
// the write side because each DMA lane simply fetches the chunk its LDS slot
// is to hold.  Rows are padded to whole 64-slot (1 KB) DMA instructions.
#pragma once

#include "smallg_common.h"

namespace gconv {
namespace smallg {
namespace {

constexpr unsigned kRingMaxLds = 160 * 1024;   // the dynamic LDS limit every ring instance is raised to
// Input rows in flight ahead of the arithmetic (the ring holds one more).
// Measured on the ResNeXt-style and 3D N=8 workloads: 6 rows ahead (2D) and
// all 8 of a 3D run's later rows issued up front time the same as 3 rows.
constexpr int kRingPF2d = 3;
constexpr int kRingPF3d = 3;

struct RingParams {
    Div dCpg, dKpg;
    int D, H, W, Do, Ho, Wo, C, K, Cpg, Kpg, GN, NT;
    int pd, ph, pw;
    int IW, RS;                   // ring pixels per plane segment, slots per ring row (mult. of 64)
    int TPB, ntb;                 // tiles per workgroup, workgroups across the channels
    int NINS;                     // DMA instructions per ring row
    int nmt, nchunk;              // M tiles per output row, row chunks per image
    unsigned in_row, img_bytes, oimg_bytes;
};

template <typename T, int S, int R, int CH8, int NTW, int CPGC, int DZ, int PF>
__global__ __launch_bounds__(kBlock) void ring_kernel(RingParams q, const T *__restrict__ x,
                                                      const T *__restrict__ w,
                                                      const T *__restrict__ bias, T *__restrict__ y)
{
    typedef typename Mfma<T>::V V;
    constexpr unsigned ES = sizeof(T);                 // bytes per element
    constexpr unsigned EPC = 16 / ES;                  // channels per 16-byte chunk
    extern __shared__ uint4 ring[];
    constexpr int NSL = 3 * CH8;             // K slices of one input row
    constexpr int NSR = (NSL + 3) / 4;       // MFMAs per (input row, tile, window row)
    constexpr int NI = (R - 1) * S + 3;      // input rows of R output rows
    static_assert(PF >= 1 && PF < NI, "rows in flight ahead of the arithmetic");
    constexpr int NR = PF + 1;               // ring rows
    constexpr int kMaxIns = 8;               // DMA instructions per wave per row
    constexpr int CVR = kWaves * NTW * CH8;  // 16-byte chunks per ring pixel (16 or 8)
    static_assert(CVR == 16 || CVR == 8, "ring pixels hold 8 or 16 chunks");
    // slot swizzle: the 16 pixels a fragment read touches land on 16 bank groups
    auto swz = [](int pp) { return CVR == 16 ? (pp / S) & 15 : ((pp / S) >> 1) & 7; };

    int tile = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int tb = tile % q.ntb;   tile /= q.ntb;
    const int mt = tile % q.nmt;   tile /= q.nmt;
    const int chunk = tile % q.nchunk;   tile /= q.nchunk;
    const int od = tile % q.Do;                  // output plane (0 in 2D)
    const int n = tile / q.Do;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    const int nn = lane & 15, kq = lane >> 4;
    const int lt0 = wave * NTW;                  // first tile of the wave within the workgroup
    const int t0 = tb * q.TPB + lt0;             // ... and among all tiles
    const int cb = tb * q.TPB * CH8;             // first channel chunk of the workgroup
    const int ow0 = mt * 16, oh0 = chunk * R;
    const int iw0 = ow0 * S - q.pw, ih0 = oh0 * S - q.ph;
    const unsigned ring_lds = (unsigned)(size_t)ring;
    const unsigned row_bytes = (unsigned)q.RS * 16u;
    const unsigned zero_slot = ring_lds + (unsigned)NR * row_bytes;   // 16 zero bytes

    // ---- DMA plan: instruction k = wave + 4 m of a ring row covers slots
    //      64 k .. 64 k + 63; lane -> ring pixel p, slot j -> chunk j ^ f(p)
    //      (a 3D ring row is DZ input planes' row segments, one after the other)
    const int nins = (q.NINS - wave + kWaves - 1) / kWaves;   // this wave's instructions per row
    const int seg = q.IW * CVR;                                // slots of one plane's segment
    unsigned dcol[kMaxIns];                                    // plane + column part of the offset, or kOob
#pragma unroll
    for (int m = 0; m < kMaxIns; ++m) {
        const int sl = (wave + kWaves * m) * 64 + lane;
        const int dz = sl / seg, rem = sl - (sl / seg) * seg;
        const int pp = rem / CVR, j = rem - (rem / CVR) * CVR;
        const int iw = iw0 + pp, id = od - q.pd + dz;
        const int c = cb + (j ^ swz(pp));
        const bool ok = m < nins && dz < DZ && id >= 0 && id < q.D && iw >= 0 && iw < q.W;
        dcol[m] = ok ? (((unsigned)id * (unsigned)(q.H * q.W) + (unsigned)iw) * (unsigned)q.C + (unsigned)c * EPC) * ES : kOob;
    }
    const rsrc_t rs = make_rsrc(x + (size_t)n * q.D * q.H * q.W * q.C, q.img_bytes);
    auto issue_row = [&](int i) __attribute__((always_inline)) {
        const int ih = ih0 + i;
        const bool rok = ih >= 0 && ih < q.H;
        const unsigned roff = (unsigned)ih * q.in_row;
        const unsigned base = ring_lds + (unsigned)(i % NR) * row_bytes;
#pragma unroll
        for (int m = 0; m < kMaxIns; ++m) {
            if (m < nins) {
                const unsigned vo = (rok && dcol[m] != kOob) ? roff + dcol[m] : kOob;
                dma16(vo, __builtin_amdgcn_readfirstlane(base + (unsigned)(wave + kWaves * m) * 1024u), rs);
            }
        }
    };

    // ---- weight fragments of all taps: W[j][dz][dy][s2], lane (row nn, slice kq)
    V wfrag[NTW][DZ][3][NSR];
    const int gout = fdiv(nn, q.dKpg), kout = nn - gout * q.Kpg;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int g0 = (t0 + j) * q.GN;
        const T *wk = w + ((size_t)(g0 + gout) * q.Kpg + kout) * (9 * DZ) * q.Cpg;
#pragma unroll
        for (int dz = 0; dz < DZ; ++dz)
#pragma unroll
            for (int dy = 0; dy < 3; ++dy)
#pragma unroll
                for (int s2 = 0; s2 < NSR; ++s2) {
                    const int k8 = 4 * s2 + kq;
                    const bool live = k8 < NSL;
                    const int dx = live ? k8 / CH8 : 0, c = live ? k8 - (k8 / CH8) * CH8 : 0;
                    const uint4 raw = weight_slice<T, CPGC>(wk, live ? (dz * 3 + dy) * 3 + dx : 0, c, gout, q.dCpg, live);
                    wfrag[j][dz][dy][s2] = *reinterpret_cast<const V *>(&raw);
                }
    }
    float bias_v[NTW][4];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias_v[j][e] = bias ? to_f32(bias[(t0 + j) * 16 + 4 * kq + e]) : 0.f;
    // LDS byte offset (within a ring row) of the lane's fragment of tile j,
    // slice s2: ring pixel nn S + dx, ring chunk (lt0 + j) CH8 + c, swizzled;
    // a dead slice reads the zero slot
    unsigned foff[NTW][NSR];
    bool fzero[NSR];
#pragma unroll
    for (int s2 = 0; s2 < NSR; ++s2) fzero[s2] = 4 * s2 + kq >= NSL;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int s2 = 0; s2 < NSR; ++s2) {
            const int k8 = 4 * s2 + kq;
            const int dx = k8 / CH8, c = k8 - (k8 / CH8) * CH8;
            const int pp = nn * S + dx;
            const int ch = (lt0 + j) * CH8 + c;
            foff[j][s2] = (unsigned)(pp * CVR + (ch ^ swz(pp))) * 16u;
        }
    const unsigned seg_bytes = (unsigned)seg * 16u;   // plane dz's segment starts dz * seg_bytes into a ring row
    // ---- output.  A completed output row goes through an LDS staging
    // buffer (two, alternating): each lane drops its four channels of pixel
    // nn there, and after the next barrier the workgroup writes the row's 16
    // pixels x TPB * 16 channels with one 16-byte store per thread and chunk
    // -- whole pixel runs instead of 8-byte (fp32: 16-byte) pieces of 16 pixels,
    // which the texture path handles far better.  y is written once and not
    // read back, so the stores are non-temporal (measured a few % faster).
    constexpr int kNonTemporal = 2;
    constexpr int kStageChunks = kWaves * NTW * (int)ES;     // 16-byte chunks per staged pixel
    constexpr int kStagePitch = kStageChunks * 16 + 16;      // bytes per staged pixel (padded)
    const unsigned stage_lds = zero_slot + 16u;
    const unsigned stage_w = (unsigned)(nn * kStagePitch) + (unsigned)lt0 * 16u * ES + (unsigned)kq * 4u * ES;   // this lane's 4 channels
    const auto ry = buf_rsrc(y + ((size_t)n * q.Do + od) * q.Ho * q.Wo * q.K, q.oimg_bytes);
    auto flush = [&](int o, int buf) __attribute__((always_inline)) {
        const unsigned sb = stage_lds + (unsigned)buf * 16u * kStagePitch;
#pragma unroll
        for (int k = (int)threadIdx.x; k < 16 * kStageChunks; k += kBlock) {
            const int pix = k / kStageChunks, ck = k - (k / kStageChunks) * kStageChunks;
            const uint4 v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(ring) +
                                                            (sb - ring_lds) + pix * kStagePitch + ck * 16);
            const bool ok = ow0 + pix < q.Wo && oh0 + o < q.Ho;
            const unsigned go = ((unsigned)((oh0 + o) * q.Wo + ow0 + pix) * (unsigned)q.K + (unsigned)(tb * q.TPB * 16)) * ES +
                                (unsigned)ck * 16u;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, ry, ok ? go : kOob, 0, kNonTemporal);
        }
    };

    // ---- prologue: the zero slot, then the first PF rows
    if (threadIdx.x == 0) *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(ring) + (size_t)NR * row_bytes) = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PF; ++i)
        if (i < NI) issue_row(i);

    f32x4 acc[R][NTW];
#pragma unroll
    for (int o = 0; o < R; ++o)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[o][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // flushes issued at step st (compile time): the output row completed at
    // step st - 1.  A flush's 16 * kStageChunks stores go to threads in order,
    // so this wave issues one store instruction per pass of 256 threads that
    // reaches its first lane, and none when the row has fewer stores than the
    // waves before it have lanes (3D rings of 8-chunk pixels: 128 stores).
    auto flushes_at = [](int st) constexpr {
        return (st >= 3 && (st - 3) % S == 0 && (st - 3) / S < R) ? 1 : 0;
    };
    constexpr int kFlushStores = 16 * kStageChunks;
    const int wave_stores = kFlushStores > wave * 64 ? (kFlushStores - wave * 64 + kBlock - 1) / kBlock : 0;
    static_for(std::make_integer_sequence<int, NI>{}, [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        // this wave's DMAs of row i are done when only later rows' DMAs and
        // the stores issued since remain: rows i+1 .. i+PF-1 and the stores
        // of steps i-PF .. i-1
        constexpr int later_rows = (i + PF - 1 < NI - 1 ? i + PF - 1 : NI - 1) - i;
        constexpr int later_flushes = [=]() constexpr {
            int n = 0;
            for (int k = i - PF; k < i; ++k) n += k >= 0 ? flushes_at(k) : 0;
            return n;
        }();
        vm_wait(later_rows * nins + later_flushes * wave_stores);
        __syncthreads();
        // the slot of row i + PF was last read at step i - 1: refill it
        if constexpr (i + PF < NI) issue_row(i + PF);
        // the output row completed at step i - 1 is staged: write it out
        constexpr int dp = i - 3;
        if constexpr (dp >= 0 && dp % S == 0 && dp / S < R) flush(dp / S, (dp / S) & 1);
        const unsigned rb = ring_lds + (unsigned)(i % NR) * row_bytes;
        V xf[DZ][NTW][NSR];
#pragma unroll
        for (int dz = 0; dz < DZ; ++dz)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int s2 = 0; s2 < NSR; ++s2) {
                    const unsigned a = fzero[s2] ? zero_slot : rb + (unsigned)dz * seg_bytes + foff[j][s2];
                    const uint4 raw = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(ring) + (a - ring_lds));
                    xf[dz][j][s2] = *reinterpret_cast<const V *>(&raw);
                }
        static_for(std::make_integer_sequence<int, 3>{}, [&](auto dyc) __attribute__((always_inline)) {
            constexpr int dy = decltype(dyc)::value;
            constexpr int d = i - dy;
            if constexpr (d >= 0 && d % S == 0 && d / S < R) {
                constexpr int o = d / S;
#pragma unroll
                for (int dz = 0; dz < DZ; ++dz)
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
#pragma unroll
                        for (int s2 = 0; s2 < NSR; ++s2)
                            acc[o][j] = Mfma<T>::run(wfrag[j][dz][dy][s2], xf[dz][j][s2], acc[o][j]);
            }
        });
        constexpr int dl = i - 2;
        if constexpr (dl >= 0 && dl % S == 0 && dl / S < R) {
            constexpr int o = dl / S;
            char *sb = reinterpret_cast<char *>(ring) + (stage_lds - ring_lds) + (o & 1) * 16 * kStagePitch + stage_w;
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                T ov[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = from_f32<T>(acc[o][j][e] + bias_v[j][e]);
                if constexpr (ES == 4)
                    *reinterpret_cast<uint4 *>(sb + j * 64) = *reinterpret_cast<const uint4 *>(ov);
                else
                    *reinterpret_cast<uint2 *>(sb + j * 32) = *reinterpret_cast<const uint2 *>(ov);
            }
        }
    });
    // the last output row (completed at the last step) is still staged
    __syncthreads();
    flush(R - 1, (R - 1) & 1);
    // no DMA may still be writing LDS when the workgroup retires
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

template <typename T, int S, int R, int CH8, int NTW, int CPGC, int DZ, int PF>
hipError_t ring_go(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    RingParams q;
    q.D = p.D; q.H = p.H; q.W = p.W; q.Do = p.Do; q.Ho = p.Ho; q.Wo = p.Wo; q.C = p.C(); q.K = p.K();
    q.Cpg = p.Cpg; q.Kpg = p.Kpg; q.GN = c.GN; q.NT = c.NT;
    q.dCpg = make_div(p.Cpg); q.dKpg = make_div(p.Kpg);
    q.pd = p.pd; q.ph = p.ph; q.pw = p.pw;
    q.IW = c.IW; q.RS = c.RS; q.NINS = c.NINS;
    q.TPB = c.TPB; q.ntb = c.ntb;
    q.nmt = c.nmt; q.nchunk = c.nchunk;
    q.in_row = (unsigned)((long long)p.W * p.C() * (long long)sizeof(T));
    q.img_bytes = (unsigned)((long long)p.D * p.H * p.W * p.C() * (long long)sizeof(T));
    q.oimg_bytes = (unsigned)((long long)p.Ho * p.Wo * p.K() * (long long)sizeof(T));
    const int blocks = c.blocks;
    auto k = ring_kernel<T, S, R, CH8, NTW, CPGC, DZ, PF>;
    static std::atomic<unsigned long long> lds_set{0};
    if (c.lds > 64 * 1024) {
        // the limit is raised to the largest LDS any configuration of this instance uses
        const hipError_t e = allow_lds((const void *)k, lds_set, kRingMaxLds);
        if (e != hipSuccess) return e;
    }
    return enqueue(k, dim3(blocks), dim3(kBlock), c.lds, s, a, q,
                   (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y);
}

template <typename T, int S, int R, int CH8, int NTW, int DZ, int PF>
hipError_t ring_go4(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    switch (p.Cpg) {
    case 1: return ring_go<T, S, R, CH8, NTW, 1, DZ, PF>(p, c, a, s);
    case 2: return ring_go<T, S, R, CH8, NTW, 2, DZ, PF>(p, c, a, s);
    case 4: return ring_go<T, S, R, CH8, NTW, 4, DZ, PF>(p, c, a, s);
    default: return ring_go<T, S, R, CH8, NTW, 8, DZ, PF>(p, c, a, s);
    }
}

}  // namespace
}  // namespace smallg
}  // namespace gconv

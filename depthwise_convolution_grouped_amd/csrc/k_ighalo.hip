// Halo-staged implicit GEMM for groups with many channels (fp16 / bf16, 2D
// and 3D, Cpg % 32 == 0, Kpg % 64 == 0), persistent and XCD-aware.
//
// Per group the convolution is a GEMM with M = output pixels, N = Kpg output
// channels and K = taps * Cpg, with K decoded into (tap, channel) and the
// channel fastest, as the implicit-GEMM A and B descriptors of rocm-libraries
// PR 10064 do (Technical Details: C is split into G x C/G and the weight
// descriptor's channel extent is C/G).  Unlike an M-tiled implicit GEMM,
// which gathers a fresh im2col tile for every (tap, channel) stage, a work
// item here is a block of output pixels of one image: RH output rows x CW
// output columns (one output plane in 3D), for one group and a block of BN
// output channels.  The input box that block reads - the output block
// widened by the filter's dilated footprint - is staged in LDS once per
// chunk of KT input channels, and every tap of the chunk reads its A operand
// from that box at a shifted offset.  Input bytes leave HBM about once; the
// only per-stage transfer is the weight slice of one (tap, chunk), which the
// group's items share through the L2 of their XCD.
//
// Pipelines, all filled by direct-to-LDS buffer loads (zero fill for
// padding from the buffer range check):
//   - input box: two chunk buffers; at a chunk's first stage the next
//     chunk's box (the next item's first chunk at an item's last chunk) is
//     loaded into the other buffer;
//   - weights: four stage buffers; stage s loads stage s+3;
//   - bias: three 1 KB blocks; an item's first stage loads the next item's.
// One barrier per stage.  Every wave waits only for its own loads with an
// explicit s_waitcnt vmcnt (loads return in order), then the barrier makes
// all waves' loads visible and ends every wave's previous stage, so the
// buffers that stage used can be refilled.
//
// Four waves split the item 2 (pixels) x 2 (channels).  Each computes up to
// 7 x NTW tiles of v_mfma_f32_16x16x32 with the weights as the first operand,
// so each lane ends with four adjacent output channels of one pixel.  An
// item's epilogue adds the bias, rounds once and stores 8 bytes per lane.
//
// Grid: two workgroups per CU where the LDS fits (it does for boxes up to
// about 20 KB per 32 channels), at most 512 workgroups, each looping over
// its items.  Items are ordered group-major and each XCD (workgroup id mod 8
// under the round-robin dispatch) takes one contiguous eighth of them, so an
// XCD's L2 holds the weights of about G/8 groups.
#include <type_traits>

#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace ighalo {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = 4;
constexpr int kMaxTiles = 14;         // M tiles (16 pixels) per item
constexpr int kMaxHaloInstr = 32;      // box load instructions per chunk (boxes up to 512 pixels)
constexpr int kHaloLPW = kMaxHaloInstr / kWaves;
constexpr int kCUs = 256;              // MI355X compute units
constexpr int kMaxLds = 160 * 1024;
constexpr int kBiasBytes = 3 * 1024;   // three 1 KB bias blocks
constexpr int kColdBytes = 128;        // per-item parameters (Cold), read from LDS
constexpr int kWBuf = 4;               // weight stage buffers
constexpr unsigned kOob = 0x80000000u;

typedef int rsrc_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Params {
    int N, G, Cpg, Kpg, C, K;
    int D, H, W, Do, Ho, Wo, Z, Y, X;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int RH, CW, nrb, ncb, nnb;   // item = RH x CW output pixels of one plane; blocks per axis
    int BD, BH, BW, BP;          // input box extents and pixel count
    int HI;                      // halo DMA instructions per chunk (64 lanes each)
    int MT;                      // M tiles of 16 pixels per item
    int items, nch, taps;
    int xcd_split;               // 1: XCD-contiguous item ranges
    int hb_bytes;                // one halo buffer (multiple of 1 KB)
    unsigned x_bytes, w_bytes;
};

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    const unsigned long long a = (unsigned long long)base;
    rsrc_t r;
    r.x = (int)(unsigned)(a & 0xffffffffull);
    r.y = (int)(unsigned)((a >> 32) & 0xffffull);
    r.z = (int)bytes;
    r.w = 0x00020000;
    return r;
}

// 16 bytes from buffer offset `voffset` to LDS M0 + 16 * lane.  The
// descriptor is wave-uniform; readfirstlane keeps it in scalar registers
// even where the compiler cannot prove that.
__device__ __forceinline__ void dma16(unsigned voffset, unsigned lds_byte, rsrc_t r)
{
    r.x = __builtin_amdgcn_readfirstlane(r.x);
    r.y = __builtin_amdgcn_readfirstlane(r.y);
    r.z = __builtin_amdgcn_readfirstlane(r.z);
    r.w = __builtin_amdgcn_readfirstlane(r.w);
    asm volatile("s_mov_b32 m0, %1\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voffset), "s"(lds_byte), "s"(r)
                 : "memory", "m0");
}


template <typename T> struct Mfma;
template <> struct Mfma<_Float16> {
    typedef f16x8 V;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<__bf16> {
    typedef bf16x8 V;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

struct Item {
    int g, nb, n, od, rb, cb;
};

// Parameters used once per chunk or item (item decode, box origin, output
// addressing).  The kernel keeps them in LDS and reads them where they are
// used, so they hold neither scalar nor vector registers across the stage
// loop (two waves share each SIMD's register file).
struct Cold {
    int N, Do, Ho, Wo, D, H, W, C, K, Kpg, Cpg, sd, sh, sw, pd, ph, pw, RH, CW, ncb, nrb, nnb;
};
static_assert(sizeof(Cold) <= kColdBytes, "Cold fits its LDS slot");

__device__ __forceinline__ int in_vgpr(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

template <typename P>
__device__ __forceinline__ Item decode(const P &q, int it)
{
    Item r;
    r.cb = it % q.ncb; it /= q.ncb;
    r.rb = it % q.nrb; it /= q.nrb;
    r.od = it % q.Do;  it /= q.Do;
    r.n = it % q.N;    it /= q.N;
    r.nb = it % q.nnb;
    r.g = it / q.nnb;
    return r;
}

// NTW: 16-channel N tiles per wave (the item's channel block is
// BN = 32 * NTW); TPW: M tiles per wave (the item has at most 2 TPW).  Every
// wave runs all TPW tiles without branches; tiles past the item's end read
// box pixel 0 and are not stored.  A stage is one tap x KT = 32 input
// channels: one MFMA K step.
//
// LDS rows (a box pixel's 32 channels, or a weight row's 32 channels) are
// four 16-byte slots with no padding; slot j of row r holds channel vector
// j ^ key(r), key(r) = (r >> 1) & 3.  The XOR swizzle is applied when the
// row is loaded (direct-to-LDS loads write each lane's 16 bytes at a fixed
// place, so the lane picks which global vector to fetch) and keeps the
// 16-byte fragment reads of eight consecutive rows in distinct banks.
//
// Two workgroups share a CU (LDS and registers are sized for it), so each
// SIMD runs two waves: while one waits for LDS, loads or the barrier, the
// other issues MFMAs.
template <typename T, int NTW, int TPW>
__global__ __launch_bounds__(kBlock, 2) void kernel(Params q, const T *__restrict__ x,
                                                    const T *__restrict__ w,
                                                    const T *__restrict__ bias, T *__restrict__ y)
{
    typedef typename Mfma<T>::V V;
    constexpr int KT = 32;
    constexpr int SPR = KT / 8;               // 16-byte slots per staged row
    constexpr int BN = 2 * NTW * 16;
    constexpr int B_INSTR = BN * SPR / 64;    // load instructions per weight stage
    static_assert(B_INSTR % kWaves == 0, "weight stage loads split evenly over the waves");
    constexpr int B_LPW = B_INSTR / kWaves;
    static_assert(B_LPW <= TPW, "weight loads are interleaved one per M tile");
    constexpr int B_BYTES = BN * SPR * 16;
    extern __shared__ uint4 lds[];

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    const int mh = wave & 1, nh = wave >> 1;
    const unsigned es = (unsigned)sizeof(T);
    const rsrc_t rx = make_rsrc(x, q.x_bytes);
    const rsrc_t rw = make_rsrc(w, q.w_bytes);
    const rsrc_t rb = make_rsrc(bias, bias ? (unsigned)(q.K * (int)sizeof(T)) : 0u);
    const unsigned lds_b = (unsigned)(size_t)lds;
    const unsigned halo_b = lds_b;                                       // 2 box buffers
    const unsigned wbuf_b = lds_b + 2u * (unsigned)q.hb_bytes;           // kWBuf weight stages
    const unsigned bias_b = wbuf_b + (unsigned)(kWBuf * B_BYTES);        // 3 bias blocks of 1 KB
    const char *lds_c = reinterpret_cast<const char *>(lds);
    const int cold_off = 2 * q.hb_bytes + kWBuf * B_BYTES + kBiasBytes;

    auto key = [](int r) { return (r >> 1) & 3; };

    // ---- this workgroup's items
    int it0, itstep, nI;
    {
        const int b = blockIdx.x, nwg = gridDim.x;
        if (q.xcd_split) {
            const int xcd = b & 7, j = b >> 3, per = nwg >> 3;
            const int lo = (int)((long long)q.items * xcd / 8);
            const int hi = (int)((long long)q.items * (xcd + 1) / 8);
            it0 = lo + j;
            itstep = per;
            nI = it0 < hi ? (hi - it0 + per - 1) / per : 0;
        } else {
            it0 = b;
            itstep = nwg;
            nI = (q.items - b + nwg - 1) / nwg;
        }
    }
    if (nI <= 0) return;
    if (t == 0) {
        Cold cv;
        cv.N = q.N; cv.Do = q.Do; cv.Ho = q.Ho; cv.Wo = q.Wo; cv.D = q.D; cv.H = q.H; cv.W = q.W;
        cv.C = q.C; cv.K = q.K; cv.Kpg = q.Kpg; cv.Cpg = q.Cpg; cv.sd = q.sd; cv.sh = q.sh; cv.sw = q.sw;
        cv.pd = q.pd; cv.ph = q.ph; cv.pw = q.pw; cv.RH = q.RH; cv.CW = q.CW; cv.ncb = q.ncb;
        cv.nrb = q.nrb; cv.nnb = q.nnb;
        *reinterpret_cast<Cold *>(reinterpret_cast<char *>(lds) + cold_off) = cv;
    }
    __syncthreads();
    const Cold &cq = *reinterpret_cast<const Cold *>(lds_c + cold_off);

    // ---- per-lane load plans (fixed for the whole kernel).  Instruction
    // k = wave + 4 i of a buffer fills its slots 64k .. 64k+63.
    int wofs[B_LPW];     // weights: element offset of this lane's vector within the block's rows
#pragma unroll
    for (int i = 0; i < B_LPW; ++i) {
        const int L = (wave + kWaves * i) * 64 + lane;
        const int row = L / SPR, j = L - row * SPR;
        wofs[i] = row * q.taps * q.Cpg + (j ^ key(row)) * 8;
    }
    int nhw = 0;          // box load instructions of this wave per chunk
#pragma unroll
    for (int i = 0; i < kHaloLPW; ++i)
        if (wave + kWaves * i < q.HI) nhw = i + 1;

    // ---- fragment addressing
    // A: tile tm of this wave = item tile T = mh * ta + tm; lane pixel m = 16 T + l16
    const int ta = (q.MT + 1) >> 1;
    const int my_tiles = mh == 0 ? ta : q.MT - ta;
    const int tbase = mh * ta;     // ta <= TPW
    int apos[TPW];                 // the pixel's row in the box (before the tap shift)
#pragma unroll
    for (int tm = 0; tm < TPW; ++tm) {
        const int m = (tbase + tm) * 16 + l16;
        const int lr = m / q.CW, lc = m - lr * q.CW;
        const bool live = tm < my_tiles && lr < q.RH;
        apos[tm] = live ? lr * q.sh * q.BW + lc * q.sw : 0;
    }
    // B: byte offset of this lane's vector for N tile 0 of a weight stage;
    // tile nt is 1 KB further (16 rows, and the swizzle key only sees l16)
    const unsigned boff0 = (unsigned)(((nh * NTW) * 16 + l16) * SPR + (kq ^ key(l16))) * 16u;

    // ---- stage sequence: item ii (local), chunk c, tap tp; stage s, chunk
    // h = ii * nch + c
    const int SPI = q.nch * q.taps;   // stages per item
    const int S = nI * SPI;
    const int nH = nI * q.nch;
    int issued = 0;   // this wave's load instructions so far (for the vmcnt waits)

    // Weight stages are issued kWBuf - 1 ahead through a cursor that only
    // counts (no divisions per stage): item, chunk, tap, ring buffer.
    auto w_rowbase = [&](int ii) {
        const Item I = decode(cq, it0 + ii * itstep);
        return (I.g * cq.Kpg + I.nb * BN) * q.taps * cq.Cpg;
    };
    int w_next = 0, w_tp = 0, w_c = 0, w_ii = 0, w_buf = 0;
    int w_row = w_rowbase(0);
    int w_vo[B_LPW];            // this lane's offsets for the next weight stage
    unsigned w_m0 = 0;          // its buffer's LDS byte address
    auto prep_w = [&]() {
        const int rowbase = w_row + w_tp * q.Cpg + w_c * KT;
#pragma unroll
        for (int i = 0; i < B_LPW; ++i) w_vo[i] = (rowbase + wofs[i]) * (int)es;
        w_m0 = wbuf_b + (unsigned)(w_buf * B_BYTES);
    };
    // Issue marks (this wave's load count right after a group of loads) are
    // named scalars that shift as the cursors advance; every write goes to
    // one fixed variable, so they stay in registers (a dynamically indexed
    // mark would live in scratch memory, whose loads count in vmcnt).
    int w_last = 0;             // mark of the last weight stage issued
    auto finish_w = [&]() {     // after a stage's B_LPW instructions are out
        issued += B_LPW;
        w_last = issued;
        ++w_next;
        if (++w_buf == kWBuf) w_buf = 0;
        if (++w_tp == q.taps) {
            w_tp = 0;
            if (++w_c == q.nch) {
                w_c = 0;
                if (++w_ii < nI) w_row = w_rowbase(w_ii);
            }
        }
    };
    auto issue_w1 = [&](int i) {
        dma16((unsigned)w_vo[i], __builtin_amdgcn_readfirstlane(w_m0 + (unsigned)((wave + kWaves * i) * 1024)), rw);
    };
    int mh_last = 0;            // mark of the last box issued
    // This lane's box vectors for channel chunk 0 of the item whose box is
    // being loaded: element offsets into x, -1 where the vector is padding
    // or past the box.  Set once per item (the only division work of the
    // box loads); chunk c adds c * KT.
    int hoff[kHaloLPW];
    auto set_box_item = [&](int ii) {
        const Item I = decode(cq, it0 + ii * itstep);
        const int iz0 = I.od * cq.sd - cq.pd;
        const int iy0 = I.rb * cq.RH * cq.sh - cq.ph;
        const int ix0 = I.cb * cq.CW * cq.sw - cq.pw;
        const int Dv = cq.D, Hv = cq.H, Wv = cq.W, Cv = cq.C;
        const int cg = I.g * cq.Cpg;
        const int plane = q.BH * q.BW;
#pragma unroll
        for (int i = 0; i < kHaloLPW; ++i) {
            // instruction wave + 4 i fills box slots 64 (wave + 4 i) + lane:
            // slot L is box pixel L / 4, vector (L % 4) ^ key(pixel)
            const int L = (wave + kWaves * i) * 64 + lane;
            const int p = L / SPR, j = L - p * SPR;
            const int bz = p / plane, r = p - bz * plane;
            const int by = r / q.BW, bx = r - by * q.BW;
            const int iz = iz0 + bz, iy = iy0 + by, ix = ix0 + bx;
            const bool in = p < q.BP && (unsigned)iz < (unsigned)Dv && (unsigned)iy < (unsigned)Hv &&
                            (unsigned)ix < (unsigned)Wv;
            hoff[i] = in ? (((I.n * Dv + iz) * Hv + iy) * Wv + ix) * Cv + cg + (j ^ key(p)) * 8 : -1;
        }
    };
    // box of chunk c (of the item set above) into box buffer hbuf
    auto issue_h = [&](int c, int hbuf) {
        const unsigned base = halo_b + (unsigned)(hbuf * q.hb_bytes);
#pragma unroll
        for (int i = 0; i < kHaloLPW; ++i) {
            if (i < nhw) {
                const int o = hoff[i];
                dma16(o >= 0 ? (unsigned)(o + c * KT) * es : kOob,
                      __builtin_amdgcn_readfirstlane(base + (unsigned)((wave + kWaves * i) * 1024)), rx);
            }
        }
        issued += nhw;
        mh_last = issued;
    };
    // Item ii's BN bias values go to LDS by the same direct loads (wave 0,
    // one instruction, block ii % 3), one item ahead, so no global load
    // result has to be waited for by a full vmcnt(0) drain.
    int mb_last = 0;            // mark of the last bias block issued (wave 0)
    auto issue_bias = [&](int ii) {
        if (!bias || wave != 0) return;
        const Item I = decode(cq, it0 + ii * itstep);
        const unsigned vo = lane < BN / 8
                                ? (unsigned)(I.g * cq.Kpg + I.nb * BN + lane * 8) * es
                                : kOob;
        dma16(vo, __builtin_amdgcn_readfirstlane(bias_b + (unsigned)((ii % 3) * 1024)), rb);
        issued += 1;
        mb_last = issued;
    };

    f32x4 acc[TPW][NTW];

    // The item's results: bias added, rounded once, 8-byte stores.
    auto finish_item = [&](int ii) {
        const Item I = decode(cq, it0 + ii * itstep);
        const int oh0 = I.rb * cq.RH, ow0 = I.cb * cq.CW;
        const char *bl = lds_c + 2 * q.hb_bytes + kWBuf * B_BYTES + (ii % 3) * 1024;
        T *yb = y + I.g * cq.Kpg + I.nb * BN + nh * NTW * 16 + 4 * kq;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int cb = (nh * NTW + nt) * 16 + 4 * kq;               // channel in the block
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (bias) {
                const uint2 braw = *reinterpret_cast<const uint2 *>(bl + cb * (int)sizeof(T));
                const T *bel = reinterpret_cast<const T *>(&braw);
#pragma unroll
                for (int i = 0; i < 4; ++i) bv[i] = to_f32(bel[i]);
            }
#pragma unroll
            for (int tm = 0; tm < TPW; ++tm) {
                // the lane's pixel in the item, recomputed here per item
                const int m = (tbase + tm) * 16 + l16;
                const int RHv = cq.RH, CWv = cq.CW;
                const int lr = m / CWv, lc = m - lr * CWv;
                const int oh = oh0 + lr, ow = ow0 + lc;
                if (tm < my_tiles && lr < RHv && oh < cq.Ho && ow < cq.Wo) {
                    T o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(acc[tm][nt][i] + bv[i]);
                    const size_t pix = ((size_t)(I.n * cq.Do + I.od) * cq.Ho + oh) * cq.Wo + ow;
                    *reinterpret_cast<uint2 *>(yb + pix * cq.K + nt * 16) = *reinterpret_cast<const uint2 *>(o);
                }
            }
        }
    };

    // ---- prologue: first item's bias, first chunk's box, weight stages
    // 0 .. kWBuf-2 (stage s issues stage s + kWBuf - 1)
    issue_bias(0);
    int mb_cur = mb_last, mb_nxt = 0;   // bias of the current item, of the next
    set_box_item(0);
    issue_h(0, 0);
    int mh_cur = mh_last, mh_nxt = 0;   // box of the current chunk, of the next
    int mw0 = 0, mw1 = 0, mw2 = 0;      // weight stages s, s+1, s+2
#pragma unroll
    for (int i = 0; i < kWBuf - 1; ++i) {
        int m = 0;
        if (w_next < S) {
            prep_w();
#pragma unroll
            for (int j = 0; j < B_LPW; ++j) issue_w1(j);
            finish_w();
            m = w_last;
        }
        if (i == 0) mw0 = m;
        else if (i == 1) mw1 = m;
        else mw2 = m;
    }

    int s = 0, kx = 0, ky = 0, kz = 0, wb = 0;
    for (int ii = 0; ii < nI; ++ii) {
#pragma unroll
        for (int a = 0; a < TPW; ++a)
#pragma unroll
            for (int b = 0; b < NTW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < q.nch; ++c) {
            const int h = ii * q.nch + c;
            for (int tp = 0; tp < q.taps; ++tp, ++s) {
                const bool last = tp == q.taps - 1 && c == q.nch - 1;
                // This wave's loads of stage s's weights and box (and, in an
                // item's last stage, of its bias) are in when no more than
                // the loads issued after the latest of them remain; the
                // barrier publishes every wave's loads.  It also ends every
                // wave's MFMAs of stage s-1, whose fragments were read before
                // them: the buffers stage s-1 used are free below.
                {
                    int need = mw0 > mh_cur ? mw0 : mh_cur;
                    if (last && mb_cur > need) need = mb_cur;
                    vm_wait(issued - need);
                    __syncthreads();
                }
                // loads that run ahead: at a chunk's first stage the next
                // chunk's box (into the buffer of chunk h-1), at an item's
                // first stage the next item's bias, and weight stage
                // s + kWBuf - 1 (into the buffer of stage s-1, between MFMAs)
                if (tp == 0 && h + 1 < nH) {
                    if (c + 1 < q.nch) {
                        issue_h(c + 1, (h + 1) & 1);
                    } else {
                        set_box_item(ii + 1);
                        issue_h(0, (h + 1) & 1);
                    }
                    mh_nxt = mh_last;
                }
                if (tp == 0 && c == 0 && ii + 1 < nI) {
                    issue_bias(ii + 1);
                    mb_nxt = mb_last;
                }
                const bool more_w = w_next < S;
                if (more_w) prep_w();

                // fragments of stage s
                const int tpx = (kz * q.dd * q.BH + ky * q.dh) * q.BW + kx * q.dw;
                const char *wbp = lds_c + 2 * q.hb_bytes + wb * B_BYTES;
                const char *hbp = lds_c + (h & 1) * q.hb_bytes;
                V wf[NTW], xf[TPW];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const uint4 raw = *reinterpret_cast<const uint4 *>(wbp + boff0 + nt * 1024);
                    wf[nt] = *reinterpret_cast<const V *>(&raw);
                }
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm) {
                    const int P = apos[tm] + tpx;
                    const uint4 raw = *reinterpret_cast<const uint4 *>(
                        hbp + (unsigned)(P * SPR + (kq ^ key(P))) * 16u);
                    xf[tm] = *reinterpret_cast<const V *>(&raw);
                }
                // MFMAs; weight load i goes out after tile i so its issue
                // hides under the matrix pipe
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm) {
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) acc[tm][nt] = Mfma<T>::run(wf[nt], xf[tm], acc[tm][nt]);
                    if (tm < B_LPW && more_w) issue_w1(tm);
                }
                if (more_w) finish_w();
                mw0 = mw1;
                mw1 = mw2;
                mw2 = more_w ? w_last : 0;

                if (++wb == kWBuf) wb = 0;
                if (++kx == q.X) {
                    kx = 0;
                    if (++ky == q.Y) {
                        ky = 0;
                        ++kz;
                    }
                }
            }
            kx = ky = kz = 0;
            mh_cur = mh_nxt;
        }
        finish_item(ii);
        mb_cur = mb_nxt;
    }
}

// ----------------------------------------------------------------- host side

struct Config {
    int NTW, TPW;
    int RH, CW, nrb, ncb, nnb;
    int BD, BH, BW, BP, HI, MT;
    int items, nch, taps, grid, xcd_split;
    int hb_bytes, lds;
};

bool configure(const Problem &p, Config &c)
{
    if (p.dtype != GCONV_F16 && p.dtype != GCONV_BF16) return false;
    // a stage is one tap x 32 input channels; a channel block is 64 or 128
    if (p.Cpg % 32 != 0 || p.Kpg % 64 != 0) return false;
    const long long xb = (long long)p.N * p.D * p.H * p.W * p.C() * 2;
    const long long wb = (long long)p.K() * p.taps() * p.Cpg * 2;
    if (xb >= (1LL << 31) || wb >= (1LL << 31)) return false;
    constexpr int KT = 32, SPR = KT / 8;
    c.NTW = p.Kpg % 128 == 0 ? 4 : 2;
    const int BN = 32 * c.NTW;
    const int b_bytes = BN * SPR * 16;
    c.nnb = p.Kpg / BN;
    c.nch = p.Cpg / KT;
    c.taps = p.taps();
    c.BD = (p.Z - 1) * p.dd + 1;
    if (c.BD > 255) return false;
    // Pick the item shape (RH rows x CW columns of output) that minimises the
    // MFMA time: rounds of items over the workgroup slots (two per CU when
    // the LDS fits half a CU, else one) x tiles per wave, then the input box
    // overhead; the box must fit two box buffers next to the weight stages.
    bool found = false;
    double best = 0.0;
    for (int CW = p.Wo < kMaxTiles * 16 ? p.Wo : kMaxTiles * 16; CW >= 1; --CW) {
        int RH = kMaxTiles * 16 / CW;
        if (RH > p.Ho) RH = p.Ho;
        for (; RH >= 1; --RH) {
            const int M = RH * CW;
            const int MT = (M + 15) / 16;
            if (MT > kMaxTiles) continue;
            const int BH = (RH - 1) * p.sh + (p.Y - 1) * p.dh + 1;
            const int BW = (CW - 1) * p.sw + (p.X - 1) * p.dw + 1;
            if (BH > 1023 || BW > 1023) continue;
            const long long BP = (long long)c.BD * BH * BW;
            const long long HI = (BP * SPR + 63) / 64;
            if (HI > kMaxHaloInstr) continue;
            const long long hb = HI * 1024;
            const long long lds = 2 * hb + kWBuf * b_bytes + kBiasBytes + kColdBytes;
            if (lds > kMaxLds) continue;
            const int per_cu = lds <= kMaxLds / 2 ? 2 : 1;
            const long long slots = (long long)kCUs * per_cu;
            const long long nrb = (p.Ho + RH - 1) / RH, ncb = (p.Wo + CW - 1) / CW;
            const long long items = (long long)p.G * c.nnb * p.N * p.Do * nrb * ncb;
            if (items >= (1LL << 30)) continue;
            const long long grid = items < slots ? items : slots;
            const long long rounds = (items + grid - 1) / grid;
            const int tpw = (MT + 1) / 2 <= 4 ? 4 : 7;
            // per-SIMD MFMA work: rounds x waves per SIMD x tiles per wave
            const double t_mfma = (double)rounds * per_cu * tpw;
            const double useful = (double)p.N * p.Do * p.Ho * p.Wo * p.G * c.nnb / (double)kCUs;
            const double box_over = (double)BP / (M * (double)p.sh * p.sw);
            const double score = useful / t_mfma / (0.9 + 0.1 * box_over);
            if (!found || score > best) {
                found = true;
                best = score;
                c.RH = RH; c.CW = CW; c.nrb = (int)nrb; c.ncb = (int)ncb; c.TPW = tpw;
                c.BH = BH; c.BW = BW; c.BP = (int)BP; c.HI = (int)HI; c.MT = MT;
                c.items = (int)items; c.grid = (int)grid; c.hb_bytes = (int)hb;
                c.lds = (int)lds;
            }
        }
    }
    if (!found) return false;
    c.xcd_split = c.grid % 8 == 0 ? 1 : 0;
    return true;
}

template <typename T, int NTW, int TPW>
hipError_t go3(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    Params q;
    q.N = p.N; q.G = p.G; q.Cpg = p.Cpg; q.Kpg = p.Kpg; q.C = p.C(); q.K = p.K();
    q.D = p.D; q.H = p.H; q.W = p.W; q.Do = p.Do; q.Ho = p.Ho; q.Wo = p.Wo;
    q.Z = p.Z; q.Y = p.Y; q.X = p.X;
    q.sd = p.sd; q.sh = p.sh; q.sw = p.sw; q.pd = p.pd; q.ph = p.ph; q.pw = p.pw;
    q.dd = p.dd; q.dh = p.dh; q.dw = p.dw;
    q.RH = c.RH; q.CW = c.CW; q.nrb = c.nrb; q.ncb = c.ncb; q.nnb = c.nnb;
    q.BD = c.BD; q.BH = c.BH; q.BW = c.BW; q.BP = c.BP; q.HI = c.HI; q.MT = c.MT;
    q.items = c.items; q.nch = c.nch; q.taps = c.taps; q.xcd_split = c.xcd_split;
    q.hb_bytes = c.hb_bytes;
    q.x_bytes = (unsigned)((long long)p.N * p.D * p.H * p.W * p.C() * 2);
    q.w_bytes = (unsigned)((long long)p.K() * p.taps() * p.Cpg * 2);
    auto k = kernel<T, NTW, TPW>;
    static std::atomic<unsigned long long> lds_set{0};
    const hipError_t e = allow_lds((const void *)k, lds_set, kMaxLds);
    if (e != hipSuccess) return e;
    return enqueue(k, dim3(c.grid), dim3(kBlock), c.lds, s, a, q, (const T *)a.x, (const T *)a.w,
                   (const T *)a.bias, (T *)a.y);
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    if (c.NTW == 4) return c.TPW == 7 ? go3<T, 4, 7>(p, c, a, s) : go3<T, 4, 4>(p, c, a, s);
    return c.TPW == 7 ? go3<T, 2, 7>(p, c, a, s) : go3<T, 2, 4>(p, c, a, s);
}

}  // namespace

// tile menu: the whole-box variant (where it applies), then the
// chunk-streaming one (where it applies); the own pick is the first
bool use_box(const Problem &p)
{
    if (!ighalo_box::supported(p)) return false;
    const int t = tile_choice();
    Config c;
    return !(t == 1 && configure(p, c));
}

bool supported(const Problem &p)
{
    Config c;
    return ighalo_box::supported(p) || configure(p, c);
}

int tiles(const Problem &p, int *picked)
{
    Config c;
    *picked = 0;
    return (ighalo_box::supported(p) ? 1 : 0) + (configure(p, c) ? 1 : 0);
}

gconv_plan plan(const Problem &p)
{
    if (use_box(p)) return ighalo_box::plan(p);
    Config c;
    configure(p, c);
    gconv_plan pl{};
    pl.path = GCONV_PATH_IGHALO;
    pl.grid[0] = (uint32_t)c.grid;
    pl.grid[1] = 1;
    pl.grid[2] = 1;
    pl.block = kBlock;
    pl.lds_bytes = (uint32_t)c.lds;
    pl.groups_per_tile = 1;
    return pl;
}

hipError_t launch(const Problem &p, const Args &a, hipStream_t s)
{
    if (use_box(p)) return ighalo_box::launch(p, a, s);
    Config c;
    if (!configure(p, c)) return hipErrorInvalidValue;
    if (p.dtype == GCONV_F16) return go<_Float16>(p, c, a, s);
    return go<__bf16>(p, c, a, s);
}

}  // namespace ighalo
}  // namespace gconv

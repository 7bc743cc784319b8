// Halo-staged implicit GEMM for groups with many channels (fp16 / bf16, 2D
// and 3D, Cpg % 64 == 0, Kpg % 64 == 0), persistent and XCD-aware.
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
// Pipelines, both filled by direct-to-LDS buffer loads (zero fill for
// padding from the buffer range check):
//   - input box: two chunk buffers; the next chunk's box (the next item's
//     first chunk at an item's end) is loaded while the current one is used;
//   - weights: four stage buffers; stage s+3 is loaded while s is used.
// One barrier per stage.  Every wave waits only for its own loads with an
// explicit s_waitcnt vmcnt (loads return in order), then the barrier makes
// all waves' loads visible.  The MFMA fragments of stage s+1 are read from
// LDS while the MFMAs of stage s run, so LDS latency and bandwidth overlap
// the matrix pipe.
//
// Four waves split the item 2 (pixels) x 2 (channels).  Each computes up to
// 7 x NTW tiles of v_mfma_f32_16x16x32 with the weights as the first operand,
// so each lane ends with four adjacent output channels of one pixel.  The
// epilogue of an item (bias, one rounding, 8-byte stores) runs at the start
// of the next item's first stage, after that stage's wait, so the stores
// overlap the next item's first MFMAs instead of delaying its loads.
//
// Grid: one workgroup per CU (the LDS reservation is above half a CU's LDS),
// at most 256 workgroups, each looping over its items.  Items are ordered
// group-major and each XCD (workgroup id mod 8 under the round-robin
// dispatch) takes one contiguous eighth of them, so an XCD's L2 holds the
// weights of about G/8 groups.
#include <type_traits>

#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace ighalo {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = 4;
constexpr int kMaxTiles = 14;         // M tiles (16 pixels) per item
constexpr int kMaxHaloInstr = 64;      // halo DMA instructions per chunk
constexpr int kHaloLPW = kMaxHaloInstr / kWaves;
constexpr int kGrid = 256;
constexpr int kMinLds = 82 * 1024;     // > half of 160 KB: one workgroup per CU
constexpr int kMaxLds = 160 * 1024;
constexpr int kBiasBytes = 3 * 1024;   // three 1 KB bias blocks
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

// s_waitcnt vmcnt(n) for a wave-uniform n (other counters not waited on).
__device__ __forceinline__ void vm_wait(int n)
{
#define GCONV_VMW(k) \
    case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (7 << 4) | (15 << 8) | (((k) >> 4) << 14)); break;
    switch (__builtin_amdgcn_readfirstlane(n)) {
        GCONV_VMW(1) GCONV_VMW(2) GCONV_VMW(3) GCONV_VMW(4) GCONV_VMW(5) GCONV_VMW(6)
        GCONV_VMW(7) GCONV_VMW(8) GCONV_VMW(9) GCONV_VMW(10) GCONV_VMW(11) GCONV_VMW(12)
        GCONV_VMW(13) GCONV_VMW(14) GCONV_VMW(15) GCONV_VMW(16) GCONV_VMW(17) GCONV_VMW(18)
        GCONV_VMW(19) GCONV_VMW(20) GCONV_VMW(21) GCONV_VMW(22) GCONV_VMW(23) GCONV_VMW(24)
        GCONV_VMW(25) GCONV_VMW(26) GCONV_VMW(27) GCONV_VMW(28) GCONV_VMW(29) GCONV_VMW(30)
        GCONV_VMW(31) GCONV_VMW(32)
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;   // vmcnt(0)
    }
#undef GCONV_VMW
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
// addressing), held in VGPRs: the scalar register file is kept for the
// per-stage state, and these are per-lane address arithmetic anyway.
struct Cold {
    int N, Do, Ho, Wo, D, H, W, C, K, Kpg, Cpg, sd, sh, sw, pd, ph, pw, RH, CW, ncb, nrb, nnb;
};

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

// KT: input channels per chunk (64: two MFMA K steps); NTW: 16-channel N tiles per wave
// (the item's channel block is BN = 32 * NTW); TPW: M tiles per wave (the
// item has at most 2 TPW).  Every wave runs all TPW tiles without branches;
// tiles past the item's end read box pixel 0 and are not stored.
//
// LDS rows (a box pixel's KT channels, or a weight row's KT channels) are
// SPR = KT/8 slots of 16 bytes with no padding; slot j of row r holds
// channel vector j ^ key(r).  The XOR swizzle is applied when the row is
// loaded (direct-to-LDS loads write each lane's 16 bytes at a fixed place,
// so the lane picks which global vector to fetch), and it keeps the 16-byte
// fragment reads of consecutive rows in distinct banks.
template <typename T, int KT, int NTW, int TPW>
__global__ __launch_bounds__(kBlock, 1) void kernel(Params q, const T *__restrict__ x,
                                                    const T *__restrict__ w,
                                                    const T *__restrict__ bias, T *__restrict__ y)
{
    typedef typename Mfma<T>::V V;
    constexpr int SPR = KT / 8;               // 16-byte slots per staged row
    constexpr int KS = KT / 32;               // MFMA K steps per stage
    constexpr int BN = 2 * NTW * 16;
    constexpr int B_INSTR = BN * SPR / 64;    // load instructions per weight stage
    static_assert(B_INSTR % kWaves == 0, "weight stage loads split evenly over the waves");
    constexpr int B_LPW = B_INSTR / kWaves;
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

    auto key = [](int r) { return SPR == 8 ? (r & 7) : ((r >> 1) & 3); };

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
    Cold cq;
    cq.N = in_vgpr(q.N); cq.Do = in_vgpr(q.Do); cq.Ho = in_vgpr(q.Ho); cq.Wo = in_vgpr(q.Wo);
    cq.D = in_vgpr(q.D); cq.H = in_vgpr(q.H); cq.W = in_vgpr(q.W); cq.C = in_vgpr(q.C);
    cq.K = in_vgpr(q.K); cq.Kpg = in_vgpr(q.Kpg); cq.Cpg = in_vgpr(q.Cpg);
    cq.sd = in_vgpr(q.sd); cq.sh = in_vgpr(q.sh); cq.sw = in_vgpr(q.sw);
    cq.pd = in_vgpr(q.pd); cq.ph = in_vgpr(q.ph); cq.pw = in_vgpr(q.pw);
    cq.RH = in_vgpr(q.RH); cq.CW = in_vgpr(q.CW);
    cq.ncb = in_vgpr(q.ncb); cq.nrb = in_vgpr(q.nrb); cq.nnb = in_vgpr(q.nnb);

    // ---- per-lane load plans (fixed for the whole kernel).  Instruction
    // k = wave + 4 i of a buffer fills its slots 64k .. 64k+63.
    int wofs[B_LPW];     // weights: element offset of this lane's vector within the block's rows
#pragma unroll
    for (int i = 0; i < B_LPW; ++i) {
        const int L = (wave + kWaves * i) * 64 + lane;
        const int row = L / SPR, j = L - row * SPR;
        wofs[i] = row * q.taps * q.Cpg + (j ^ key(row)) * 8;
    }
    int hpack[kHaloLPW];  // box: packed (bz, by, bx, vector), -1 past the box
    int nhw = 0;
#pragma unroll
    for (int i = 0; i < kHaloLPW; ++i) {
        const int k = wave + kWaves * i;
        hpack[i] = -1;
        if (k < q.HI) {
            nhw = i + 1;
            const int L = k * 64 + lane;
            const int p = L / SPR, j = L - p * SPR;
            if (p < q.BP) {
                const int plane = q.BH * q.BW;
                const int bz = p / plane, r = p - bz * plane;
                const int by = r / q.BW, bx = r - by * q.BW;
                hpack[i] = (bz << 23) | (by << 13) | (bx << 3) | (j ^ key(p));
            }
        }
    }

    // ---- fragment addressing
    // A: tile tm of this wave = item tile T = mh * ta + tm; lane pixel m = 16 T + l16
    const int ta = (q.MT + 1) >> 1;
    const int my_tiles = mh == 0 ? ta : q.MT - ta;
    const int tbase = mh * ta;     // ta <= TPW
    int apos[TPW];                 // the pixel's row in the box (before the tap shift)
    int pix_rc[TPW];               // pixel's row << 16 | column in the item, -1 = padding lane
#pragma unroll
    for (int tm = 0; tm < TPW; ++tm) {
        const int m = (tbase + tm) * 16 + l16;
        const int lr = m / q.CW, lc = m - lr * q.CW;
        const bool live = tm < my_tiles && lr < q.RH;
        pix_rc[tm] = live ? (lr << 16) | lc : -1;
        apos[tm] = live ? lr * q.sh * q.BW + lc * q.sw : 0;
    }
    unsigned boff[NTW];            // B: byte offset of this lane's first K-step vector
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int r = (nh * NTW + nt) * 16 + l16;
        boff[nt] = (unsigned)(r * SPR + (kq ^ key(r))) * 16u;
    }
    // K step ks of a row is slot (kq + 4 ks) ^ key = (kq ^ key) ^ 4 ks: byte offset ^ 64 ks
    auto read_frags = [&](V (&wf)[KS][NTW], V (&xf)[KS][TPW], int hbuf, int wbuf, int tpx) {
        const char *wb = lds_c + 2 * q.hb_bytes + wbuf * B_BYTES;
        const char *hb = lds_c + hbuf * q.hb_bytes;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(wb + (boff[nt] ^ (unsigned)(64 * ks)));
                wf[ks][nt] = *reinterpret_cast<const V *>(&raw);
            }
#pragma unroll
        for (int tm = 0; tm < TPW; ++tm) {
            const int P = apos[tm] + tpx;
            const unsigned a0 = (unsigned)(P * SPR + (kq ^ key(P))) * 16u;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(hb + (a0 ^ (unsigned)(64 * ks)));
                xf[ks][tm] = *reinterpret_cast<const V *>(&raw);
            }
        }
    };

    // ---- stage sequence: item ii (local), chunk c, tap tp; stage s, chunk
    // h = ii * nch + c.  A stage is two K steps of 32 (KT = 64).
    static_assert(KS == 2, "a stage is two K steps");
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
        const int rowbase = w_row + w_tp * cq.Cpg + w_c * KT;
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
    int mh_next = 0;            // mark of the last box issued
    auto issue_h = [&](int h) {
        const int c = h % q.nch;
        const int ii = h / q.nch;
        const Item I = decode(cq, it0 + ii * itstep);
        const int iz0 = I.od * cq.sd - cq.pd;
        const int iy0 = I.rb * cq.RH * cq.sh - cq.ph;
        const int ix0 = I.cb * cq.CW * cq.sw - cq.pw;
        const int cbase = I.g * cq.Cpg + c * KT;
        const unsigned base = halo_b + (unsigned)((h & 1) * q.hb_bytes);
#pragma unroll
        for (int i = 0; i < kHaloLPW; ++i) {
            if (i < nhw) {
                unsigned vo = kOob;
                int pk = hpack[i];
                // opaque to the optimiser: the unpacked fields are recomputed
                // here, once per chunk, instead of being held live in
                // registers across the whole stage loop
                asm volatile("" : "+v"(pk));
                if (pk >= 0) {
                    const int iz = iz0 + (pk >> 23), iy = iy0 + ((pk >> 13) & 1023),
                              ix = ix0 + ((pk >> 3) & 1023);
                    if (iz >= 0 && iz < cq.D && iy >= 0 && iy < cq.H && ix >= 0 && ix < cq.W)
                        vo = ((unsigned)(((I.n * cq.D + iz) * cq.H + iy) * cq.W + ix) * (unsigned)cq.C +
                              (unsigned)(cbase + (pk & 7) * 8)) * es;
                }
                dma16(vo, __builtin_amdgcn_readfirstlane(base + (unsigned)((wave + kWaves * i) * 1024)), rx);
            }
        }
        issued += nhw;
        mh_next = issued;
    };
    // Item ii's BN bias values go to LDS by the same direct loads (wave 0,
    // one instruction, block ii % 3), one item ahead, so no global load
    // result has to be waited for by a full vmcnt(0) drain.
    int mb_next = 0;            // mark of the last bias block issued (wave 0)
    auto issue_bias = [&](int ii) {
        if (!bias || wave != 0) return;
        const Item I = decode(cq, it0 + ii * itstep);
        const unsigned vo = lane < BN / 8
                                ? (unsigned)(I.g * cq.Kpg + I.nb * BN + lane * 8) * es
                                : kOob;
        dma16(vo, __builtin_amdgcn_readfirstlane(bias_b + (unsigned)((ii % 3) * 1024)), rb);
        issued += 1;
        mb_next = issued;
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
                // opaque: address arithmetic is redone per item, not held live
                const int rc = in_vgpr(pix_rc[tm]);
                const int oh = oh0 + (rc >> 16), ow = ow0 + (rc & 0xffff);
                if (rc >= 0 && oh < cq.Ho && ow < cq.Wo) {
                    T o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(acc[tm][nt][i] + bv[i]);
                    const size_t pix = ((size_t)(I.n * cq.Do + I.od) * cq.Ho + oh) * cq.Wo + ow;
                    *reinterpret_cast<uint2 *>(yb + pix * cq.K + nt * 16) = *reinterpret_cast<const uint2 *>(o);
                }
            }
        }
    };

    // ---- fragment sets: one K step of this wave's B (NTW) and A (TPW)
    // vectors.  Set 0 holds K step 0 of a stage, set 1 K step 1; each is read
    // while the other one multiplies.
    V wf0[NTW], xf0[TPW], wf1[NTW], xf1[TPW];
    auto read_step = [&](V (&wfs)[NTW], V (&xfs)[TPW], int hbuf, int wbuf, int tpx, int ks) {
        const char *wb = lds_c + 2 * q.hb_bytes + wbuf * B_BYTES;
        const char *hb = lds_c + hbuf * q.hb_bytes;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(wb + (boff[nt] ^ (unsigned)(64 * ks)));
            wfs[nt] = *reinterpret_cast<const V *>(&raw);
        }
#pragma unroll
        for (int tm = 0; tm < TPW; ++tm) {
            const int P = apos[tm] + tpx;
            const unsigned a0 = (unsigned)(P * SPR + (kq ^ key(P))) * 16u;
            const uint4 raw = *reinterpret_cast<const uint4 *>(hb + (a0 ^ (unsigned)(64 * ks)));
            xfs[tm] = *reinterpret_cast<const V *>(&raw);
        }
    };
    // MFMAs of one K step; weight load i of the stage being issued (if any)
    // goes out after tile i, so its issue hides under the matrix pipe
    auto mfma_step = [&](V (&wfs)[NTW], V (&xfs)[TPW], bool with_w) {
#pragma unroll
        for (int tm = 0; tm < TPW; ++tm) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) acc[tm][nt] = Mfma<T>::run(wfs[nt], xfs[tm], acc[tm][nt]);
            if (tm < B_LPW && with_w) issue_w1(tm);
        }
    };

    // ---- prologue: first item's bias, first chunk's box, weight stages
    // 0 .. kWBuf-1; stage 0's first K step; then the loads a first stage of
    // a chunk and of an item issue (next chunk's box, next item's bias)
    issue_bias(0);
    const int mb0 = mb_next;
    issue_h(0);
    const int mh0 = mh_next;
    int mw0 = 0, mw1 = 0, mw2 = 0;      // marks of weight stages next, next+1, next+2
    int mw3 = 0;
#pragma unroll
    for (int i = 0; i < kWBuf; ++i) {
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
        else if (i == 2) mw2 = m;
        else mw3 = m;
    }
    {
        int need = mw0 > mh0 ? mw0 : mh0;
        if (SPI == 1 && mb0 > need) need = mb0;
        vm_wait(issued - need);
        __syncthreads();
        read_step(wf0, xf0, 0, 0, 0, 0);
    }
    mw0 = mw1;          // from here on the marks describe stage 1 onwards
    mw1 = mw2;
    mw2 = mw3;
    if (1 < nH) issue_h(1);
    if (1 < nI) issue_bias(1);

    // Cursors: current stage s (tap offset cur_tpx, box buffer cur_hb,
    // weight buffer cur_wb) and next stage s+1 (n_*).
    int cur_tpx = 0, cur_hb = 0, cur_wb = 0;
    int n_ii = 0, n_c = 0, n_tp = 0, n_kx = 0, n_ky = 0, n_kz = 0, n_wb = 0;
    // mark bookkeeping: box of the next stage's chunk and of the chunk after
    // it, bias of the next stage's item and of the item after it
    int mh_for_next = mh0, mb_for_next = mb0;
    int mh_pending = 1 < nH ? mh_next : 0, mb_pending = 1 < nI ? mb_next : 0;
    auto advance_n = [&]() {
        if (++n_wb == kWBuf) n_wb = 0;
        if (++n_kx == q.X) {
            n_kx = 0;
            if (++n_ky == q.Y) {
                n_ky = 0;
                ++n_kz;
            }
        }
        if (++n_tp == q.taps) {
            n_tp = 0;
            n_kx = n_ky = n_kz = 0;
            mh_for_next = mh_pending;
            mh_pending = 0;
            if (++n_c == q.nch) {
                n_c = 0;
                ++n_ii;
                mb_for_next = mb_pending;
                mb_pending = 0;
            }
        }
    };
    advance_n();   // next = stage 1

    int s = 0;
    for (int ii = 0; ii < nI; ++ii) {
#pragma unroll
        for (int a = 0; a < TPW; ++a)
#pragma unroll
            for (int b = 0; b < NTW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < SPI; ++j, ++s) {
            // step A: K step 1 of stage s into set 1; MFMAs of K step 0
            read_step(wf1, xf1, cur_hb, cur_wb, cur_tpx, 1);
            mfma_step(wf0, xf0, false);

            // step B: stage s+1 becomes readable; its first K step into set 0;
            // MFMAs of K step 1 with the weight loads that run ahead
            bool more_w = false;
            const bool have_next = s + 1 < S;
            const bool next_ends_item = n_tp == q.taps - 1 && n_c == q.nch - 1;
            {
                // stage s+1's weights and box, and, if it ends its item, the
                // item's bias: this wave's loads are in when no more than the
                // loads issued after the latest of them remain.  The fragment
                // reads of stage s are complete too (lgkmcnt(0)), so after the
                // barrier every buffer stage s used is free.
                int need = 0;
                if (have_next) {
                    need = mw0 > mh_for_next ? mw0 : mh_for_next;
                    if (next_ends_item && mb_for_next > need) need = mb_for_next;
                }
                __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
                vm_wait(issued - need);
                __syncthreads();
            }
            if (have_next) {
                // loads that run ahead: at the first stage of a chunk the
                // chunk after it; at an item's first stage the next item's
                // bias; weight stage s+1+kWBuf-1 into the buffer of stage s
                const int nh_ = n_ii * q.nch + n_c;
                if (n_tp == 0 && nh_ + 1 < nH) {
                    issue_h(nh_ + 1);
                    mh_pending = mh_next;
                }
                if (n_tp == 0 && n_c == 0 && n_ii + 1 < nI) {
                    issue_bias(n_ii + 1);
                    mb_pending = mb_next;
                }
                more_w = w_next < S;
                if (more_w) prep_w();
                const int n_tpx = (n_kz * q.dd * q.BH + n_ky * q.dh) * q.BW + n_kx * q.dw;
                read_step(wf0, xf0, nh_ & 1, n_wb, n_tpx, 0);
                cur_tpx = n_tpx;
                cur_hb = nh_ & 1;
                cur_wb = n_wb;
            }
            mfma_step(wf1, xf1, more_w);
            if (more_w) finish_w();
            mw0 = mw1;
            mw1 = mw2;
            mw2 = more_w ? w_last : 0;
            advance_n();
        }
        finish_item(ii);
    }
}

// ----------------------------------------------------------------- host side

struct Config {
    int KT, NTW, TPW;
    int RH, CW, nrb, ncb, nnb;
    int BD, BH, BW, BP, HI, MT;
    int items, nch, taps, grid, xcd_split;
    int hb_bytes, lds;
};

bool configure(const Problem &p, Config &c)
{
    if (p.dtype != GCONV_F16 && p.dtype != GCONV_BF16) return false;
    // a stage is one tap x 64 input channels (two MFMA K steps)
    if (p.Cpg % 64 != 0 || p.Kpg % 64 != 0) return false;
    const long long xb = (long long)p.N * p.D * p.H * p.W * p.C() * 2;
    const long long wb = (long long)p.K() * p.taps() * p.Cpg * 2;
    if (xb >= (1LL << 31) || wb >= (1LL << 31)) return false;
    c.KT = 64;
    c.NTW = p.Kpg % 128 == 0 ? 4 : 2;
    const int BN = 32 * c.NTW;
    const int SPR = c.KT / 8;
    const int b_bytes = BN * SPR * 16;
    c.nnb = p.Kpg / BN;
    c.nch = p.Cpg / c.KT;
    c.taps = p.taps();
    c.BD = (p.Z - 1) * p.dd + 1;
    if (c.BD > 255) return false;
    // Pick the item shape (RH rows x CW columns of output) that minimises the
    // MFMA time: rounds of items over the grid x tiles per wave, then the
    // input box overhead; the box must fit two box buffers next to the
    // weight stage buffers.
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
            if (2 * hb + kWBuf * b_bytes + kBiasBytes > kMaxLds) continue;
            const long long nrb = (p.Ho + RH - 1) / RH, ncb = (p.Wo + CW - 1) / CW;
            const long long items = (long long)p.G * c.nnb * p.N * p.Do * nrb * ncb;
            if (items >= (1LL << 30)) continue;
            const long long grid = items < kGrid ? items : kGrid;
            const long long rounds = (items + grid - 1) / grid;
            const int tpw = (MT + 1) / 2 <= 4 ? 4 : 7;
            const double t_mfma = (double)rounds * tpw * 16.0;   // per-wave pixel rows
            const double useful = (double)p.N * p.Do * p.Ho * p.Wo * p.G * c.nnb / grid;
            const double box_over = (double)BP / (M * (double)p.sh * p.sw);
            const double score = useful / t_mfma / (0.9 + 0.1 * box_over);
            if (!found || score > best) {
                found = true;
                best = score;
                c.RH = RH; c.CW = CW; c.nrb = (int)nrb; c.ncb = (int)ncb; c.TPW = tpw;
                c.BH = BH; c.BW = BW; c.BP = (int)BP; c.HI = (int)HI; c.MT = MT;
                c.items = (int)items; c.grid = (int)grid; c.hb_bytes = (int)hb;
            }
        }
    }
    if (!found) return false;
    c.xcd_split = c.grid % 8 == 0 ? 1 : 0;
    c.lds = 2 * c.hb_bytes + kWBuf * b_bytes + kBiasBytes;
    if (c.lds < kMinLds) c.lds = kMinLds;
    return true;
}

template <typename T, int KT, int NTW, int TPW>
hipError_t go4(const Problem &p, const Config &c, const Args &a, hipStream_t s)
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
    auto k = kernel<T, KT, NTW, TPW>;
    static bool lds_set = false;
    if (!lds_set) {
        (void)hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        lds_set = true;
    }
    return enqueue(k, dim3(c.grid), dim3(kBlock), c.lds, s, a, q, (const T *)a.x, (const T *)a.w,
                   (const T *)a.bias, (T *)a.y);
}

template <typename T, int KT, int NTW>
hipError_t go3(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    return c.TPW == 7 ? go4<T, KT, NTW, 7>(p, c, a, s) : go4<T, KT, NTW, 4>(p, c, a, s);
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    return c.NTW == 4 ? go3<T, 64, 4>(p, c, a, s) : go3<T, 64, 2>(p, c, a, s);
}

}  // namespace

bool supported(const Problem &p)
{
    Config c;
    return configure(p, c);
}

gconv_plan plan(const Problem &p)
{
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
    Config c;
    if (!configure(p, c)) return hipErrorInvalidValue;
    if (p.dtype == GCONV_F16) return go<_Float16>(p, c, a, s);
    return go<__bf16>(p, c, a, s);
}

}  // namespace ighalo
}  // namespace gconv

// Halo implicit GEMM with the whole input box resident in LDS (fp16 / bf16,
// 2D and 3D, Cpg = 64 or 128, Kpg % 64 == 0): the variant of the halo path
// that runs when the box of every input channel of a group fits in LDS.
//
// The GEMM per group is the one of rocm-libraries PR 10064 (Technical
// Details: the group splits C into G x C/G, the weight descriptor's channel
// extent is C/G, the output channel is g * Kpg + k): M = output pixels,
// N = Kpg, K = taps x Cpg with the channel fastest.  A work item is RH x CW
// output pixels of one output plane, one group and a block of BN output
// channels.  Its input box - the block widened by the dilated filter
// footprint - is loaded once, all Cpg channels of it, into LDS; every
// (tap, 32-channel) step of the reduction then reads its pixel operand
// from the box at a shifted pixel offset, and its weight operand straight
// from global memory into registers.  The weights of a group are shared by
// every item of the group, so they are L2 (and L1) hits; they never pass
// through LDS.  The reduction loop therefore has no barrier and no explicit
// memory wait: one box load, one barrier, then taps x Cpg/32 steps of
// 16x16x32 MFMAs fed by immediate-offset LDS reads and register loads that
// run one tap ahead.
//
// Box layout: pixel-major rows of Cpg channels plus 16 bytes of padding
// (PS = 2 Cpg + 16 bytes).  Sixteen lanes read sixteen consecutive pixels at
// the same channel offset; with the 16-byte pad their addresses fall in
// distinct 16-byte bank groups.  The box is filled by direct-to-LDS buffer
// loads (each lane writes 16 bytes at M0 + 16 * lane); a lane whose slot is
// a pad slot, a padding pixel or past the box loads from past the end of the
// buffer, which returns zeros.
//
// Four waves split the item 2 (pixels) x 2 (channels); each computes up to
// TPW x NT tiles with the weights as the first MFMA operand, so a lane ends
// with four adjacent output channels of one pixel.  The epilogue adds the
// bias, rounds once and stores 8 bytes per lane.  When a workgroup has
// another item, the next box load is issued before the epilogue's stores.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace ighalo_box {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = 4;
constexpr int kCUs = 256;              // MI355X compute units
constexpr int kMaxLds = 160 * 1024;
constexpr unsigned kOob = 0x80000000u;

typedef int rsrc_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Params {
    int N, G, Cpg, Kpg, C, K;
    int D, H, W, Do, Ho, Wo, Y, X;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int RH, CW, nrb, ncb, nnb;   // item = RH x CW output pixels of one plane; blocks per axis
    int VW;                      // pixels per output row in the tile order (CW, or BW: see below)
    int BH, BW, BP;              // input box rows, columns, pixels (BD planes)
    int HI;                      // box load instructions (64 lanes x 16 bytes each)
    int MT;                      // M tiles of 16 pixels per item
    int items, taps, xcd_split;
    int nch;                     // channel chunks per group (32 CC channels each), one box each
    unsigned x_bytes, w_bytes;
    float rplane, rbw;           // 1 / (BH BW), 1 / BW
};

// n / d for 0 <= n < 2^22 from a float reciprocal of d: the estimate is off
// by at most one, which the remainder test corrects.
__device__ __forceinline__ int fdiv(int n, int d, float rd)
{
    int v = (int)((float)n * rd);
    const int r = n - v * d;
    v += r >= d ? 1 : 0;
    v -= r < 0 ? 1 : 0;
    return v;
}

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

// 16 bytes from buffer offset `voffset` to LDS M0 + 16 * lane.
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

__device__ __forceinline__ Item decode(const Params &q, int it)
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

// WM: waves along the item's pixels (1 or 2; the other 4 / WM waves split
// its channels); NT: 16-channel N tiles per wave (item channel block
// BN = 16 NT 4 / WM); TPW: M tiles per wave (the item has at most WM TPW);
// CC: 32-channel steps per tap (Cpg = 32 CC).
template <typename T, int WM, int NT, int TPW, int CC>
__global__ __launch_bounds__(kBlock, 2) void kernel(Params q, const T *__restrict__ x,
                                                    const T *__restrict__ w,
                                                    const T *__restrict__ bias, T *__restrict__ y)
{
    typedef typename Mfma<T>::V V;
    constexpr int WN = kWaves / WM;
    constexpr int BN = WN * NT * 16;
    constexpr int SPP = CC * 4 + 1;           // 16-byte slots per box pixel (last one is padding)
    constexpr int PS = SPP * 16;              // box pixel stride in bytes
    constexpr int OP = BN * (int)sizeof(T) + 16;   // staged output pixel stride in bytes
    extern __shared__ uint4 lds[];

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    const int mh = wave % WM, nh = wave / WM;
    const rsrc_t rx = make_rsrc(x, q.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)w, (short)0, (int)q.w_bytes, 0x00020000);
    const unsigned lds_b = (unsigned)(size_t)lds;
    const char *lds_c = reinterpret_cast<const char *>(lds);

    // ---- this workgroup's items: XCD-contiguous ranges when the grid is a
    // multiple of 8 (workgroup b runs on XCD b % 8)
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

    // ---- fragment addressing (fixed for the kernel)
    const int ta = (q.MT + WM - 1) / WM;
    const int my_tiles = mh == 0 ? ta : q.MT - ta;
    const int tbase = mh * ta;
    int aoff[TPW];      // byte offset of this lane's pixel (tap 0) and channel slot in the box
#pragma unroll
    for (int tm = 0; tm < TPW; ++tm) {
        const int m = (tbase + tm) * 16 + l16;
        const int lr = m / q.VW, lc = m - lr * q.VW;
        const bool live = tm < my_tiles && lr < q.RH;
        const int P = live ? lr * q.sh * q.BW + lc * q.sw : 0;
        aoff[tm] = P * PS + kq * 16;
    }
    const int kstride = q.taps * q.Cpg;                   // elements per weight row
    // this lane's weight row and channel slot within the group's channel block
    const unsigned woff_lane = (unsigned)(((nh * NT * 16 + l16) * kstride + kq * 8) * (int)sizeof(T));
    const unsigned wtile_b = (unsigned)(16 * kstride * (int)sizeof(T));   // N tile stride in bytes

    // the box of item ii, channel chunk ch: direct-to-LDS loads, instruction
    // k fills slots 64k .. 64k+63
    auto issue_box = [&](int ii, int ch) {
        const Item I = decode(q, it0 + ii * itstep);
        const int iz0 = I.od * q.sd - q.pd;
        const int iy0 = I.rb * q.RH * q.sh - q.ph;
        const int ix0 = I.cb * q.CW * q.sw - q.pw;
        const int plane = q.BH * q.BW;
        const int cg = I.g * q.Cpg + ch * 32 * CC;
        // wave-uniform loop (scalar branch); the box-pixel divisions use
        // host-computed reciprocals and one exact correction step
        for (int k = __builtin_amdgcn_readfirstlane(wave); k < q.HI; k += kWaves) {
            const int L = k * 64 + lane;
            const int p = L / SPP, j = L - p * SPP;
            const int bz = fdiv(p, plane, q.rplane), r = p - bz * plane;
            const int by = fdiv(r, q.BW, q.rbw), bx = r - by * q.BW;
            const int iz = iz0 + bz, iy = iy0 + by, ix = ix0 + bx;
            const bool in = j < SPP - 1 && p < q.BP && (unsigned)iz < (unsigned)q.D &&
                            (unsigned)iy < (unsigned)q.H && (unsigned)ix < (unsigned)q.W;
            const unsigned vo =
                in ? (unsigned)(((((I.n * q.D + iz) * q.H + iy) * q.W + ix) * q.C + cg + j * 8) *
                                (int)sizeof(T))
                   : kOob;
            dma16(vo, __builtin_amdgcn_readfirstlane(lds_b + (unsigned)(k * 1024)), rx);
        }
    };

    issue_box(0, 0);
    for (int ii = 0; ii < nI; ++ii) {
        const Item I = decode(q, it0 + ii * itstep);
        // weights of this item's channel block: a wave-uniform byte offset
        // (soffset) plus this lane's row and channel slot (voffset)
        const int wg_b = (I.g * q.Kpg + I.nb * BN) * kstride * (int)sizeof(T);
        int cho = 0;    // byte offset of the current channel chunk in a weight row's tap
        auto wload = [&](int tap, int cc, int nt) -> V {
            const int so = wg_b + nt * (int)wtile_b + (tap * q.Cpg + cc * 32) * (int)sizeof(T) + cho;
            return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)woff_lane,
                                                                               __builtin_amdgcn_readfirstlane(so), 0));
        };
        f32x4 acc[TPW][NT];
#pragma unroll
        for (int a = 0; a < TPW; ++a)
#pragma unroll
            for (int b = 0; b < NT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int ch = 0; ch < q.nch; ++ch) {
        if (ch > 0) {
            // every wave is done with the previous chunk's box
            __syncthreads();
            issue_box(ii, ch);
        }
        cho = ch * 32 * CC * (int)sizeof(T);
        // the weight fragments of one whole tap in flight: step (tap, cc)
        // uses buffer cc, refilled with (tap + 1, cc) after its MFMAs
        constexpr int NB = CC;
        V bq[NB][NT];
#pragma unroll
        for (int cc = 0; cc < NB; ++cc)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bq[cc][nt] = wload(0, cc, nt);

        // the box is in once this wave's loads are back and every wave has passed here
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        // Pixel fragments go in runs of R <= 7 tiles (bounded registers),
        // double-buffered: the next run's LDS reads are issued before this
        // run's MFMAs, so they are in flight while the matrix pipe works.
        // Within a step the order reads, MFMAs, then the weight loads for
        // a later step is kept (loads return in order: a load issued before
        // these MFMAs would have to be back before they could start).
        constexpr int R = TPW < 7 ? TPW : 7;
        constexpr int NR = (TPW + R - 1) / R;       // runs per step; CC * NR is even
        V af[2][R];
        auto read_run = [&](V *dst, int tofs_, int cc_, int r_) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(lds_c + aoff[r_ * R + i] + tofs_ + cc_ * 64);
                dst[i] = *reinterpret_cast<const V *>(&raw);
            }
        };
        int kx = 0, ky = 0, kz = 0;
        int tofs = 0;                                // tap 0 reads the box at offset 0
        read_run(af[0], 0, 0, 0);
        for (int tap = 0; tap < q.taps; ++tap) {
            const bool more = tap + 1 < q.taps;
            if (++kx == q.X) {
                kx = 0;
                if (++ky == q.Y) {
                    ky = 0;
                    ++kz;
                }
            }
            // the next tap's offset (the last tap re-reads its own: in
            // bounds, unused; a branch would make the wait counts at the
            // join conservative)
            const int tofs_n = more ? ((kz * q.dd * q.BH + ky * q.dh) * q.BW + kx * q.dw) * PS : tofs;
#pragma unroll
            for (int cc = 0; cc < CC; ++cc) {
                const int b = cc % NB;
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const int cur = (cc * NR + r) & 1;
                    if (r + 1 < NR) read_run(af[cur ^ 1], tofs, cc, r + 1);
                    else if (cc + 1 < CC) read_run(af[cur ^ 1], tofs, cc + 1, 0);
                    else read_run(af[cur ^ 1], tofs_n, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < R; ++i)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[r * R + i][nt] = Mfma<T>::run(bq[b][nt], af[cur][i], acc[r * R + i][nt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // step s + NB: same tap while cc + NB < CC, else the next tap
                // (unconditional: past the last tap it reloads the last
                // tap's weights, in bounds and unused)
                const int ncc = cc + NB < CC ? cc + NB : cc + NB - CC;
                const bool nxt_tap = cc + NB >= CC;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bq[b][nt] = wload(nxt_tap && more ? tap + 1 : tap, ncc, nt);
                __builtin_amdgcn_sched_barrier(0);
            }
            tofs = tofs_n;
        }
        }   // channel chunks

        // The results leave through LDS (the box is dead once every wave is
        // past the loop): each lane drops its four channels (bias added,
        // rounded once) of each of its pixels into a staging row per pixel,
        // then the workgroup writes whole BN-channel pixel runs with one
        // 16-byte non-temporal store per thread and chunk - full lines
        // instead of 8-byte pieces of 16 pixels.
        __syncthreads();
        const int kb = I.g * q.Kpg + I.nb * BN;
        {
            const int cw = nh * NT * 16 + 4 * kq;    // this lane's channel in the block
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float bv[4] = {0.f, 0.f, 0.f, 0.f};
                if (bias) {
                    const uint2 braw = *reinterpret_cast<const uint2 *>(bias + kb + cw + nt * 16);
                    const T *bel = reinterpret_cast<const T *>(&braw);
#pragma unroll
                    for (int i = 0; i < 4; ++i) bv[i] = to_f32(bel[i]);
                }
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm) {
                    if (tm < my_tiles) {
                        const int m = (tbase + tm) * 16 + l16;
                        T o[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(acc[tm][nt][i] + bv[i]);
                        *reinterpret_cast<uint2 *>(reinterpret_cast<char *>(lds) + m * OP + (cw + nt * 16) * (int)sizeof(T)) =
                            *reinterpret_cast<const uint2 *>(o);
                    }
                }
            }
        }
        __syncthreads();
        {
            constexpr int CPP = BN * (int)sizeof(T) / 16;     // 16-byte chunks per pixel
            constexpr int PPP = kBlock / CPP;                 // pixels per pass
            const int ck = t % CPP;
            const int oh0 = I.rb * q.RH, ow0 = I.cb * q.CW;
            const int M = q.RH * q.VW;
            const size_t plane = (size_t)(I.n * q.Do + I.od) * q.Ho;
            for (int m = t / CPP; m < M; m += PPP) {
                const int lr = m / q.VW, lc = m - lr * q.VW;
                const int oh = oh0 + lr, ow = ow0 + lc;
                if (lc < q.CW && oh < q.Ho && ow < q.Wo) {
                    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(lds_c + m * OP + ck * 16);
                    T *dst = y + ((plane + oh) * q.Wo + ow) * q.K + kb + ck * 8;
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
                }
            }
        }
        // every wave has read its staged results: the next box may load
        __syncthreads();
        if (ii + 1 < nI) issue_box(ii + 1, 0);
    }
}

// ----------------------------------------------------------------- host side

struct Config {
    int WM, NT, TPW, CC, nch;
    int RH, CW, nrb, ncb, nnb, VW;
    int BH, BW, BP, HI, MT;
    int items, grid, xcd_split, lds;
};

// The item shape for boxes of 32 CC channels (Cpg / (32 CC) chunks).
bool search(const Problem &p, Config &c, int CC)
{
    c.CC = CC;
    c.nch = p.Cpg / (32 * CC);
    // Channel blocks of 128 are split over the four waves (each wave takes
    // every pixel tile of the item and two N tiles, so no two waves of a
    // workgroup load the same weights); blocks of 64 over two waves.
    c.WM = p.Kpg % 128 == 0 ? 1 : 2;
    c.NT = 2;
    const int BN = (kWaves / c.WM) * c.NT * 16;
    c.nnb = p.Kpg / BN;
    const int BD = (p.Z - 1) * p.dd + 1;
    const int max_tiles = 14;
    // Item shape (RH rows x CW columns of output): minimise the MFMA time -
    // rounds of items over the workgroup slots (two per CU when the box fits
    // half the LDS) x tiles per wave - then the box overhead.
    bool found = false;
    double best = 0.0;
    for (int CW = p.Wo < max_tiles * 16 ? p.Wo : max_tiles * 16; CW >= 1; --CW) {
        int RH = max_tiles * 16 / CW;
        if (RH > p.Ho) RH = p.Ho;
        for (; RH >= 1; --RH) {
            const long long BH = (long long)(RH - 1) * p.sh + (long long)(p.Y - 1) * p.dh + 1;
            const long long BW = (long long)(CW - 1) * p.sw + (long long)(p.X - 1) * p.dw + 1;
            // At stride 1 the tiles run over whole box rows (VW = BW pixels
            // per row, the last BW - CW of them computed and dropped): then
            // the 16 pixels of a tile are 16 consecutive box pixels, whose
            // rows (PS = 17 x 16 bytes apart) start in 16 distinct 16-byte
            // bank groups.  Over output rows only, a tile straddling a row
            // end skips the halo pixels and two of its lanes share a bank
            // group with two others (measured: LDS bank conflicts were
            // about half of the LDS cycles).
            const int VW = p.sw == 1 && RH * BW <= max_tiles * 16 ? (int)BW : CW;
            const int M = RH * VW;
            const int MT = (M + 15) / 16;
            if (MT > max_tiles) continue;
            const long long BP = BD * BH * BW;
            const long long slots_needed = BP * (c.CC * 4 + 1);
            const long long HI = (slots_needed + 63) / 64;
            // the box (whole load instructions, >= BP * PS), and the staged
            // output rows, which reuse it
            const long long stage = ((long long)MT * 16 * (BN * 2 + 16) + 1023) / 1024 * 1024;
            // the dropped columns of the last rows read up to (X-1) dw
            // pixels past the box
            long long lds = HI * 1024 > stage ? HI * 1024 : stage;
            const long long reach = (BP + (long long)(p.X - 1) * p.dw) * (c.CC * 4 + 1) * 16;
            if (reach > lds) lds = (reach + 1023) / 1024 * 1024;
            if (lds > kMaxLds) continue;
            const int per_cu = lds <= kMaxLds / 2 ? 2 : 1;
            // the two-wave kernel needs two workgroups per CU to fill its SIMDs
            const long long slots = (long long)kCUs * per_cu;
            const long long nrb = (p.Ho + RH - 1) / RH, ncb = (p.Wo + CW - 1) / CW;
            const long long items = (long long)p.G * c.nnb * p.N * p.Do * nrb * ncb;
            if (items >= (1LL << 30)) continue;
            const long long grid = items < slots ? items : slots;
            const long long rounds = (items + grid - 1) / grid;
            // One round only: a workgroup's later items would wait for their
            // box with nothing to overlap it (the staged output reuses the
            // box), and the chunk-streaming variant measured faster there.
            if (rounds > 1) continue;
            const int tpw = c.WM == 2 ? ((MT + 1) / 2 <= 4 ? 4 : 7) : (MT <= 7 ? 7 : 14);
            // one workgroup per CU leaves one wave per SIMD, which hides
            // little of the LDS and load latency (measured about 1.3x)
            const double t_mfma = (double)rounds * per_cu * tpw * (per_cu == 1 ? 1.3 : 1.0);
            const double useful = (double)p.N * p.Do * p.Ho * p.Wo * p.G * c.nnb / (double)kCUs;
            const double box_over = (double)BP / ((double)RH * CW * p.sh * p.sw);
            const double score = useful / t_mfma / (0.9 + 0.1 * box_over);
            if (!found || score > best) {
                found = true;
                best = score;
                c.RH = RH; c.CW = CW; c.VW = VW; c.nrb = (int)nrb; c.ncb = (int)ncb; c.TPW = tpw;
                c.BH = (int)BH; c.BW = (int)BW; c.BP = (int)BP; c.HI = (int)HI; c.MT = MT;
                c.items = (int)items; c.grid = (int)grid; c.lds = (int)lds;
            }
        }
    }
    if (!found) return false;
    c.xcd_split = c.grid % 8 == 0 ? 1 : 0;
    return true;
}

bool configure(const Problem &p, Config &c)
{
    if (p.dtype != GCONV_F16 && p.dtype != GCONV_BF16) return false;
    if (p.Cpg % 64 != 0 || p.Kpg % 64 != 0) return false;
    const long long xb = (long long)p.N * p.D * p.H * p.W * p.C() * 2;
    const long long wb = (long long)p.K() * p.taps() * p.Cpg * 2;
    if (xb >= (1LL << 31) || wb >= (1LL << 31)) return false;
    // the whole Cpg in one box where it fits, else chunks of 128, else of 64
    if ((p.Cpg == 64 || p.Cpg == 128) && search(p, c, p.Cpg / 32)) return true;
    if (p.Cpg % 128 == 0 && p.Cpg > 128 && search(p, c, 4)) return true;
    return p.Cpg > 64 && search(p, c, 2);
}

Params params(const Problem &p, const Config &c)
{
    Params q;
    q.N = p.N; q.G = p.G; q.Cpg = p.Cpg; q.Kpg = p.Kpg; q.C = p.C(); q.K = p.K();
    q.D = p.D; q.H = p.H; q.W = p.W; q.Do = p.Do; q.Ho = p.Ho; q.Wo = p.Wo;
    q.Y = p.Y; q.X = p.X;
    q.sd = p.sd; q.sh = p.sh; q.sw = p.sw; q.pd = p.pd; q.ph = p.ph; q.pw = p.pw;
    q.dd = p.dd; q.dh = p.dh; q.dw = p.dw;
    q.RH = c.RH; q.CW = c.CW; q.VW = c.VW; q.nrb = c.nrb; q.ncb = c.ncb; q.nnb = c.nnb;
    q.BH = c.BH; q.BW = c.BW; q.BP = c.BP; q.HI = c.HI; q.MT = c.MT;
    q.items = c.items; q.taps = p.taps(); q.xcd_split = c.xcd_split; q.nch = c.nch;
    q.x_bytes = (unsigned)((long long)p.N * p.D * p.H * p.W * p.C() * 2);
    q.w_bytes = (unsigned)((long long)p.K() * p.taps() * p.Cpg * 2);
    q.rplane = 1.0f / (float)(c.BH * c.BW);
    q.rbw = 1.0f / (float)c.BW;
    return q;
}

template <typename T, int WM, int NT, int TPW, int CC>
hipError_t go4(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    Params q = params(p, c);
    auto k = kernel<T, WM, NT, TPW, CC>;
    static std::atomic<unsigned long long> lds_set{0};
    const hipError_t e = allow_lds((const void *)k, lds_set, kMaxLds);
    if (e != hipSuccess) return e;
    return enqueue(k, dim3(c.grid), dim3(kBlock), c.lds, s, a, q, (const T *)a.x, (const T *)a.w,
                   (const T *)a.bias, (T *)a.y);
}

template <typename T, int CC>
hipError_t go2(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    if (c.WM == 1) return c.TPW == 14 ? go4<T, 1, 2, 14, CC>(p, c, a, s) : go4<T, 1, 2, 7, CC>(p, c, a, s);
    return c.TPW == 7 ? go4<T, 2, 2, 7, CC>(p, c, a, s) : go4<T, 2, 2, 4, CC>(p, c, a, s);
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    return c.CC == 4 ? go2<T, 4>(p, c, a, s) : go2<T, 2>(p, c, a, s);
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

}  // namespace ighalo_box
}  // namespace gconv

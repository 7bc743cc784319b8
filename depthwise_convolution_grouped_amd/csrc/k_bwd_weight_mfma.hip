// Backward weight on the matrix cores (fp16 / bf16): stage 1 of the
// two-stage deterministic reduction (partial sums per chunk of output
// pixels), as an implicit GEMM per group.
//
// The backward-weight variant of the CK grouped_conv tile-engine README
// (introduction), whose runner takes X and dY (CK Python examples README,
// Runner argument contract), with the two-stage fp32 workspace of its
// two_stage option (Config-options harness).  Per group g the result is a
// GEMM whose reduction runs over output pixels p:
//
//   dw[g][k][t][c] = sum_p dy[p][g][k] * x[p shifted by tap t][g][c]
//
// M = output channels k, N = (tap t, input channel c), K = output pixels.
// Both operands are stored pixel-major in memory (channels contiguous), so
// the reduction index is the row index of both.  gfx950's transposing LDS
// read (ds_read_b64_tr_b16) delivers them as MFMA operands anyway: within
// each group of 16 lanes, lane 4j + m points at four consecutive channels
// 4m..4m+3 of pixel j, and lane i receives channel i of pixels 0..3; two
// such reads give a lane the eight pixels of its 16x16x32 operand.  So the
// operand tiles sit in LDS exactly as they come from memory and are filled
// by direct-to-LDS loads.
//
// Small groups are merged: GN consecutive groups form one super-group of
// Kq = GN Kpg output and Cq = GN Cpg input channels (both multiples of 16),
// the product is computed for the whole super-group, and only its diagonal
// blocks (k and c of the same group) are kept (the num_groups_to_merge
// option of the same harness).
//
// Work decomposition.  A step is SR output rows x SC output columns of one
// output plane of one image (SP pixels, a multiple of 32, the tail zeroed).
// Its dy tile (SP pixels x the workgroup's output channels) and its input
// box (the step's pixels widened by the dilated filter footprint, the
// workgroup's input channels) are loaded into LDS, double-buffered: the next
// step's loads are in flight while this step's MFMAs run.  Every tap reads
// the same box at a shifted pixel offset, so x crosses into LDS once per
// step, not once per tap.  Wave (sg, wk, wc) of the workgroup owns, in its
// super-group sg, KW output tiles of 16 channels x all taps x one input
// tile of 16 channels; a workgroup whose tiles cover whole super-groups
// takes SG consecutive ones, so its loads read longer channel runs.  Pixel
// rows of 128 bytes or more in LDS get one 16-byte pad slot, which spreads
// the four pixels of a transposing read over distinct banks.  A workgroup
// owns a chunk of consecutive steps and writes its partial sums once:
// [chunk][g][k][t][c] in the fp32 workspace, or dw itself, rounded once,
// when there is a single chunk.
#include "device_common.h"
#include "gconv_internal.h"
#include "smallg_common.h"

namespace gconv {
namespace bwdw_mfma {
namespace {

using smallg::dma16;
using smallg::f32x4;
using smallg::make_rsrc;
using smallg::Mfma;
using smallg::rsrc_t;

constexpr unsigned kOob = 0x80000000u;   // a buffer offset past any tensor: loads zero
constexpr int kMaxBoxIns = 16;           // box DMA instructions per wave and step
constexpr int kMaxDyIns = 8;             // dy-tile DMA instructions per wave and step
constexpr int kMaxLds = 80 * 1024;       // both buffers: two workgroups per CU
// Chunks for one round of 8 waves per CU (two 4-wave workgroups, or one of
// 8 waves): measured against 512 .. 8192 waves on the ResNeXt-style, 3D
// 2-in/4-out and large-group shapes, 2048 was fastest on all of them (1.2-1.6x
// over two rounds: fewer chunks of partial sums for stage 2 and no second,
// partly filled round)
constexpr int kTargetWaves = 2048;
// chunks are also capped so that stage 2 (which reads every chunk's partial
// sums) moves at most kStage2Share x the bytes of x and dy
constexpr double kStage2Share = 1.0;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

struct Params {
    int N, G, D, H, W, Do, Ho, Wo, C, K;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int Y, X, taps;
    int Cpg, Kpg, GN, Kq, Cq;
    int SR, SC, SP;          // step shape: SR x SC output pixels, SP of them rounded up to 32
    int BH, BW, BP;          // input box rows, columns, pixels (all planes)
    int nrb, nwb;            // row and column blocks per output plane
    int nkb, ncb;            // output- and input-channel blocks per super-group
    int WK, WC, SG;          // waves along output tiles, along input tiles, super-groups per workgroup
    int SPB, SPD;            // 16-byte slots per box pixel / dy-tile pixel (a pad slot included)
    int CB, CD;              // channels per box pixel / dy-tile pixel (the workgroup's)
    int steps, spc;          // steps in all, steps per chunk
    int box_ins, dy_ins;     // DMA instructions per step (whole workgroup)
    unsigned box_bytes, buf_bytes;
    unsigned x_bytes, dy_bytes;
    int welems;
    float rbhw, rbw;         // 1 / (BH BW), 1 / BW
    float rspb, rspd;        // 1 / SPB, 1 / SPD
};

// n / d for 0 <= n < 2^22 from a float reciprocal of d (off by at most one
// before the correction).
__device__ __forceinline__ int fdivr(int n, int d, float rd)
{
    int v = (int)((float)n * rd);
    const int r = n - v * d;
    v += r >= d ? 1 : 0;
    v -= r < 0 ? 1 : 0;
    return v;
}

// One operand half: four channels of four pixels (see the file comment).
__device__ __forceinline__ v4s tr_read(const char *lds_c, unsigned off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(lds_c + off));
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::V operand(v4s lo, v4s hi)
{
    struct {
        v4s a, b;
    } pair{lo, hi};
    return __builtin_bit_cast(typename Mfma<T>::V, pair);
}

template <typename T, int KW, int TAPS>
__global__ __launch_bounds__(256) void kernel(Params q, const T *__restrict__ x,
                                                        const T *__restrict__ dy, float *__restrict__ ws,
                                                        T *__restrict__ dwout)
{
    const int NW = q.WK * q.WC * q.SG;
    const int PS = 16 * q.SPB;              // box pixel stride, bytes
    const int PD = 16 * q.SPD;              // dy-tile pixel stride, bytes
    constexpr int NKC = 4;                  // at most 4 x 32 pixels per step
    typedef typename Mfma<T>::V V;
    extern __shared__ uint4 lds[];
    const char *lds_c = reinterpret_cast<const char *>(lds);
    const unsigned lds_b = (unsigned)(size_t)lds;

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    const int wc = wave % q.WC, wk = (wave / q.WC) % q.WK, sg = wave / (q.WC * q.WK);
    const int s16 = lane & 15, qg = lane >> 4;

    int tile = (int)blockIdx.x;
    const int cbk = tile % q.ncb;  tile /= q.ncb;
    const int kbk = tile % q.nkb;
    const int gq = tile / q.nkb;
    const int chunk = (int)blockIdx.y;
    const int c0 = cbk * 16 * q.WC;               // first input channel of the block (in the super-group)
    const int k0 = kbk * 16 * KW * q.WK;          // first output channel of the block
    const int st0 = chunk * q.spc;
    const int st1 = st0 + q.spc < q.steps ? st0 + q.spc : q.steps;

    // ---- step-invariant DMA plans.  Box slot L (16 bytes) = pixel L / SPB,
    //      channel chunk L % SPB (the pad slot, if any, loads zeros); dy-tile
    //      slot L = pixel L / SPD, chunk L % SPD.
    unsigned bplan[kMaxBoxIns];   // bz << 24 | by << 12 | bx, with the chunk in the top bits; ~0: dead
    unsigned dplan[kMaxDyIns];    // r << 16 | c << 4 | chunk; ~0: dead
#pragma unroll
    for (int m = 0; m < kMaxBoxIns; ++m) {
        const int ins = wave + NW * m;
        const int L = ins * 64 + lane;
        const int P = fdivr(L, q.SPB, q.rspb), j = L - P * q.SPB;
        bplan[m] = ~0u;
        if (ins < q.box_ins && P < q.BP && j * 8 < q.CB) {
            const int bz = fdivr(P, q.BH * q.BW, q.rbhw);
            const int rem = P - bz * q.BH * q.BW;
            const int by = fdivr(rem, q.BW, q.rbw), bx = rem - by * q.BW;
            bplan[m] = ((unsigned)j << 29) | ((unsigned)bz << 24) | ((unsigned)by << 12) | (unsigned)bx;
        }
    }
#pragma unroll
    for (int m = 0; m < kMaxDyIns; ++m) {
        const int ins = wave + NW * m;
        const int L = ins * 64 + lane;
        const int pix = fdivr(L, q.SPD, q.rspd), j = L - pix * q.SPD;
        dplan[m] = ~0u;
        if (ins < q.dy_ins && pix < q.SR * q.SC && j * 8 < q.CD) {
            const int r = pix / q.SC, c = pix - (pix / q.SC) * q.SC;
            dplan[m] = ((unsigned)r << 16) | ((unsigned)c << 4) | (unsigned)j;
        }
    }
    const int nbox = (q.box_ins - wave + NW - 1) / NW;   // this wave's DMA instructions per step
    const int ndy = (q.dy_ins - wave + NW - 1) / NW;
    const rsrc_t rx = make_rsrc(x, q.x_bytes);
    const rsrc_t rd = make_rsrc(dy, q.dy_bytes);
    const unsigned cx = (unsigned)(gq * q.SG * q.Cq + c0);   // first x channel of the block
    const unsigned cy = (unsigned)(gq * q.SG * q.Kq + k0);   // first dy channel of the block

    auto issue = [&](int st, int buf) __attribute__((always_inline)) {
        int r = st;
        const int wb = r % q.nwb;  r /= q.nwb;
        const int rb = r % q.nrb;  r /= q.nrb;
        const int od = r % q.Do;
        const int n = r / q.Do;
        const int oh0 = rb * q.SR, ow0 = wb * q.SC;
        const int iz0 = od * q.sd - q.pd, iy0 = oh0 * q.sh - q.ph, ix0 = ow0 * q.sw - q.pw;
        const unsigned base = lds_b + (unsigned)buf * q.buf_bytes;
#pragma unroll
        for (int m = 0; m < kMaxBoxIns; ++m) {
            if (m < nbox) {
                const unsigned pl = bplan[m];
                const int bx = (int)(pl & 4095u), by = (int)((pl >> 12) & 4095u), bz = (int)((pl >> 24) & 31u);
                const int j = (int)(pl >> 29);
                const int iz = iz0 + bz, iy = iy0 + by, ix = ix0 + bx;
                const bool in = pl != ~0u && (unsigned)iz < (unsigned)q.D && (unsigned)iy < (unsigned)q.H &&
                                (unsigned)ix < (unsigned)q.W;
                const unsigned vo =
                    in ? ((unsigned)(((n * q.D + iz) * q.H + iy) * q.W + ix) * (unsigned)q.C + cx + (unsigned)j * 8u) *
                             (unsigned)sizeof(T)
                       : kOob;
                dma16(vo, __builtin_amdgcn_readfirstlane(base + (unsigned)(wave + NW * m) * 1024u), rx);
            }
        }
#pragma unroll
        for (int m = 0; m < kMaxDyIns; ++m) {
            if (m < ndy) {
                const unsigned pl = dplan[m];
                const int j = (int)(pl & 15u), c = (int)((pl >> 4) & 4095u), rr = (int)(pl >> 16);
                const int oh = oh0 + rr, ow = ow0 + c;
                const bool in = pl != ~0u && oh < q.Ho && ow < q.Wo;
                const unsigned vo =
                    in ? ((unsigned)(((n * q.Do + od) * q.Ho + oh) * q.Wo + ow) * (unsigned)q.K + cy + (unsigned)j * 8u) *
                             (unsigned)sizeof(T)
                       : kOob;
                dma16(vo, __builtin_amdgcn_readfirstlane(base + q.box_bytes + (unsigned)(wave + NW * m) * 1024u), rd);
            }
        }
    };

    // ---- operand addressing.  Source lane s16 of lane group qg reads, for
    //      32-pixel slice kc and half h, pixel 32 kc + 8 qg + 4 h + s16 / 4 at
    //      channels 4 (s16 % 4) .. + 3 of its tile.
    unsigned aoff[NKC][2];   // dy tile: byte offset of that pixel row (tile channel 0)
    unsigned boff[NKC][2];   // box: byte offset of that pixel's tap-0 input
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int pix = 32 * kc + 8 * qg + 4 * h + (s16 >> 2);
            const bool live = pix < q.SR * q.SC;
            const int r = live ? pix / q.SC : 0, c = live ? pix - (pix / q.SC) * q.SC : 0;
            aoff[kc][h] = (unsigned)pix * PD;
            boff[kc][h] = (unsigned)((r * q.sh) * q.BW + c * q.sw) * PS;
        }
    // this wave's channels within a box / dy-tile pixel
    const unsigned a_ch = (unsigned)(sg * 16 * KW * q.WK + 4 * (s16 & 3)) * 2u;
    const unsigned b_ch = (unsigned)(sg * 16 * q.WC + 16 * wc + 4 * (s16 & 3)) * 2u;
    int tofs[TAPS];   // box byte offset of each tap
#pragma unroll
    for (int t = 0; t < TAPS; ++t) {
        const int tx = t % q.X, ty = (t / q.X) % q.Y, tz = t / (q.X * q.Y);
        tofs[t] = ((tz * q.dd * q.BH + ty * q.dh) * q.BW + tx * q.dw) * PS;
    }

    f32x4 acc[KW][TAPS];
#pragma unroll
    for (int a = 0; a < KW; ++a)
#pragma unroll
        for (int t = 0; t < TAPS; ++t) acc[a][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkc = q.SP / 32;
    if (st0 < st1) issue(st0, 0);
    for (int st = st0; st < st1; ++st) {
        const int buf = (st - st0) & 1;
        // every wave is done with the other buffer (read by the previous step)
        __syncthreads();
        const bool more = st + 1 < st1;
        if (more) issue(st + 1, buf ^ 1);
        // this wave's loads of step st are back once only the next step's remain
        vm_wait(more ? nbox + ndy : 0);
        __syncthreads();
        const unsigned bb = (unsigned)buf * q.buf_bytes;
        const unsigned db = bb + q.box_bytes;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            if (kc < nkc) {
                V af[KW];
#pragma unroll
                for (int a = 0; a < KW; ++a) {
                    const unsigned ch = (unsigned)(16 * (wk * KW + a)) * 2u + a_ch;   // sg's tile wk * KW + a
                    af[a] = operand<T>(tr_read(lds_c, db + aoff[kc][0] + ch), tr_read(lds_c, db + aoff[kc][1] + ch));
                }
#pragma unroll
                for (int t = 0; t < TAPS; ++t) {
                    const V bf = operand<T>(tr_read(lds_c, bb + boff[kc][0] + (unsigned)tofs[t] + b_ch),
                                            tr_read(lds_c, bb + boff[kc][1] + (unsigned)tofs[t] + b_ch));
#pragma unroll
                    for (int a = 0; a < KW; ++a) acc[a][t] = Mfma<T>::run(af[a], bf, acc[a][t]);
                }
            }
        }
    }
    // no DMA may still be writing LDS when the workgroup retires
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

    // ---- results: lane holds rows 4 qg + i (output channels) of column s16
    //      (input channel) of each 16 x 16 tile; only a group's own block counts
    const int cq = c0 + 16 * wc + s16;            // input channel in super-group gq * SG + sg
    const int gc = cq / q.Cpg, c = cq - gc * q.Cpg;
#pragma unroll
    for (int a = 0; a < KW; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kq = k0 + 16 * (wk * KW + a) + 4 * qg + i;
            const int gk = kq / q.Kpg, k = kq - gk * q.Kpg;
            if (gk != gc) continue;
            const int g = (gq * q.SG + sg) * q.GN + gk;
            const size_t fb = ((size_t)(g * q.Kpg + k) * q.taps) * q.Cpg + c;
#pragma unroll
            for (int t = 0; t < TAPS; ++t) {
                const size_t f = fb + (size_t)t * q.Cpg;
                if (dwout) dwout[f] = from_f32<T>(acc[a][t][i]);
                else ws[(size_t)chunk * q.welems + f] = acc[a][t][i];
            }
        }
}

// ----------------------------------------------------------------- host side

struct Config {
    int GN, KW, WK, WC, SG, taps;
    Params q;
    int tiles, nch, threads, lds;
};

bool configure(const Problem &p, Config &c)
{
    if (p.dtype != GCONV_F16 && p.dtype != GCONV_BF16) return false;
    if (p.Cpg == 1 && p.Kpg == 1) return false;     // depthwise keeps its channel-vector kernel
    const int taps = p.taps();
    if (taps != 1 && taps != 9 && taps != 25 && taps != 27) return false;
    c.GN = 0;
    for (int g : {1, 2, 4, 8, 16})
        if (p.G % g == 0 && (g * p.Kpg) % 16 == 0 && (g * p.Cpg) % 16 == 0) {
            c.GN = g;
            break;
        }
    if (c.GN == 0) return false;
    const int Kq = c.GN * p.Kpg, Cq = c.GN * p.Cpg;
    const int KTn = Kq / 16, CTn = Cq / 16;
    c.taps = taps;
    c.KW = taps <= 9 && KTn % 2 == 0 ? 2 : 1;
    c.WC = CTn % 2 == 0 ? 2 : 1;
    const int kgroups = KTn / c.KW;
    c.WK = 1;
    for (int w : {4, 2})
        if (w * c.WC <= 4 && kgroups % w == 0) {
            c.WK = w;
            break;
        }
    Params &q = c.q;
    q.N = p.N; q.G = p.G; q.D = p.D; q.H = p.H; q.W = p.W; q.Do = p.Do; q.Ho = p.Ho; q.Wo = p.Wo;
    q.C = p.C(); q.K = p.K();
    q.sd = p.sd; q.sh = p.sh; q.sw = p.sw; q.pd = p.pd; q.ph = p.ph; q.pw = p.pw;
    q.dd = p.dd; q.dh = p.dh; q.dw = p.dw;
    q.Y = p.Y; q.X = p.X; q.taps = taps;
    q.Cpg = p.Cpg; q.Kpg = p.Kpg; q.GN = c.GN; q.Kq = Kq; q.Cq = Cq;
    // Layout search: super-groups per workgroup (a workgroup whose tiles
    // cover whole super-groups takes up to four waves' worth of them; more
    // is preferred: longer channel runs per load), then the step columns SC
    // and rows SR for the best use of the 32-pixel MFMA slices over the
    // steps, within the LDS and DMA-instruction budgets; on a tie, the fewest
    // load instructions per output pixel (less halo).  SC is the whole row
    // when it has <= 64 columns, or half of it: a 56-column row in two
    // 28-column blocks takes 2-row steps where whole rows only fit 1-row ones
    // in the LDS budget (measured: ResNeXt-style stage 1 about 7% faster).
    const int sc_full = p.Wo <= 64 ? p.Wo : 32;
    const int sc_half = p.Wo <= 64 && p.Wo > 16 ? (p.Wo + 1) / 2 : 0;
    const long long BD = (long long)(p.Z - 1) * p.dd + 1;
    if (BD >= 32) return false;
    long long BW = 0;
    bool found = false;
    for (int sgn : {4, 2, 1}) {
        if (sgn > 1 && !(kgroups == c.WK && CTn == c.WC && sgn * c.WK * c.WC <= 4 && (p.G / c.GN) % sgn == 0))
            continue;
        const int NW = c.WK * c.WC * sgn;
        const int CB = 16 * c.WC * sgn, CD = 16 * c.KW * c.WK * sgn;
        const int SPB = CB / 8 + (CB / 8 % 8 == 0 ? 1 : 0);
        const int SPD = CD / 8 + (CD / 8 % 8 == 0 ? 1 : 0);
        double best = -1.0, best_ipp = 1e30;
        for (int SC : {sc_full, sc_half}) {
            if (SC == 0) continue;
            const long long bw = (long long)(SC - 1) * p.sw + (long long)(p.X - 1) * p.dw + 1;
            if (bw >= 4096) continue;
            const int nwb = (p.Wo + SC - 1) / SC;
            for (int sr = 1; sr * SC <= 128 && sr <= p.Ho; ++sr) {
                const long long BH = (long long)(sr - 1) * p.sh + (long long)(p.Y - 1) * p.dh + 1;
                if (BH >= 4096) break;
                const int SP = (sr * SC + 31) / 32 * 32;
                const long long box_ins = (BD * BH * bw * SPB + 63) / 64;
                const long long dy_ins = ((long long)SP * SPD + 63) / 64;
                if (box_ins > kMaxBoxIns * NW || dy_ins > kMaxDyIns * NW) continue;
                if (2 * (box_ins + dy_ins) * 1024 > kMaxLds) continue;   // at least two buffers
                const int nrb = (p.Ho + sr - 1) / sr;
                const double steps_img = (double)nrb * nwb;
                const double use = (double)p.Ho * p.Wo / (steps_img * SP);
                const double ipp = (double)(box_ins + dy_ins) * steps_img / ((double)p.Ho * p.Wo);
                if (use > best + 1e-9 || (use >= best - 1e-9 && ipp <= best_ipp)) {
                    best = use;
                    best_ipp = ipp;
                    found = true;
                    c.SG = sgn;
                    q.SC = SC;
                    BW = bw;
                    q.SR = sr;
                    q.SP = SP;
                    q.BH = (int)BH;
                    q.SPB = SPB; q.SPD = SPD; q.CB = CB; q.CD = CD;
                    q.box_ins = (int)box_ins;
                    q.dy_ins = (int)dy_ins;
                }
            }
        }
        if (found) break;
    }
    if (!found) return false;
    q.WK = c.WK; q.WC = c.WC; q.SG = c.SG;
    q.rspb = 1.0f / (float)q.SPB;
    q.rspd = 1.0f / (float)q.SPD;
    q.BW = (int)BW;
    q.BP = (int)(BD * q.BH * BW);
    const long long BH = q.BH;
    q.nrb = (p.Ho + q.SR - 1) / q.SR;
    q.nwb = (p.Wo + q.SC - 1) / q.SC;
    q.nkb = kgroups / c.WK;
    q.ncb = CTn / c.WC;
    const long long steps = (long long)p.N * p.Do * q.nrb * q.nwb;
    if (steps >= (1LL << 30)) return false;
    q.steps = (int)steps;
    const int NW = c.WK * c.WC * c.SG;
    q.box_bytes = (unsigned)q.box_ins * 1024u;
    q.buf_bytes = q.box_bytes + (unsigned)q.dy_ins * 1024u;
    c.lds = 2 * (int)q.buf_bytes;
    const long long xb = (long long)p.N * p.D * p.H * p.W * p.C() * 2;
    const long long yb = (long long)p.N * p.Do * p.Ho * p.Wo * p.K() * 2;
    if (xb >= (1LL << 31) || yb >= (1LL << 31)) return false;
    q.x_bytes = (unsigned)xb;
    q.dy_bytes = (unsigned)yb;
    q.welems = p.G * p.Kpg * taps * p.Cpg;
    q.rbhw = 1.0f / (float)(BH * BW);
    q.rbw = 1.0f / (float)BW;
    c.tiles = (p.G / c.GN / c.SG) * q.nkb * q.ncb;
    c.threads = 64 * NW;
    // chunks: enough workgroups for about kTargetWaves waves, each chunk at
    // least two steps (the loads of one overlap the MFMAs of the other)
    long long want = ((long long)kTargetWaves / NW + c.tiles - 1) / c.tiles;
    if (want > (steps + 1) / 2) want = (steps + 1) / 2;
    const double s2cap = kStage2Share * (double)(xb + yb) / ((double)q.welems * 4.0);
    if (want > (long long)s2cap) want = (long long)s2cap;
    if (want > 65535) want = 65535;
    if (want < 1) want = 1;
    q.spc = (int)((steps + want - 1) / want);
    c.nch = (int)((steps + q.spc - 1) / q.spc);
    return true;
}

template <typename T, int KW, int TAPS>
hipError_t go3(const Config &c, const void *x, const void *dy, float *ws, void *dw, int nch, int *used,
               hipStream_t s)
{
    Params q = c.q;
    // fewer chunks than the ideal (a smaller workspace): longer ones
    q.spc = (q.steps + nch - 1) / nch;
    const int n = (q.steps + q.spc - 1) / q.spc;
    *used = n;
    static std::atomic<unsigned long long> lds_set{0};
    if (c.lds > 64 * 1024) {
        const hipError_t e = allow_lds((const void *)kernel<T, KW, TAPS>, lds_set, kMaxLds);
        if (e != hipSuccess) return e;
    }
    Args a{};
    return enqueue(kernel<T, KW, TAPS>, dim3((unsigned)c.tiles, (unsigned)n), dim3((unsigned)c.threads),
                   (unsigned)c.lds, s, a, q, (const T *)x, (const T *)dy, ws, (T *)dw);
}

template <typename T>
hipError_t go(const Config &c, const void *x, const void *dy, float *ws, void *dw, int nch, int *used,
              hipStream_t s)
{
    // two output tiles per wave only for windows of up to 9 taps
    if (c.KW == 2) {
        if (c.taps == 1) return go3<T, 2, 1>(c, x, dy, ws, dw, nch, used, s);
        return go3<T, 2, 9>(c, x, dy, ws, dw, nch, used, s);
    }
    switch (c.taps) {
    case 1: return go3<T, 1, 1>(c, x, dy, ws, dw, nch, used, s);
    case 9: return go3<T, 1, 9>(c, x, dy, ws, dw, nch, used, s);
    case 25: return go3<T, 1, 25>(c, x, dy, ws, dw, nch, used, s);
    default: return go3<T, 1, 27>(c, x, dy, ws, dw, nch, used, s);
    }
}

}  // namespace

bool supported(const Problem &p)
{
    Config c;
    return configure(p, c);
}

int chunks(const Problem &p)
{
    Config c;
    return configure(p, c) ? c.nch : 1;
}

hipError_t stage1(const Problem &p, const void *x, const void *dy, float *ws, void *dw, int nch, int *used,
                  hipStream_t s)
{
    Config c;
    if (!configure(p, c)) return hipErrorInvalidValue;
    if (nch < 1) nch = 1;
    if (p.dtype == GCONV_F16) return go<_Float16>(c, x, dy, ws, dw, nch, used, s);
    return go<__bf16>(c, x, dy, ws, dw, nch, used, s);
}

}  // namespace bwdw_mfma
}  // namespace gconv

// Implicit-GEMM grouped convolution on the matrix cores (fp16 / bf16 on
// 16x16x32 MFMAs, fp32 on four chained 16x16x4 ones; 2D and 3D), for groups
// of 8k (fp32: 4k) input and 4k output channels that the small-group kernels
// do not take (wider groups, or more output than input channels).
//
// Per group g the convolution is a GEMM: M = output pixels (N * Do * Ho *
// Wo), N = Kpg output channels, K = taps * Cpg.  The group is the grid's z
// coordinate and the grid is (M tiles, N tiles, G), after the grid-per-group
// scheme of rocm-libraries PR 10064 (Technical Details: the launch grid is
// (gn, gm, groups)).  K is decoded into (tap, channel in group) with the
// channel fastest, as that page's A descriptor does, so the im2col operand is
// never materialised.  When KT divides Cpg a K stage is one tap and KT
// consecutive channels: each output pixel needs KT contiguous input channels
// of one input pixel, or zeros when the tap falls into the padding.  Other
// widths (Cpg = 8, 16, 24, 40, ...) walk K in 8-channel chunks q = tap *
// Cpg/8 + c8, KT/8 chunks per stage, so a stage may span taps: each 16-byte
// slot decodes its own (tap, chunk), and chunks past taps * Cpg/8 are zero.
// Either way the weight operand of a stage is KT contiguous values of each
// output channel's GKZYXC row (the B descriptor's channel extent is Cpg).
// For fp32 a 16-byte slot holds 4 channels, so the chunks above are 4
// channels and a stage of KT channels has KT / 16 MFMA K steps.
// Output-channel tiles past Kpg (Kpg not a multiple of BN) read zero weights
// and store nothing.
//
// A workgroup (4 waves, 2 x 2) computes a BM x BN output tile.  Every K stage
// of both operands is staged in LDS by direct-to-LDS buffer loads (zero fill
// from the buffer range check), double-buffered: the loads of stage s+1 are
// in flight while stage s is multiplied (v_mfma_f32_16x16x32, fp32
// accumulators).  Rows are padded by one 16-byte slot so the 16 rows read by
// one MFMA operand fall in different LDS banks.  The weights are the first
// MFMA operand, so each lane ends with four adjacent output channels of one
// pixel: the fused epilogue adds the bias, rounds and stores 8 bytes.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace igemm {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = 4;
constexpr int BM = 128;
constexpr unsigned kOob = 0x80000000u;

typedef int rsrc_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Params {
    int N, G, Cpg, Kpg, C, K;
    int D, H, W, Do, Ho, Wo, Z, Y, X;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int M;                 // N * Do * Ho * Wo
    int mtiles, ntiles;    // grid x, y
    int stages;            // K stages: ceil(taps * Cpg / KT)
    int nq8;               // 8-channel chunks of K: taps * Cpg / 8
    Div dCH8, dX, dY;      // Cpg / 8, X, Y (chunk decode of the general K walk)
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

__device__ __forceinline__ void dma16(unsigned voffset, unsigned lds_byte, rsrc_t r)
{
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
// fp32: a 16-byte slot holds 4 channels; element e of both operands' slots
// feeds the e-th of four 16x16x4 MFMAs (k = lane / 16 in each), so the four
// cover the 16 channels of the lanes' four slots in a permuted order that
// both operands share.
template <> struct Mfma<float> {
    typedef f32x4 V;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    }
};

// BN: output channels per tile (32, 64 or 128; each of the two waves along
// N takes BN / 2); KT: K per stage (32 or 64, fp32 16 or 32); CHUNKED: K
// walked in 16-byte chunks (8 channels, fp32 4) across taps (KT does not
// divide Cpg).
template <typename T, int BN, int KT, bool CHUNKED>
__global__ __launch_bounds__(kBlock) void kernel(Params q, const T *__restrict__ x,
                                                 const T *__restrict__ w,
                                                 const T *__restrict__ bias, T *__restrict__ y)
{
    typedef typename Mfma<T>::V V;
    constexpr int EPC = 16 / (int)sizeof(T);    // channels per 16-byte slot
    constexpr int RS = KT / EPC + 1;            // 16-byte slots per staged row (one pad)
    constexpr int A_SLOTS = BM * RS, B_SLOTS = BN * RS;
    constexpr int A_INSTR = (A_SLOTS + 63) / 64, B_INSTR = (B_SLOTS + 63) / 64;
    constexpr int INSTR = A_INSTR + B_INSTR;    // load instructions per stage (all waves)
    constexpr int LPW = (INSTR + kWaves - 1) / kWaves;
    constexpr int STAGE_BYTES = (A_SLOTS + B_SLOTS) * 16;
    constexpr int WM = BM / 2, WN = BN / 2;     // wave tile
    constexpr int TM = WM / 16, TN = WN / 16;   // MFMA tiles per wave
    constexpr int KS = KT / (4 * EPC);          // MFMA K steps per stage (four slots each)
    static_assert(KS >= 1, "a stage holds at least one K step");
    extern __shared__ uint4 lds[];

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int g = blockIdx.z;
    const int nb = blockIdx.y;
    const int mb = (int)blockIdx.x;
    const int m0 = mb * BM, n0 = nb * BN;
    const int taps = q.Z * q.Y * q.X;
    const unsigned es = (unsigned)sizeof(T);
    const rsrc_t rx = make_rsrc(x, q.x_bytes);
    const rsrc_t rw = make_rsrc(w, q.w_bytes);
    const unsigned lds_b = (unsigned)(size_t)lds;

    // ---- this lane's share of a stage's loads: instruction k = wave + 4 i.
    // Instructions [0, A_INSTR) fill the input tile (row = output pixel),
    // the rest the weight tile (row = output channel).  Slot j of a row is
    // channel vector j of the stage; slot RS-1 is the zero pad.
    int ld_kind[LPW];           // 0 none, 1 input, 2 weight
    int ld_slot[LPW];           // slot within its row
    int ld_pix_n[LPW], ld_pix_d[LPW], ld_pix_h[LPW], ld_pix_w[LPW];   // input row: pixel origin
    int ld_wrow[LPW];           // weight row: output channel index g*Kpg + n
    unsigned ld_m0[LPW];        // LDS byte offset inside a stage buffer
    int nld = 0;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int k = wave + kWaves * i;
        ld_kind[i] = 0; ld_slot[i] = RS - 1; ld_pix_n[i] = -1; ld_pix_d[i] = 0; ld_pix_h[i] = 0;
        ld_pix_w[i] = 0; ld_wrow[i] = -1; ld_m0[i] = 0;
        if (k < A_INSTR) {
            const int L = k * 64 + lane;
            nld = i + 1;
            ld_kind[i] = L < A_SLOTS ? 1 : 0;
            ld_m0[i] = (unsigned)(k * 64) * 16u;
            const int row = L / RS;
            ld_slot[i] = L - row * RS;
            const int m = m0 + row;
            if (L < A_SLOTS && m < q.M) {
                int r = m;
                const int ow = r % q.Wo; r /= q.Wo;
                const int oh = r % q.Ho; r /= q.Ho;
                const int od = r % q.Do;
                ld_pix_n[i] = r / q.Do;
                ld_pix_d[i] = od * q.sd - q.pd;
                ld_pix_h[i] = oh * q.sh - q.ph;
                ld_pix_w[i] = ow * q.sw - q.pw;
            }
        } else if (k < INSTR) {
            const int L = (k - A_INSTR) * 64 + lane;
            nld = i + 1;
            ld_kind[i] = L < B_SLOTS ? 2 : 0;
            ld_m0[i] = (unsigned)(A_SLOTS * 16) + (unsigned)((k - A_INSTR) * 64) * 16u;
            const int row = L / RS;
            ld_slot[i] = L - row * RS;
            if (L < B_SLOTS && n0 + row < q.Kpg) ld_wrow[i] = g * q.Kpg + n0 + row;
        }
    }
    // issue stage st into buffer b: tap st / (Cpg/KT), channels c0 .. c0+KT-1,
    // or, chunked, chunks st * KT/EPC .. st * KT/EPC + KT/EPC - 1 of the K walk
    const int cstages = CHUNKED ? 1 : q.Cpg / KT;
    auto issue = [&](int st, int b) {
        int tap = st / cstages;
        int c0 = (st - tap * cstages) * KT;
        int xx = tap % q.X, yy = (tap / q.X) % q.Y, zz = tap / (q.X * q.Y);
        const unsigned base = lds_b + (unsigned)(b * STAGE_BYTES);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            if (i < nld) {
                unsigned vo = kOob;
                bool live = true;
                if constexpr (CHUNKED) {
                    // this slot's chunk: its own tap and EPC channels
                    const int q8 = st * (KT / EPC) + ld_slot[i];
                    live = q8 < q.nq8;
                    tap = fdiv(q8, q.dCH8);
                    c0 = (q8 - tap * q.dCH8.d) * EPC - ld_slot[i] * EPC;
                    const int t1 = fdiv(tap, q.dX);
                    xx = tap - t1 * q.X;
                    zz = fdiv(t1, q.dY);
                    yy = t1 - zz * q.Y;
                }
                if (ld_kind[i] == 1 && ld_slot[i] < RS - 1 && ld_pix_n[i] >= 0 && live) {
                    const int id = ld_pix_d[i] + zz * q.dd, ih = ld_pix_h[i] + yy * q.dh,
                              iw = ld_pix_w[i] + xx * q.dw;
                    if (id >= 0 && id < q.D && ih >= 0 && ih < q.H && iw >= 0 && iw < q.W)
                        vo = ((unsigned)(((ld_pix_n[i] * q.D + id) * q.H + ih) * q.W + iw) * (unsigned)q.C +
                              (unsigned)(g * q.Cpg + c0 + ld_slot[i] * EPC)) * es;
                } else if (ld_kind[i] == 2 && ld_slot[i] < RS - 1 && ld_wrow[i] >= 0 && live) {
                    vo = ((unsigned)(ld_wrow[i] * taps + tap) * (unsigned)q.Cpg +
                          (unsigned)(c0 + ld_slot[i] * EPC)) * es;
                }
                if (ld_kind[i] != 0) {
                    // input instructions read through the x buffer, weight ones through w
                    const int k = wave + kWaves * i;
                    if (k < A_INSTR) dma16(vo, __builtin_amdgcn_readfirstlane(base + ld_m0[i]), rx);
                    else dma16(vo, __builtin_amdgcn_readfirstlane(base + ld_m0[i]), rw);
                }
            }
        }
    };

    // ---- fragments: lane (l16 = lane % 16, kq = lane / 16)
    const int l16 = lane & 15, kq = lane >> 4;
    const int wm = (wave & 1) * WM, wn = (wave >> 1) * WN;
    f32x4 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nst = q.stages;
    issue(0, 0);
    for (int st = 0; st < nst; ++st) {
        const int b = st & 1;
        // this wave's loads of stage st are in when none issued later remain
        vm_wait(0);
        __syncthreads();
        if (st + 1 < nst) issue(st + 1, b ^ 1);   // buffer b^1 was last read before the barrier
        const char *sb = reinterpret_cast<const char *>(lds) + b * STAGE_BYTES;
        const char *sa = sb;                                  // input tile rows (pixels)
        const char *sw_ = sb + A_SLOTS * 16;                  // weight tile rows (channels)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            V wf[TN], xf[TM];
#pragma unroll
            for (int nt = 0; nt < TN; ++nt) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(sw_ + ((wn + nt * 16 + l16) * RS + ks * 4 + kq) * 16);
                wf[nt] = *reinterpret_cast<const V *>(&raw);
            }
#pragma unroll
            for (int mt = 0; mt < TM; ++mt) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(sa + ((wm + mt * 16 + l16) * RS + ks * 4 + kq) * 16);
                xf[mt] = *reinterpret_cast<const V *>(&raw);
            }
#pragma unroll
            for (int mt = 0; mt < TM; ++mt)
#pragma unroll
                for (int nt = 0; nt < TN; ++nt) acc[mt][nt] = Mfma<T>::run(wf[nt], xf[mt], acc[mt][nt]);
        }
    }

    // ---- epilogue: acc[mt][nt][i] = channel n0 + wn + nt*16 + 4 kq + i of pixel m0 + wm + mt*16 + l16
#pragma unroll
    for (int nt = 0; nt < TN; ++nt) {
        const int ch = n0 + wn + nt * 16 + 4 * kq;            // channel within the group
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias && ch < q.Kpg) {
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = to_f32(bias[g * q.Kpg + ch + i]);
        }
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) {
            const int m = m0 + wm + mt * 16 + l16;
            if (m < q.M && ch < q.Kpg) {
                T o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(acc[mt][nt][i] + bv[i]);
                if constexpr (sizeof(T) == 4)
                    *reinterpret_cast<uint4 *>(y + (size_t)m * q.K + g * q.Kpg + ch) = *reinterpret_cast<const uint4 *>(o);
                else
                    *reinterpret_cast<uint2 *>(y + (size_t)m * q.K + g * q.Kpg + ch) = *reinterpret_cast<const uint2 *>(o);
            }
        }
    }
}

// ----------------------------------------------------------------- host side

struct Config {
    int BN, KT, mtiles, ntiles, stages, nq8, lds;
    bool chunked;
};

// Groups of 32k input and output channels ("wide") run one tap per stage;
// other widths need 8k input and 4k output channels and walk K in chunks.
bool wide(const Problem &p) { return p.Cpg % 32 == 0 && p.Kpg % 32 == 0; }

// Tile menu: (BN, KT) pairs, widest first.  Wide groups take BN dividing Kpg
// and KT dividing Cpg; other widths take BN of 32, or 64 and 128 while the
// tile is less than twice Kpg, each with both KT.
int menu(const Problem &p, int (*m)[2])
{
    const bool wd = wide(p);
    const bool f32 = p.dtype == GCONV_F32;   // fp32 stages of 32 or 16 channels (twice the bytes)
    int n = 0;
    for (int bn : {128, 64, 32})
        for (int kt0 : {64, 32}) {
            const int kt = f32 ? kt0 / 2 : kt0;
            const bool ok = wd ? (p.Kpg % bn == 0 && p.Cpg % kt == 0) : (bn == 32 || bn < 2 * p.Kpg);
            if (ok) {
                m[n][0] = bn;
                m[n][1] = kt;
                ++n;
            }
        }
    return n;
}

// Own pick (from the tile sweep).  Wide groups: the widest output-channel
// tile with 32-channel reduction steps (half the LDS, more workgroups
// resident); with fewer 128-channel tiles than CUs, 64-channel tiles with
// 64-channel steps; with fewer than two tiles per CU, 64-channel steps.  Other widths: the widest tile that pads Kpg no more
// than 32-channel tiles do, with 32-channel steps.
void own_pick_half(const Problem &p, long long mt, Config &c)
{
    c.KT = 32;
    if (wide(p)) {
        c.BN = p.Kpg % 128 == 0 ? 128 : (p.Kpg % 64 == 0 ? 64 : 32);
        const long long tiles = mt * (p.Kpg / c.BN) * p.G;
        if (p.ndim == 3) {
            // 27-tap windows: 128-channel tiles with 64-channel steps below
            // four tiles per CU (1.1-1.2x over the 2D choices in the sweep)
            if (tiles < 1024 && p.Cpg % 64 == 0) c.KT = 64;
        } else if (c.BN == 128 && tiles < 256 && p.Cpg % 64 == 0) {
            c.BN = 64;
            c.KT = 64;
        } else if (tiles < 512 && p.Cpg % 64 == 0) {
            c.KT = 64;
        }
        return;
    }
    const int pad32 = (p.Kpg + 31) / 32 * 32;
    c.BN = 32;
    for (int bn : {128, 64})
        if (bn < 2 * p.Kpg && (p.Kpg + bn - 1) / bn * bn <= pad32) {
            c.BN = bn;
            break;
        }
}

void own_pick(const Problem &p, long long mt, Config &c)
{
    own_pick_half(p, mt, c);
    if (p.dtype != GCONV_F32) return;
    // fp32: stages of half the channels, the same bytes per staged row; with
    // fewer than 128 tiles, 32-channel tiles for more workgroups (fp32 tile
    // sweep: 1.3-1.8x on 3D images of one batch)
    c.KT /= 2;
    if (mt * ((p.Kpg + c.BN - 1) / c.BN) * p.G < 128) c.BN = 32;
    // groups of 32k channels with fewer than 512 tiles: 32-channel stages
    // (as the half types' 64-channel steps under two tiles per CU; 1.2x on
    // a 2-group 32/32 problem of 356 tiles)
    if (wide(p) && c.KT == 16 && p.Cpg % 32 == 0 && mt * ((p.Kpg + c.BN - 1) / c.BN) * p.G < 512) c.KT = 32;
}

bool configure(const Problem &p, Config &c)
{
    if (p.dtype != GCONV_F16 && p.dtype != GCONV_BF16 && p.dtype != GCONV_F32) return false;
    const int epc = p.dtype == GCONV_F32 ? 4 : 8;     // channels per 16-byte slot
    const long long es = p.dtype == GCONV_F32 ? 4 : 2;
    if (p.Cpg % epc != 0 || p.Kpg % 4 != 0) return false;
    const long long xb = (long long)p.N * p.D * p.H * p.W * p.C() * es;
    const long long wb = (long long)p.K() * p.taps() * p.Cpg * es;
    if (xb >= (1LL << 31) || wb >= (1LL << 31)) return false;
    const long long M = (long long)p.N * p.Do * p.Ho * p.Wo;
    if (M >= (1LL << 31)) return false;
    // the chunk decode divides exactly below 2^16
    const long long nq8 = (long long)p.taps() * (p.Cpg / epc);
    if (nq8 + 8 >= (1LL << 16)) return false;
    const long long mt = (M + BM - 1) / BM;
    own_pick(p, mt, c);
    const int t = tile_choice();
    int m[6][2];
    if (t >= 0 && t < menu(p, m)) {
        c.BN = m[t][0];
        c.KT = m[t][1];
    }
    c.chunked = p.Cpg % c.KT != 0;
    c.nq8 = (int)nq8;
    c.mtiles = (int)mt;
    c.ntiles = (p.Kpg + c.BN - 1) / c.BN;
    c.stages = (int)((nq8 + c.KT / epc - 1) / (c.KT / epc));
    const int RS = c.KT / epc + 1;
    c.lds = 2 * (BM + c.BN) * RS * 16;
    return c.mtiles < (1 << 30) && c.ntiles < 65536 && p.G < 65536;
}

template <typename T, int BN, int KT, bool CHUNKED>
hipError_t go4(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    Params q;
    q.N = p.N; q.G = p.G; q.Cpg = p.Cpg; q.Kpg = p.Kpg; q.C = p.C(); q.K = p.K();
    q.D = p.D; q.H = p.H; q.W = p.W; q.Do = p.Do; q.Ho = p.Ho; q.Wo = p.Wo;
    q.Z = p.Z; q.Y = p.Y; q.X = p.X;
    q.sd = p.sd; q.sh = p.sh; q.sw = p.sw; q.pd = p.pd; q.ph = p.ph; q.pw = p.pw;
    q.dd = p.dd; q.dh = p.dh; q.dw = p.dw;
    q.M = p.N * p.Do * p.Ho * p.Wo;
    q.mtiles = c.mtiles; q.ntiles = c.ntiles; q.stages = c.stages; q.nq8 = c.nq8;
    const long long es = (long long)sizeof(T);
    q.dCH8 = make_div(p.Cpg / (16 / (int)sizeof(T))); q.dX = make_div(p.X); q.dY = make_div(p.Y);
    q.x_bytes = (unsigned)((long long)p.N * p.D * p.H * p.W * p.C() * es);
    q.w_bytes = (unsigned)((long long)p.K() * p.taps() * p.Cpg * es);
    auto k = kernel<T, BN, KT, CHUNKED>;
    static std::atomic<unsigned long long> lds_set{0};
    if (c.lds > 64 * 1024) {
        const hipError_t e = allow_lds((const void *)k, lds_set, 160 * 1024);
        if (e != hipSuccess) return e;
    }
    return enqueue(k, dim3(c.mtiles, c.ntiles, p.G), dim3(kBlock), c.lds, s, a, q,
                   (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y);
}

template <typename T, int BN, int KT>
hipError_t go3(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    return c.chunked ? go4<T, BN, KT, true>(p, c, a, s) : go4<T, BN, KT, false>(p, c, a, s);
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    if constexpr (sizeof(T) == 4) {
        // fp32: stages of 32 or 16 channels
        if (c.BN == 128) return c.KT == 32 ? go3<T, 128, 32>(p, c, a, s) : go3<T, 128, 16>(p, c, a, s);
        if (c.BN == 64) return c.KT == 32 ? go3<T, 64, 32>(p, c, a, s) : go3<T, 64, 16>(p, c, a, s);
        return c.KT == 32 ? go3<T, 32, 32>(p, c, a, s) : go3<T, 32, 16>(p, c, a, s);
    } else {
        if (c.BN == 128) return c.KT == 64 ? go3<T, 128, 64>(p, c, a, s) : go3<T, 128, 32>(p, c, a, s);
        if (c.BN == 64) return c.KT == 64 ? go3<T, 64, 64>(p, c, a, s) : go3<T, 64, 32>(p, c, a, s);
        return c.KT == 64 ? go3<T, 32, 64>(p, c, a, s) : go3<T, 32, 32>(p, c, a, s);
    }
}

}  // namespace

bool supported(const Problem &p)
{
    Config c;
    return configure(p, c);
}

int tiles(const Problem &p, int *picked)
{
    const int saved = tile_choice();
    tile_choice() = -1;
    Config c;
    const bool ok = configure(p, c);
    tile_choice() = saved;
    int m[6][2];
    const int n = menu(p, m);
    *picked = 0;
    for (int i = 0; i < n; ++i)
        if (ok && m[i][0] == c.BN && m[i][1] == c.KT) *picked = i;
    return n < 1 ? 1 : n;
}

gconv_plan plan(const Problem &p)
{
    Config c;
    configure(p, c);
    gconv_plan pl{};
    pl.path = GCONV_PATH_IGEMM;
    pl.grid[0] = (uint32_t)c.mtiles;
    pl.grid[1] = (uint32_t)c.ntiles;
    pl.grid[2] = (uint32_t)p.G;
    pl.block = kBlock;
    pl.lds_bytes = (uint32_t)c.lds;
    pl.groups_per_tile = 1;
    return pl;
}

hipError_t launch(const Problem &p, const Args &a, hipStream_t s)
{
    Config c;
    if (!configure(p, c)) return hipErrorInvalidValue;
    if (p.dtype == GCONV_F32) return go<float>(p, c, a, s);
    if (p.dtype == GCONV_F16) return go<_Float16>(p, c, a, s);
    return go<__bf16>(p, c, a, s);
}

}  // namespace igemm
}  // namespace gconv

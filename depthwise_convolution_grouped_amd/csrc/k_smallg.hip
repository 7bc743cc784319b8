// Small-group direct convolution on the matrix cores (fp16 / bf16, 2D and 3D).
//
// Grouped conv with few channels per group (ResNeXt-style 8/8, the 3D 2/4 case
// of the TileOPs PR 1568 review) is a batch of tiny GEMMs: per group, M =
// output pixels, N = Kpg, K = taps * Cpg.  One v_mfma_f32_16x16x32 tile is
// 16 output channels x 16 pixels, so GN = 16 / Kpg consecutive groups share
// one tile (group merging, as num_groups_to_merge in the CK Python examples
// README, Config-options harness) and the weight operand is block diagonal:
// output channel n (group n / Kpg) only sees input channels of its own group.
//
// K is ordered (tap, 8-channel chunk), so every 8-element K slice of the input
// operand is one 16-byte vector of input channels at one tap: a single LDS
// read per lane.  The merged groups' CH = GN * Cpg input channels are
// contiguous in NDHWGC, CH / 8 chunks per tap.  The weights are the first
// MFMA operand and the inputs the second, so the accumulator comes out as
// D[channel][pixel]: each lane ends with four adjacent output channels of one
// pixel and stores them with one 8-byte write.
//
// Per workgroup: one image, a box of output pixels (TD x TH x TW) and a slab
// of NS merged-group tiles.  The input halo box for the slab is brought into
// LDS by direct-to-LDS buffer loads (zero padding from the buffer range
// check).  Each halo pixel occupies VPP + 1 16-byte slots: the odd stride
// spreads the 16 pixels of one read over all LDS banks, and the extra slot is
// zero, which is where lanes of an unused K slice read.  Each wave owns NTW
// tiles, keeps their weight fragments in registers and walks the box's
// 16-pixel M tiles, ending in the fused epilogue (bias, round, store).
#include "smallg_common.h"

namespace gconv {
namespace smallg {
namespace {

constexpr int kLdsTile = 80 * 1024;          // halo box budget (two workgroups per CU)

struct Params {
    int N, G, Cpg, Kpg, C, K;
    int D, H, W, Do, Ho, Wo, Z, Y, X;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int GN, CH8, slices, nmf, NT, NS, VPP, VS;   // merged tiles, K slices, slab vectors, pixel stride
    int TD, TH, TW, ID, IH, IW, MT;              // output box, halo box, M tiles per box
    int ntd, nth, ntw, nslab;
    Div dVS, dTW, dTH, dIH, dCPR;
    Div dCH8, dX, dY, dKpg, dCpg;                 // divisors of the fragment set-up
    int CPR;                                      // 64-slot chunks per halo row
    int stage_off, SP;                            // LDS byte offset of the output staging, bytes per staged pixel
    Div dSC;                                      // 16-byte chunks per staged pixel (2 NS)
    unsigned img_bytes;
};

// NMF: MFMAs per tile (>= nmf), NTW: merged-group tiles per wave, CPGC: the
// channels-per-group class (1, 2, 4, or 8 for any multiple of 8).
template <typename T, int NMF, int NTW, int CPGC>
__global__ __launch_bounds__(kBlock) void kernel(Params q, const T *__restrict__ x,
                                                 const T *__restrict__ w,
                                                 const T *__restrict__ bias, T *__restrict__ y)
{
    typedef typename Mfma<T>::V V;
    extern __shared__ uint4 halo[];
    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;

    // ---- which box: XCD-aware order, width tiles fastest
    const int nblocks = q.ntw * q.nth * q.ntd * q.nslab * q.N;
    int tile = xcd_tile((int)blockIdx.x, nblocks);
    const int tw = tile % q.ntw;   tile /= q.ntw;
    const int th = tile % q.nth;   tile /= q.nth;
    const int td = tile % q.ntd;   tile /= q.ntd;
    const int slab = tile % q.nslab;
    const int n = tile / q.nslab;
    const int od0 = td * q.TD, oh0 = th * q.TH, ow0 = tw * q.TW;
    const int id0 = od0 * q.sd - q.pd, ih0 = oh0 * q.sh - q.ph, iw0 = ow0 * q.sw - q.pw;
    const int vec0 = slab * q.NS * q.CH8;          // first channel vector of the slab
    const int cvec = q.C / 8;                      // channel vectors per input pixel
    const unsigned es = 2u;

    // ---- halo box -> LDS: slot P * VS + s holds channel vector s of halo
    // pixel P (s < VPP); slot VPP of every pixel is zero.  A halo row (fixed
    // depth and height) is IW * VS consecutive slots, fetched in 64-slot
    // chunks; (row, chunk) pairs are dealt round-robin to the waves.
    {
        const rsrc_t rs = make_rsrc(x + (size_t)n * q.D * q.H * q.W * q.C, q.img_bytes);
        const int rows = q.ID * q.IH;
        const int row_slots = q.IW * q.VS;
        const unsigned base = (unsigned)(size_t)halo;
        const int total = rows * q.CPR;
        for (int k = wave; k < total; k += kWaves) {
            const int r = fdiv(k, q.dCPR), c = k - r * q.CPR;     // wave-uniform
            const int pz = fdiv(r, q.dIH), py = r - pz * q.IH;
            const int j = c * 64 + lane;                           // slot within the row
            if (j < row_slots) {
                const int px = fdiv(j, q.dVS), sl = j - px * q.VS;
                const int gd = id0 + pz, gh = ih0 + py, gw = iw0 + px, gv = vec0 + sl;
                unsigned vo = kOob;
                if (sl < q.VPP && gv < cvec && gd >= 0 && gd < q.D && gh >= 0 && gh < q.H &&
                    gw >= 0 && gw < q.W)
                    vo = ((unsigned)((gd * q.H + gh) * q.W + gw) * (unsigned)q.C + (unsigned)gv * 8u) * es;
                const unsigned m0 = base + (unsigned)(r * row_slots + c * 64) * 16u;
                dma16(vo, __builtin_amdgcn_readfirstlane(m0), rs);
            }
        }
    }

    // ---- weight fragments of this wave's tiles (block diagonal), from w.
    // Lane (nn = lane % 16, kq = lane / 16) holds W[nn][8 kq + e] of each K
    // step: output channel nn against the 8 input channels of one (tap,
    // chunk) slice.  Only the channels of nn's own group are nonzero; they are
    // contiguous in w ([g][k][tap][c]).  Every lane loads unconditionally from
    // a clamped address and zeroes afterwards, so the loads issue together.
    const int nn = lane & 15, kq = lane >> 4;
    const int taps = q.Z * q.Y * q.X;
    V wfrag[NTW][NMF];
    int aoff[NTW][NMF];         // LDS byte offset of this lane's input slice, relative to its pixel
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int tl = wave * NTW + j;
        const int ntile = slab * q.NS + tl;
        const bool tile_ok = ntile < q.NT && tl < q.NS;
        const int g0 = tile_ok ? ntile * q.GN : 0;
        const int gout = fdiv(nn, q.dKpg), kout = nn - gout * q.Kpg;   // group within tile, channel
        const T *wk = w + ((size_t)(g0 + gout) * q.Kpg + kout) * taps * q.Cpg;
#pragma unroll
        for (int s = 0; s < NMF; ++s) {
            const int k8 = 4 * s + kq;
            const bool live = tile_ok && s < q.nmf && k8 < q.slices;
            const int kk = live ? k8 : 0;
            const int tap = fdiv(kk, q.dCH8), c = kk - tap * q.CH8;
            // input slice: tap offset inside the halo box, chunk of this tile;
            // an unused slice reads the zero slot of the lane's own pixel
            const int t1 = fdiv(tap, q.dX), xx = tap - t1 * q.X;
            const int zz = fdiv(t1, q.dY), yy = t1 - zz * q.Y;
            const int tp = ((zz * q.dd) * q.IH + yy * q.dh) * q.IW + xx * q.dw;
            aoff[j][s] = (live ? tp * q.VS + tl * q.CH8 + c : q.VPP) * 16;
            const uint4 raw = wslice<T, CPGC>(wk, tap, c, gout, q.dCpg, live);
            wfrag[j][s] = *reinterpret_cast<const V *>(&raw);
        }
    }
    // bias of the four output channels 4 kq .. 4 kq + 3 of each tile
    float bias_v[NTW][4];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int ntile = slab * q.NS + wave * NTW + j;
        const int chb = (ntile < q.NT ? ntile : 0) * 16 + 4 * kq;
        uint2 braw = make_uint2(0u, 0u);
        if (bias) braw = *reinterpret_cast<const uint2 *>(bias + chb);
        const T *bel = reinterpret_cast<const T *>(&braw);
#pragma unroll
        for (int i = 0; i < 4; ++i) bias_v[j][i] = bias ? to_f32(bel[i]) : 0.f;
    }

    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): halo and weights are in
    __syncthreads();

    const int box = q.TD * q.TH * q.TW;
    const int Do_Ho_Wo = q.Do * q.Ho * q.Wo;
    const char *hb = reinterpret_cast<const char *>(halo);
    char *stage = reinterpret_cast<char *>(halo) + q.stage_off;
    for (int mt = 0; mt < q.MT; ++mt) {
        // lane's pixel: m = lane % 16 of this M tile (reads clamped inside the box)
        const int pix = mt * 16 + nn;
        const int pc = min(pix, box - 1);
        const int r1 = fdiv(pc, q.dTW), ax = pc - r1 * q.TW;
        const int az = fdiv(r1, q.dTH), ay = r1 - az * q.TH;
        const char *pbase = hb + (size_t)((((az * q.sd) * q.IH + ay * q.sh) * q.IW + ax * q.sw) * q.VS) * 16;
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int tl = wave * NTW + j;               // tile within the slab
            const int ntile = slab * q.NS + tl;
            if (tl >= q.NS || ntile >= q.NT) continue;   // wave-uniform
            // all input slices of this tile first (one LDS wait), then the MFMAs
            V afrag[NMF];
#pragma unroll
            for (int s = 0; s < NMF; ++s) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(pbase + aoff[j][s]);
                afrag[s] = *reinterpret_cast<const V *>(&raw);
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NMF; ++s) acc = Mfma<T>::run(wfrag[j][s], afrag[s], acc);
            // acc[i] = output channel ntile*16 + 4 kq + i (= g*Kpg + k) of this lane's pixel
            if (pix < box) {
                T o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(acc[i] + bias_v[j][i]);
                *reinterpret_cast<uint2 *>(stage + pix * q.SP + tl * 32 + kq * 8) = *reinterpret_cast<const uint2 *>(o);
            }
        }
    }
    // ---- the box's outputs leave from the LDS staging area as whole runs of
    // the slab's channels per pixel (NS x 32 bytes), one 16-byte
    // non-temporal store per thread and chunk: 8-byte pieces of 16 pixels per
    // lane are much slower through the texture path
    __syncthreads();
    const int sc = 2 * q.NS;                        // 16-byte chunks per staged pixel
    const int ch0 = slab * q.NS * 16;               // first output channel of the slab
    const auto ry = __builtin_amdgcn_make_buffer_rsrc(y + (size_t)n * Do_Ho_Wo * q.K, (short)0,
                                                      (int)((unsigned)Do_Ho_Wo * (unsigned)q.K * 2u), 0x00020000);
    for (int k = t; k < box * sc; k += kBlock) {
        const int pix = fdiv(k, q.dSC), ck = k - pix * sc;
        const int r1 = fdiv(pix, q.dTW), ax = pix - r1 * q.TW;
        const int az = fdiv(r1, q.dTH), ay = r1 - az * q.TH;
        const int gd = od0 + az, gh = oh0 + ay, gw = ow0 + ax;
        const int ch = ch0 + ck * 8;
        const bool ok = gd < q.Do && gh < q.Ho && gw < q.Wo && ch < q.K;
        const uint4 v = *reinterpret_cast<const uint4 *>(stage + pix * q.SP + ck * 16);
        const unsigned go = ((unsigned)((gd * q.Ho + gh) * q.Wo + gw) * (unsigned)q.K + (unsigned)ch) * 2u;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, ry, ok ? go : kOob, 0, 2);
    }
}


// ----------------------------------------------------------------- host side

struct Config {
    int GN, CH8, slices, nmf, NMF, NTW, NT, NS, VPP, VS, CPR;
    int TD, TH, TW, ID, IH, IW, MT, ntd, nth, ntw, nslab, lds, stage_off;
};

int pick_nmf(int nmf)
{
    const int opts[] = {5, 7, 9, 16, 28};
    for (int o : opts)
        if (nmf <= o) return o;
    return 0;
}

bool shape_ok(const Problem &p)
{
    if (p.dtype != GCONV_F16 && p.dtype != GCONV_BF16) return false;
    if (p.Kpg < 1 || p.Kpg > 16 || 16 % p.Kpg != 0) return false;
    const int GN = 16 / p.Kpg;
    if (p.G % GN != 0) return false;
    if ((GN * p.Cpg) % 8 != 0) return false;
    if (!(p.Cpg == 1 || p.Cpg == 2 || p.Cpg == 4 || p.Cpg % 8 == 0)) return false;
    const int slices = p.taps() * GN * p.Cpg / 8;
    if (pick_nmf((slices + 3) / 4) == 0) return false;
    if ((long long)p.D * p.H * p.W * p.G * p.Cpg * 2 >= (1LL << 31)) return false;
    // one image of y must be addressable by a 32-bit buffer offset
    if ((long long)p.Do * p.Ho * p.Wo * p.G * p.Kpg * 2 >= (1LL << 31)) return false;
    return true;
}

bool configure(const Problem &p, Config &c)
{
    c.GN = 16 / p.Kpg;
    c.CH8 = c.GN * p.Cpg / 8;
    c.slices = p.taps() * c.CH8;
    c.nmf = (c.slices + 3) / 4;
    c.NMF = pick_nmf(c.nmf);
    c.NTW = c.NMF <= 5 ? 4 : (c.NMF <= 9 ? 2 : 1);
    c.NT = p.G / c.GN;
    c.NS = c.NT < kWaves * c.NTW ? c.NT : kWaves * c.NTW;
    c.VPP = c.NS * c.CH8;
    c.VS = c.VPP + 1;
    // output box: a few shapes (<= 128 pixels) scored by useful outputs per
    // MFMA row and per halo pixel, and by how well the grid fills the chip
    const int tds[] = {4, 2, 1}, ths[] = {16, 8, 4, 2, 1}, tws[] = {32, 28, 16, 14, 8, 7, 4, 2, 1};
    double best = -1.0;
    bool found = false;
    for (int TD : tds) {
        if (TD > p.Do && TD != 1) continue;
        for (int TH : ths) {
            if (TH > p.Ho && TH != 1) continue;
            for (int TW : tws) {
                if (TW > p.Wo && TW != 1) continue;
                const int pix = TD * TH * TW;
                if (pix > 128) continue;
                const int ID = (TD - 1) * p.sd + (p.Z - 1) * p.dd + 1;
                const int IH = (TH - 1) * p.sh + (p.Y - 1) * p.dh + 1;
                const int IW = (TW - 1) * p.sw + (p.X - 1) * p.dw + 1;
                const long long slots = (long long)ID * IH * IW * c.VS;
                const long long stage_bytes = (long long)((pix + 15) / 16 * 16) * (c.NS * 32 + 16);
                if (slots * 16 + stage_bytes > kLdsTile || slots >= 65536) continue;
                const int MT = (pix + 15) / 16;
                const int ntd = (p.Do + TD - 1) / TD, nth = (p.Ho + TH - 1) / TH, ntw = (p.Wo + TW - 1) / TW;
                const double useful = (double)p.Do * p.Ho * p.Wo / ((double)ntd * nth * ntw);
                const double blocks = (double)ntd * nth * ntw * ((c.NT + c.NS - 1) / c.NS) * p.N;
                const double fill = blocks >= 512.0 ? 1.0 : blocks / 512.0;
                const double score = useful / (MT * 16.0) * useful / (ID * IH * IW) * fill * (pix >= 64 ? 1.0 : 0.85);
                if (score > best) {
                    best = score;
                    found = true;
                    c.TD = TD; c.TH = TH; c.TW = TW; c.ID = ID; c.IH = IH; c.IW = IW;
                    c.MT = MT; c.ntd = ntd; c.nth = nth; c.ntw = ntw;
                    c.lds = (int)(slots * 16 + stage_bytes);
                    c.stage_off = (int)(slots * 16);
                }
            }
        }
    }
    if (!found) return false;
    c.CPR = (c.IW * c.VS + 63) / 64;
    c.nslab = (c.NT + c.NS - 1) / c.NS;
    const long long blocks = (long long)c.ntw * c.nth * c.ntd * c.nslab * p.N;
    return blocks < (1LL << 31) && (long long)c.ID * c.IH * c.CPR < 65536 &&
           c.IW * c.VS < 65536 && c.MT * 16 < 65536;
}

template <typename T, int NMF, int NTW, int CPGC>
hipError_t go4(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    Params q;
    q.N = p.N; q.G = p.G; q.Cpg = p.Cpg; q.Kpg = p.Kpg; q.C = p.C(); q.K = p.K();
    q.D = p.D; q.H = p.H; q.W = p.W; q.Do = p.Do; q.Ho = p.Ho; q.Wo = p.Wo;
    q.Z = p.Z; q.Y = p.Y; q.X = p.X;
    q.sd = p.sd; q.sh = p.sh; q.sw = p.sw; q.pd = p.pd; q.ph = p.ph; q.pw = p.pw;
    q.dd = p.dd; q.dh = p.dh; q.dw = p.dw;
    q.GN = c.GN; q.CH8 = c.CH8; q.slices = c.slices; q.nmf = c.nmf; q.NT = c.NT; q.NS = c.NS;
    q.VPP = c.VPP; q.VS = c.VS;
    q.TD = c.TD; q.TH = c.TH; q.TW = c.TW; q.ID = c.ID; q.IH = c.IH; q.IW = c.IW; q.MT = c.MT;
    q.ntd = c.ntd; q.nth = c.nth; q.ntw = c.ntw; q.nslab = c.nslab;
    q.dVS = make_div(c.VS); q.dTW = make_div(c.TW); q.dTH = make_div(c.TH);
    q.dIH = make_div(c.IH); q.dCPR = make_div(c.CPR); q.CPR = c.CPR;
    q.stage_off = c.stage_off; q.SP = c.NS * 32 + 16; q.dSC = make_div(2 * c.NS);
    q.dCH8 = make_div(c.CH8); q.dX = make_div(p.X); q.dY = make_div(p.Y);
    q.dKpg = make_div(p.Kpg); q.dCpg = make_div(p.Cpg);
    q.img_bytes = (unsigned)((long long)p.D * p.H * p.W * p.C() * 2);
    const int blocks = c.ntw * c.nth * c.ntd * c.nslab * p.N;
    auto k = kernel<T, NMF, NTW, CPGC>;
    static std::atomic<unsigned long long> lds_set{0};   // one attribute call per kernel instance and device
    if (c.lds > 64 * 1024) {
        const hipError_t e = allow_lds((const void *)k, lds_set, kLdsTile);
        if (e != hipSuccess) return e;
    }
    return enqueue(k, dim3(blocks), dim3(kBlock), c.lds, s, a, q, (const T *)a.x,
                   (const T *)a.w, (const T *)a.bias, (T *)a.y);
}

template <typename T, int CPGC>
hipError_t go3(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    switch (c.NMF) {
    case 5: return go4<T, 5, 4, CPGC>(p, c, a, s);
    case 7: return go4<T, 7, 2, CPGC>(p, c, a, s);
    case 9: return go4<T, 9, 2, CPGC>(p, c, a, s);
    case 16: return go4<T, 16, 1, CPGC>(p, c, a, s);
    default: return go4<T, 28, 1, CPGC>(p, c, a, s);
    }
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    switch (p.Cpg) {
    case 1: return go3<T, 1>(p, c, a, s);
    case 2: return go3<T, 2>(p, c, a, s);
    case 4: return go3<T, 4>(p, c, a, s);
    default: return go3<T, 8>(p, c, a, s);
    }
}

}  // namespace

namespace {

// Tile menu: the LDS ring (rows per workgroup 14 and 28 for 2D stride 1, 7 and
// 2 in 3D, its own value otherwise), then the row-streaming variant, then the halo
// box, each where it takes the problem.  The own pick is the first variant
// that applies, with the ring's own row count, except at stride 2, where the
// row-streaming variant measured faster than the ring (tile sweep: 1.2-1.3x
// on 16-channel groups).
enum Var { kRing, kRows, kBox };
struct Choice {
    int var, rows;
};

int menu(const Problem &p, Choice *m, int *own)
{
    int n = 0;
    *own = -1;
    // fp32 runs on the ring variant only (16x16x4 MFMAs)
    if (!shape_ok(p) && p.dtype != GCONV_F32) return 0;
    RingConfig gc;
    if (ring_configure(p, gc)) {
        if (p.ndim == 2 && p.sh == 1) {
            m[n++] = {kRing, 14};
            m[n++] = {kRing, 28};
            *own = gc.R == 28 ? 1 : 0;
        } else if (p.ndim == 3) {
            m[n++] = {kRing, 7};
            m[n++] = {kRing, 2};
            *own = gc.R == 2 ? 1 : 0;
        } else {
            m[n++] = {kRing, gc.R};
            *own = 0;
        }
    }
    if (p.dtype == GCONV_F32) return n;
    RowConfig rc;
    if (rows_configure(p, rc)) {
        if (*own < 0 || (p.ndim == 2 && p.sh == 2)) *own = n;
        m[n++] = {kRows, 0};
    }
    Config c;
    if (configure(p, c)) {
        if (*own < 0) *own = n;
        m[n++] = {kBox, 0};
    }
    return n;
}

Choice choose(const Problem &p)
{
    Choice m[4];
    int own = 0;
    const int n = menu(p, m, &own);
    const int t = tile_choice();
    if (n == 0) return {kBox, 0};
    return t >= 0 && t < n ? m[t] : m[own];
}

}  // namespace

bool supported(const Problem &p)
{
    Config c;
    RingConfig gc;
    if (p.dtype == GCONV_F32) return ring_configure(p, gc);
    return shape_ok(p) && configure(p, c);
}

bool streams(const Problem &p)
{
    RingConfig gc;
    RowConfig rc;
    if (p.dtype == GCONV_F32) return ring_configure(p, gc);
    return shape_ok(p) && (ring_configure(p, gc) || rows_configure(p, rc));
}

int tiles(const Problem &p, int *picked)
{
    Choice m[4];
    int own = 0;
    const int n = menu(p, m, &own);
    *picked = own < 0 ? 0 : own;
    return n < 1 ? 1 : n;
}

gconv_plan plan(const Problem &p)
{
    const Choice ch = choose(p);
    RingConfig gc;
    if (ch.var == kRing && ring_configure(p, gc)) {
        ring_set_rows(p, gc, ch.rows);
        gconv_plan pl{};
        pl.path = GCONV_PATH_SMALLG;
        pl.grid[0] = (uint32_t)gc.blocks;
        pl.grid[1] = pl.grid[2] = 1;
        pl.block = kBlock;
        pl.lds_bytes = (uint32_t)gc.lds;
        pl.groups_per_tile = (uint32_t)gc.GN;
        return pl;
    }
    RowConfig rc;
    if (ch.var == kRows && rows_configure(p, rc)) {
        gconv_plan pl{};
        pl.path = GCONV_PATH_SMALLG;
        pl.grid[0] = (uint32_t)(rc.nmt * rc.ntb * p.N);
        pl.grid[1] = pl.grid[2] = 1;
        pl.block = kBlock;
        pl.lds_bytes = 0;
        pl.groups_per_tile = (uint32_t)rc.GN;
        return pl;
    }
    Config c;
    configure(p, c);
    gconv_plan pl{};
    pl.path = GCONV_PATH_SMALLG;
    pl.grid[0] = (uint32_t)(c.ntw * c.nth * c.ntd * c.nslab * p.N);
    pl.grid[1] = pl.grid[2] = 1;
    pl.block = kBlock;
    pl.lds_bytes = (uint32_t)c.lds;
    pl.groups_per_tile = (uint32_t)c.GN;
    return pl;
}

hipError_t launch(const Problem &p, const Args &a, hipStream_t s)
{
    // 2D 3x3 windows (stride 1 or 2, no dilation) stream rows; the rest
    // stages halo boxes
    const Choice ch = choose(p);
    RingConfig gc;
    if (ch.var == kRing && (shape_ok(p) || p.dtype == GCONV_F32) && ring_configure(p, gc)) {
        ring_set_rows(p, gc, ch.rows);
        return ring_launch(p, gc, a, s);
    }
    if (p.dtype == GCONV_F32) return hipErrorInvalidValue;
    RowConfig rc;
    if (ch.var == kRows && shape_ok(p) && rows_configure(p, rc)) return rows_launch(p, rc, a, s);
    Config c;
    if (!configure(p, c)) return hipErrorInvalidValue;
    if (p.dtype == GCONV_F16) return go<_Float16>(p, c, a, s);
    return go<__bf16>(p, c, a, s);
}

}  // namespace smallg
}  // namespace gconv

// Depthwise direct convolution (Cpg = Kpg = 1, 2D): input rows streamed into an
// LDS ring by direct-to-LDS buffer loads, 16-byte channel vectors, fp32 FMA on
// the VALU, fused bias/convert epilogue.
//
// Depthwise conv is the G == C case of the grouped forward conv (TileOPs PR
// 1568 review, summary: MobileNetV2 depthwise benchmark cases).  With one
// input and one output channel per group there is no contraction for the
// matrix cores; the work is bound by HBM traffic (about 4.5 FLOP per byte for
// 3x3 fp16), so the kernel is built to read x and write y once each with long
// coalesced vector accesses and to keep many bytes in flight.
//
// Work decomposition.  A workgroup (4 waves) owns one image n, a strip of TW
// output columns, a slab of CV channel vectors (VEC channels, 16 bytes each)
// and a chunk of output rows.  Thread t computes channel vector t % CV of
// output column t / CV.  In NHWC a row segment of the strip is IW * CV
// vectors; when the slab spans all channels it is one contiguous run.
//
// Input rows live in an LDS ring of NR rows (ring row rr = ih + pad_h ->
// slot rr % NR).  Each row is fetched with buffer_load_dwordx4 ... lds: one
// instruction moves 64 consecutive 16-byte vectors (lane l -> LDS + 16 l)
// without passing through registers; offsets outside the image (padding,
// slab tail) are out of the buffer range and land as zeros.  Output rows are
// produced in bands of RB rows; a band needs IR = (RB-1)*SH + (Y-1)*DH + 1
// input rows and brings NEW = RB*SH new ones.  The loads of the next DEPTH
// bands are always in flight.  With NR = IR + (DEPTH+1)*NEW, the band issued
// at the top of iteration b lands in slots last read in iteration b-1, so one
// barrier per band orders every reuse of a slot.
//
// The compiler does not see these loads (inline asm), so it inserts no
// conservative wait before the LDS reads; each wave waits with s_waitcnt
// vmcnt for its own loads of the band it is about to read (loads return in
// order, and only loads issued after that band are allowed to stay
// outstanding), then the barrier makes every wave's rows visible.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace depthwise {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kLds = 160 * 1024;      // LDS per CU on gfx950
constexpr int kMaxLw = 12;            // ring-load instructions per wave per band
constexpr unsigned kOob = 0x80000000u; // buffer offset past any image: reads zero

struct Params {
    int N, C, Cv;          // images, channels, channel vectors
    int H, W, Ho, Wo;
    int sw, dw, ph, pw;
    int CV, TW, IW, P, NCH;// slab vectors, strip width out/in, vectors per row, 64-vector chunks per row
    int RH;                // output rows per workgroup (multiple of RB)
    int ncol, nslab, nchunk;
    int DEPTH, NR;         // bands in flight, ring rows
    unsigned img_bytes;    // bytes of one image of x
    unsigned w_bytes, b_bytes;  // bytes of w and of bias (0: no bias)
};

template <typename T> struct VecOf;
template <> struct VecOf<float> { static constexpr int n = 4; };
template <> struct VecOf<_Float16> { static constexpr int n = 8; };
template <> struct VecOf<__bf16> { static constexpr int n = 8; };

typedef int rsrc_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    const unsigned long long a = (unsigned long long)base;
    rsrc_t r;
    r.x = (int)(unsigned)(a & 0xffffffffull);
    r.y = (int)(unsigned)((a >> 32) & 0xffffull);   // stride 0
    r.z = (int)bytes;                                // num_records (bytes)
    r.w = 0x00020000;                                // raw 32-bit dword format
    return r;
}

// One direct-to-LDS 16-byte load per active lane: lane l writes LDS[m0 + 16 l].
__device__ __forceinline__ void dma16(unsigned voffset, unsigned lds_byte, rsrc_t r)
{
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
        GCONV_VMW(31) GCONV_VMW(32) GCONV_VMW(33) GCONV_VMW(34) GCONV_VMW(35) GCONV_VMW(36)
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;   // vmcnt(0)
    }
#undef GCONV_VMW
}

template <typename T, int SH, int DH>
struct Shape {
    static constexpr int Y = 3, X = 3;
    static constexpr int RB = 2;                          // output rows per band
    static constexpr int IR = (RB - 1) * SH + (Y - 1) * DH + 1;
    static constexpr int NEW = RB * SH;
};

template <typename T, int SH, int DH>
__global__ __launch_bounds__(kBlock) void kernel(Params q, const T *__restrict__ x,
                                                 const T *__restrict__ w,
                                                 const T *__restrict__ bias, T *__restrict__ y)
{
    using S = Shape<T, SH, DH>;
    constexpr int VEC = VecOf<T>::n, Y = S::Y, X = S::X, RB = S::RB, IR = S::IR, NEW = S::NEW;
    typedef T vecT __attribute__((ext_vector_type(VEC)));
    extern __shared__ uint4 ring[];

    // ---- tile (XCD-aware order, column strips fastest)
    const int nblocks = q.ncol * q.nslab * q.nchunk * q.N;
    int tile = xcd_tile((int)blockIdx.x, nblocks);
    const int col = tile % q.ncol;   tile /= q.ncol;
    const int slab = tile % q.nslab; tile /= q.nslab;
    const int chunk = tile % q.nchunk;
    const int n = tile / q.nchunk;

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int ow0 = col * q.TW;
    const int cv0 = slab * q.CV;
    const int oh_begin = chunk * q.RH;
    const int oh_end = min(oh_begin + q.RH, q.Ho);
    const int nbands = (oh_end - oh_begin + RB - 1) / RB;
    const int iw0 = ow0 * q.sw - q.pw;
    const unsigned ring_lds = (unsigned)(size_t)ring;
    const unsigned row_bytes = (unsigned)q.P * 16u;
    const rsrc_t rs = make_rsrc(x + (size_t)n * q.H * q.W * q.C, q.img_bytes);
    const unsigned es = (unsigned)sizeof(T);

    // Column part of the buffer offset of vector j of a ring row, or kOob.
    auto col_voff = [&](int j) -> unsigned {
        const int px = j / q.CV, cvl = j - (j / q.CV) * q.CV;
        const int iw = iw0 + px, cv = cv0 + cvl;
        if (iw < 0 || iw >= q.W || cv >= q.Cv) return kOob;
        return ((unsigned)iw * (unsigned)q.C + (unsigned)cv * VEC) * es;
    };
    auto row_voff = [&](int rr) -> int {   // ring row -> image row offset, or -1 outside
        const int ih = rr - q.ph;
        return (ih >= 0 && ih < q.H) ? ih * q.W * q.C * (int)es : -1;
    };

    // ---- this thread's output column / channel vector
    const int cvl = t % q.CV;
    const int owl = t / q.CV;
    const int ow = ow0 + owl;
    const int cv = cv0 + cvl;
    const bool active = owl < q.TW && ow < q.Wo && cv < q.Cv;

    // ---- prologue.  First the slab's weights and bias (the VEC channels of
    // one vector own Y*X*VEC consecutive weights, [c][y][x] with G = C and
    // Kpg = Cpg = 1, i.e. Y*X whole vectors; the slab's are contiguous), then
    // the first band's IR rows.  All of it travels by the same direct-to-LDS
    // loads, so nothing waits before the ring starts.
    constexpr int WV = Y * X * VEC * (int)sizeof(T) / 16;   // weight vectors per channel vector
    static_assert(Y * X * VEC * sizeof(T) % 16 == 0, "weight block must be whole vectors");
    const unsigned wlds = ring_lds + (unsigned)q.NR * row_bytes;   // CV * WV vectors
    const unsigned blds = wlds + (unsigned)(q.CV * WV) * 16u;      // CV vectors
    {
        const rsrc_t rw = make_rsrc(w + (size_t)cv0 * VEC * Y * X, q.w_bytes - (unsigned)cv0 * WV * 16u);
        const int nwv = q.CV * WV, nwc = (nwv + 63) / 64;
        for (int c = wave; c < nwc; c += kWaves)
            if (c * 64 + lane < nwv)
                dma16((unsigned)(c * 64 + lane) * 16u, __builtin_amdgcn_readfirstlane(wlds + (unsigned)c * 1024u), rw);
        if (q.b_bytes && wave == kWaves - 1) {
            const rsrc_t rb = make_rsrc(bias + (size_t)cv0 * VEC, q.b_bytes - (unsigned)cv0 * 16u);
            for (int c = 0; c * 64 < q.CV; ++c)
                if (c * 64 + lane < q.CV)
                    dma16((unsigned)(c * 64 + lane) * 16u, __builtin_amdgcn_readfirstlane(blds + (unsigned)c * 1024u), rb);
        }
    }
    const int rr_first = oh_begin * SH;
    {
        const int total = IR * q.NCH;
        for (int k = wave; k < total; k += kWaves) {
            const int r = k / q.NCH, c = k - (k / q.NCH) * q.NCH;
            const int j = c * 64 + lane;
            if (j < q.P) {
                const int ro = row_voff(rr_first + r);
                const unsigned cvo = col_voff(j);
                const unsigned vo = (ro < 0 || cvo == kOob) ? kOob : (unsigned)ro + cvo;
                const unsigned m0 = ring_lds + (unsigned)((rr_first + r) % q.NR) * row_bytes + (unsigned)c * 1024u;
                dma16(vo, __builtin_amdgcn_readfirstlane(m0), rs);
            }
        }
    }
    // Deeper bands are requested only once band 0 has landed: band 0 of every
    // workgroup then reaches the front of the memory queues first.

    // (computed while the prologue loads are in flight)
    // ---- per-thread plan of one band's loads: instruction k = wave + 4 i
    //      covers row k / NCH of the band and 64-vector chunk k % NCH.
    const int band_instr = NEW * q.NCH;
    int lw = 0;                                  // this wave's instructions per band
    unsigned plan_col[kMaxLw];                   // column offset (or kOob) of this lane
    int plan_row[kMaxLw], plan_chunk[kMaxLw];
    bool plan_lane[kMaxLw];                      // lane has a vector in that chunk
#pragma unroll
    for (int i = 0; i < kMaxLw; ++i) {
        const int k = wave + kWaves * i;
        plan_row[i] = 0; plan_chunk[i] = 0; plan_col[i] = kOob; plan_lane[i] = false;
        if (k < band_instr) {
            ++lw;
            plan_row[i] = k / q.NCH;
            plan_chunk[i] = k - plan_row[i] * q.NCH;
            const int j = plan_chunk[i] * 64 + lane;
            plan_lane[i] = j < q.P;
            if (plan_lane[i]) plan_col[i] = col_voff(j);
        }
    }
    // issue the NEW rows starting at ring row rr0; band index beyond the chunk -> all zeros
    auto issue_band = [&](int rr0, bool real) {
        int slot0 = rr0 % q.NR;
#pragma unroll
        for (int i = 0; i < kMaxLw; ++i) {
            if (i < lw) {
                int slot = slot0 + plan_row[i];
                if (slot >= q.NR) slot -= q.NR;
                const int ro = real ? row_voff(rr0 + plan_row[i]) : -1;
                const unsigned vo = (ro < 0 || plan_col[i] == kOob) ? kOob : (unsigned)ro + plan_col[i];
                const unsigned m0 = ring_lds + (unsigned)slot * row_bytes + (unsigned)plan_chunk[i] * 1024u;
                if (plan_lane[i]) dma16(vo, __builtin_amdgcn_readfirstlane(m0), rs);
            }
        }
    };

    T *yn = y + (size_t)n * q.Ho * q.Wo * q.C;
    const int cbase = owl * q.sw * q.CV + cvl;
    float wf[Y][X][VEC];
    float bf[VEC];
    for (int b = 0; b < nbands; ++b) {
        const int oh0 = oh_begin + b * RB;
        const int rr0 = oh0 * SH;
        // this wave's loads of band b are done when at most DEPTH * lw younger
        // ones remain (none yet for band 0)
        vm_wait(b == 0 ? 0 : q.DEPTH * lw);
        __syncthreads();
        if (b == 0) {
            // bands 1 .. DEPTH+1: the ring slots they use are all still free
            for (int d = 1; d <= q.DEPTH + 1; ++d)
                issue_band(rr_first + IR + (d - 1) * NEW, d < nbands);
        } else {
            // band b+DEPTH+1 lands in the slots band b-1 read before the barrier
            issue_band(rr0 + IR + q.DEPTH * NEW, b + 1 + q.DEPTH < nbands);
        }
        if (b == 0) {   // weights and bias arrived with the first band
            const uint4 *wl = reinterpret_cast<const uint4 *>(ring + q.NR * q.P) + (active ? cvl : 0) * WV;
            uint4 wraw[WV];
#pragma unroll
            for (int i = 0; i < WV; ++i) wraw[i] = wl[i];
            uint4 braw = make_uint4(0, 0, 0, 0);
            if (q.b_bytes) braw = (reinterpret_cast<const uint4 *>(ring + q.NR * q.P + q.CV * WV))[active ? cvl : 0];
            const T *wel = reinterpret_cast<const T *>(wraw);
            const T *bel = reinterpret_cast<const T *>(&braw);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
#pragma unroll
                for (int yy = 0; yy < Y; ++yy)
#pragma unroll
                    for (int xx = 0; xx < X; ++xx) wf[yy][xx][j] = to_f32(wel[(j * Y + yy) * X + xx]);
                bf[j] = q.b_bytes ? to_f32(bel[j]) : 0.f;
            }
        }

        float acc[RB][VEC];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[r][j] = 0.f;
        if (active) {
            const int slot0 = rr0 % q.NR;
#pragma unroll
            for (int ir = 0; ir < IR; ++ir) {
                int slot = slot0 + ir;
                if (slot >= q.NR) slot -= q.NR;
                const uint4 *row = ring + slot * q.P + cbase;
#pragma unroll
                for (int xx = 0; xx < X; ++xx) {
                    uint4 raw = row[xx * q.dw * q.CV];
                    vecT v = *reinterpret_cast<vecT *>(&raw);
                    float vf[VEC];
#pragma unroll
                    for (int j = 0; j < VEC; ++j) vf[j] = to_f32(v[j]);
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        const int dy = ir - r * SH;      // compile-time after unrolling
                        if (dy >= 0 && dy % DH == 0 && dy / DH < Y) {
#pragma unroll
                            for (int j = 0; j < VEC; ++j)
                                acc[r][j] = fmaf(vf[j], wf[dy / DH][xx][j], acc[r][j]);
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int oh = oh0 + r;
                if (oh < oh_end) {
                    vecT o;
#pragma unroll
                    for (int j = 0; j < VEC; ++j) o[j] = from_f32<T>(acc[r][j] + bf[j]);
                    *reinterpret_cast<vecT *>(yn + ((size_t)oh * q.Wo + ow) * q.C + cv * VEC) = o;
                }
            }
        }
    }
    // drain: no ring load may still be writing LDS when the workgroup retires
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// ----------------------------------------------------------------- host side

struct Config {
    int RB, IR, NEW, CV, TW, IW, P, NCH, RH, ncol, nslab, nchunk, DEPTH, NR, lds;
};

int vec_of(int dtype) { return dtype == GCONV_F32 ? 4 : 8; }

bool shape_ok(const Problem &p)
{
    if (p.ndim != 2 || p.Cpg != 1 || p.Kpg != 1) return false;
    if ((p.G % vec_of(p.dtype)) != 0) return false;
    if (p.Y != 3 || p.X != 3) return false;
    if ((p.sh != 1 && p.sh != 2) || (p.dh != 1 && p.dh != 2)) return false;
    // one image must be addressable by a 32-bit buffer offset
    if ((long long)p.H * p.W * p.G * elem_size(p.dtype) >= (1LL << 31)) return false;
    return true;
}

bool configure(const Problem &p, Config &c)
{
    const int VEC = vec_of(p.dtype);
    const int Cv = p.G / VEC;
    c.RB = 2;
    c.IR = (c.RB - 1) * p.sh + (p.Y - 1) * p.dh + 1;
    c.NEW = c.RB * p.sh;
    c.CV = Cv < 64 ? Cv : 64;
    c.TW = kBlock / c.CV;
    if (c.TW > p.Wo) c.TW = p.Wo;
    // largest strip whose ring fits; prefer deeper prefetch, then two workgroups per CU
    for (;;) {
        c.IW = (c.TW - 1) * p.sw + (p.X - 1) * p.dw + 1;
        c.P = c.IW * c.CV;
        c.NCH = (c.P + 63) / 64;
        bool fits = false;
        for (int depth = 3; depth >= 1 && !fits; --depth) {
            const int nr = c.IR + (depth + 1) * c.NEW;
            const int lw = (c.NEW * c.NCH + kWaves - 1) / kWaves;
            if (nr * c.P * 16 + c.CV * 10 * 16 <= kLds && lw <= kMaxLw && depth * lw <= 36) {
                c.DEPTH = depth;
                c.NR = nr;
                fits = true;
            }
        }
        if (fits) break;
        if (c.TW == 1) return false;
        --c.TW;
    }
    c.lds = c.NR * c.P * 16 + c.CV * 9 * 16 + c.CV * 16;
    const int per_cu = kLds / c.lds;
    c.ncol = (p.Wo + c.TW - 1) / c.TW;
    c.nslab = (Cv + c.CV - 1) / c.CV;
    // row chunks: about one workgroup per resident slot, whole bands each
    const long long strips = (long long)c.ncol * c.nslab * p.N;
    const long long slots = 256LL * (per_cu > 0 ? per_cu : 1);
    long long chunks = (slots + strips - 1) / strips;
    const int max_chunks = (p.Ho + c.RB - 1) / c.RB;
    if (chunks > max_chunks) chunks = max_chunks;
    if (chunks < 1) chunks = 1;
    const int bands = (int)(((p.Ho + chunks - 1) / chunks + c.RB - 1) / c.RB);
    c.RH = bands * c.RB;
    c.nchunk = (p.Ho + c.RH - 1) / c.RH;
    return strips * c.nchunk < (1LL << 31);
}

template <typename T, int SH, int DH>
hipError_t go3(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    Params q;
    q.N = p.N; q.C = p.G; q.Cv = p.G / VecOf<T>::n;
    q.H = p.H; q.W = p.W; q.Ho = p.Ho; q.Wo = p.Wo;
    q.sw = p.sw; q.dw = p.dw; q.ph = p.ph; q.pw = p.pw;
    q.CV = c.CV; q.TW = c.TW; q.IW = c.IW; q.P = c.P; q.NCH = c.NCH; q.RH = c.RH;
    q.ncol = c.ncol; q.nslab = c.nslab; q.nchunk = c.nchunk;
    q.DEPTH = c.DEPTH; q.NR = c.NR;
    q.img_bytes = (unsigned)((long long)p.H * p.W * p.G * sizeof(T));
    q.w_bytes = (unsigned)((long long)p.G * p.Y * p.X * sizeof(T));
    q.b_bytes = a.bias ? (unsigned)(p.G * sizeof(T)) : 0u;
    const int blocks = c.ncol * c.nslab * c.nchunk * p.N;
    auto k = kernel<T, SH, DH>;
    if (c.lds > 64 * 1024)
        hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, c.lds);
    return enqueue(k, dim3(blocks), dim3(kBlock), c.lds, s, a, q, (const T *)a.x,
                   (const T *)a.w, (const T *)a.bias, (T *)a.y);
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    if (p.sh == 1) return p.dh == 1 ? go3<T, 1, 1>(p, c, a, s) : go3<T, 1, 2>(p, c, a, s);
    return p.dh == 1 ? go3<T, 2, 1>(p, c, a, s) : go3<T, 2, 2>(p, c, a, s);
}

}  // namespace

bool supported(const Problem &p)
{
    Config c;
    return shape_ok(p) && configure(p, c);
}

gconv_plan plan(const Problem &p)
{
    Config c;
    configure(p, c);
    gconv_plan pl{};
    pl.path = GCONV_PATH_DEPTHWISE;
    pl.grid[0] = (uint32_t)(c.ncol * c.nslab * c.nchunk * p.N);
    pl.grid[1] = pl.grid[2] = 1;
    pl.block = kBlock;
    pl.lds_bytes = (uint32_t)c.lds;
    pl.groups_per_tile = (uint32_t)(c.CV * vec_of(p.dtype));
    return pl;
}

hipError_t launch(const Problem &p, const Args &a, hipStream_t s)
{
    Config c;
    if (!configure(p, c)) return hipErrorInvalidValue;
    switch (p.dtype) {
    case GCONV_F32: return go<float>(p, c, a, s);
    case GCONV_F16: return go<_Float16>(p, c, a, s);
    default: return go<__bf16>(p, c, a, s);
    }
}

}  // namespace depthwise
}  // namespace gconv

// Depthwise direct convolution (Cpg = Kpg = 1, 2D, 3x3 window): every wave
// streams its own input rows straight into registers, with 16-byte channel
// vectors, fp32 accumulation on the VALU and a fused bias/convert epilogue.
//
// Depthwise conv is the G == C case of the grouped forward conv (TileOPs PR
// 1568 review, summary: MobileNetV2 depthwise benchmark cases).  With one
// input and one output channel per group there is no contraction for the
// matrix cores; the work is bound by HBM traffic (about 4.5 FLOP per byte for
// 3x3 fp16), so the kernel is built like a copy: each byte of x and y crosses
// HBM once, every access is a long coalesced 16-byte-per-lane buffer access,
// and nothing makes waves wait for one another (no LDS, no barriers).
//
// Work decomposition.  An output row of one image, flattened NHWC style, is
// Wo * Cv channel vectors (Cv = C / VEC, VEC channels per 16 bytes).  A wave
// owns 64 consecutive ones of them (lane -> output column ow and channel
// vector cv) over R consecutive output rows; a workgroup is four such waves
// side by side.  The wave walks the (R - 1) * SH + 2 * DH + 1 input rows that
// the R output rows need, in order.  Each input row costs three 16-byte loads
// per lane (the three window columns; a neighbour's loads of the same bytes
// hit in the caches) and is folded into every output row whose window covers
// it (input stationary), so an output row is written as soon as its last
// input row has been folded in.  The whole walk is unrolled into one basic
// block of straight-line code: the compiler is free to issue loads for rows
// far ahead of the arithmetic, which is what hides the HBM latency.
//
// Zero padding and ragged edges cost no branches: a column outside the image
// (or a lane past the row) gets a buffer offset beyond the buffer's range, so
// its loads return zeros and its stores are dropped by the hardware; a row
// outside the image gets the same treatment for all lanes.
//
// fp16: no element is ever converted.  The taps of window columns 0 and 1
// go through v_dot2_f32_f16 (two fp16 products summed into an fp32
// accumulator) on (x[dx=0], x[dx=1]) pairs built once per input row with one
// byte permute per channel, and column 2 through v_fma_mix_f32, which reads
// both fp16 factors in place (either half of a register) and accumulates in
// fp32.  Both run at the same rate, so 9 taps cost 6 instructions.  bf16 and
// fp32 convert the input once per load and keep the weights in fp32.
#include <utility>

#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace depthwise {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTargetWaves = 1024;      // one wave per SIMD
constexpr unsigned kOob = 0x80000000u;   // buffer offset past any image: loads zero, stores dropped
constexpr int kRawBuffer = 0x00020000;   // buffer descriptor word 3: raw 32-bit dwords
// Cache policy of the accesses (buffer instruction bits: 1 sc0, 2 nt,
// 16 sc1).  y is written once and never read back, so its stores are
// non-temporal, which lets the memory system stream them (measured: about
// 10% faster for this kernel).  x stays on the default policy: its halo rows
// and the neighbouring window columns are re-read from L1/L2, and
// non-temporal loads lose those hits.
constexpr int kLoadPolicy = 0;
constexpr int kStorePolicy = 2;

struct Params {
    int C, Cv;             // channels, channel vectors per pixel
    int H, W, Ho, Wo;
    int sw, dw, ph, pw;
    int nseg;              // 64-vector segments per output row
    int nsb, nchunk;       // segment blocks (4 segments) per row, row chunks per image
    unsigned in_row, out_row;       // bytes of one row of x / of y
    unsigned img_bytes, oimg_bytes; // bytes of one image of x / of y
    unsigned w_bytes, b_bytes;      // bytes of w and of bias (0: no bias)
    int flip;              // read each channel's window reversed (w[t] as w[8 - t])
};

template <typename T> struct VecOf { static constexpr int n = 16 / (int)sizeof(T); };

// f(integral_constant<int, I>) for I = 0, 1, ..., in order
template <int... Is, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Is...>, F &&f)
{
    (f(std::integral_constant<int, Is>{}), ...);
}

typedef unsigned u4 __attribute__((ext_vector_type(4)));

// The lane's 9 * VEC weights (channel e, tap t at element 9 e + t, VEC
// channels in nine 16-byte vectors) with every channel's taps reversed:
// element 9 e + t takes element 9 e + 8 - t.  Indices are compile-time, so
// this is register moves (and half-word merges for 2-byte types).
template <typename T>
__device__ __forceinline__ void reverse_taps(u4 (&w)[9])
{
    constexpr int ES = (int)sizeof(T);
    constexpr int VEC = 16 / ES;
    auto src_of = [](int k) { return (k / 9) * 9 + 8 - k % 9; };
    u4 o[9];
    if constexpr (ES == 4) {
#pragma unroll
        for (int k = 0; k < 9 * VEC; ++k) {
            const int sidx = src_of(k);
            o[k >> 2][k & 3] = w[sidx >> 2][sidx & 3];
        }
    } else {
        auto half_at = [&](int k) -> unsigned {
            const unsigned d = w[k >> 3][(k & 7) >> 1];
            return (k & 1) ? (d >> 16) : (d & 0xffffu);
        };
#pragma unroll
        for (int d = 0; d < 9 * VEC / 2; ++d) {
            const unsigned lo = half_at(src_of(2 * d)), hi = half_at(src_of(2 * d + 1));
            o[d >> 2][d & 3] = lo | (hi << 16);
        }
    }
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = o[i];
}
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// acc += a.lo * b.lo + a.hi * b.hi (fp16 pairs, fp32 accumulation)
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float acc)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), acc, false);
}
// (half S0 of r0, half S1 of r1) as one fp16 pair
template <int S0, int S1> __device__ __forceinline__ unsigned pair_halves(unsigned r0, unsigned r1)
{
    constexpr unsigned sel = (2u * S0) | ((2u * S0 + 1u) << 8) | ((4u + 2u * S1) << 16) | ((5u + 2u * S1) << 24);
    return __builtin_amdgcn_perm(r1, r0, sel);
}

// acc + x.half(XS) * w.half(WS), both fp16, accumulated in fp32: written as
// a plain fma of widened halves, which the compiler emits as one
// v_fma_mix_f32 (op_sel picks the halves), and being ordinary code it is
// covered by the compiler's hazard checks.
template <int XS, int WS>
__device__ __forceinline__ float fma_mix(unsigned xr, unsigned wr, float acc)
{
    const h2 xh = __builtin_bit_cast(h2, xr), wh = __builtin_bit_cast(h2, wr);
    return __builtin_fmaf((float)xh[XS], (float)wh[WS], acc);
}

// Element e of a 16-byte vector as fp32 (bf16 / fp32 inputs).
template <typename T> __device__ __forceinline__ float elem_f32(const u4 &v, int e);
template <> __device__ __forceinline__ float elem_f32<float>(const u4 &v, int e)
{
    const unsigned r = v[e];   // (bit-casting the element expression itself reads element 0)
    return __builtin_bit_cast(float, r);
}
template <> __device__ __forceinline__ float elem_f32<__bf16>(const u4 &v, int e)
{
    const unsigned r = v[e >> 1];
    return __builtin_bit_cast(float, (e & 1) ? (r & 0xffff0000u) : (r << 16));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBuffer);
}

template <typename T, int SH, int DH, int R, int PF>
__global__ __launch_bounds__(kBlock) void kernel(Params q, const T *__restrict__ x,
                                                 const T *__restrict__ w,
                                                 const T *__restrict__ bias, T *__restrict__ y)
{
    constexpr int VEC = VecOf<T>::n;
    constexpr int NI = (R - 1) * SH + 2 * DH + 1;      // input rows of R output rows
    constexpr bool kF16 = __is_same(T, _Float16);

    // ---- tile: (image, row chunk, block of 4 segments); neighbours in the
    //      tile order share halo rows and columns, so keep them on one XCD
    int tile = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int sb = tile % q.nsb;   tile /= q.nsb;
    const int chunk = tile % q.nchunk;
    const int n = tile / q.nchunk;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    const int seg = sb * kWaves + wave;
    if (seg >= q.nseg) return;     // whole wave idle (last block of a row)

    const int j = seg * 64 + lane;
    const bool jok = j < q.Wo * q.Cv;
    const int ow = j / q.Cv, cv = j - (j / q.Cv) * q.Cv;
    const unsigned es = (unsigned)sizeof(T);
    unsigned coff[3];              // byte offset of the lane's vector in an input row, per window column
#pragma unroll
    for (int dx = 0; dx < 3; ++dx) {
        const int iw = ow * q.sw - q.pw + dx * q.dw;
        coff[dx] = (jok && iw >= 0 && iw < q.W) ? ((unsigned)iw * (unsigned)q.C + (unsigned)cv * VEC) * es : kOob;
    }
    const unsigned ooff = jok ? ((unsigned)ow * (unsigned)q.C + (unsigned)cv * VEC) * es : kOob;

    const auto rx = rsrc(x + (size_t)n * q.H * q.W * q.C, q.img_bytes);
    const auto ry = rsrc(y + (size_t)n * q.Ho * q.Wo * q.C, q.oimg_bytes);

    // ---- weights of the lane's VEC channels: [c][y][x], 9 * VEC consecutive
    //      elements = 9 vectors; bias: one vector (zeros without bias)
    const auto rw = rsrc(w, q.w_bytes);
    u4 wraw[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) wraw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (unsigned)(cv * 9 + i) * 16u, 0, 0);
    if (q.flip) reverse_taps<T>(wraw);
    const auto rb = rsrc(bias, q.b_bytes);
    const u4 braw = __builtin_amdgcn_raw_buffer_load_b128(rb, q.b_bytes ? (unsigned)cv * 16u : kOob, 0, 0);
    // weight (e, dy, dx) is element e * 9 + dy * 3 + dx of the lane's 9 * VEC.
    // fp16: the (dx = 0, dx = 1) weights of each (e, dy) as one fp16 pair for
    // v_dot2, and the dx = 2 weights of channels (2m, 2m + 1) as one pair for
    // v_fma_mix (36 registers in all, like the raw block).
    unsigned wp[kF16 ? 3 : 1][kF16 ? VEC : 1];
    unsigned w2[kF16 ? 3 : 1][kF16 ? VEC / 2 : 1];
    if constexpr (kF16) {
#pragma unroll
        for (int m = 0; m < VEC / 2; ++m)
#pragma unroll
            for (int dy = 0; dy < 3; ++dy) {
                const int k0 = 2 * m * 9 + dy * 3 + 2, k1 = k0 + 9;
                const unsigned r0 = wraw[k0 >> 3][(k0 & 7) >> 1], r1 = wraw[k1 >> 3][(k1 & 7) >> 1];
                if (k0 & 1) w2[dy][m] = pair_halves<1, 0>(r0, r1);   // k1 = k0 + 9 has the other parity
                else w2[dy][m] = pair_halves<0, 1>(r0, r1);
            }
#pragma unroll
        for (int e = 0; e < VEC; ++e)
#pragma unroll
            for (int dy = 0; dy < 3; ++dy) {
                const int k = e * 9 + dy * 3;
                const unsigned lo = wraw[k >> 3][(k & 7) >> 1];
                const int k1 = k + 1;
                const unsigned hi = wraw[k1 >> 3][(k1 & 7) >> 1];
                wp[dy][e] = (k & 1) ? pair_halves<1, 0>(lo, hi) : lo;
            }
    }
    float wf[kF16 ? 1 : VEC][3][3];
    if constexpr (!kF16) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                const int k = e * 9 + t;
                wf[e][t / 3][t % 3] = elem_f32<T>(wraw[k / VEC], k % VEC);
            }
    }

    const int oh0 = chunk * R;
    const int ih0 = oh0 * SH - q.ph;
    float acc[R][VEC];
#pragma unroll
    for (int o = 0; o < R; ++o)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[o][e] = 0.f;

    // Input row i, three window columns (zeros outside the image).
    u4 xbuf[NI][3];
    auto load_row = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int ih = ih0 + i;
        const bool rok = ih >= 0 && ih < q.H;
        const unsigned soff = rok ? (unsigned)ih * q.in_row : 0u;
#pragma unroll
        for (int dx = 0; dx < 3; ++dx)
            xbuf[i][dx] = __builtin_amdgcn_raw_buffer_load_b128(rx, rok ? coff[dx] : kOob, soff, kLoadPolicy);
    };
    // The loads run PF rows ahead of the arithmetic; the scheduling barriers
    // keep the compiler from sinking them next to their use.
    static_for(std::make_integer_sequence<int, (PF < NI ? PF : NI)>{}, load_row);
    // one input row per step; i is a compile-time constant in each step, so
    // the row -> output-row mapping below costs nothing at run time
    static_for(std::make_integer_sequence<int, NI>{}, [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + PF < NI) load_row(std::integral_constant<int, i + PF>{});
        __builtin_amdgcn_sched_barrier(0);
        const u4 *xv = xbuf[i];
        unsigned xp[kF16 ? VEC : 1];   // fp16: (dx = 0, dx = 1) input pair of each channel
        if constexpr (kF16) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                xp[e] = (e & 1) ? pair_halves<1, 1>(xv[0][e >> 1], xv[1][e >> 1])
                                : pair_halves<0, 0>(xv[0][e >> 1], xv[1][e >> 1]);
        }
        float xf[kF16 ? 1 : 3][VEC];
        if constexpr (!kF16) {
#pragma unroll
            for (int dx = 0; dx < 3; ++dx)
#pragma unroll
                for (int e = 0; e < VEC; ++e) xf[dx][e] = elem_f32<T>(xv[dx], e);
        }
        // fold row i into every output row o with o * SH + dy * DH == i
        static_for(std::make_integer_sequence<int, 3>{}, [&](auto dyc) __attribute__((always_inline)) {
            constexpr int dy = decltype(dyc)::value;
            constexpr int d = i - dy * DH;
            if constexpr (d >= 0 && d % SH == 0 && d / SH < R) {
                constexpr int o = d / SH;
                if constexpr (kF16) {
                    // dx = 0 and 1 in one v_dot2, dx = 2 by v_fma_mix
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        acc[o][e] = dot2(xp[e], wp[dy][e], acc[o][e]);
                        if (e & 1) acc[o][e] = fma_mix<1, 1>(xv[2][e >> 1], w2[dy][e >> 1], acc[o][e]);
                        else acc[o][e] = fma_mix<0, 0>(xv[2][e >> 1], w2[dy][e >> 1], acc[o][e]);
                    }
                } else {
#pragma unroll
                    for (int dx = 0; dx < 3; ++dx)
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[o][e] = fmaf(xf[dx][e], wf[e][dy][dx], acc[o][e]);
                }
            }
        });
        // the output row whose window ends at input row i is complete
        constexpr int dl = i - 2 * DH;
        if constexpr (dl >= 0 && dl % SH == 0 && dl / SH < R) {
            constexpr int o = dl / SH;
            const int oh = oh0 + o;
            const T *bel = reinterpret_cast<const T *>(&braw);
            T ov[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) ov[e] = from_f32<T>(acc[o][e] + to_f32(bel[e]));
            const u4 packed = *reinterpret_cast<const u4 *>(ov);
            const bool ook = oh < q.Ho;
            __builtin_amdgcn_raw_buffer_store_b128(packed, ry, ook ? ooff : kOob, ook ? (unsigned)oh * q.out_row : 0u, kStorePolicy);
        }
    });
}

// ----------------------------------------------------------------- host side

struct Config {
    int R, nseg, nsb, nchunk;
};

int vec_of(int dtype) { return dtype == GCONV_F32 ? 4 : 8; }

bool shape_ok(const Problem &p)
{
    if (p.ndim != 2 || p.Cpg != 1 || p.Kpg != 1) return false;
    if ((p.G % vec_of(p.dtype)) != 0) return false;
    if (p.Y != 3 || p.X != 3) return false;
    if ((p.sh != 1 && p.sh != 2) || (p.dh != 1 && p.dh != 2)) return false;
    // one image of x and of y must be addressable by a 32-bit buffer offset
    const long long es = elem_size(p.dtype);
    if ((long long)p.H * p.W * p.G * es >= (1LL << 31)) return false;
    if ((long long)p.Ho * p.Wo * p.G * es >= (1LL << 31)) return false;
    return true;
}

bool configure(const Problem &p, Config &c)
{
    const int Cv = p.G / vec_of(p.dtype);
    const long long row_vecs = (long long)p.Wo * Cv;
    c.nseg = (int)((row_vecs + 63) / 64);
    c.nsb = (c.nseg + kWaves - 1) / kWaves;
    // Rows per wave: long runs amortise the 2 * DH halo rows and the setup
    // (weights, offsets), short runs give more waves to hide latency with.
    // Measured on the MobileNetV2 shapes, about one wave per SIMD (1024 in
    // all) with the longest run that gives is best; R comes from a small menu
    // of compiled run lengths (shorter for stride 2, whose runs read twice
    // the rows).  The tile sweep over random shapes found the next longer
    // run still best up to 1.5x the run that gives 1024 waves.
    const long long wave_rows = (long long)p.Ho * c.nseg * p.N;
    const long long want = (wave_rows + kTargetWaves - 1) / kTargetWaves;
    c.R = 4;
    for (int r : {7, 14, 28})
        if (2 * r <= 3 * want && (p.sh == 1 || r <= 14)) c.R = r;
    // no run past the image, and no ragged last run where the image's whole
    // height is a menu entry at most twice the run: the held-out tile sweep
    // measured both 1.2-1.4x faster on 7-row images
    while (c.R > 4 && c.R > p.Ho) c.R = c.R == 28 ? 14 : c.R == 14 ? 7 : 4;
    for (int r : {7, 14, 28})
        if (r == p.Ho && p.Ho % c.R != 0 && r <= 2 * c.R && (p.sh == 1 || r <= 14)) c.R = r;
    // tile menu: R = 4, 7, 14 (and 28 at stride 1)
    const int t = tile_choice();
    if (t >= 0 && t < (p.sh == 1 ? 4 : 3)) c.R = t == 0 ? 4 : t == 1 ? 7 : t == 2 ? 14 : 28;
    c.nchunk = (p.Ho + c.R - 1) / c.R;
    return row_vecs < (1LL << 30) && (long long)c.nsb * c.nchunk * p.N < (1LL << 31);
}

template <typename T, int SH, int DH, int R, int PF>
hipError_t go4(const Problem &p, const Config &c, const Args &a, hipStream_t s, bool flip)
{
    Params q;
    q.flip = flip ? 1 : 0;
    q.C = p.G; q.Cv = p.G / VecOf<T>::n;
    q.H = p.H; q.W = p.W; q.Ho = p.Ho; q.Wo = p.Wo;
    q.sw = p.sw; q.dw = p.dw; q.ph = p.ph; q.pw = p.pw;
    q.nseg = c.nseg; q.nsb = c.nsb; q.nchunk = c.nchunk;
    q.in_row = (unsigned)((long long)p.W * p.G * sizeof(T));
    q.out_row = (unsigned)((long long)p.Wo * p.G * sizeof(T));
    q.img_bytes = (unsigned)((long long)p.H * p.W * p.G * sizeof(T));
    q.oimg_bytes = (unsigned)((long long)p.Ho * p.Wo * p.G * sizeof(T));
    q.w_bytes = (unsigned)((long long)p.G * 9 * sizeof(T));
    q.b_bytes = a.bias ? (unsigned)(p.G * sizeof(T)) : 0u;
    const int blocks = c.nsb * c.nchunk * p.N;
    return enqueue(kernel<T, SH, DH, R, PF>, dim3(blocks), dim3(kBlock), 0, s, a, q, (const T *)a.x,
                   (const T *)a.w, (const T *)a.bias, (T *)a.y);
}

template <typename T, int R>
hipError_t go3(const Problem &p, const Config &c, const Args &a, hipStream_t s, bool flip)
{
    if (p.sh == 1)
        return p.dh == 1 ? go4<T, 1, 1, R, 3>(p, c, a, s, flip) : go4<T, 1, 2, R, 3>(p, c, a, s, flip);
    if constexpr (R <= 14)
        return p.dh == 1 ? go4<T, 2, 1, R, 3>(p, c, a, s, flip) : go4<T, 2, 2, R, 3>(p, c, a, s, flip);
    return hipErrorInvalidValue;   // configure() never picks R > 14 for stride 2
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s, bool flip)
{
    switch (c.R) {
    case 4: return go3<T, 4>(p, c, a, s, flip);
    case 7: return go3<T, 7>(p, c, a, s, flip);
    case 14: return go3<T, 14>(p, c, a, s, flip);
    default: return go3<T, 28>(p, c, a, s, flip);
    }
}

hipError_t launch_as(const Problem &p, const Args &a, hipStream_t s, bool flip)
{
    Config c;
    if (!configure(p, c)) return hipErrorInvalidValue;
    switch (p.dtype) {
    case GCONV_F32: return go<float>(p, c, a, s, flip);
    case GCONV_F16: return go<_Float16>(p, c, a, s, flip);
    default: return go<__bf16>(p, c, a, s, flip);
    }
}

}  // namespace

bool supported(const Problem &p)
{
    Config c;
    return shape_ok(p) && configure(p, c);
}

int tiles(const Problem &p, int *picked)
{
    const int saved = tile_choice();
    tile_choice() = -1;
    Config c;
    configure(p, c);
    tile_choice() = saved;
    *picked = c.R == 4 ? 0 : c.R == 7 ? 1 : c.R == 14 ? 2 : 3;
    return p.sh == 1 ? 4 : 3;
}

gconv_plan plan(const Problem &p)
{
    Config c;
    configure(p, c);
    gconv_plan pl{};
    pl.path = GCONV_PATH_DEPTHWISE;
    pl.grid[0] = (uint32_t)(c.nsb * c.nchunk * p.N);
    pl.grid[1] = pl.grid[2] = 1;
    pl.block = kBlock;
    pl.lds_bytes = 0;
    pl.groups_per_tile = (uint32_t)vec_of(p.dtype);
    return pl;
}

hipError_t launch(const Problem &p, const Args &a, hipStream_t s) { return launch_as(p, a, s, false); }

hipError_t launch_flipped(const Problem &p, const Args &a, hipStream_t s) { return launch_as(p, a, s, true); }

}  // namespace depthwise
}  // namespace gconv

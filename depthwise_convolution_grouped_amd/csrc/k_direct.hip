// Register-blocked direct kernels on the vector ALUs: the path for grouped
// problems the matrix-core kernels do not take (group widths off the
// 4-channel grid, and what fp32 leaves to it; the TileOPs PR 1568 review's
// grouped kernels and the CK tile engine's datatypes include fp32; CK
// grouped_conv tile-engine README, Hardware).  Two kernels: the per-thread
// one below, and a wave-uniform-weight one further down.
//
// A thread owns KB output channels of one group x PW consecutive output
// pixels of one output row.  For each tap of the window and each vector of
// VC input channels of the group it loads the PW input vectors (one per
// output pixel, shared by its KB channels) and the KB weight vectors (shared
// by its PW pixels) and does KB x PW x VC fused multiply-adds in fp32, so a
// 16-byte load feeds up to 32 FMAs.  Consecutive threads take consecutive
// (channel block, group) pairs of the same pixels: their x loads are
// neighbouring channel vectors of one pixel and their stores neighbouring
// runs of its output channels.  Taps outside the input contribute nothing
// (their loads are skipped).  The epilogue adds the bias, rounds once and
// stores.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace direct {
namespace {

constexpr int kBlock = 256;
constexpr int kPW = 4;                  // output pixels per thread along a row
constexpr long long kMinThreads = 32768;  // below this the generic kernel's split reductions win

template <typename T, int VC> struct VecT;
template <typename T> struct VecT<T, 1> {
    static __device__ __forceinline__ void load(const T *p, float (&v)[1]) { v[0] = to_f32(p[0]); }
};
template <> struct VecT<float, 4> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[4])
    {
        const float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
};
template <typename T> struct VecT<T, 4> {   // fp16 / bf16: 8 bytes
    static __device__ __forceinline__ void load(const T *p, float (&v)[4])
    {
        const uint2 q = *reinterpret_cast<const uint2 *>(p);
        const T *e = reinterpret_cast<const T *>(&q);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = to_f32(e[i]);
    }
};

template <typename T, int KB, int VC>
__global__ __launch_bounds__(kBlock) void kernel(Problem p, const T *__restrict__ x, const T *__restrict__ w,
                                                 const T *__restrict__ bias, T *__restrict__ y, int nkb,
                                                 int nwb, int total)
{
    const int tid = blockIdx.x * kBlock + threadIdx.x;
    if (tid >= total) return;
    int r = tid;
    const int kb = r % nkb;   r /= nkb;
    const int g = r % p.G;    r /= p.G;
    const int wb = r % nwb;   r /= nwb;
    const int oh = r % p.Ho;  r /= p.Ho;
    const int od = r % p.Do;
    const int n = r / p.Do;
    const int k0 = kb * KB, ow0 = wb * kPW;
    const int C = p.G * p.Cpg, K = p.G * p.Kpg, taps = p.Z * p.Y * p.X;
    float acc[KB][kPW];
#pragma unroll
    for (int a = 0; a < KB; ++a)
#pragma unroll
        for (int j = 0; j < kPW; ++j) acc[a][j] = 0.f;
    for (int z = 0; z < p.Z; ++z) {
        const int id = od * p.sd - p.pd + z * p.dd;
        if (id < 0 || id >= p.D) continue;
        for (int yy = 0; yy < p.Y; ++yy) {
            const int ih = oh * p.sh - p.ph + yy * p.dh;
            if (ih < 0 || ih >= p.H) continue;
            const T *xrow = x + ((size_t)((n * p.D + id) * p.H + ih) * p.W) * C + g * p.Cpg;
            for (int xx = 0; xx < p.X; ++xx) {
                const int tap = (z * p.Y + yy) * p.X + xx;
                const T *wt = w + ((size_t)(g * p.Kpg + k0) * taps + tap) * p.Cpg;
                int iw[kPW];
                bool ok[kPW];
#pragma unroll
                for (int j = 0; j < kPW; ++j) {
                    iw[j] = (ow0 + j) * p.sw - p.pw + xx * p.dw;
                    ok[j] = ow0 + j < p.Wo && iw[j] >= 0 && iw[j] < p.W;
                }
                for (int c = 0; c < p.Cpg; c += VC) {
                    float xv[kPW][VC], wv[KB][VC];
#pragma unroll
                    for (int j = 0; j < kPW; ++j) {
                        if (ok[j]) VecT<T, VC>::load(xrow + (size_t)iw[j] * C + c, xv[j]);
                        else
#pragma unroll
                            for (int v = 0; v < VC; ++v) xv[j][v] = 0.f;
                    }
#pragma unroll
                    for (int a = 0; a < KB; ++a) VecT<T, VC>::load(wt + (size_t)a * taps * p.Cpg + c, wv[a]);
#pragma unroll
                    for (int v = 0; v < VC; ++v)
#pragma unroll
                        for (int a = 0; a < KB; ++a)
#pragma unroll
                            for (int j = 0; j < kPW; ++j) acc[a][j] = fmaf(xv[j][v], wv[a][v], acc[a][j]);
                }
            }
        }
    }
    const int ch0 = g * p.Kpg + k0;
#pragma unroll
    for (int j = 0; j < kPW; ++j) {
        if (ow0 + j >= p.Wo) continue;
        T *yp = y + ((size_t)((n * p.Do + od) * p.Ho + oh) * p.Wo + ow0 + j) * K + ch0;
#pragma unroll
        for (int a = 0; a < KB; ++a) yp[a] = finish<T>(acc[a][j], bias, ch0 + a);
    }
}

// Wave-uniform weights.  A wave owns one group, KB of its output channels
// and 64 PW output pixels of one output plane (lane l takes pixels
// l, l + 64, ... of the block, so each input load instruction covers 64
// consecutive pixels).  The weights of a (tap, channel vector) are then the
// same for every lane of the wave: they come through the scalar cache into
// scalar registers, which the FMAs read directly, and the vector memory path
// carries only the input vectors - one per pixel and channel vector, shared
// by the KB output channels.  The four waves of a workgroup take four
// neighbouring groups of the same pixels, so their input loads share cache
// lines; workgroups of one XCD take neighbouring pixel blocks (halo rows).
template <typename T, int KB, int VC, int PW>
__global__ __launch_bounds__(kBlock) void wave_kernel(Problem p, const T *__restrict__ x,
                                                      const T *__restrict__ w,
                                                      const T *__restrict__ bias, T *__restrict__ y,
                                                      int nkb, int ngb, int npb)
{
    constexpr int kWaves = kBlock / 64;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    int r = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int kbi = r % nkb;  r /= nkb;
    const int gb = r % ngb;   r /= ngb;
    const int pb = r % npb;   r /= npb;
    const int od = r % p.Do;
    const int n = r / p.Do;
    const int g = __builtin_amdgcn_readfirstlane(gb * kWaves + wave);
    if (g >= p.G) return;
    const int k0 = kbi * KB;
    const int C = p.G * p.Cpg, K = p.G * p.Kpg, taps = p.Z * p.Y * p.X;
    const int plane = p.Ho * p.Wo;
    int ihb[PW], iwb[PW];
    bool live[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const int m = pb * 64 * PW + j * 64 + lane;
        live[j] = m < plane;
        const int oh = live[j] ? m / p.Wo : 0, ow = live[j] ? m - (m / p.Wo) * p.Wo : 0;
        ihb[j] = oh * p.sh - p.ph;
        iwb[j] = ow * p.sw - p.pw;
    }
    float acc[KB][PW];
#pragma unroll
    for (int a = 0; a < KB; ++a)
#pragma unroll
        for (int j = 0; j < PW; ++j) acc[a][j] = 0.f;
    const T *wg = w + (size_t)(g * p.Kpg + k0) * taps * p.Cpg;
    // Within a depth plane of the window, steps (row, column, channel
    // vector), channel vector fastest; the input vectors of step s + 1 are
    // requested before the FMAs of step s, so each wave keeps two steps of
    // loads in flight.
    const int ncv = p.Cpg / VC;
    const int nst = p.Y * p.X * ncv;
    for (int z = 0; z < p.Z; ++z) {
        const int id = od * p.sd - p.pd + z * p.dd;
        if (id < 0 || id >= p.D) continue;
        const T *xplane = x + (size_t)(n * p.D + id) * p.H * p.W * C + g * p.Cpg;
        const T *wz = wg + (size_t)z * p.Y * p.X * p.Cpg;
        auto load_x = [&](float (&xv)[PW][VC], int st) {
            const int rc = st / ncv, cv = st - rc * ncv;
            const int yy = rc / p.X, xx = rc - yy * p.X;
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                const int ih = ihb[j] + yy * p.dh, iw = iwb[j] + xx * p.dw;
                if (live[j] && (unsigned)ih < (unsigned)p.H && (unsigned)iw < (unsigned)p.W)
                    VecT<T, VC>::load(xplane + (size_t)(ih * p.W + iw) * C + cv * VC, xv[j]);
                else
#pragma unroll
                    for (int v = 0; v < VC; ++v) xv[j][v] = 0.f;
            }
        };
        float xb[2][PW][VC];
        load_x(xb[0], 0);
        for (int s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int st = s0 + u;
                if (st < nst) {
                    if (st + 1 < nst) load_x(xb[u ^ 1], st + 1);
                    // the window tap and channel vector of this step: the
                    // weight offset (tap-major rows of Cpg channels) is just
                    // st * VC within the depth plane's taps
                    float wv[KB][VC];
#pragma unroll
                    for (int a = 0; a < KB; ++a) VecT<T, VC>::load(wz + (size_t)a * taps * p.Cpg + st * VC, wv[a]);
#pragma unroll
                    for (int v = 0; v < VC; ++v)
#pragma unroll
                        for (int a = 0; a < KB; ++a)
#pragma unroll
                            for (int j = 0; j < PW; ++j) acc[a][j] = fmaf(xb[u][j][v], wv[a][v], acc[a][j]);
                }
            }
        }
    }
    const int ch0 = g * p.Kpg + k0;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        if (!live[j]) continue;
        const int m = pb * 64 * PW + j * 64 + lane;
        T *yp = y + ((size_t)(n * p.Do + od) * plane + m) * K + ch0;
#pragma unroll
        for (int a = 0; a < KB; ++a) yp[a] = finish<T>(acc[a][j], bias, ch0 + a);
    }
}

struct Config {
    bool wave;            // wave-uniform-weight kernel
    int KB, VC, PW, nkb, nwb, ngb, npb;
    long long threads;    // threads (per-thread kernel) or lanes (wave kernel) launched
};

// channel blocks among 8, 4, 2, 1 that divide Kpg
int kb_list(const Problem &p, int *kb)
{
    int n = 0;
    for (int v : {8, 4, 2, 1})
        if (p.Kpg % v == 0) kb[n++] = v;
    return n;
}

// tile menu: the per-thread kernel with each channel block, then the
// wave-uniform-weight kernel with each channel block
int kb_menu(const Problem &p, int *kb, bool *wave)
{
    int one[4];
    const int n = kb_list(p, one);
    for (int i = 0; i < n; ++i) {
        kb[i] = one[i];
        wave[i] = false;
        kb[n + i] = one[i];
        wave[n + i] = true;
    }
    return 2 * n;
}

int pw_of(const Problem &p)
{
    const long long plane = (long long)p.Ho * p.Wo;
    return plane >= 256 ? 4 : plane >= 128 ? 2 : 1;
}

long long threads_at(const Problem &p, int KB, bool wave)
{
    if (wave) {
        const int PW = pw_of(p);
        const long long npb = ((long long)p.Ho * p.Wo + 64 * PW - 1) / (64 * PW);
        return (long long)p.N * p.Do * npb * ((p.G + 3) / 4) * (p.Kpg / KB) * kBlock;
    }
    return (long long)p.N * p.Do * p.Ho * ((p.Wo + kPW - 1) / kPW) * p.G * (p.Kpg / KB);
}

// own pick: the widest channel block of at least 4 that still leaves
// kMinThreads threads (the tile sweep: a large-group fp32 problem of few
// pixels ran 8x faster on 4-channel blocks than on the generic kernel it
// fell to with 8; with 1- or 2-channel blocks the generic kernel's split
// reductions measured slightly faster)
int own_kb(const Problem &p, const int *kb, const bool *wave, int n)
{
    // Wide groups over many workgroups: the wave-uniform-weight kernel with
    // 8-channel blocks (fp32 tile sweep: 1.1-2.4x faster than the per-thread
    // kernel with 16+ input channels per group and 1000+ workgroups; with
    // fewer workgroups, or 4-channel blocks, the per-thread kernel measured
    // as fast or up to 1.2x faster)
    if (p.Cpg >= 16)
        for (int i = 0; i < n; ++i)
            if (wave[i] && kb[i] == 8 && threads_at(p, kb[i], true) / kBlock >= 1024) return i;
    for (int i = 0; i < n; ++i)
        if (!wave[i] && kb[i] >= 4 && threads_at(p, kb[i], false) >= kMinThreads) return i;
    return 0;
}

void configure(const Problem &p, Config &c)
{
    int kb[8];
    bool wave[8];
    const int n = kb_menu(p, kb, wave);
    const int t = tile_choice();
    const int i = t >= 0 && t < n ? t : own_kb(p, kb, wave, n);
    c.KB = kb[i];
    c.wave = wave[i];
    c.VC = p.Cpg % 4 == 0 ? 4 : 1;
    c.nkb = p.Kpg / c.KB;
    c.nwb = (p.Wo + kPW - 1) / kPW;
    c.PW = pw_of(p);
    c.ngb = (p.G + 3) / 4;
    c.npb = (int)(((long long)p.Ho * p.Wo + 64 * c.PW - 1) / (64 * c.PW));
    c.threads = threads_at(p, c.KB, c.wave);
}

template <typename T, int KB, int VC>
hipError_t go_wave(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    const dim3 grid((unsigned)(c.threads / kBlock));
    auto run = [&](auto k) {
        return enqueue(k, grid, dim3(kBlock), 0, s, a, p, (const T *)a.x, (const T *)a.w, (const T *)a.bias,
                       (T *)a.y, c.nkb, c.ngb, c.npb);
    };
    if (c.PW == 4) return run(wave_kernel<T, KB, VC, 4>);
    if (c.PW == 2) return run(wave_kernel<T, KB, VC, 2>);
    return run(wave_kernel<T, KB, VC, 1>);
}

template <typename T, int KB>
hipError_t go2(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    if (c.wave) return c.VC == 4 ? go_wave<T, KB, 4>(p, c, a, s) : go_wave<T, KB, 1>(p, c, a, s);
    const int total = (int)c.threads;
    const dim3 grid((unsigned)((c.threads + kBlock - 1) / kBlock));
    if (c.VC == 4)
        return enqueue(kernel<T, KB, 4>, grid, dim3(kBlock), 0, s, a, p, (const T *)a.x, (const T *)a.w,
                       (const T *)a.bias, (T *)a.y, c.nkb, c.nwb, total);
    return enqueue(kernel<T, KB, 1>, grid, dim3(kBlock), 0, s, a, p, (const T *)a.x, (const T *)a.w,
                   (const T *)a.bias, (T *)a.y, c.nkb, c.nwb, total);
}

template <typename T>
hipError_t go(const Problem &p, const Config &c, const Args &a, hipStream_t s)
{
    switch (c.KB) {
    case 8: return go2<T, 8>(p, c, a, s);
    case 4: return go2<T, 4>(p, c, a, s);
    case 2: return go2<T, 2>(p, c, a, s);
    default: return go2<T, 1>(p, c, a, s);
    }
}

}  // namespace

bool supported(const Problem &p)
{
    Config c;
    configure(p, c);
    return c.threads < (1LL << 31);
}

int tiles(const Problem &p, int *picked)
{
    int kb[8];
    bool wave[8];
    const int n = kb_menu(p, kb, wave);
    *picked = own_kb(p, kb, wave, n);
    return n;
}

// Whether the dispatcher should prefer this path over the generic kernel:
// enough threads to fill the chip with register-blocked work.
bool preferred(const Problem &p)
{
    const int saved = tile_choice();
    tile_choice() = -1;
    Config c;
    configure(p, c);
    tile_choice() = saved;
    return c.threads >= kMinThreads && c.threads < (1LL << 31);
}

gconv_plan plan(const Problem &p)
{
    Config c;
    configure(p, c);
    gconv_plan pl{};
    pl.path = GCONV_PATH_DIRECT;
    pl.grid[0] = (uint32_t)((c.threads + kBlock - 1) / kBlock);
    pl.grid[1] = pl.grid[2] = 1;
    pl.block = kBlock;
    pl.lds_bytes = 0;
    pl.groups_per_tile = 1;
    return pl;
}

hipError_t launch(const Problem &p, const Args &a, hipStream_t s)
{
    Config c;
    configure(p, c);
    if (c.threads >= (1LL << 31)) return hipErrorInvalidValue;
    switch (p.dtype) {
    case GCONV_F32: return go<float>(p, c, a, s);
    case GCONV_F16: return go<_Float16>(p, c, a, s);
    default: return go<__bf16>(p, c, a, s);
    }
}

}  // namespace direct
}  // namespace gconv

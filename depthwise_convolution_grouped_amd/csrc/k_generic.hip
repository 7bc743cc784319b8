// Generic direct kernel: any shape, any dtype.  It is the fallback for
// shapes the tiled paths do not take and the first, simplest HIP form of the
// operation declared in gconv.h.
//
// L consecutive threads own y[n][od][oh][ow][g][k] (flat NDHWGK index e):
// thread j of the L walks the window taps (z, y, x) and the input channels
// c = j, j + L, ... of the group, accumulating in fp32; the L partial sums
// are added by cross-lane exchanges (L divides the wave) and the first
// thread ends in the shared bias/convert epilogue.  L = 1 for large outputs;
// small problems (few outputs, long reductions) spread each reduction over
// up to 16 threads, so the whole chip works and each thread's loads are few
// and independent instead of one long dependent chain per output.  Windows
// of at most 9 taps with at most 4 channels per thread take a flat form that
// issues all of a thread's loads before its first product, so the thread
// waits for one memory latency instead of one per tap.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace generic {
namespace {

constexpr int kBlock = 256;

template <typename T, int L>
__global__ __launch_bounds__(kBlock) void kernel(Problem p, const T *__restrict__ x,
                                                 const T *__restrict__ w,
                                                 const T *__restrict__ bias, T *__restrict__ y,
                                                 int total)
{
    const int tid = blockIdx.x * kBlock + threadIdx.x;
    const int e = tid / L, part = tid - (tid / L) * L;
    float acc = 0.f;
    int g = 0, k = 0;
    if (e < total) {
        int r = e;
        k = r % p.Kpg;  r /= p.Kpg;
        g = r % p.G;    r /= p.G;
        const int ow = r % p.Wo;  r /= p.Wo;
        const int oh = r % p.Ho;  r /= p.Ho;
        const int od = r % p.Do;  r /= p.Do;
        const int n = r;
        const int C = p.G * p.Cpg;
        for (int z = 0; z < p.Z; ++z) {
            const int id = od * p.sd - p.pd + z * p.dd;
            if (id < 0 || id >= p.D) continue;
            for (int yy = 0; yy < p.Y; ++yy) {
                const int ih = oh * p.sh - p.ph + yy * p.dh;
                if (ih < 0 || ih >= p.H) continue;
                for (int xx = 0; xx < p.X; ++xx) {
                    const int iw = ow * p.sw - p.pw + xx * p.dw;
                    if (iw < 0 || iw >= p.W) continue;
                    const T *xp = x + ((((n * p.D + id) * p.H + ih) * p.W + iw) * C + g * p.Cpg);
                    const T *wp = w + ((((g * p.Kpg + k) * p.Z + z) * p.Y + yy) * p.X + xx) * p.Cpg;
                    for (int c = part; c < p.Cpg; c += L) acc = fmaf(to_f32(xp[c]), to_f32(wp[c]), acc);
                }
            }
        }
    }
    // the L partial sums of one output sit in L consecutive lanes of a wave
#pragma unroll
    for (int m = L / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m);
    if (e < total && part == 0) y[e] = finish<T>(acc, bias, g * p.Kpg + k);
}

// The flat form: taps and channel slots unrolled to fixed bounds.  A slot
// outside the window, the input or the group loads from a valid address and
// its product is dropped by a select (never multiplied by zero, so a
// non-finite weight next to the padding stays out of the sum); the products
// are added in the loop form's order (taps outer, channels c = part + j L
// inner), so both forms give the same bits.
constexpr int kFlatTaps = 9, kFlatCh = 4;

template <typename T, int L>
__global__ __launch_bounds__(kBlock) void flat_kernel(Problem p, const T *__restrict__ x,
                                                      const T *__restrict__ w,
                                                      const T *__restrict__ bias, T *__restrict__ y,
                                                      int total)
{
    const int tid = blockIdx.x * kBlock + threadIdx.x;
    const int e = tid / L, part = tid - (tid / L) * L;
    const bool live = e < total;
    int r = live ? e : 0;
    const int k = r % p.Kpg;  r /= p.Kpg;
    const int g = r % p.G;    r /= p.G;
    const int ow = r % p.Wo;  r /= p.Wo;
    const int oh = r % p.Ho;  r /= p.Ho;
    const int od = r % p.Do;  r /= p.Do;
    const int n = r;
    const int C = p.G * p.Cpg, taps = p.Z * p.Y * p.X;
    const T *wk = w + (size_t)(g * p.Kpg + k) * taps * p.Cpg;
    float xv[kFlatTaps][kFlatCh], wv[kFlatTaps][kFlatCh];
    bool use[kFlatTaps][kFlatCh];
    int z = 0, yy = 0, xx = 0;   // tap t = (z Y + yy) X + xx
#pragma unroll
    for (int t = 0; t < kFlatTaps; ++t) {
        const int id = od * p.sd - p.pd + z * p.dd;
        const int ih = oh * p.sh - p.ph + yy * p.dh;
        const int iw = ow * p.sw - p.pw + xx * p.dw;
        const bool in = live && t < taps && (unsigned)id < (unsigned)p.D && (unsigned)ih < (unsigned)p.H &&
                        (unsigned)iw < (unsigned)p.W;
        const size_t xo = (size_t)(((n * p.D + id) * p.H + ih) * p.W + iw) * C + g * p.Cpg;
#pragma unroll
        for (int j = 0; j < kFlatCh; ++j) {
            const int c = part + j * L;
            use[t][j] = in && c < p.Cpg;
            xv[t][j] = to_f32(x[use[t][j] ? xo + c : 0]);
            wv[t][j] = to_f32(wk[use[t][j] ? (size_t)t * p.Cpg + c : 0]);
        }
        if (++xx == p.X) {
            xx = 0;
            if (++yy == p.Y) {
                yy = 0;
                ++z;
            }
        }
    }
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < kFlatTaps; ++t)
#pragma unroll
        for (int j = 0; j < kFlatCh; ++j) acc = use[t][j] ? fmaf(xv[t][j], wv[t][j], acc) : acc;
#pragma unroll
    for (int m = L / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m);
    if (live && part == 0) y[e] = finish<T>(acc, bias, g * p.Kpg + k);
}

bool flat_ok(const Problem &p, int L) { return p.taps() <= kFlatTaps && (p.Cpg + L - 1) / L <= kFlatCh; }

// threads per output: doubled while the launch stays under 2^21 threads
// (eight waves per SIMD on 256 CUs), at most the channels a thread would
// otherwise walk alone (tile sweep: a 1728-long reduction over 200k outputs
// ran 8x faster on 8 threads per output than on one)
int own_lanes(const Problem &p)
{
    const long long outs = p.y_elems();
    int L = 1;
    while (L < 16 && outs * 2 * L <= (1LL << 21) && 2 * L <= p.Cpg * p.taps()) L *= 2;
    return L;
}

// tile menu: L = 1, 2, 4, 8, 16 threads per output
int lanes_for(const Problem &p)
{
    const int t = tile_choice();
    return t >= 0 && t < 5 ? 1 << t : own_lanes(p);
}

template <int DT, int L>
hipError_t go2(const Problem &p, const Args &a, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    const int total = (int)p.y_elems();
    const int blocks = (int)(((long long)total * L + kBlock - 1) / kBlock);
    if (flat_ok(p, L))
        return enqueue(flat_kernel<T, L>, dim3(blocks), dim3(kBlock), 0, s, a, p,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, total);
    return enqueue(kernel<T, L>, dim3(blocks), dim3(kBlock), 0, s, a, p,
                   (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, total);
}

template <int DT>
hipError_t go(const Problem &p, const Args &a, hipStream_t s)
{
    switch (lanes_for(p)) {
    case 1: return go2<DT, 1>(p, a, s);
    case 2: return go2<DT, 2>(p, a, s);
    case 4: return go2<DT, 4>(p, a, s);
    case 8: return go2<DT, 8>(p, a, s);
    default: return go2<DT, 16>(p, a, s);
    }
}

}  // namespace

bool supported(const Problem &) { return true; }

int tiles(const Problem &p, int *picked)
{
    int L = own_lanes(p), i = 0;
    while ((1 << i) < L) ++i;
    *picked = i;
    return 5;
}

gconv_plan plan(const Problem &p)
{
    gconv_plan pl{};
    pl.path = GCONV_PATH_GENERIC;
    pl.grid[0] = (uint32_t)((p.y_elems() * lanes_for(p) + kBlock - 1) / kBlock);
    pl.grid[1] = pl.grid[2] = 1;
    pl.block = kBlock;
    pl.lds_bytes = 0;
    pl.groups_per_tile = 1;
    return pl;
}

hipError_t launch(const Problem &p, const Args &a, hipStream_t s)
{
    switch (p.dtype) {
    case GCONV_F32: return go<GCONV_F32>(p, a, s);
    case GCONV_F16: return go<GCONV_F16>(p, a, s);
    default: return go<GCONV_BF16>(p, a, s);
    }
}

}  // namespace generic
}  // namespace gconv

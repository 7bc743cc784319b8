// Generic direct kernel: one thread per output element, any shape, any
// dtype.  It is the fallback for shapes the tiled paths do not take and the
// first, simplest HIP form of the operation declared in gconv.h.
//
// Thread e owns y[n][od][oh][ow][g][k] (flat NDHWGK index e), walks the
// window taps (z, y, x) and the group's Cpg input channels, accumulates in
// fp32 and ends in the shared bias/convert epilogue.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace generic {
namespace {

constexpr int kBlock = 256;

template <typename T>
__global__ __launch_bounds__(kBlock) void kernel(Problem p, const T *__restrict__ x,
                                                 const T *__restrict__ w,
                                                 const T *__restrict__ bias, T *__restrict__ y,
                                                 int total)
{
    int e = blockIdx.x * kBlock + threadIdx.x;
    if (e >= total) return;
    int r = e;
    const int k = r % p.Kpg;  r /= p.Kpg;
    const int g = r % p.G;    r /= p.G;
    const int ow = r % p.Wo;  r /= p.Wo;
    const int oh = r % p.Ho;  r /= p.Ho;
    const int od = r % p.Do;  r /= p.Do;
    const int n = r;
    const int C = p.G * p.Cpg;
    float acc = 0.f;
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
                for (int c = 0; c < p.Cpg; ++c) acc = fmaf(to_f32(xp[c]), to_f32(wp[c]), acc);
            }
        }
    }
    y[e] = finish<T>(acc, bias, g * p.Kpg + k);
}

template <int DT>
hipError_t go(const Problem &p, const Args &a, hipStream_t s)
{
    using T = typename Elem<DT>::T;
    const int total = (int)p.y_elems();
    const int blocks = (total + kBlock - 1) / kBlock;
    return enqueue(kernel<T>, dim3(blocks), dim3(kBlock), 0, s, a, p,
                   (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, total);
}

}  // namespace

bool supported(const Problem &) { return true; }

gconv_plan plan(const Problem &p)
{
    gconv_plan pl{};
    pl.path = GCONV_PATH_GENERIC;
    pl.grid[0] = (uint32_t)((p.y_elems() + kBlock - 1) / kBlock);
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

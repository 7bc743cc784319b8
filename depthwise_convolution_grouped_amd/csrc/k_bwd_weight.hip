// Backward weight: dw, the gradient with respect to w, from x and dy.  It is
// the third grouped-convolution variant the CK grouped_conv tile-engine
// README lists (forward, backward-data, backward-weight); the CK Python
// examples README's runner for it takes X and dY (Runner argument contract).
// Layouts are the forward ones: x [N][D][H][W][G][Cpg],
// dy [N][Do][Ho][Wo][G][Kpg], dw [G][Kpg][Z][Y][X][Cpg].
//
//   dw[g,k,t,c] = sum over output pixels o whose tap t reads an in-bounds
//                 input i = o stride - pad + t dil of dy[n,o,g,k] x[n,i,g,c]
//
// A reduction over N Do Ho Wo per weight element, done in two deterministic
// stages (no atomics, a fixed summation order):
//   1. partial sums: thread (chunk, f) sums the terms of weight element f
//      over one chunk of output rows (n, od, oh) into an fp32 workspace
//      [chunk][f]; consecutive threads take consecutive input channels c,
//      so their x reads are contiguous and their dy reads shared;
//   2. the chunks of each element are added in chunk order and rounded once.
// With one chunk (no workspace, or a problem with enough weight elements to
// fill the chip) stage 1 writes dw directly.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace bwdw {
namespace {

constexpr int kBlock = 256;

template <typename T, bool kFinal>
__global__ __launch_bounds__(kBlock) void partial_kernel(Problem p, const T *__restrict__ x,
                                                         const T *__restrict__ dy, float *__restrict__ ws,
                                                         T *__restrict__ dw, int welems, int rows_per_chunk)
{
    const int f = blockIdx.x * kBlock + threadIdx.x;
    const int ch = blockIdx.y;
    if (f >= welems) return;
    int r = f;
    const int c = r % p.Cpg;  r /= p.Cpg;
    const int xx = r % p.X;   r /= p.X;
    const int yy = r % p.Y;   r /= p.Y;
    const int z = r % p.Z;    r /= p.Z;
    const int k = r % p.Kpg;  r /= p.Kpg;
    const int g = r;
    const int C = p.G * p.Cpg, K = p.G * p.Kpg;
    const int rows = p.N * p.Do * p.Ho;
    const int r0 = ch * rows_per_chunk;
    const int r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
    // the output columns whose tap xx reads inside the input: iw = ow sw - pw + xx dw in [0, W)
    int ow_lo = 0, ow_hi = p.Wo;   // [lo, hi)
    {
        const int off = xx * p.dw - p.pw;          // iw = ow sw + off
        if (off < 0) ow_lo = (-off + p.sw - 1) / p.sw;
        const int lim = p.W - off;                 // ow sw < lim
        const int hi = lim <= 0 ? 0 : (lim + p.sw - 1) / p.sw;
        if (hi < ow_hi) ow_hi = hi;
    }
    float acc = 0.f;
    for (int rr = r0; rr < r1; ++rr) {
        const int oh = rr % p.Ho, t = rr / p.Ho;
        const int od = t % p.Do, n = t / p.Do;
        const int id = od * p.sd - p.pd + z * p.dd;
        const int ih = oh * p.sh - p.ph + yy * p.dh;
        if (id < 0 || id >= p.D || ih < 0 || ih >= p.H) continue;
        const T *dyr = dy + ((size_t)((n * p.Do + od) * p.Ho + oh) * p.Wo) * K + g * p.Kpg + k;
        const T *xr = x + ((size_t)((n * p.D + id) * p.H + ih) * p.W) * C + g * p.Cpg + c;
        for (int ow = ow_lo; ow < ow_hi; ++ow) {
            const int iw = ow * p.sw - p.pw + xx * p.dw;
            acc = fmaf(to_f32(dyr[(size_t)ow * K]), to_f32(xr[(size_t)iw * C]), acc);
        }
    }
    if (kFinal) dw[f] = from_f32<T>(acc);
    else ws[(size_t)ch * welems + f] = acc;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void reduce_kernel(const float *__restrict__ ws, T *__restrict__ dw,
                                                        int welems, int nch)
{
    const int f = blockIdx.x * kBlock + threadIdx.x;
    if (f >= welems) return;
    float acc = 0.f;
    for (int ch = 0; ch < nch; ++ch) acc += ws[(size_t)ch * welems + f];
    dw[f] = from_f32<T>(acc);
}

template <typename T>
hipError_t go(const Problem &p, const void *x, const void *dy, void *dw, float *ws, int nch, hipStream_t s)
{
    const int welems = p.G * p.Kpg * p.taps() * p.Cpg;
    const int rows = p.N * p.Do * p.Ho;
    const int rpc = (rows + nch - 1) / nch;
    nch = (rows + rpc - 1) / rpc;                  // no empty chunk
    const dim3 grid((unsigned)((welems + kBlock - 1) / kBlock), (unsigned)nch);
    Args a{};
    if (nch == 1)
        return enqueue(partial_kernel<T, true>, grid, dim3(kBlock), 0, s, a, p, (const T *)x, (const T *)dy,
                       (float *)nullptr, (T *)dw, welems, rpc);
    hipError_t e = enqueue(partial_kernel<T, false>, grid, dim3(kBlock), 0, s, a, p, (const T *)x,
                           (const T *)dy, ws, (T *)nullptr, welems, rpc);
    if (e != hipSuccess) return e;
    return enqueue(reduce_kernel<T>, dim3((unsigned)((welems + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, a,
                   (const float *)ws, (T *)dw, welems, nch);
}

}  // namespace

// Chunks that fill the chip: about 256 K stage-1 threads, at most one chunk
// per output row, at most 65535 (the grid's y extent).
int ideal_chunks(const Problem &p)
{
    const long long welems = (long long)p.G * p.Kpg * p.taps() * p.Cpg;
    const long long rows = (long long)p.N * p.Do * p.Ho;
    long long n = (262144 + welems - 1) / welems;
    if (n > rows) n = rows;
    if (n > 65535) n = 65535;
    return n < 1 ? 1 : (int)n;
}

hipError_t launch(const Problem &p, const void *x, const void *dy, void *dw, float *ws, int nch, hipStream_t s)
{
    switch (p.dtype) {
    case GCONV_F32: return go<float>(p, x, dy, dw, ws, nch, s);
    case GCONV_F16: return go<_Float16>(p, x, dy, dw, ws, nch, s);
    default: return go<__bf16>(p, x, dy, dw, ws, nch, s);
    }
}

}  // namespace bwdw
}  // namespace gconv

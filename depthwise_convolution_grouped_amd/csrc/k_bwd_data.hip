// Backward data: dx, the gradient with respect to x, from dy and w.  It is
// the second of the three grouped-convolution variants the CK grouped_conv
// tile-engine README lists (forward, backward-data, backward-weight); the
// CK Python examples README's runner for it takes dY and W (Runner argument
// contract).  Layouts are the forward ones: dy [N][Do][Ho][Wo][G][Kpg],
// w [G][Kpg][Z][Y][X][Cpg], dx [N][D][H][W][G][Cpg].
//
//   dx[n,i,g,c] = sum over taps t and k with o = (i + pad - t dil) / stride an
//                 integer in [0, out) of dy[n,o,g,k] w[g,k,t,c]   (per axis)
//
// Two kernels live here:
//   - a direct kernel for every shape: L consecutive threads own one dx
//     element, walk the taps whose output coordinate is integral and in
//     range, and split the Kpg output channels of the group between them
//     (partial sums joined by lane exchanges), fp32 accumulation;
//   - the weight transform of the stride-1 route: at stride 1, dx is the
//     forward convolution of dy with the weights flipped in space and with
//     C and K exchanged (wt[g][c][Z-1-z][Y-1-y][X-1-x][k] = w[g][k][z][y][x][c]:
//     reversing the flat tap index reverses all three axes)
//     under padding dil (k - 1) - pad, so the host runs this transform into
//     a caller workspace and then the forward dispatcher.
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace bwd {
namespace {

constexpr int kBlock = 256;

template <typename T, int L>
__global__ __launch_bounds__(kBlock) void direct_kernel(Problem p, const T *__restrict__ dy,
                                                        const T *__restrict__ w, T *__restrict__ dx,
                                                        int total)
{
    const int tid = blockIdx.x * kBlock + threadIdx.x;
    const int e = tid / L, part = tid - (tid / L) * L;
    float acc = 0.f;
    if (e < total) {
        int r = e;
        const int c = r % p.Cpg;  r /= p.Cpg;
        const int g = r % p.G;    r /= p.G;
        const int iw = r % p.W;   r /= p.W;
        const int ih = r % p.H;   r /= p.H;
        const int id = r % p.D;   r /= p.D;
        const int n = r;
        const int K = p.G * p.Kpg;
        for (int z = 0; z < p.Z; ++z) {
            const int td = id + p.pd - z * p.dd;
            if (td < 0 || td % p.sd != 0 || td / p.sd >= p.Do) continue;
            const int od = td / p.sd;
            for (int yy = 0; yy < p.Y; ++yy) {
                const int th = ih + p.ph - yy * p.dh;
                if (th < 0 || th % p.sh != 0 || th / p.sh >= p.Ho) continue;
                const int oh = th / p.sh;
                for (int xx = 0; xx < p.X; ++xx) {
                    const int tw = iw + p.pw - xx * p.dw;
                    if (tw < 0 || tw % p.sw != 0 || tw / p.sw >= p.Wo) continue;
                    const int ow = tw / p.sw;
                    const T *dyp = dy + ((((n * p.Do + od) * p.Ho + oh) * p.Wo + ow) * K + g * p.Kpg);
                    const T *wp = w + (((g * p.Kpg * p.Z + z) * p.Y + yy) * p.X + xx) * p.Cpg + c;
                    const int kstep = p.Z * p.Y * p.X * p.Cpg;    // w elements between output channels
                    for (int k = part; k < p.Kpg; k += L) acc = fmaf(to_f32(dyp[k]), to_f32(wp[k * kstep]), acc);
                }
            }
        }
    }
#pragma unroll
    for (int m = L / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m);
    if (e < total && part == 0) dx[e] = from_f32<T>(acc);
}

// wt[g][c][t][k] = w[g][k][T-1-t][c] (t the flat tap (z, y, x), so T-1-t
// flips all three axes at once): for each (group, tap) a Kpg x Cpg matrix
// transposed through LDS in 32 x 32 tiles, read along c and written along
// k so both sides are coalesced; a copy of element bits
template <typename U>
__global__ __launch_bounds__(kBlock) void flip_kernel(Problem p, const U *__restrict__ w, U *__restrict__ wt)
{
    __shared__ U tile[32][33];
    const int T = p.Z * p.Y * p.X;
    const int nct = (p.Cpg + 31) / 32;
    const int gt = blockIdx.x / nct;            // g * T + t (destination tap t)
    const int g = gt / T, t = gt - g * T;
    const int c0 = (blockIdx.x - gt * nct) * 32, k0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8 threads
    const U *src = w + ((size_t)g * p.Kpg * T + (T - 1 - t)) * p.Cpg;   // + k * T * Cpg + c
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
        const int k = k0 + ty + j, c = c0 + tx;
        if (k < p.Kpg && c < p.Cpg) tile[ty + j][tx] = src[(size_t)k * T * p.Cpg + c];
    }
    __syncthreads();
    U *dst = wt + ((size_t)g * p.Cpg * T + t) * p.Kpg;                  // + c * T * Kpg + k
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
        const int c = c0 + ty + j, k = k0 + tx;
        if (c < p.Cpg && k < p.Kpg) dst[(size_t)c * T * p.Kpg + k] = tile[tx][ty + j];
    }
}

int lanes_for(const Problem &p, long long elems)
{
    int L = 1;
    while (L < 16 && elems * L < 256LL * kBlock && 2 * L <= p.Kpg) L *= 2;
    return L;
}

template <typename T, int L>
hipError_t go2(const Problem &p, const void *dy, const void *w, void *dx, hipStream_t s)
{
    const long long elems = (long long)p.N * p.D * p.H * p.W * p.G * p.Cpg;
    const int blocks = (int)((elems * L + kBlock - 1) / kBlock);
    Args a{};
    return enqueue(direct_kernel<T, L>, dim3(blocks), dim3(kBlock), 0, s, a, p, (const T *)dy,
                   (const T *)w, (T *)dx, (int)elems);
}

template <typename T>
hipError_t go(const Problem &p, const void *dy, const void *w, void *dx, hipStream_t s)
{
    const long long elems = (long long)p.N * p.D * p.H * p.W * p.G * p.Cpg;
    switch (lanes_for(p, elems)) {
    case 1: return go2<T, 1>(p, dy, w, dx, s);
    case 2: return go2<T, 2>(p, dy, w, dx, s);
    case 4: return go2<T, 4>(p, dy, w, dx, s);
    case 8: return go2<T, 8>(p, dy, w, dx, s);
    default: return go2<T, 16>(p, dy, w, dx, s);
    }
}

}  // namespace

hipError_t launch_direct(const Problem &p, const void *dy, const void *w, void *dx, hipStream_t s)
{
    switch (p.dtype) {
    case GCONV_F32: return go<float>(p, dy, w, dx, s);
    case GCONV_F16: return go<_Float16>(p, dy, w, dx, s);
    default: return go<__bf16>(p, dy, w, dx, s);
    }
}

hipError_t launch_flip(const Problem &p, const void *w, void *wt, hipStream_t s)
{
    // x: (group, tap, 32-channel tile of c), y: 32-channel tile of k
    const dim3 grid((unsigned)((long long)p.G * p.taps() * ((p.Cpg + 31) / 32)), (p.Kpg + 31) / 32, 1);
    Args a{};
    if (elem_size(p.dtype) == 4)
        return enqueue(flip_kernel<uint32_t>, grid, dim3(kBlock), 0, s, a, p, (const uint32_t *)w, (uint32_t *)wt);
    return enqueue(flip_kernel<uint16_t>, grid, dim3(kBlock), 0, s, a, p, (const uint16_t *)w, (uint16_t *)wt);
}

}  // namespace bwd
}  // namespace gconv

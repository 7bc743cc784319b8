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
// Kernels here:
//   - a direct kernel for every shape: L consecutive threads own one dx
//     element, walk the taps whose output coordinate is integral and in
//     range, and split the Kpg output channels of the group between them
//     (partial sums joined by lane exchanges), fp32 accumulation; for
//     depthwise problems with 16-byte aligned dy and dx, a channel-vector
//     form of it (and, for 3x3 windows at stride 2, one over 2 x 2 blocks of
//     dx pixels);
//   - the weight transform of the stride-1 route: at stride 1, dx is the
//     forward convolution of dy with the weights flipped in space and with
//     C and K exchanged (wt[g][c][Z-1-z][Y-1-y][X-1-x][k] = w[g][k][z][y][x][c]:
//     reversing the flat tap index reverses all three axes)
//     under padding dil (k - 1) - pad, so the host runs this transform into
//     a caller workspace and then the forward dispatcher;
//   - the two kernels of the strided (polyphase) route: at stride s > 1 the
//     dx positions of one residue class r (i = r + s m per axis) receive only
//     the taps t with (t dil - r - pad) divisible by s, which form the
//     progression t0, t0 + s', ... (s' = s / gcd(dil, s)); in m they are a
//     stride-1 convolution of dy with that sub-kernel, reversed and with C and
//     K exchanged, at dilation dil / gcd(dil, s).  phase_flip_kernel writes
//     one class's sub-kernel, the forward dispatcher computes the class into
//     a dense buffer, and phase_scatter_kernel places it (or zeros, for a
//     class no tap reaches) at its positions of dx.
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

// Depthwise (Cpg = Kpg = 1, so group g is channel g): one thread owns VEC
// consecutive channels (16 bytes) of one dx pixel.  The tap walk and its
// index arithmetic are shared by the VEC channels, dy is read and dx written
// as 16-byte vectors, and the whole weight tensor sits in LDS transposed to
// [tap][channel], so the VEC weights of a tap are one 16-byte LDS read (a
// gather from global memory would touch a different line per lane).
constexpr int kDwLdsBytes = 32 * 1024;
// S: the stride on every axis when it is 1 or 2 (the divisibility tests
// and divisions become bit operations), 0 for any stride
template <typename T, int S>
__global__ __launch_bounds__(kBlock) void depthwise_kernel(Problem p, const T *__restrict__ dy,
                                                           const T *__restrict__ w, T *__restrict__ dx,
                                                           int total)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    extern __shared__ uint4 wl4[];
    T *wl = reinterpret_cast<T *>(wl4);
    const int T9 = p.Z * p.Y * p.X;
    for (int i = threadIdx.x; i < p.G * T9; i += kBlock) {   // w[g][t] -> wl[t][g]
        const int g = i / T9, t = i - g * T9;
        wl[t * p.G + g] = w[i];
    }
    __syncthreads();
    // grid-stride over (pixel, channel vector): a few blocks per CU, each
    // staging the weights once
    for (int e = blockIdx.x * kBlock + threadIdx.x; e < total; e += gridDim.x * kBlock) {
        const int Cv = p.G / VEC;
        int r = e;
        const int cv = r % Cv;  r /= Cv;
        const int iw = r % p.W; r /= p.W;
        const int ih = r % p.H; r /= p.H;
        const int id = r % p.D; r /= p.D;
        const int n = r;
        const int g0 = cv * VEC;
        const int sd = S ? S : p.sd, sh = S ? S : p.sh, sw = S ? S : p.sw;
        float acc[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
        for (int z = 0; z < p.Z; ++z) {
            const int td = id + p.pd - z * p.dd;
            if (td < 0 || td % sd != 0 || td / sd >= p.Do) continue;
            const int od = td / sd;
            for (int yy = 0; yy < p.Y; ++yy) {
                const int th = ih + p.ph - yy * p.dh;
                if (th < 0 || th % sh != 0 || th / sh >= p.Ho) continue;
                const int oh = th / sh;
                for (int xx = 0; xx < p.X; ++xx) {
                    const int tw = iw + p.pw - xx * p.dw;
                    if (tw < 0 || tw % sw != 0 || tw / sw >= p.Wo) continue;
                    const int ow = tw / sw;
                    const uint4 raw = *reinterpret_cast<const uint4 *>(
                        dy + (((size_t)(n * p.Do + od) * p.Ho + oh) * p.Wo + ow) * p.G + g0);
                    const T *dv = reinterpret_cast<const T *>(&raw);
                    const int t = (z * p.Y + yy) * p.X + xx;
                    const uint4 wraw = *reinterpret_cast<const uint4 *>(wl + t * p.G + g0);
                    const T *wv = reinterpret_cast<const T *>(&wraw);
#pragma unroll
                    for (int j = 0; j < VEC; ++j) acc[j] = fmaf(to_f32(dv[j]), to_f32(wv[j]), acc[j]);
                }
            }
        }
        T o[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) o[j] = from_f32<T>(acc[j]);
        *reinterpret_cast<uint4 *>(dx + (size_t)e * VEC) = *reinterpret_cast<const uint4 *>(o);
    }
}

// Depthwise 2D, 3x3 window, stride 2, dilation 1 (the strided depthwise
// layer of MobileNet-style blocks): one thread owns a 2 x 2 block of dx
// pixels (rows 2a, 2a + 1, columns 2b, 2b + 1) and one 16-byte channel
// vector.  Row i = 2a + ry receives the taps ty with (i + pad - ty) even, at
// dy row (i + pad - ty) / 2; for both rows of the block these are the two dy
// rows a + f and a + f + 1, f = floor((pad - 1) / 2) (likewise for columns).
// So the thread loads the 2 x 2 dy vectors its block reads once (zero
// outside dy) instead of once per dx pixel that reads them, and adds each
// dx pixel's products in the tap order of the plain kernel.  PH and PW are
// the pads' parities: with them every tap's dy slot is a constant (odd pad:
// (ry - ty + 1) / 2, even pad: (ry - ty) / 2 + 1).
template <typename T, int PH, int PW>
__global__ __launch_bounds__(kBlock) void depthwise_s2_kernel(Problem p, const T *__restrict__ dy,
                                                              const T *__restrict__ w, T *__restrict__ dx,
                                                              int total)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    extern __shared__ uint4 wl4[];
    T *wl = reinterpret_cast<T *>(wl4);
    for (int i = threadIdx.x; i < p.G * 9; i += kBlock) {   // w[g][t] -> wl[t][g]
        const int g = i / 9, t = i - g * 9;
        wl[t * p.G + g] = w[i];
    }
    __syncthreads();
    const int Cv = p.G / VEC;
    const int Hb = (p.H + 1) / 2, Wb = (p.W + 1) / 2;
    const int fh = p.ph == 0 ? -1 : (p.ph - 1) / 2, fw = p.pw == 0 ? -1 : (p.pw - 1) / 2;
    for (int e = blockIdx.x * kBlock + threadIdx.x; e < total; e += gridDim.x * kBlock) {
        int r = e;
        const int cv = r % Cv;  r /= Cv;
        const int b = r % Wb;   r /= Wb;
        const int a = r % Hb;   r /= Hb;
        const int n = r;
        const int g0 = cv * VEC;
        // the 2 x 2 dy vectors of the block (rows a + fh + u, columns b + fw + v)
        float d[2][2][VEC];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int oh = a + fh + u, ow = b + fw + v;
                const bool in = (unsigned)oh < (unsigned)p.Ho && (unsigned)ow < (unsigned)p.Wo;
                uint4 raw = make_uint4(0u, 0u, 0u, 0u);
                if (in) raw = *reinterpret_cast<const uint4 *>(dy + (((size_t)n * p.Ho + oh) * p.Wo + ow) * p.G + g0);
                const T *dv = reinterpret_cast<const T *>(&raw);
#pragma unroll
                for (int j = 0; j < VEC; ++j) d[u][v][j] = to_f32(dv[j]);
            }
#pragma unroll
        for (int ry = 0; ry < 2; ++ry)
#pragma unroll
            for (int rx = 0; rx < 2; ++rx) {
                const int ih = 2 * a + ry, iw = 2 * b + rx;
                float acc[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
#pragma unroll
                for (int ty = 0; ty < 3; ++ty) {
                    if ((ry + PH - ty) & 1) continue;         // the tap misses row ih
                    const int u = PH ? (ry - ty + 1) / 2 : (ry - ty) / 2 + 1;   // dy row a + fh + u
#pragma unroll
                    for (int tx = 0; tx < 3; ++tx) {
                        if ((rx + PW - tx) & 1) continue;
                        const int v = PW ? (rx - tx + 1) / 2 : (rx - tx) / 2 + 1;
                        const uint4 wraw = *reinterpret_cast<const uint4 *>(wl + (ty * 3 + tx) * p.G + g0);
                        const T *wv = reinterpret_cast<const T *>(&wraw);
#pragma unroll
                        for (int j = 0; j < VEC; ++j) acc[j] = fmaf(d[u][v][j], to_f32(wv[j]), acc[j]);
                    }
                }
                if (ih < p.H && iw < p.W) {
                    T o[VEC];
#pragma unroll
                    for (int j = 0; j < VEC; ++j) o[j] = from_f32<T>(acc[j]);
                    *reinterpret_cast<uint4 *>(dx + (((size_t)n * p.H + ih) * p.W + iw) * p.G + g0) =
                        *reinterpret_cast<const uint4 *>(o);
                }
            }
    }
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

// The same transform for narrow groups (Cpg or Kpg under 32, where the
// 32 x 32 tiles would be mostly empty): one thread per element of wt, in wt's
// order (k fastest), each reading its source element
template <typename U>
__global__ __launch_bounds__(kBlock) void flip_small_kernel(Problem p, const U *__restrict__ w, U *__restrict__ wt,
                                                            int total)
{
    const int e = blockIdx.x * kBlock + threadIdx.x;
    if (e >= total) return;
    const int T = p.Z * p.Y * p.X;
    int r = e;
    const int k = r % p.Kpg;  r /= p.Kpg;
    const int t = r % T;      r /= T;
    const int c = r % p.Cpg;
    const int g = r / p.Cpg;
    wt[e] = w[(((size_t)g * p.Kpg + k) * T + (T - 1 - t)) * p.Cpg + c];
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

// the 2 x 2 block form: 2D, 3x3, stride 2, dilation 1 on both axes
static bool s2_ok(const Problem &p)
{
    return p.ndim == 2 && p.Y == 3 && p.X == 3 && p.sh == 2 && p.sw == 2 && p.dh == 1 && p.dw == 1 &&
           p.ph >= 0 && p.pw >= 0;
}

template <typename T>
hipError_t go_dw(const Problem &p, const void *dy, const void *w, void *dx, hipStream_t s)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    const long long total = (long long)p.N * p.D * p.H * p.W * (p.G / VEC);
    Args a{};
    const long long blocks = (total + kBlock - 1) / kBlock;
    const dim3 grid((unsigned)(blocks < 2048 ? blocks : 2048));   // 8 per CU, grid-stride beyond
    const bool same = p.sh == p.sw && (p.ndim == 2 || p.sd == p.sh);   // 2D: sd is 1 and unused
    const unsigned lds = (unsigned)(p.G * p.taps() * (int)sizeof(T));
    if (s2_ok(p)) {
        const long long tq = (long long)p.N * ((p.H + 1) / 2) * ((p.W + 1) / 2) * (p.G / VEC);
        const long long bq = (tq + kBlock - 1) / kBlock;
        auto k2 = (p.ph & 1) ? ((p.pw & 1) ? depthwise_s2_kernel<T, 1, 1> : depthwise_s2_kernel<T, 1, 0>)
                             : ((p.pw & 1) ? depthwise_s2_kernel<T, 0, 1> : depthwise_s2_kernel<T, 0, 0>);
        return enqueue(k2, dim3((unsigned)(bq < 2048 ? bq : 2048)), dim3(kBlock), lds, s, a, p,
                       (const T *)dy, (const T *)w, (T *)dx, (int)tq);
    }
    auto k = same && p.sh == 1 ? depthwise_kernel<T, 1> : same && p.sh == 2 ? depthwise_kernel<T, 2>
                                                                             : depthwise_kernel<T, 0>;
    return enqueue(k, grid, dim3(kBlock), lds, s, a, p, (const T *)dy, (const T *)w, (T *)dx, (int)total);
}

bool depthwise_ok(const Problem &p)
{
    return p.Cpg == 1 && p.Kpg == 1 && p.G % (16 / elem_size(p.dtype)) == 0 &&
           (long long)p.G * p.taps() * elem_size(p.dtype) <= kDwLdsBytes;
}

hipError_t launch_direct(const Problem &p, const void *dy, const void *w, void *dx, hipStream_t s)
{
    const bool vec_ok = depthwise_ok(p) && ((uintptr_t)dy & 15) == 0 && ((uintptr_t)dx & 15) == 0;
    if (vec_ok) {
        switch (p.dtype) {
        case GCONV_F32: return go_dw<float>(p, dy, w, dx, s);
        case GCONV_F16: return go_dw<_Float16>(p, dy, w, dx, s);
        default: return go_dw<__bf16>(p, dy, w, dx, s);
        }
    }
    switch (p.dtype) {
    case GCONV_F32: return go<float>(p, dy, w, dx, s);
    case GCONV_F16: return go<_Float16>(p, dy, w, dx, s);
    default: return go<__bf16>(p, dy, w, dx, s);
    }
}

namespace {

template <typename U>
__global__ __launch_bounds__(kBlock) void phase_flip_kernel(Problem p, PhaseTaps ph, const U *__restrict__ w,
                                                            U *__restrict__ wt)
{
    __shared__ U tile[32][33];
    const int T = p.Z * p.Y * p.X;
    const int Tp = ph.J[0] * ph.J[1] * ph.J[2];
    const int nct = (p.Cpg + 31) / 32;
    const int gt = blockIdx.x / nct;            // g * Tp + destination tap
    const int g = gt / Tp, tp = gt - g * Tp;
    // destination tap (jz, jy, jx), x fastest; its source tap runs backwards
    // through the class's progression on every axis
    const int jx = tp % ph.J[2], jy = (tp / ph.J[2]) % ph.J[1], jz = tp / (ph.J[2] * ph.J[1]);
    const int sz = ph.t0[0] + (ph.J[0] - 1 - jz) * ph.st[0];
    const int sy = ph.t0[1] + (ph.J[1] - 1 - jy) * ph.st[1];
    const int sx = ph.t0[2] + (ph.J[2] - 1 - jx) * ph.st[2];
    const int ts = (sz * p.Y + sy) * p.X + sx;
    const int c0 = (blockIdx.x - gt * nct) * 32, k0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8 threads
    const U *src = w + ((size_t)g * p.Kpg * T + ts) * p.Cpg;  // + k * T * Cpg + c
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
        const int k = k0 + ty + j, c = c0 + tx;
        if (k < p.Kpg && c < p.Cpg) tile[ty + j][tx] = src[(size_t)k * T * p.Cpg + c];
    }
    __syncthreads();
    U *dst = wt + ((size_t)g * p.Cpg * Tp + tp) * p.Kpg;     // + c * Tp * Kpg + k
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
        const int c = c0 + ty + j, k = k0 + tx;
        if (c < p.Cpg && k < p.Kpg) dst[(size_t)c * Tp * p.Kpg + k] = tile[tx][ty + j];
    }
}

// dx[n][r0 + s0 m0][r1 + s1 m1][r2 + s2 m2][v] = src[n][m0][m1][m2][v] (v: a
// channel unit, 16 bytes when the channels allow), or 0 for a class no tap
// reaches.
template <typename U>
__global__ __launch_bounds__(kBlock) void phase_scatter_kernel(PhaseScatter q, const U *__restrict__ src,
                                                               U *__restrict__ dx)
{
    const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
    if (i >= q.total) return;
    long long r = i / q.cv;
    const int v = (int)(i - r * q.cv);
    const int m2 = (int)(r % q.M[2]); r /= q.M[2];
    const int m1 = (int)(r % q.M[1]); r /= q.M[1];
    const int m0 = (int)(r % q.M[0]);
    const int n = (int)(r / q.M[0]);
    const int z = q.r[0] + q.s[0] * m0, y = q.r[1] + q.s[1] * m1, x = q.r[2] + q.s[2] * m2;
    const size_t o = ((((size_t)n * q.D + z) * q.H + y) * q.W + x) * q.cv + v;
    if (q.zero) dx[o] = U{};
    else dx[o] = src[i];
}

}  // namespace

hipError_t launch_phase_flip(const Problem &p, const PhaseTaps &ph, const void *w, void *wt, hipStream_t s)
{
    const int Tp = ph.J[0] * ph.J[1] * ph.J[2];
    const dim3 grid((unsigned)((long long)p.G * Tp * ((p.Cpg + 31) / 32)), (p.Kpg + 31) / 32, 1);
    Args a{};
    if (elem_size(p.dtype) == 4)
        return enqueue(phase_flip_kernel<uint32_t>, grid, dim3(kBlock), 0, s, a, p, ph, (const uint32_t *)w,
                       (uint32_t *)wt);
    return enqueue(phase_flip_kernel<uint16_t>, grid, dim3(kBlock), 0, s, a, p, ph, (const uint16_t *)w,
                   (uint16_t *)wt);
}

hipError_t launch_phase_scatter(PhaseScatter q, int elem, const void *src, void *dx, hipStream_t s)
{
    // 16-byte units when a pixel's channels are whole units and both buffers are aligned
    const long long bytes = (long long)q.cv * elem;   // q.cv holds the channels on entry
    const bool vec = bytes % 16 == 0 && ((uintptr_t)src & 15) == 0 && ((uintptr_t)dx & 15) == 0;
    const int unit = vec ? 16 : elem;
    q.cv = (int)(bytes / unit);
    q.total = (long long)q.N * q.M[0] * q.M[1] * q.M[2] * q.cv;
    if (q.total == 0) return hipSuccess;
    const dim3 grid((unsigned)((q.total + kBlock - 1) / kBlock));
    Args a{};
    if (unit == 16) return enqueue(phase_scatter_kernel<uint4>, grid, dim3(kBlock), 0, s, a, q, (const uint4 *)src, (uint4 *)dx);
    if (unit == 4) return enqueue(phase_scatter_kernel<uint32_t>, grid, dim3(kBlock), 0, s, a, q, (const uint32_t *)src, (uint32_t *)dx);
    return enqueue(phase_scatter_kernel<uint16_t>, grid, dim3(kBlock), 0, s, a, q, (const uint16_t *)src, (uint16_t *)dx);
}

hipError_t launch_flip(const Problem &p, const void *w, void *wt, hipStream_t s)
{
    const long long total = (long long)p.G * p.Cpg * p.taps() * p.Kpg;
    if ((p.Cpg < 32 || p.Kpg < 32) && total < (1LL << 31)) {
        const dim3 g1((unsigned)((total + kBlock - 1) / kBlock));
        Args a{};
        if (elem_size(p.dtype) == 4)
            return enqueue(flip_small_kernel<uint32_t>, g1, dim3(kBlock), 0, s, a, p, (const uint32_t *)w,
                           (uint32_t *)wt, (int)total);
        return enqueue(flip_small_kernel<uint16_t>, g1, dim3(kBlock), 0, s, a, p, (const uint16_t *)w,
                       (uint16_t *)wt, (int)total);
    }
    // x: (group, tap, 32-channel tile of c), y: 32-channel tile of k
    const dim3 grid((unsigned)((long long)p.G * p.taps() * ((p.Cpg + 31) / 32)), (p.Kpg + 31) / 32, 1);
    Args a{};
    if (elem_size(p.dtype) == 4)
        return enqueue(flip_kernel<uint32_t>, grid, dim3(kBlock), 0, s, a, p, (const uint32_t *)w, (uint32_t *)wt);
    return enqueue(flip_kernel<uint16_t>, grid, dim3(kBlock), 0, s, a, p, (const uint16_t *)w, (uint16_t *)wt);
}

}  // namespace bwd
}  // namespace gconv

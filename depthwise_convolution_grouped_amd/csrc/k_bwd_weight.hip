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
//      then output channels k, so their x reads are contiguous or shared and
//      their dy reads contiguous;
//   2. the chunks of each element are added in a fixed order (lane groups
//      with eight running sums each, then a fixed tree) and rounded once.
// With one chunk (no workspace, or a problem with enough weight elements to
// fill the chip) stage 1 writes dw directly.  Depthwise 3x3 problems take a
// channel-vector form of stage 1 (below).
#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace bwdw {
namespace {

constexpr int kBlock = 256;

constexpr int kU = 8;        // output columns per step of the plain kernel

template <typename T, bool kFinal>
__global__ __launch_bounds__(kBlock) void partial_kernel(Problem p, const T *__restrict__ x,
                                                         const T *__restrict__ dy, float *__restrict__ ws,
                                                         T *__restrict__ dw, int welems, int rows_per_chunk)
{
    // thread order (c, k, g, tap), c fastest: a wave's lanes share one tap
    // where they can, so one x load reads a contiguous run of a pixel's
    // channels across groups (and neighbouring k share it) and one dy load a
    // run of the output pixel's; f is the element's place in dw [g][k][tap][c]
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int ch = blockIdx.y;
    if (i >= welems) return;
    int r = i;
    const int c = r % p.Cpg;  r /= p.Cpg;
    const int k = r % p.Kpg;  r /= p.Kpg;
    const int g = r % p.G;    r /= p.G;
    const int xx = r % p.X;   r /= p.X;
    const int yy = r % p.Y;   r /= p.Y;
    const int z = r;
    const int f = ((((g * p.Kpg + k) * p.Z + z) * p.Y + yy) * p.X + xx) * p.Cpg + c;
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
        // kU columns per step, their loads issued before the first product
        // (the sum still runs over ow in order)
        int ow = ow_lo;
        for (; ow + kU <= ow_hi; ow += kU) {
            T dv[kU], xv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int iw = (ow + u) * p.sw - p.pw + xx * p.dw;
                dv[u] = dyr[(size_t)(ow + u) * K];
                xv[u] = xr[(size_t)iw * C];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) acc = fmaf(to_f32(dv[u]), to_f32(xv[u]), acc);
        }
        for (; ow < ow_hi; ++ow) {
            const int iw = ow * p.sw - p.pw + xx * p.dw;
            acc = fmaf(to_f32(dyr[(size_t)ow * K]), to_f32(xr[(size_t)iw * C]), acc);
        }
    }
    if (kFinal) dw[f] = from_f32<T>(acc);
    else ws[(size_t)ch * welems + f] = acc;
}

// acc[i][j] += dy channel i * x channel j over one pixel: 4 dy values (8
// bytes) against 8 x values (16 bytes)
template <typename T>
__device__ __forceinline__ void tile_fma(float (&acc)[4][8], uint4 xv4, uint2 dv2)
{
    const T *xv = reinterpret_cast<const T *>(&xv4);
    const T *dv = reinterpret_cast<const T *>(&dv2);
    float xf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xf[j] = to_f32(xv[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float d = to_f32(dv[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(d, xf[j], acc[i][j]);
    }
}

// Grouped, half types, Cpg % 8 == 0 and Kpg % 4 == 0: a register-tiled
// stage 1.  Thread (chunk, tile) owns 4 output channels x 8 input channels
// of one tap of one group; per output pixel it loads the 8 input channels
// of x (16 bytes) and the 4 output channels of dy (8 bytes) and does 32
// FMAs.  Consecutive threads take consecutive 8-channel vectors of x, so a
// wave's x loads are contiguous runs.  Partial sums go to [chunk][f] as in
// the plain kernel (or to dw with one chunk).
template <typename T, bool kFinal>
__global__ __launch_bounds__(kBlock) void tile_partial_kernel(Problem p, const T *__restrict__ x,
                                                              const T *__restrict__ dy, float *__restrict__ ws,
                                                              T *__restrict__ dw, int ntiles, int rows_per_chunk)
{
    const int tile = blockIdx.x * kBlock + threadIdx.x;
    const int ch = blockIdx.y;
    if (tile >= ntiles) return;
    // tile order (c vector, k tile, tap, g); putting g before the taps (as
    // the plain kernel does) measured 5% slower on 8-channel groups
    const int ncv = p.Cpg / 8, nkt = p.Kpg / 4;
    int r = tile;
    const int cv = r % ncv;  r /= ncv;
    const int kt = r % nkt;  r /= nkt;
    const int xx = r % p.X;  r /= p.X;
    const int yy = r % p.Y;  r /= p.Y;
    const int z = r % p.Z;   r /= p.Z;
    const int g = r;
    const int c0 = cv * 8, k0 = kt * 4;
    const int C = p.G * p.Cpg, K = p.G * p.Kpg;
    const int rows = p.N * p.Do * p.Ho;
    const int r0 = ch * rows_per_chunk;
    const int r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
    int ow_lo = 0, ow_hi = p.Wo;
    {
        const int off = xx * p.dw - p.pw;
        if (off < 0) ow_lo = (-off + p.sw - 1) / p.sw;
        const int lim = p.W - off;
        const int hi = lim <= 0 ? 0 : (lim + p.sw - 1) / p.sw;
        if (hi < ow_hi) ow_hi = hi;
    }
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int rr = r0; rr < r1; ++rr) {
        const int oh = rr % p.Ho, t = rr / p.Ho;
        const int od = t % p.Do, n = t / p.Do;
        const int id = od * p.sd - p.pd + z * p.dd;
        const int ih = oh * p.sh - p.ph + yy * p.dh;
        if (id < 0 || id >= p.D || ih < 0 || ih >= p.H) continue;
        const T *dyr = dy + ((size_t)((n * p.Do + od) * p.Ho + oh) * p.Wo) * K + g * p.Kpg + k0;
        const T *xr = x + ((size_t)((n * p.D + id) * p.H + ih) * p.W) * C + g * p.Cpg + c0;
        // one column per step: four columns per step (their loads first)
        // measured 14% slower on 8-channel groups, 7% faster on 128-channel
        for (int ow = ow_lo; ow < ow_hi; ++ow) {
            const int iw = ow * p.sw - p.pw + xx * p.dw;
            tile_fma<T>(acc, *reinterpret_cast<const uint4 *>(xr + (size_t)iw * C),
                        *reinterpret_cast<const uint2 *>(dyr + (size_t)ow * K));
        }
    }
    const int T9 = p.Z * p.Y * p.X;
    const int welems = p.G * p.Kpg * T9 * p.Cpg;
    const int tap = (z * p.Y + yy) * p.X + xx;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int f0 = ((g * p.Kpg + k0 + i) * T9 + tap) * p.Cpg + c0;   // dw [g][k][tap][c]
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (kFinal) dw[f0 + j] = from_f32<T>(acc[i][j]);
            else ws[(size_t)ch * welems + f0 + j] = acc[i][j];
        }
    }
}

// Stage 2: a workgroup owns E weight elements; its kBlock / E lane groups
// split their chunks (group q takes chunks q, q + kBlock / E, ...; eight
// running sums each, loads in flight together), and the group sums are added
// in group order through LDS.  A fixed order throughout: deterministic.  E is
// 64 (whole 256-byte rows of the workspace per wave) unless the weight is
// small, where 16 gives four times the workgroups and a quarter of the
// dependent rounds per lane.
template <typename T, int E>
__global__ __launch_bounds__(kBlock) void reduce_kernel(const float *__restrict__ ws, T *__restrict__ dw,
                                                        int welems, int nch)
{
    constexpr int NQ = kBlock / E;
    __shared__ float part[NQ][E];
    const int l = threadIdx.x % E, q = threadIdx.x / E;
    const int f = blockIdx.x * E + l;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (f < welems) {
        int ch = q;
        for (; ch + 7 * NQ < nch; ch += 8 * NQ)
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] += ws[(size_t)(ch + u * NQ) * welems + f];
        for (; ch < nch; ch += NQ) a[0] += ws[(size_t)ch * welems + f];
    }
    part[q][l] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    __syncthreads();
    if (q == 0 && f < welems) {
        float sum = part[0][l];
#pragma unroll
        for (int r = 1; r < NQ; ++r) sum += part[r][l];
        dw[f] = from_f32<T>(sum);
    }
}

template <typename T>
hipError_t reduce(const float *ws, T *dw, int welems, int nch, hipStream_t s)
{
    Args a{};
    if (welems < 8192)
        return enqueue(reduce_kernel<T, 16>, dim3((unsigned)((welems + 15) / 16)), dim3(kBlock), 0, s, a, ws, dw,
                       welems, nch);
    return enqueue(reduce_kernel<T, 64>, dim3((unsigned)((welems + 63) / 64)), dim3(kBlock), 0, s, a, ws, dw,
                   welems, nch);
}

// Depthwise 3x3 (Cpg = Kpg = 1, nine taps, at most 256 channel vectors of
// 16 bytes): a workgroup owns every channel of one chunk of output pixels.
// Lane `tid` takes channel vector v = tid % nv of pixel slot tid / nv, so
// the lanes of a wave read whole pixels (all C channels, contiguous) of dy
// and of the nine x pixels the taps read; each lane keeps 9 x VEC fp32 sums
// over the pixels of its slot.  Per tap the slots' sums are added in slot
// order through LDS and one partial per (tap, channel) is written:
// [chunk][g][tap], or dw itself when there is one chunk.
constexpr int kDwTaps = 9;
constexpr int kDwPix = 2;   // pixels per lane per iteration (3 measured slower)
constexpr int kDwChunks = 512;   // two workgroups per CU (768, three per CU, measured slower)

// 16 zero bytes: the operand of a tap that falls outside the input
__device__ __align__(16) uint4 kZero16 = {0u, 0u, 0u, 0u};

template <typename T, bool kFinal>
__global__ __launch_bounds__(kBlock) void dw_partial_kernel(Problem p, const T *__restrict__ x,
                                                            const T *__restrict__ dy, float *__restrict__ ws,
                                                            T *__restrict__ dw, int ppc)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    __shared__ float red[kBlock * VEC];          // [slot][channel]
    const int tid = threadIdx.x, ch = blockIdx.x;
    const int nv = p.G / VEC, slots = kBlock / nv;
    const int v = tid % nv, slot = tid / nv;
    const bool active = slot < slots;
    const int g0 = v * VEC;
    const int M = p.N * p.Do * p.Ho * p.Wo;
    const int m0 = ch * ppc;
    const int m1 = m0 + ppc < M ? m0 + ppc : M;
    float acc[kDwTaps][VEC];
    int oz[kDwTaps], oy[kDwTaps], ox[kDwTaps];   // input offset of each tap (tap * dil - pad)
#pragma unroll
    for (int t = 0; t < kDwTaps; ++t) {
        oz[t] = (t / (p.Y * p.X)) * p.dd - p.pd;
        oy[t] = ((t / p.X) % p.Y) * p.dh - p.ph;
        ox[t] = (t % p.X) * p.dw - p.pw;
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[t][j] = 0.f;
    }
    if (active) {
        // kDwPix pixels of the slot per iteration (m, m + slots, ...), all
        // their loads in flight before the first product.  A tap outside the
        // input reads 16 zero bytes (kZero16) instead of its pixel, and a
        // pixel past the chunk's end reads them for dy and every x: the choice
        // is made on the address, so no loaded value is touched before the
        // products (each tap's sum still runs over the slot's pixels in order)
        const T *zero = reinterpret_cast<const T *>(&kZero16);
        for (int m = m0 + slot; m < m1; m += kDwPix * slots) {
            uint4 dr[kDwPix];
            uint4 xr[kDwPix][kDwTaps];
#pragma unroll
            for (int u = 0; u < kDwPix; ++u) {
                const int mu = m + u * slots;
                const bool pad = mu >= m1;
                int r = mu;
                const int ow = r % p.Wo; r /= p.Wo;
                const int oh = r % p.Ho; r /= p.Ho;
                const int od = r % p.Do; r /= p.Do;
                const int n = r;
                dr[u] = *reinterpret_cast<const uint4 *>(pad ? zero : dy + (size_t)mu * p.G + g0);
#pragma unroll
                for (int t = 0; t < kDwTaps; ++t) {
                    const int id = od * p.sd + oz[t];
                    const int ih = oh * p.sh + oy[t];
                    const int iw = ow * p.sw + ox[t];
                    const bool in = !pad && (unsigned)id < (unsigned)p.D && (unsigned)ih < (unsigned)p.H &&
                                    (unsigned)iw < (unsigned)p.W;
                    const T *src = in ? x + (((size_t)(n * p.D + id) * p.H + ih) * p.W + iw) * p.G + g0 : zero;
                    xr[u][t] = *reinterpret_cast<const uint4 *>(src);
                }
            }
            float df[kDwPix][VEC];
#pragma unroll
            for (int u = 0; u < kDwPix; ++u) {
                const T *dv = reinterpret_cast<const T *>(&dr[u]);
#pragma unroll
                for (int j = 0; j < VEC; ++j) df[u][j] = to_f32(dv[j]);
            }
#pragma unroll
            for (int u = 0; u < kDwPix; ++u)
#pragma unroll
                for (int t = 0; t < kDwTaps; ++t) {
                    const T *xv = reinterpret_cast<const T *>(&xr[u][t]);
#pragma unroll
                    for (int j = 0; j < VEC; ++j) acc[t][j] = fmaf(df[u][j], to_f32(xv[j]), acc[t][j]);
                }
        }
    }
    const int welems = p.G * kDwTaps;
#pragma unroll
    for (int t = 0; t < kDwTaps; ++t) {
        if (active) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) red[slot * p.G + g0 + j] = acc[t][j];
        }
        __syncthreads();
        for (int g = tid; g < p.G; g += kBlock) {
            float sum = 0.f;
            for (int q = 0; q < slots; ++q) sum += red[q * p.G + g];
            const int f = g * kDwTaps + t;             // dw [g][k = 0][tap][c = 0]
            if (kFinal) dw[f] = from_f32<T>(sum);
            else ws[(size_t)ch * welems + f] = sum;
        }
        __syncthreads();
    }
}

// The row-run form of the depthwise kernel for 2D 3x3 windows at stride S
// (1 or 2) and dilation 1: an item is kDwRun<S> output rows of one image at
// `slots` consecutive columns; lane (slot, v) owns one column and one
// channel vector.  It loads each input row of the run once (three columns:
// the window's) instead of once per output pixel and tap, and the run's dy
// vectors, all before the first product, then adds the products row by row.
// Outside the input, past the last column and for rows past the image's
// output, the loads read 16 zero bytes; a row past the output adds nothing.
// Each lane walks its chunk's items in order, and the slots are joined per
// tap through LDS in slot order, as in the plain form.  Runs of 8 rows at
// stride 1 (10 input rows, 248 VGPRs in fp16, no spills) and 4 at stride 2
// (measured on the MobileNet-style stride-1 case against runs of 4: 31.8 ->
// 29.5 us per call; the plain form took 36.2).
template <int S> constexpr int kDwRun = S == 1 ? 8 : 4;

template <typename T, bool kFinal, int S>
__global__ __launch_bounds__(kBlock) void dw_rows_kernel(Problem p, const T *__restrict__ x,
                                                         const T *__restrict__ dy, float *__restrict__ ws,
                                                         T *__restrict__ dw, int ipc, int items)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int RUN = kDwRun<S>;
    constexpr int NXR = (RUN - 1) * S + 3;        // input rows of a run
    __shared__ float red[kBlock * VEC];          // [slot][channel]
    const int tid = threadIdx.x, ch = blockIdx.x;
    const int nv = p.G / VEC, slots = kBlock / nv;
    const int v = tid % nv, slot = tid / nv;
    const bool active = slot < slots;
    const int g0 = v * VEC;
    const int ncb = (p.Wo + slots - 1) / slots, nrb = (p.Ho + RUN - 1) / RUN;
    const int it0 = ch * ipc, it1 = it0 + ipc < items ? it0 + ipc : items;
    const T *zero = reinterpret_cast<const T *>(&kZero16);
    float acc[kDwTaps][VEC];
#pragma unroll
    for (int t = 0; t < kDwTaps; ++t)
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[t][j] = 0.f;
    if (active) {
        for (int it = it0; it < it1; ++it) {
            int r = it;
            const int cb = r % ncb;  r /= ncb;
            const int rb = r % nrb;
            const int n = r / nrb;
            const int ow = cb * slots + slot;
            const bool col = ow < p.Wo;
            const int oh0 = rb * RUN;
            const int ih0 = oh0 * S - p.ph, iw0 = ow * S - p.pw;
            uint4 xr[NXR][3];
            uint4 dr[RUN];
#pragma unroll
            for (int i = 0; i < NXR; ++i)
#pragma unroll
                for (int tx = 0; tx < 3; ++tx) {
                    const int ih = ih0 + i, iw = iw0 + tx;
                    const bool in = col && (unsigned)ih < (unsigned)p.H && (unsigned)iw < (unsigned)p.W;
                    xr[i][tx] = *reinterpret_cast<const uint4 *>(
                        in ? x + (((size_t)n * p.H + ih) * p.W + iw) * p.G + g0 : zero);
                }
#pragma unroll
            for (int k = 0; k < RUN; ++k) {
                const bool in = col && oh0 + k < p.Ho;
                dr[k] = *reinterpret_cast<const uint4 *>(
                    in ? dy + (((size_t)n * p.Ho + oh0 + k) * p.Wo + ow) * p.G + g0 : zero);
            }
#pragma unroll
            for (int k = 0; k < RUN; ++k) {
                if (oh0 + k >= p.Ho) break;              // the same for every lane of the item
                const T *dv = reinterpret_cast<const T *>(&dr[k]);
                float df[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) df[j] = to_f32(dv[j]);
#pragma unroll
                for (int ty = 0; ty < 3; ++ty)
#pragma unroll
                    for (int tx = 0; tx < 3; ++tx) {
                        const T *xv = reinterpret_cast<const T *>(&xr[k * S + ty][tx]);
#pragma unroll
                        for (int j = 0; j < VEC; ++j)
                            acc[ty * 3 + tx][j] = fmaf(df[j], to_f32(xv[j]), acc[ty * 3 + tx][j]);
                    }
            }
        }
    }
    const int welems = p.G * kDwTaps;
#pragma unroll
    for (int t = 0; t < kDwTaps; ++t) {
        if (active) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) red[slot * p.G + g0 + j] = acc[t][j];
        }
        __syncthreads();
        for (int g = tid; g < p.G; g += kBlock) {
            float sum = 0.f;
            for (int q = 0; q < slots; ++q) sum += red[q * p.G + g];
            const int f = g * kDwTaps + t;             // dw [g][k = 0][tap][c = 0]
            if (kFinal) dw[f] = from_f32<T>(sum);
            else ws[(size_t)ch * welems + f] = sum;
        }
        __syncthreads();
    }
}

// the row-run form: 2D, 3x3, dilation 1, the same stride 1 or 2 on both axes
bool rows_ok(const Problem &p)
{
    return p.ndim == 2 && p.Y == 3 && p.X == 3 && p.dh == 1 && p.dw == 1 && p.sh == p.sw &&
           (p.sh == 1 || p.sh == 2) && p.ph >= 0 && p.pw >= 0;
}

bool dw_ok(const Problem &p)
{
    const int vec = 16 / elem_size(p.dtype);
    return p.Cpg == 1 && p.Kpg == 1 && p.taps() == kDwTaps && p.G % vec == 0 && p.G / vec <= kBlock;
}

// Stage 1 of the depthwise kernel: two workgroups per CU, at most `nch`
// chunks (what the workspace holds) and at most kDwChunks so stage 2 stays
// short; one chunk writes dw directly when dw is given.
template <typename T>
hipError_t go_dw(const Problem &p, const void *x, const void *dy, void *dw, float *ws, int nch, int *used,
                 hipStream_t s)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    const int slots = kBlock / (p.G / VEC);
    Args a{};
    if (rows_ok(p)) {
        const int run = p.sh == 1 ? kDwRun<1> : kDwRun<2>;
        const long long items = (long long)p.N * ((p.Ho + run - 1) / run) * ((p.Wo + slots - 1) / slots);
        long long want = kDwChunks;
        if (want > nch) want = nch;
        if (want > items) want = items;
        if (want < 1) want = 1;
        const int ipc = (int)((items + want - 1) / want);
        const int chunks = (int)((items + ipc - 1) / ipc);
        *used = chunks;
        if (chunks == 1 && dw) {
            auto k = p.sh == 1 ? dw_rows_kernel<T, true, 1> : dw_rows_kernel<T, true, 2>;
            return enqueue(k, dim3(1), dim3(kBlock), 0, s, a, p, (const T *)x, (const T *)dy, (float *)nullptr,
                           (T *)dw, ipc, (int)items);
        }
        auto k = p.sh == 1 ? dw_rows_kernel<T, false, 1> : dw_rows_kernel<T, false, 2>;
        return enqueue(k, dim3(chunks), dim3(kBlock), 0, s, a, p, (const T *)x, (const T *)dy, ws, (T *)nullptr,
                       ipc, (int)items);
    }
    const long long M = (long long)p.N * p.Do * p.Ho * p.Wo;
    long long want = kDwChunks;
    if (want > nch) want = nch;
    if (want > (M + slots - 1) / slots) want = (M + slots - 1) / slots;
    if (want < 1) want = 1;
    const int ppc = (int)((M + want - 1) / want);
    const int chunks = (int)((M + ppc - 1) / ppc);
    *used = chunks;
    if (chunks == 1 && dw)
        return enqueue(dw_partial_kernel<T, true>, dim3(1), dim3(kBlock), 0, s, a, p, (const T *)x,
                       (const T *)dy, (float *)nullptr, (T *)dw, ppc);
    return enqueue(dw_partial_kernel<T, false>, dim3(chunks), dim3(kBlock), 0, s, a, p, (const T *)x,
                   (const T *)dy, ws, (T *)nullptr, ppc);
}

bool tile_ok(const Problem &p)
{
    return p.dtype != GCONV_F32 && p.Cpg % 8 == 0 && p.Kpg % 4 == 0;
}

// Stage 1 of the register-tiled and plain kernels: chunks of output rows.
template <typename T>
hipError_t go(const Problem &p, const void *x, const void *dy, void *dw, float *ws, int nch, int *used,
              hipStream_t s)
{
    const int welems = p.G * p.Kpg * p.taps() * p.Cpg;
    const int rows = p.N * p.Do * p.Ho;
    const int rpc = (rows + nch - 1) / nch;
    nch = (rows + rpc - 1) / rpc;                  // no empty chunk
    *used = nch;
    const bool final_ = nch == 1 && dw;
    const dim3 grid((unsigned)((welems + kBlock - 1) / kBlock), (unsigned)nch);
    Args a{};
    if (tile_ok(p) && ((uintptr_t)x & 15) == 0 && ((uintptr_t)dy & 7) == 0) {
        const int ntiles = welems / 32;
        const dim3 tg((unsigned)((ntiles + kBlock - 1) / kBlock), (unsigned)nch);
        if (final_)
            return enqueue(tile_partial_kernel<T, true>, tg, dim3(kBlock), 0, s, a, p, (const T *)x, (const T *)dy,
                           (float *)nullptr, (T *)dw, ntiles, rpc);
        return enqueue(tile_partial_kernel<T, false>, tg, dim3(kBlock), 0, s, a, p, (const T *)x,
                       (const T *)dy, ws, (T *)nullptr, ntiles, rpc);
    }
    if (final_)
        return enqueue(partial_kernel<T, true>, grid, dim3(kBlock), 0, s, a, p, (const T *)x, (const T *)dy,
                       (float *)nullptr, (T *)dw, welems, rpc);
    return enqueue(partial_kernel<T, false>, grid, dim3(kBlock), 0, s, a, p, (const T *)x,
                   (const T *)dy, ws, (T *)nullptr, welems, rpc);
}

bool vec_aligned(const void *x, const void *dy)
{
    return ((uintptr_t)x & 15) == 0 && ((uintptr_t)dy & 15) == 0;
}

}  // namespace

// Chunks that fill the chip: the MFMA route's own count; else about 256 K
// stage-1 threads (one per weight element, or per 4 x 8 tile on the tiled
// route), at most one chunk per output row, at most 65535 (the grid's y
// extent); for the depthwise kernel, up to kDwChunks workgroups of one
// chunk each.
int ideal_chunks(const Problem &p)
{
    if (dw_ok(p)) {   // the depthwise kernel: up to kDwChunks workgroups, one chunk each
        const long long slots = kBlock / (p.G / (16 / elem_size(p.dtype)));
        const long long m = ((long long)p.N * p.Do * p.Ho * p.Wo + slots - 1) / slots;
        return (int)(m < kDwChunks ? (m < 1 ? 1 : m) : kDwChunks);
    }
    if (bwdw_mfma::supported(p)) return bwdw_mfma::chunks(p);
    const long long welems = (long long)p.G * p.Kpg * p.taps() * p.Cpg;
    const long long rows = (long long)p.N * p.Do * p.Ho;
    const long long threads = tile_ok(p) ? welems / 32 : welems;   // stage-1 threads per chunk
    long long n = (262144 + threads - 1) / threads;
    if (n > rows) n = rows;
    if (n > 65535) n = 65535;
    return n < 1 ? 1 : (int)n;
}

hipError_t stage1(const Problem &p, const void *x, const void *dy, float *ws, void *dw, int nch, int *used,
                  hipStream_t s)
{
    if (nch < 1) nch = 1;
    const bool vec_ok = vec_aligned(x, dy);
    if (dw_ok(p) && vec_ok) {
        switch (p.dtype) {
        case GCONV_F32: return go_dw<float>(p, x, dy, dw, ws, nch, used, s);
        case GCONV_F16: return go_dw<_Float16>(p, x, dy, dw, ws, nch, used, s);
        default: return go_dw<__bf16>(p, x, dy, dw, ws, nch, used, s);
        }
    }
    if (vec_ok && bwdw_mfma::supported(p)) return bwdw_mfma::stage1(p, x, dy, ws, dw, nch, used, s);
    switch (p.dtype) {
    case GCONV_F32: return go<float>(p, x, dy, dw, ws, nch, used, s);
    case GCONV_F16: return go<_Float16>(p, x, dy, dw, ws, nch, used, s);
    default: return go<__bf16>(p, x, dy, dw, ws, nch, used, s);
    }
}

hipError_t stage2(const Problem &p, const float *ws, void *dw, int nch, hipStream_t s)
{
    const int welems = p.G * p.Kpg * p.taps() * p.Cpg;
    switch (p.dtype) {
    case GCONV_F32: return reduce<float>(ws, (float *)dw, welems, nch, s);
    case GCONV_F16: return reduce<_Float16>(ws, (_Float16 *)dw, welems, nch, s);
    default: return reduce<__bf16>(ws, (__bf16 *)dw, welems, nch, s);
    }
}

}  // namespace bwdw
}  // namespace gconv

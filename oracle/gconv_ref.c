/*
 * gconv_ref.c -- plain CPU oracle for grouped / depthwise convolution forward,
 * backward data and backward weight.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * path (the HIP library and its Python binding) never does, and shares no
 * code, header or constant with this file.
 *
 * What it computes is the grouped cross-correlation written out from its
 * definition, in double precision, one output element at a time:
 *
 *   input channel of group g, channel c   = g*Cpg + c
 *     (rocm-libraries PR 10064, Technical Details: the A descriptor embeds
 *      (group, c_in_group) into the channel index)
 *   output channel of group g, channel k  = g*Kpg + k
 *     (same page, Technical Details: B/D fold k_out = g*kpg + n)
 *   taps: the filter is not flipped (cross-correlation, as the PyTorch
 *     convolution the TileOPs PR 1568 review uses as its comparator);
 *   input coordinate of tap t along one axis = o*stride - pad + t*dilation,
 *     taps that fall outside the input read zero (symmetric zero padding, one
 *     pad value per axis as in the CK grouped_conv tile-engine README,
 *     Problem Registry field list);
 *   output extent = floor((in + 2*pad - dil*(k-1) - 1) / stride) + 1.
 *
 * Layouts (last index fastest), the forward layouts the CK Python examples
 * README names in its Examples table (NHWGC input, GKYXC weight), extended to
 * 3D with a leading depth axis:
 *   x    [N][D][H][W][G][Cpg]
 *   w    [G][Kpg][Z][Y][X][Cpg]
 *   y    [N][Do][Ho][Wo][G][Kpg]
 *   bias [G*Kpg]                    (NULL = no bias)
 * A 2D problem is the 3D one with D = Z = 1, stride/dil 1 and pad 0 in depth.
 *
 * Besides y the oracle returns, per output element, scale = sum of |x*w| over
 * the taps it summed plus |bias|, which the parity tolerance is written
 * against.  Accumulation is in double; inputs are the exact values of the
 * fp32/fp16/bf16 tensors widened to double by the caller.
 *
 * Built with gcc -O2 -fopenmp (no fast-math): the only parallelism is an
 * OpenMP split over independent output rows.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>

/* Number of output positions along one axis; 0 when no window fits. */
int64_t gref_out_extent(int64_t in, int64_t k, int64_t stride, int64_t pad,
                        int64_t dil)
{
    int64_t span = dil * (k - 1) + 1; /* extent of the dilated filter */
    int64_t room = in + 2 * pad - span;
    if (in <= 0 || k <= 0 || stride <= 0 || dil <= 0 || pad < 0 || room < 0)
        return 0;
    return room / stride + 1;
}

/* One output element, the definition written out. */
static void one_output(int64_t G, int64_t Cpg, int64_t Kpg,
                       const int64_t in[3], const int64_t filt[3],
                       const int64_t stride[3], const int64_t pad[3],
                       const int64_t dil[3],
                       const double *x, const double *w, const double *bias,
                       int64_t n, int64_t od, int64_t oh, int64_t ow,
                       int64_t g, int64_t k, double *y_out, double *s_out)
{
    const int64_t D = in[0], H = in[1], W = in[2];
    const int64_t Z = filt[0], Y = filt[1], X = filt[2];
    double acc = 0.0, s = 0.0;
    for (int64_t z = 0; z < Z; ++z) {
        int64_t id = od * stride[0] - pad[0] + z * dil[0];
        if (id < 0 || id >= D) continue;
        for (int64_t yy = 0; yy < Y; ++yy) {
            int64_t ih = oh * stride[1] - pad[1] + yy * dil[1];
            if (ih < 0 || ih >= H) continue;
            for (int64_t xx = 0; xx < X; ++xx) {
                int64_t iw = ow * stride[2] - pad[2] + xx * dil[2];
                if (iw < 0 || iw >= W) continue;
                for (int64_t c = 0; c < Cpg; ++c) {
                    int64_t xi = ((((n * D + id) * H + ih) * W + iw) * G + g) * Cpg + c;
                    int64_t wi = ((((g * Kpg + k) * Z + z) * Y + yy) * X + xx) * Cpg + c;
                    double t = x[xi] * w[wi];
                    acc += t;
                    s += fabs(t);
                }
            }
        }
    }
    if (bias) {
        double b = bias[g * Kpg + k];
        acc += b;
        s += fabs(b);
    }
    *y_out = acc;
    *s_out = s;
}

/*
 * Full forward: fills y and scale ([N][Do][Ho][Wo][G][Kpg] each).
 * Returns 0, or -1 when the sizes are inconsistent (C or K not divisible by
 * G, a non-positive size, or an empty output).
 */
int gref_conv_fwd(int64_t N, int64_t G, int64_t C, int64_t K,
                  const int64_t in[3], const int64_t filt[3],
                  const int64_t stride[3], const int64_t pad[3],
                  const int64_t dil[3],
                  const double *x, const double *w, const double *bias,
                  double *y, double *scale)
{
    if (N <= 0 || G <= 0 || C <= 0 || K <= 0 || C % G != 0 || K % G != 0)
        return -1;
    const int64_t Cpg = C / G, Kpg = K / G;
    int64_t out[3];
    for (int a = 0; a < 3; ++a) {
        out[a] = gref_out_extent(in[a], filt[a], stride[a], pad[a], dil[a]);
        if (out[a] <= 0) return -1;
    }
    const int64_t Do = out[0], Ho = out[1], Wo = out[2];
    const int64_t rows = N * Do * Ho;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t oh = r % Ho;
        int64_t od = (r / Ho) % Do;
        int64_t n = r / (Ho * Do);
        for (int64_t ow = 0; ow < Wo; ++ow)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t k = 0; k < Kpg; ++k) {
                    int64_t yi = ((((n * Do + od) * Ho + oh) * Wo + ow) * G + g) * Kpg + k;
                    one_output(G, Cpg, Kpg, in, filt, stride, pad, dil, x, w, bias,
                               n, od, oh, ow, g, k, &y[yi], &scale[yi]);
                }
    }
    return 0;
}

/*
 * Selected outputs only: idx[i] is a flat index into y's
 * [N][Do][Ho][Wo][G][Kpg] layout; y_out[i], s_out[i] receive that element.
 * Used to check full-size problems at sampled positions.
 * Returns 0, or -1 on inconsistent sizes or an index out of range.
 */
int gref_conv_fwd_points(int64_t N, int64_t G, int64_t C, int64_t K,
                         const int64_t in[3], const int64_t filt[3],
                         const int64_t stride[3], const int64_t pad[3],
                         const int64_t dil[3],
                         const double *x, const double *w, const double *bias,
                         const int64_t *idx, int64_t npts,
                         double *y_out, double *s_out)
{
    if (N <= 0 || G <= 0 || C <= 0 || K <= 0 || C % G != 0 || K % G != 0)
        return -1;
    const int64_t Cpg = C / G, Kpg = K / G;
    int64_t out[3];
    for (int a = 0; a < 3; ++a) {
        out[a] = gref_out_extent(in[a], filt[a], stride[a], pad[a], dil[a]);
        if (out[a] <= 0) return -1;
    }
    const int64_t Do = out[0], Ho = out[1], Wo = out[2];
    const int64_t total = N * Do * Ho * Wo * G * Kpg;
    for (int64_t i = 0; i < npts; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -1;

    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t e = idx[i];
        int64_t k = e % Kpg;   e /= Kpg;
        int64_t g = e % G;     e /= G;
        int64_t ow = e % Wo;   e /= Wo;
        int64_t oh = e % Ho;   e /= Ho;
        int64_t od = e % Do;   e /= Do;
        int64_t n = e;
        one_output(G, Cpg, Kpg, in, filt, stride, pad, dil, x, w, bias,
                   n, od, oh, ow, g, k, &y_out[i], &s_out[i]);
    }
    return 0;
}

/*
 * Backward data: the gradient of a loss with respect to x, given its
 * gradient dy with respect to y and the weights w (the backward-data variant
 * the CK grouped_conv tile-engine README lists next to forward, and whose
 * runner takes dY and W in the Python examples README, Runner argument
 * contract).  It is the adjoint of the forward map above: every forward term
 * x[n,id,ih,iw,g,c] * w[g,k,z,y,x,c] feeds y[n,od,oh,ow,g,k] with
 * id = od*stride - pad + z*dil (and likewise in h, w), so
 *
 *   dx[n,id,ih,iw,g,c] = sum over (z, y, x, k) with od = (id + pad - z*dil) / stride
 *                        an integer in [0, Do) (likewise oh, ow) of
 *                        dy[n,od,oh,ow,g,k] * w[g,k,z,y,x,c].
 *
 * Layouts: dy [N][Do][Ho][Wo][G][Kpg], w [G][Kpg][Z][Y][X][Cpg],
 * dx [N][D][H][W][G][Cpg]; in[] gives (D, H, W), which a strided forward does
 * not determine from dy.  scale receives sum |dy*w| over the terms summed.
 * Returns 0, or -1 on inconsistent sizes.
 */
int gref_conv_bwd_data(int64_t N, int64_t G, int64_t C, int64_t K,
                       const int64_t in[3], const int64_t filt[3],
                       const int64_t stride[3], const int64_t pad[3],
                       const int64_t dil[3],
                       const double *dy, const double *w, double *dx, double *scale)
{
    if (N <= 0 || G <= 0 || C <= 0 || K <= 0 || C % G != 0 || K % G != 0)
        return -1;
    const int64_t Cpg = C / G, Kpg = K / G;
    int64_t out[3];
    for (int a = 0; a < 3; ++a) {
        out[a] = gref_out_extent(in[a], filt[a], stride[a], pad[a], dil[a]);
        if (out[a] <= 0) return -1;
    }
    const int64_t D = in[0], H = in[1], W = in[2];
    const int64_t Z = filt[0], Y = filt[1], X = filt[2];
    const int64_t Do = out[0], Ho = out[1], Wo = out[2];
    const int64_t rows = N * D * H;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t ih = r % H;
        const int64_t id = (r / H) % D;
        const int64_t n = r / (H * D);
        for (int64_t iw = 0; iw < W; ++iw)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t c = 0; c < Cpg; ++c) {
                    double acc = 0.0, s = 0.0;
                    for (int64_t z = 0; z < Z; ++z) {
                        const int64_t td = id + pad[0] - z * dil[0];
                        if (td < 0 || td % stride[0] != 0 || td / stride[0] >= Do) continue;
                        const int64_t od = td / stride[0];
                        for (int64_t yy = 0; yy < Y; ++yy) {
                            const int64_t th = ih + pad[1] - yy * dil[1];
                            if (th < 0 || th % stride[1] != 0 || th / stride[1] >= Ho) continue;
                            const int64_t oh = th / stride[1];
                            for (int64_t xx = 0; xx < X; ++xx) {
                                const int64_t tw = iw + pad[2] - xx * dil[2];
                                if (tw < 0 || tw % stride[2] != 0 || tw / stride[2] >= Wo) continue;
                                const int64_t ow = tw / stride[2];
                                for (int64_t k = 0; k < Kpg; ++k) {
                                    const int64_t yi = ((((n * Do + od) * Ho + oh) * Wo + ow) * G + g) * Kpg + k;
                                    const int64_t wi = ((((g * Kpg + k) * Z + z) * Y + yy) * X + xx) * Cpg + c;
                                    const double t = dy[yi] * w[wi];
                                    acc += t;
                                    s += fabs(t);
                                }
                            }
                        }
                    }
                    const int64_t xi = ((((n * D + id) * H + ih) * W + iw) * G + g) * Cpg + c;
                    dx[xi] = acc;
                    scale[xi] = s;
                }
    }
    return 0;
}

/*
 * Backward weight: the gradient of a loss with respect to w, given x and dy
 * (the third variant of the CK grouped_conv tile-engine README, introduction;
 * its runner takes X and dY in the Python examples README, Runner argument
 * contract).  Every forward term x[n,id,ih,iw,g,c] * w[g,k,z,y,x,c] feeds
 * y[n,od,oh,ow,g,k], so
 *
 *   dw[g,k,z,y,x,c] = sum over n, od, oh, ow with id = od*stride - pad + z*dil
 *                     (likewise ih, iw) inside the input of
 *                     dy[n,od,oh,ow,g,k] * x[n,id,ih,iw,g,c].
 *
 * Layouts: x [N][D][H][W][G][Cpg], dy [N][Do][Ho][Wo][G][Kpg],
 * dw [G][Kpg][Z][Y][X][Cpg].  scale receives sum |dy*x| over the terms
 * summed.  Returns 0, or -1 on inconsistent sizes.
 */
int gref_conv_bwd_weight(int64_t N, int64_t G, int64_t C, int64_t K,
                         const int64_t in[3], const int64_t filt[3],
                         const int64_t stride[3], const int64_t pad[3],
                         const int64_t dil[3],
                         const double *x, const double *dy, double *dw, double *scale)
{
    if (N <= 0 || G <= 0 || C <= 0 || K <= 0 || C % G != 0 || K % G != 0)
        return -1;
    const int64_t Cpg = C / G, Kpg = K / G;
    int64_t out[3];
    for (int a = 0; a < 3; ++a) {
        out[a] = gref_out_extent(in[a], filt[a], stride[a], pad[a], dil[a]);
        if (out[a] <= 0) return -1;
    }
    const int64_t D = in[0], H = in[1], W = in[2];
    const int64_t Z = filt[0], Y = filt[1], X = filt[2];
    const int64_t Do = out[0], Ho = out[1], Wo = out[2];
    const int64_t rows = G * Kpg;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t g = r / Kpg, k = r % Kpg;
        for (int64_t z = 0; z < Z; ++z)
            for (int64_t yy = 0; yy < Y; ++yy)
                for (int64_t xx = 0; xx < X; ++xx)
                    for (int64_t c = 0; c < Cpg; ++c) {
                        double acc = 0.0, s = 0.0;
                        for (int64_t n = 0; n < N; ++n)
                            for (int64_t od = 0; od < Do; ++od) {
                                const int64_t id = od * stride[0] - pad[0] + z * dil[0];
                                if (id < 0 || id >= D) continue;
                                for (int64_t oh = 0; oh < Ho; ++oh) {
                                    const int64_t ih = oh * stride[1] - pad[1] + yy * dil[1];
                                    if (ih < 0 || ih >= H) continue;
                                    for (int64_t ow = 0; ow < Wo; ++ow) {
                                        const int64_t iw = ow * stride[2] - pad[2] + xx * dil[2];
                                        if (iw < 0 || iw >= W) continue;
                                        const int64_t yi = ((((n * Do + od) * Ho + oh) * Wo + ow) * G + g) * Kpg + k;
                                        const int64_t xi = ((((n * D + id) * H + ih) * W + iw) * G + g) * Cpg + c;
                                        const double t = dy[yi] * x[xi];
                                        acc += t;
                                        s += fabs(t);
                                    }
                                }
                            }
                        const int64_t wi = ((((g * Kpg + k) * Z + z) * Y + yy) * X + xx) * Cpg + c;
                        dw[wi] = acc;
                        scale[wi] = s;
                    }
    }
    return 0;
}

/* Threads OpenMP will use for the parallel loops above. */
int gref_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

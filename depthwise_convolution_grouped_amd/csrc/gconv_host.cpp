// Host side of the C ABI declared in include/gconv.h: descriptor validation,
// output extents, path selection, launch shapes and the single launch per
// call.  Validation, extents, selection and plans make no HIP call, so they
// run (and are tested) on machines without a GPU.
//
// Validation follows rocm-libraries PR 10064 (Technical Details: the
// dispatcher checks C % G == 0 and K % G == 0 and accepts bf16 besides fp16
// and fp32) and the TileOPs PR 1568 review (summary: the forward ops route
// grouped problems to grouped kernels and check the expected weight shape;
// here the weight shape is implied by the descriptor).
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "gconv_internal.h"

#define GCONV_API extern "C" __attribute__((visibility("default")))

namespace gconv {

int &tile_choice()
{
    static thread_local int choice = -1;
    return choice;
}

namespace {

constexpr int64_t kMaxElems = (int64_t)INT32_MAX;  // elements a launch may index in 32 bits
constexpr int64_t kLim = (int64_t)INT32_MAX;       // bytes a launch's tensor may span (32-bit buffer offsets)

// out = floor((in + 2 pad - dil (k - 1) - 1) / stride) + 1, or 0 if no window fits.
int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d)
{
    int64_t room = in + 2 * p - d * (k - 1) - 1;
    return room < 0 ? 0 : room / s + 1;
}

// Product with saturation at INT64_MAX/2 so absurd descriptors cannot overflow.
int64_t sat_mul(int64_t a, int64_t b)
{
    const int64_t cap = INT64_MAX / 2;
    if (a <= 0 || b <= 0) return a * b;
    if (a > cap / b) return cap;
    return a * b;
}

int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// The spatial axis a call too large for one launch per image is split
// along: the outermost one (planes in 3D, rows in 2D), whose slices are
// contiguous in every layout.
int split_axis(const gconv_desc *d) { return d->ndim == 3 ? 0 : 1; }

// Bytes of one slice along the split axis: inner extents x channels.
int64_t slice_bytes(const gconv_desc *d, const int64_t ext[3], int64_t ch)
{
    int64_t b = ch * elem_size(d->dtype);
    for (int a = split_axis(d) + 1; a < 3; ++a) b = sat_mul(b, ext[a]);
    return b;
}

// Output slices per launch of a forward call split along the axis: the
// most whose input window (with its halo) and output each span < 2^31 bytes.
int64_t fwd_slices_per_launch(const gconv_desc *d, const int64_t out[3])
{
    const int a = split_axis(d);
    const int64_t xs = slice_bytes(d, d->in, d->C), ys = slice_bytes(d, out, d->K);
    const int64_t reach = d->dil[a] * (d->filt[a] - 1) + 1;     // input slices one output slice reads
    const int64_t by_y = kLim / ys, in_fit = kLim / xs;
    const int64_t by_x = in_fit < reach ? 0 : (in_fit - reach) / d->stride[a] + 1;
    return min64(by_y, by_x);
}

// dx slices per launch of a backward-data call split along the axis: dx,
// and the dy slices that reach it, each span < 2^31 bytes.
int64_t bwd_slices_per_launch(const gconv_desc *d, const int64_t out[3])
{
    const int a = split_axis(d);
    const int64_t xs = slice_bytes(d, d->in, d->C), ys = slice_bytes(d, out, d->K);
    const int64_t reach = d->dil[a] * (d->filt[a] - 1);
    const int64_t by_x = kLim / xs;
    // n dx slices read at most floor((n - 1 + reach) / s) + 2 dy slices
    const int64_t dy_fit = kLim / ys;
    const int64_t by_y = dy_fit < 2 ? 0 : (dy_fit - 2) * d->stride[a] + 1 - reach;
    return max64(0, min64(by_x, by_y));
}

int check_desc(const gconv_desc *d, int64_t out[3])
{
    if (!d) return GCONV_ERR_NULL_PTR;
    if (d->ndim != 2 && d->ndim != 3) return GCONV_ERR_BAD_DESC;
    if (d->dtype != GCONV_F32 && d->dtype != GCONV_F16 && d->dtype != GCONV_BF16)
        return GCONV_ERR_BAD_DESC;
    if (d->N <= 0 || d->G <= 0 || d->C <= 0 || d->K <= 0) return GCONV_ERR_BAD_DESC;
    if (d->C % d->G != 0 || d->K % d->G != 0) return GCONV_ERR_BAD_DESC;
    for (int a = 0; a < 3; ++a) {
        if (d->in[a] <= 0 || d->filt[a] <= 0 || d->stride[a] <= 0 || d->dil[a] <= 0 ||
            d->pad[a] < 0)
            return GCONV_ERR_BAD_DESC;
        // keep every per-axis quantity far from int32 overflow
        if (d->in[a] > kMaxElems || d->filt[a] > kMaxElems || d->stride[a] > kMaxElems ||
            d->dil[a] > kMaxElems || d->pad[a] > kMaxElems)
            return GCONV_ERR_TOO_LARGE;
    }
    if (d->ndim == 2 && (d->in[0] != 1 || d->filt[0] != 1 || d->stride[0] != 1 ||
                         d->dil[0] != 1 || d->pad[0] != 0))
        return GCONV_ERR_BAD_DESC;
    for (int a = 0; a < 3; ++a) {
        out[a] = out_extent(d->in[a], d->filt[a], d->stride[a], d->pad[a], d->dil[a]);
        if (out[a] <= 0) return GCONV_ERR_BAD_OUT_DIMS;
    }
    const int64_t Cpg = d->C / d->G, Kpg = d->K / d->G;
    int64_t x_el = sat_mul(sat_mul(sat_mul(sat_mul(d->N, d->in[0]), d->in[1]), d->in[2]), d->C);
    int64_t y_el = sat_mul(sat_mul(sat_mul(sat_mul(d->N, out[0]), out[1]), out[2]), d->K);
    int64_t w_el = sat_mul(sat_mul(sat_mul(sat_mul(d->K, d->filt[0]), d->filt[1]), d->filt[2]), Cpg);
    int64_t span = 0;
    for (int a = 0; a < 3; ++a)  // padded extent must also stay in int32
        span = span > d->in[a] + 2 * d->pad[a] ? span : d->in[a] + 2 * d->pad[a];
    if (w_el >= kMaxElems || span >= kMaxElems || d->K >= kMaxElems || d->C >= kMaxElems ||
        Kpg >= kMaxElems || d->N >= kMaxElems || x_el >= INT64_MAX / 4 || y_el >= INT64_MAX / 4)
        return GCONV_ERR_TOO_LARGE;
    // x and y may span more than a launch's 32-bit reach: calls then split
    // the batch into launches of whole images, and an image too large for
    // one launch into slices along the outermost spatial axis.  A slice
    // window that alone exceeds the reach cannot be split further.
    if (fwd_slices_per_launch(d, out) < 1 || bwd_slices_per_launch(d, out) < 1)
        return GCONV_ERR_TOO_LARGE;
    return GCONV_OK;
}

// Images per launch: the whole batch when x and y each span < 2^31 bytes,
// else the most whole images that keep both below; 0 when one image alone
// does not fit (the image is then split into slices).  The vector paths
// address a launch's tensors with 32-bit byte offsets, so a byte limit keeps
// every launch on the path the dispatcher would pick for its shape.
int64_t images_per_launch(const gconv_desc *d, const int64_t out[3])
{
    const int64_t es = elem_size(d->dtype);
    const int64_t x_img = d->in[0] * d->in[1] * d->in[2] * d->C * es;
    const int64_t y_img = out[0] * out[1] * out[2] * d->K * es;
    const int64_t nx = kLim / x_img, ny = kLim / y_img;
    const int64_t n = nx < ny ? nx : ny;
    return n < d->N ? n : d->N;
}

Problem to_problem(const gconv_desc *d, const int64_t out[3])
{
    Problem p;
    p.ndim = d->ndim;
    p.dtype = d->dtype;
    p.N = (int)d->N;
    p.G = (int)d->G;
    p.Cpg = (int)(d->C / d->G);
    p.Kpg = (int)(d->K / d->G);
    p.D = (int)d->in[0];  p.H = (int)d->in[1];  p.W = (int)d->in[2];
    p.Z = (int)d->filt[0]; p.Y = (int)d->filt[1]; p.X = (int)d->filt[2];
    p.Do = (int)out[0];   p.Ho = (int)out[1];   p.Wo = (int)out[2];
    p.sd = (int)d->stride[0]; p.sh = (int)d->stride[1]; p.sw = (int)d->stride[2];
    p.pd = (int)d->pad[0];    p.ph = (int)d->pad[1];    p.pw = (int)d->pad[2];
    p.dd = (int)d->dil[0];    p.dh = (int)d->dil[1];    p.dw = (int)d->dil[2];
    return p;
}

// Sets a problem's input extent, leading pad and output extent along axis a.
void set_axis(Problem &p, int a, int in, int pad, int out)
{
    if (a == 0) { p.D = in; p.pd = pad; p.Do = out; }
    else { p.H = in; p.ph = pad; p.Ho = out; }
}

// One launch of a call: a problem whose tensors each span < 2^31 bytes and
// the byte offsets of its input-side and output-side tensors (x and y for
// forward, dy and dx for backward data) in the caller's buffers.  Its leading
// pad along the split axis may differ from the trailing one (the window of
// a slice can start inside the image); kernels take the leading pad and
// the extents, never a symmetric pad.
struct Piece {
    Problem p;
    size_t in_off, out_off;
};

// Calls f(piece, first, last) for the launches of a forward call: one
// launch of the whole batch, else launches of whole images, else, image by
// image, launches of output slices along the split axis whose input windows
// (halo included) are taken from the image.  Stops at the first non-zero
// status f returns.
template <class F>
int for_fwd_pieces(const gconv_desc *d, const int64_t out[3], F &&f)
{
    const size_t es = (size_t)elem_size(d->dtype);
    const size_t x_img = (size_t)(d->in[0] * d->in[1] * d->in[2] * d->C) * es;
    const size_t y_img = (size_t)(out[0] * out[1] * out[2] * d->K) * es;
    const int64_t nl = images_per_launch(d, out);
    if (nl >= 1) {
        for (int64_t n0 = 0; n0 < d->N; n0 += nl) {
            const int64_t n = d->N - n0 < nl ? d->N - n0 : nl;
            Piece pc{to_problem(d, out), (size_t)n0 * x_img, (size_t)n0 * y_img};
            pc.p.N = (int)n;
            const int rc = f(pc, n0 == 0, n0 + n >= d->N);
            if (rc != GCONV_OK) return rc;
        }
        return GCONV_OK;
    }
    const int a = split_axis(d);
    const int64_t I = d->in[a], O = out[a], s = d->stride[a], pd = d->pad[a];
    const int64_t reach = d->dil[a] * (d->filt[a] - 1) + 1;
    const int64_t per = fwd_slices_per_launch(d, out);
    const size_t xs = (size_t)slice_bytes(d, d->in, d->C), ys = (size_t)slice_bytes(d, out, d->K);
    for (int64_t n = 0; n < d->N; ++n) {
        for (int64_t o0 = 0; o0 < O; o0 += per) {
            const int64_t o1 = min64(O, o0 + per);
            const int64_t i_lo = o0 * s - pd, i_hi = (o1 - 1) * s - pd + reach;
            int64_t lo = max64(i_lo, 0), hi = min64(i_hi, I);
            // a window wholly inside the trailing padding keeps one real
            // slice; its leading pad is then negative (generic kernel)
            if (hi <= lo) {
                lo = min64(lo, I - 1);
                hi = lo + 1;
            }
            Piece pc{to_problem(d, out), (size_t)n * x_img + (size_t)lo * xs, (size_t)n * y_img + (size_t)o0 * ys};
            pc.p.N = 1;
            set_axis(pc.p, a, (int)(hi - lo), (int)(lo - i_lo), (int)(o1 - o0));
            const int rc = f(pc, n == 0 && o0 == 0, n + 1 == d->N && o1 == O);
            if (rc != GCONV_OK) return rc;
        }
    }
    return GCONV_OK;
}

// The same for backward data: launches of whole images, else of dx slices
// along the split axis with the dy slices that reach them.  In a piece's
// problem the input extent is dx's and the output extent dy's.
template <class F>
int for_bwd_pieces(const gconv_desc *d, const int64_t out[3], F &&f)
{
    const size_t es = (size_t)elem_size(d->dtype);
    const size_t x_img = (size_t)(d->in[0] * d->in[1] * d->in[2] * d->C) * es;
    const size_t y_img = (size_t)(out[0] * out[1] * out[2] * d->K) * es;
    const int64_t nl = images_per_launch(d, out);
    if (nl >= 1) {
        for (int64_t n0 = 0; n0 < d->N; n0 += nl) {
            const int64_t n = d->N - n0 < nl ? d->N - n0 : nl;
            Piece pc{to_problem(d, out), (size_t)n0 * y_img, (size_t)n0 * x_img};
            pc.p.N = (int)n;
            const int rc = f(pc, n0 == 0, n0 + n >= d->N);
            if (rc != GCONV_OK) return rc;
        }
        return GCONV_OK;
    }
    const int a = split_axis(d);
    const int64_t I = d->in[a], O = out[a], s = d->stride[a], pd = d->pad[a];
    const int64_t reach = d->dil[a] * (d->filt[a] - 1);
    const int64_t per = bwd_slices_per_launch(d, out);
    const size_t xs = (size_t)slice_bytes(d, d->in, d->C), ys = (size_t)slice_bytes(d, out, d->K);
    for (int64_t n = 0; n < d->N; ++n) {
        for (int64_t i0 = 0; i0 < I; i0 += per) {
            const int64_t i1 = min64(I, i0 + per);
            // dy slices o with o s - pad + t dil in [i0, i1) for some tap t;
            // taking the lower end rounded down keeps the leading pad
            // pad + i0 - oa s >= dil (k - 1) >= 0 (extra slices add nothing)
            int64_t oa = floor_div(i0 + pd - reach, s), ob = floor_div(i1 - 1 + pd, s);
            oa = max64(0, min64(oa, O - 1));
            ob = max64(oa, min64(ob, O - 1));
            Piece pc{to_problem(d, out), (size_t)n * y_img + (size_t)oa * ys, (size_t)n * x_img + (size_t)i0 * xs};
            pc.p.N = 1;
            set_axis(pc.p, a, (int)(i1 - i0), (int)(pd + i0 - oa * s), (int)(ob - oa + 1));
            const int rc = f(pc, n == 0 && i0 == 0, n + 1 == d->N && i1 == I);
            if (rc != GCONV_OK) return rc;
        }
    }
    return GCONV_OK;
}

// The first launch of a forward call (what selection and plans describe).
Problem first_piece(const gconv_desc *d, const int64_t out[3])
{
    Problem first{};
    for_fwd_pieces(d, out, [&](const Piece &pc, bool, bool) {
        first = pc.p;
        return 1;   // stop after the first
    });
    return first;
}

bool path_ok(const Problem &p, int path)
{
    // a slice whose window starts below the image (negative leading pad)
    // runs on the generic kernel only
    if (path != GCONV_PATH_GENERIC && (p.pd < 0 || p.ph < 0 || p.pw < 0)) return false;
    switch (path) {
    case GCONV_PATH_GENERIC: return generic::supported(p);
    case GCONV_PATH_DEPTHWISE: return depthwise::supported(p);
    case GCONV_PATH_SMALLG: return smallg::supported(p);
    case GCONV_PATH_IGEMM: return igemm::supported(p);
    case GCONV_PATH_IGHALO: return ighalo::supported(p);
    case GCONV_PATH_DIRECT: return direct::supported(p);
    default: return false;
    }
}

// Channels-per-group dispatcher.  Depthwise (Cpg = Kpg = 1) goes to the VALU
// direct kernel; large per-group contractions (Cpg, Kpg >= 32, half types)
// are a real GEMM per group and go to the implicit-GEMM MFMA kernel; small
// groups in half types merge several groups into one block-diagonal MFMA
// tile; half-type groups neither takes (8k input channels that are not 32k,
// more than 16 output channels over narrow inputs) run the M-tiled implicit
// GEMM with its K walked in 8-channel chunks; the rest (fp32 grouped above
// all) takes the register-blocked VALU kernel when there is enough work to
// fill the chip, else the generic one.
//
// Between the two implicit GEMMs: the halo kernel reuses each staged input
// pixel across the window's taps, which pays at stride 1 with a window of
// more than one tap on 2D images, on 3D planes of up to 16 x 16 pixels and
// wherever its whole-box variant covers the problem in one round of
// workgroups; the M-tiled one measured faster elsewhere (the tile sweep: 3D
// planes of 28 x 28 and 56 x 56 in several rounds, stride 2, 1 x 1
// windows).  A 1 x 1 window over groups of fewer than 8 input channels
// measured faster on the VALU kernel.  Small groups that only the halo-box
// variant of the small-group kernel takes measured faster on the M-tiled
// implicit GEMM when a window of at most 9 taps is dilated (1.1-1.5x on
// 8-channel groups; a dilated 3x3x3 window measured faster on the box) or it
// has at most 4 taps, where the box's halo load and staging outweigh its
// reuse (1.7-2.4x on 8- and 16-channel groups with 1x1, 1x2 and 2x2
// windows: the residue classes of a stride-2 backward data); with 25 taps
// the box won by 2-3x.
bool halo_pays(const Problem &p)
{
    if (p.sd != 1 || p.sh != 1 || p.sw != 1 || p.taps() == 1) return false;
    if (p.ndim == 2) {
        // the box's extra pixels against the window's reuse: a 7x7 image
        // under a dilated 3x3 window (121 box pixels for 49 outputs, 9 taps)
        // ran 1.3-1.4x faster on M tiles, the same box under a dilated 5x5
        // window (25 taps) 1.3-2.9x faster on the halo kernel
        const long long box = (long long)(p.Ho + p.dh * (p.Y - 1)) * (p.Wo + p.dw * (p.X - 1));
        return 4 * box <= (long long)p.taps() * p.Ho * p.Wo;
    }
    return (long long)p.Ho * p.Wo <= 256 || ighalo_box::supported(p);
}

int select(const Problem &p)
{
    if (p.pd < 0 || p.ph < 0 || p.pw < 0) return GCONV_PATH_GENERIC;
    if (depthwise::supported(p)) return GCONV_PATH_DEPTHWISE;
    if (p.dtype != GCONV_F32 && p.Cpg >= 32 && p.Kpg >= 32) {
        const bool halo = halo_pays(p);
        if (halo && ighalo::supported(p)) return GCONV_PATH_IGHALO;
        if (igemm::supported(p)) return GCONV_PATH_IGEMM;
        if (ighalo::supported(p)) return GCONV_PATH_IGHALO;
    }
    if (p.taps() == 1 && p.Cpg < 8 && direct::preferred(p)) return GCONV_PATH_DIRECT;
    // fp32 on the implicit GEMM from 2048 output pixels x groups (16 M tiles'
    // worth): below that (a 2-group 8x8 image) the generic kernel's split
    // reductions measured 3x faster
    const bool small_f32 = p.dtype == GCONV_F32 && (long long)p.N * p.Do * p.Ho * p.Wo * p.G < 2048;
    const bool dilated = p.dd > 1 || p.dh > 1 || p.dw > 1;
    if (((dilated && p.taps() <= 9) || p.taps() <= 4) && !smallg::streams(p) && !small_f32 && igemm::supported(p))
        return GCONV_PATH_IGEMM;
    if (smallg::supported(p)) return GCONV_PATH_SMALLG;
    if (ighalo::supported(p)) return GCONV_PATH_IGHALO;
    if (!small_f32 && igemm::supported(p)) return GCONV_PATH_IGEMM;
    if (direct::preferred(p)) return GCONV_PATH_DIRECT;
    return GCONV_PATH_GENERIC;
}

int tiles_of(const Problem &p, int path, int *picked)
{
    switch (path) {
    case GCONV_PATH_DEPTHWISE: return depthwise::tiles(p, picked);
    case GCONV_PATH_SMALLG: return smallg::tiles(p, picked);
    case GCONV_PATH_IGEMM: return igemm::tiles(p, picked);
    case GCONV_PATH_IGHALO: return ighalo::tiles(p, picked);
    case GCONV_PATH_DIRECT: return direct::tiles(p, picked);
    default: return generic::tiles(p, picked);
    }
}

// Sets the tile choice of this host thread for the length of one call.
struct TileScope {
    int saved;
    explicit TileScope(int t) : saved(tile_choice()) { tile_choice() = t; }
    ~TileScope() { tile_choice() = saved; }
};

gconv_plan plan_of(const Problem &p, int path)
{
    switch (path) {
    case GCONV_PATH_DEPTHWISE: return depthwise::plan(p);
    case GCONV_PATH_SMALLG: return smallg::plan(p);
    case GCONV_PATH_IGEMM: return igemm::plan(p);
    case GCONV_PATH_IGHALO: return ighalo::plan(p);
    case GCONV_PATH_DIRECT: return direct::plan(p);
    default: return generic::plan(p);
    }
}

bool aligned(const void *ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// The path one launch takes (GCONV_PATH_AUTO: the dispatcher's pick, the
// generic kernel for pointers the 16-byte vector paths cannot take), or a
// negative status for a forced path that cannot run it.
int launch_path(const Problem &p, int path, const void *x, const void *w, const void *bias, const void *y)
{
    const bool vec_ok = aligned(x, 16) && aligned(w, 16) && aligned(y, 16) && (!bias || aligned(bias, 16));
    if (path == GCONV_PATH_AUTO) return vec_ok ? select(p) : GCONV_PATH_GENERIC;
    if (path < 0 || path >= GCONV_NUM_PATHS) return GCONV_ERR_BAD_PATH;
    if (!path_ok(p, path)) return GCONV_ERR_PATH_UNSUPPORTED;
    if (path != GCONV_PATH_GENERIC && !vec_ok) return GCONV_ERR_MISALIGNED;
    return path;
}

int launch_problem(const Problem &p, int path, const Args &a, hipStream_t s)
{
    hipError_t e;
    switch (path) {
    case GCONV_PATH_DEPTHWISE: e = depthwise::launch(p, a, s); break;
    case GCONV_PATH_SMALLG: e = smallg::launch(p, a, s); break;
    case GCONV_PATH_IGEMM: e = igemm::launch(p, a, s); break;
    case GCONV_PATH_IGHALO: e = ighalo::launch(p, a, s); break;
    case GCONV_PATH_DIRECT: e = direct::launch(p, a, s); break;
    default: e = generic::launch(p, a, s); break;
    }
    return e == hipSuccess ? GCONV_OK : GCONV_ERR_LAUNCH;
}

int run(const gconv_desc *d, int path, const void *x, const void *w, const void *bias,
        void *y, void *stream, void *ev_start = nullptr, void *ev_stop = nullptr)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    if (!x || !w || !y) return GCONV_ERR_NULL_PTR;
    const uintptr_t es = (uintptr_t)elem_size(d->dtype);
    if (!aligned(x, es) || !aligned(w, es) || !aligned(y, es) || (bias && !aligned(bias, es)))
        return GCONV_ERR_MISALIGNED;
    // every launch's path is settled before the first is enqueued, so a
    // forced path that cannot take one of them launches nothing
    rc = for_fwd_pieces(d, out, [&](const Piece &pc, bool, bool) {
        const int pth = launch_path(pc.p, path, (const char *)x + pc.in_off, w, bias, (const char *)y + pc.out_off);
        return pth < 0 ? pth : (int)GCONV_OK;
    });
    if (rc != GCONV_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    return for_fwd_pieces(d, out, [&](const Piece &pc, bool first, bool last) {
        const void *xp = (const char *)x + pc.in_off;
        void *yp = (char *)y + pc.out_off;
        const int pth = launch_path(pc.p, path, xp, w, bias, yp);
        // the start event is bound to the first launch, the stop event to the last
        Args a{xp, w, bias, yp, first ? (hipEvent_t)ev_start : nullptr, last ? (hipEvent_t)ev_stop : nullptr};
        return launch_problem(pc.p, pth, a, s);
    });
}

// Backward data at stride 1 is a forward convolution of dy (the input, with
// C' = K channels) with the flipped, C/K-exchanged weights (K' = C) under
// padding dil (k - 1) - pad, which must not be negative.
bool bwd_as_forward(const gconv_desc *d)
{
    for (int a = 0; a < 3; ++a)
        if (d->stride[a] != 1 || d->dil[a] * (d->filt[a] - 1) - d->pad[a] < 0) return false;
    return true;
}

// The forward problem that computes a backward-data piece at stride 1:
// input dy (the piece's output extents, K channels), output dx (its input
// extents, C channels), leading pad dil (k - 1) - pad per axis; false when a
// pad would be negative.
bool bwd_forward_problem(const Problem &q, Problem &t)
{
    t = q;
    t.Cpg = q.Kpg;
    t.Kpg = q.Cpg;
    t.D = q.Do; t.H = q.Ho; t.W = q.Wo;
    t.Do = q.D; t.Ho = q.H; t.Wo = q.W;
    t.sd = t.sh = t.sw = 1;
    t.pd = q.dd * (q.Z - 1) - q.pd;
    t.ph = q.dh * (q.Y - 1) - q.ph;
    t.pw = q.dw * (q.X - 1) - q.pw;
    return q.sd == 1 && q.sh == 1 && q.sw == 1 && t.pd >= 0 && t.ph >= 0 && t.pw >= 0;
}

size_t weight_bytes(const gconv_desc *d)
{
    return (size_t)d->K * (size_t)d->filt[0] * (size_t)d->filt[1] * (size_t)d->filt[2] *
           (size_t)(d->C / d->G) * (size_t)elem_size(d->dtype);
}

// ---- backward data at stride > 1: the polyphase route
//
// Per axis, the dx positions i = r + s m of residue class r receive the taps
// t with (t dil - r - pad) divisible by s: the progression t0 + j s' (s' =
// s / gcd(dil, s), J terms), which read dy at m - q0 - j dil' (q0 = (t0 dil -
// r - pad) / s, dil' = dil / gcd(dil, s)).  Taken in reverse order that is a
// stride-1 forward convolution of dy at dilation dil' under leading pad
// q0 + (J - 1) dil', whose outputs are the class's ceil((in - r) / s)
// positions.  Each combination of the axes' classes is one forward launch
// (the forward dispatcher on the class's problem, weights transformed into
// the workspace) into a dense buffer, and one scatter of it into dx; a
// combination with no tap on some axis scatters zeros.
struct AxisPhase {
    int t0, st, J, M, P, dl;
};

int gcd_int(int a, int b)
{
    while (b) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

AxisPhase axis_phase(int k, int s, int dil, int pad, int r, int in)
{
    AxisPhase a{};
    const int g = gcd_int(dil, s);
    a.st = s / g;
    a.dl = dil / g;
    a.M = r < in ? (in - r + s - 1) / s : 0;
    // the taps of the class form one residue class modulo s / gcd(dil, s),
    // so the first of them, if any, is below that
    a.t0 = -1;
    for (int t = 0; t < k && t < a.st; ++t)
        if (((t * dil - r - pad) % s + s) % s == 0) {
            a.t0 = t;
            break;
        }
    if (a.t0 < 0) {
        a.t0 = 0;
        a.J = 0;
        return a;
    }
    a.J = (k - 1 - a.t0) / a.st + 1;
    a.P = (a.t0 * dil - r - pad) / s + (a.J - 1) * a.dl;   // an exact division
    return a;
}

struct BwdPhase {
    bwd::PhaseTaps taps;
    int r[3], M[3], P[3], dl[3];
    bool any;        // every axis has a tap
    size_t w_off;    // the class's weights in the workspace
};

constexpr int kMaxPhases = 64;

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

// The classes of a strided backward data and the workspace they need
// (transformed weights, then the dense buffer of the largest class); false
// where the route does not apply: stride 1, depthwise problems (their
// channel-vector direct kernel is faster), more than kMaxPhases classes, or
// tensors that would need more than one launch.
bool bwd_phases(const Problem &p, BwdPhase *ph, int *nph, size_t *w_bytes, size_t *tmp_bytes)
{
    const int st[3] = {p.sd, p.sh, p.sw}, kk[3] = {p.Z, p.Y, p.X}, dl[3] = {p.dd, p.dh, p.dw};
    const int pd[3] = {p.pd, p.ph, p.pw}, in[3] = {p.D, p.H, p.W};
    if (st[0] == 1 && st[1] == 1 && st[2] == 1) return false;
    if (p.Cpg == 1 && p.Kpg == 1) return false;
    const long long n = (long long)st[0] * st[1] * st[2];
    if (n > kMaxPhases) return false;
    const long long es = elem_size(p.dtype);
    if ((long long)p.N * p.D * p.H * p.W * p.C() * es >= kLim ||
        (long long)p.N * p.Do * p.Ho * p.Wo * p.K() * es >= kLim)
        return false;
    size_t wb = 0, tb = 0;
    int cnt = 0;
    for (int r0 = 0; r0 < st[0]; ++r0)
        for (int r1 = 0; r1 < st[1]; ++r1)
            for (int r2 = 0; r2 < st[2]; ++r2) {
                BwdPhase &f = ph[cnt++];
                const int r[3] = {r0, r1, r2};
                f.any = true;
                long long taps = 1, pix = 1;
                for (int a = 0; a < 3; ++a) {
                    const AxisPhase x = axis_phase(kk[a], st[a], dl[a], pd[a], r[a], in[a]);
                    f.taps.t0[a] = x.t0;
                    f.taps.st[a] = x.st;
                    f.taps.J[a] = x.J;
                    f.r[a] = r[a];
                    f.M[a] = x.M;
                    f.P[a] = x.P;
                    f.dl[a] = x.dl;
                    f.any = f.any && x.J > 0;
                    taps *= x.J;
                    pix *= x.M;
                }
                f.w_off = wb;
                if (f.any) wb += round256((size_t)(p.G * (long long)p.Kpg * p.Cpg * taps * es));
                const size_t cls = (size_t)(p.N * pix * p.C() * es);
                if (f.any && round256(cls) > tb) tb = round256(cls);
            }
    *nph = cnt;
    *w_bytes = wb;
    *tmp_bytes = tb;
    return true;
}

// The forward problem computing class f: input dy, output the class's dense
// positions, the class's sub-kernel at stride 1.
Problem phase_problem(const Problem &p, const BwdPhase &f)
{
    Problem t = p;
    t.Cpg = p.Kpg;
    t.Kpg = p.Cpg;
    t.D = p.Do; t.H = p.Ho; t.W = p.Wo;
    t.Z = f.taps.J[0]; t.Y = f.taps.J[1]; t.X = f.taps.J[2];
    t.Do = f.M[0]; t.Ho = f.M[1]; t.Wo = f.M[2];
    t.sd = t.sh = t.sw = 1;
    t.pd = f.P[0]; t.ph = f.P[1]; t.pw = f.P[2];
    t.dd = f.dl[0]; t.dh = f.dl[1]; t.dw = f.dl[2];
    return t;
}

int run_bwd_polyphase(const Problem &p, const BwdPhase *ph, int nph, size_t w_bytes, const void *dy,
                      const void *w, void *dx, void *ws, hipStream_t s)
{
    char *wsb = (char *)ws;
    void *tmp = wsb + w_bytes;
    for (int i = 0; i < nph; ++i)
        if (ph[i].any && bwd::launch_phase_flip(p, ph[i].taps, w, wsb + ph[i].w_off, s) != hipSuccess)
            return GCONV_ERR_LAUNCH;
    for (int i = 0; i < nph; ++i) {
        const BwdPhase &f = ph[i];
        if ((long long)f.M[0] * f.M[1] * f.M[2] == 0) continue;
        if (f.any) {
            const Problem t = phase_problem(p, f);
            const int pth = launch_path(t, GCONV_PATH_AUTO, dy, wsb + f.w_off, nullptr, tmp);
            if (pth < 0) return pth;
            Args a{dy, wsb + f.w_off, nullptr, tmp};
            const int rc = launch_problem(t, pth, a, s);
            if (rc != GCONV_OK) return rc;
        }
        bwd::PhaseScatter q{};
        q.N = p.N; q.D = p.D; q.H = p.H; q.W = p.W;
        for (int a = 0; a < 3; ++a) {
            q.M[a] = f.M[a];
            q.r[a] = f.r[a];
        }
        q.s[0] = p.sd; q.s[1] = p.sh; q.s[2] = p.sw;
        q.cv = p.C();
        q.zero = f.any ? 0 : 1;
        if (bwd::launch_phase_scatter(q, elem_size(p.dtype), tmp, dx, s) != hipSuccess) return GCONV_ERR_LAUNCH;
    }
    return GCONV_OK;
}

// Stride-1 backward data whose transposed problem is depthwise: the forward
// depthwise kernel reverses the windows itself.
bool bwd_dw_reversed(const gconv_desc *d, const int64_t *out)
{
    Problem t;
    return bwd_as_forward(d) && bwd_forward_problem(to_problem(d, out), t) && depthwise::supported(t);
}

int run_bwd_data(const gconv_desc *d, const void *dy, const void *w, void *dx, void *ws,
                 size_t ws_bytes, bool direct, void *stream)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    if (!dy || !w || !dx) return GCONV_ERR_NULL_PTR;
    const uintptr_t es = (uintptr_t)elem_size(d->dtype);
    if (!aligned(dy, es) || !aligned(w, es) || !aligned(dx, es)) return GCONV_ERR_MISALIGNED;
    hipStream_t s = (hipStream_t)stream;
    if (!direct && ws && aligned(ws, 16)) {
        const Problem whole = to_problem(d, out);
        BwdPhase ph[kMaxPhases];
        int nph = 0;
        size_t wb = 0, tb = 0;
        if (bwd_phases(whole, ph, &nph, &wb, &tb) && ws_bytes >= wb + tb)
            return run_bwd_polyphase(whole, ph, nph, wb, dy, w, dx, ws, s);
    }
    // depthwise: the forward kernel reads the windows reversed itself, so no
    // transformed weight copy (and no workspace) is needed
    const bool dw_reversed = !direct && bwd_dw_reversed(d, out);
    const bool route = !direct && bwd_as_forward(d) &&
                       (dw_reversed || (ws && ws_bytes >= weight_bytes(d) && aligned(ws, 16)));
    if (route && !dw_reversed && bwd::launch_flip(to_problem(d, out), w, ws, s) != hipSuccess) return GCONV_ERR_LAUNCH;
    return for_bwd_pieces(d, out, [&](const Piece &pc, bool, bool) {
        const void *dyp = (const char *)dy + pc.in_off;
        void *dxp = (char *)dx + pc.out_off;
        Problem t;
        // the depthwise kernel's vector accesses need what launch_path checks
        // for the forward call; otherwise the direct kernel runs
        if (route && dw_reversed && aligned(dyp, 16) && aligned(dxp, 16) && aligned(w, 16) &&
            bwd_forward_problem(pc.p, t) && depthwise::supported(t)) {
            Args a{dyp, w, nullptr, dxp};
            return depthwise::launch_flipped(t, a, s) == hipSuccess ? (int)GCONV_OK : (int)GCONV_ERR_LAUNCH;
        }
        if (route && !dw_reversed && bwd_forward_problem(pc.p, t)) {
            const int pth = launch_path(t, GCONV_PATH_AUTO, dyp, ws, nullptr, dxp);
            Args a{dyp, ws, nullptr, dxp};
            return launch_problem(t, pth, a, s);
        }
        return bwd::launch_direct(pc.p, dyp, w, dxp, s) == hipSuccess ? (int)GCONV_OK : (int)GCONV_ERR_LAUNCH;
    });
}

// Backward weight reduces over every output pixel of the batch.  Stage 1
// runs as the forward call's launches (the whole batch, else whole images,
// else, image by image, output slices with the input windows they read),
// each writing its own chunks of partial sums into the workspace
// (consecutive ranges, in launch order), and one stage 2 adds them all in
// chunk order.  The launches' chunk counts, and so the summation order,
// depend only on the descriptor and the workspace size.
struct BwdwPlan {
    int64_t launches;
    int want;          // chunks a launch would take to fill the GPU
    int per;           // chunks per launch (a launch may use fewer)
    int total;         // chunks in all (1: stage 1 writes dw itself)
    size_t per_chunk;  // bytes of one chunk of partial sums
};

// Launches and the ideal chunk count (from the first launch, the largest:
// later ones are shorter runs of images or slices), before any workspace.
void bwdw_launches(const gconv_desc *d, const int64_t out[3], BwdwPlan &pl)
{
    Problem first{};
    pl.launches = 0;
    for_fwd_pieces(d, out, [&](const Piece &pc, bool, bool) {
        if (pl.launches++ == 0) first = pc.p;
        return (int)GCONV_OK;
    });
    pl.want = bwdw::ideal_chunks(first);
    pl.per_chunk = (size_t)first.G * first.Kpg * first.taps() * first.Cpg * sizeof(float);
}

int bwdw_plan(const gconv_desc *d, const int64_t out[3], size_t ws_bytes, bool have_ws, BwdwPlan &pl)
{
    bwdw_launches(d, out, pl);
    const int64_t room = have_ws ? (int64_t)(ws_bytes / pl.per_chunk) : 0;
    if (pl.launches == 1) {
        pl.per = (int)(room >= 2 ? min64(pl.want, room) : 1);
        pl.total = pl.per;
        return GCONV_OK;
    }
    // every launch needs at least one chunk of its own in the workspace (and
    // the chunk count in all stays an int)
    if (room < pl.launches || pl.launches > INT32_MAX) return GCONV_ERR_TOO_LARGE;
    pl.per = (int)max64(1, min64(min64(pl.want, room / pl.launches), INT32_MAX / pl.launches));
    pl.total = (int)(pl.per * pl.launches);
    return GCONV_OK;
}

int run_bwd_weight(const gconv_desc *d, const void *x, const void *dy, void *dw, void *ws,
                   size_t ws_bytes, void *stream)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    if (!x || !dy || !dw) return GCONV_ERR_NULL_PTR;
    const uintptr_t es = (uintptr_t)elem_size(d->dtype);
    if (!aligned(x, es) || !aligned(dy, es) || !aligned(dw, es)) return GCONV_ERR_MISALIGNED;
    const bool have_ws = ws && aligned(ws, 4);
    BwdwPlan pl;
    rc = bwdw_plan(d, out, ws_bytes, have_ws, pl);
    if (rc != GCONV_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    const Problem whole = to_problem(d, out);
    const size_t welems = (size_t)whole.G * whole.Kpg * whole.taps() * whole.Cpg;
    const bool final_ = pl.total == 1;
    int base = 0;
    // a slice whose window lies wholly in the padding (negative leading pad)
    // reads no input: the kernels' bounds checks leave its chunks zero
    rc = for_fwd_pieces(d, out, [&](const Piece &pc, bool, bool) {
        int used = 0;
        if (bwdw::stage1(pc.p, (const char *)x + pc.in_off, (const char *)dy + pc.out_off,
                         final_ ? nullptr : (float *)ws + (size_t)base * welems, final_ ? dw : nullptr, pl.per,
                         &used, s) != hipSuccess)
            return (int)GCONV_ERR_LAUNCH;
        base += used;
        return (int)GCONV_OK;
    });
    if (rc != GCONV_OK) return rc;
    if (pl.total > 1 && bwdw::stage2(whole, (const float *)ws, dw, base, s) != hipSuccess) return GCONV_ERR_LAUNCH;
    return GCONV_OK;
}

// ---- the entry point that allocates nothing
//
// Its partial sums live in a file-scope device array, one copy per GPU,
// allocated when the library's code object is loaded and held until the
// process ends.  Host code must not pass the array's name to a kernel (in
// host code it is a stand-in, not a device address): each device's address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and kept here.
constexpr size_t kScratchBytes = GCONV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// The scratch array's address on the current device (nullptr on failure).
void *scratch_ptr()
{
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> ptrs[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = ptrs[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    ptrs[dev].store(q, std::memory_order_release);   // a racing caller stores the same address
    return q;
}

}  // namespace
}  // namespace gconv

using namespace gconv;

GCONV_API int gconv_validate(const gconv_desc *d)
{
    int64_t out[3];
    return check_desc(d, out);
}

GCONV_API int gconv_out_dims(const gconv_desc *d, int64_t out[3])
{
    if (!out) return GCONV_ERR_NULL_PTR;
    int64_t o[3];
    int rc = check_desc(d, o);
    if (rc != GCONV_OK) return rc;
    memcpy(out, o, sizeof(o));
    return GCONV_OK;
}

// Selection and plans describe one launch (the first, for a call split
// into launches); support covers every launch of the call.
GCONV_API int gconv_select_path(const gconv_desc *d)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    return select(first_piece(d, out));
}

GCONV_API int gconv_path_supported(const gconv_desc *d, int path)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    if (path < 0 || path >= GCONV_NUM_PATHS) return GCONV_ERR_BAD_PATH;
    bool ok = true;
    for_fwd_pieces(d, out, [&](const Piece &pc, bool, bool) {
        ok = ok && path_ok(pc.p, path);
        return ok ? (int)GCONV_OK : 1;
    });
    return ok ? 1 : 0;
}

GCONV_API int gconv_get_plan(const gconv_desc *d, int path, gconv_plan *plan)
{
    if (!plan) return GCONV_ERR_NULL_PTR;
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    const Problem p = first_piece(d, out);
    if (path == GCONV_PATH_AUTO) path = select(p);
    else if (path < 0 || path >= GCONV_NUM_PATHS) return GCONV_ERR_BAD_PATH;
    else if (!path_ok(p, path)) return GCONV_ERR_PATH_UNSUPPORTED;
    TileScope own(-1);
    *plan = plan_of(p, path);
    return GCONV_OK;
}

GCONV_API int gconv_tile_count(const gconv_desc *d, int path, int *picked)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    const Problem p = first_piece(d, out);
    if (path == GCONV_PATH_AUTO) path = select(p);
    else if (path < 0 || path >= GCONV_NUM_PATHS) return GCONV_ERR_BAD_PATH;
    else if (!path_ok(p, path)) return GCONV_ERR_PATH_UNSUPPORTED;
    TileScope own(-1);
    int pk = 0;
    const int n = tiles_of(p, path, &pk);
    if (picked) *picked = pk;
    return n;
}

GCONV_API int gconv_fwd_tile(const gconv_desc *d, int path, int tile, const void *x, const void *w,
                             const void *bias, void *y, void *stream)
{
    if (path == GCONV_PATH_AUTO) return GCONV_ERR_BAD_PATH;
    const int n = gconv_tile_count(d, path, nullptr);
    if (n < 0) return n;
    if (tile < -1 || tile >= n) return GCONV_ERR_BAD_PATH;
    TileScope scope(tile);
    return run(d, path, x, w, bias, y, stream);
}

GCONV_API int gconv_fwd(const gconv_desc *d, const void *x, const void *w, const void *bias,
                        void *y, void *stream)
{
    return run(d, GCONV_PATH_AUTO, x, w, bias, y, stream);
}

GCONV_API int gconv_fwd_path(const gconv_desc *d, int path, const void *x, const void *w,
                             const void *bias, void *y, void *stream)
{
    return run(d, path, x, w, bias, y, stream);
}

GCONV_API int gconv_fwd_timed(const gconv_desc *d, int path, const void *x, const void *w,
                              const void *bias, void *y, void *stream, void *ev_start,
                              void *ev_stop)
{
    return run(d, path, x, w, bias, y, stream, ev_start, ev_stop);
}

GCONV_API int gconv_bwd_data_workspace(const gconv_desc *d, size_t *bytes)
{
    if (!bytes) return GCONV_ERR_NULL_PTR;
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    BwdPhase ph[kMaxPhases];
    int nph = 0;
    size_t wb = 0, tb = 0;
    if (bwd_phases(to_problem(d, out), ph, &nph, &wb, &tb)) *bytes = wb + tb;
    else *bytes = bwd_as_forward(d) && !bwd_dw_reversed(d, out) ? weight_bytes(d) : 0;
    return GCONV_OK;
}

GCONV_API int gconv_bwd_data(const gconv_desc *d, const void *dy, const void *w, void *dx,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    return run_bwd_data(d, dy, w, dx, workspace, workspace_bytes, false, stream);
}

GCONV_API int gconv_bwd_data_direct(const gconv_desc *d, const void *dy, const void *w, void *dx,
                                    void *stream)
{
    return run_bwd_data(d, dy, w, dx, nullptr, 0, true, stream);
}

GCONV_API int gconv_bwd_weight_workspace(const gconv_desc *d, size_t *bytes)
{
    if (!bytes) return GCONV_ERR_NULL_PTR;
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    BwdwPlan pl;
    bwdw_launches(d, out, pl);
    // one launch: the ideal chunks (none when one chunk fills the chip); a
    // call split into launches: the ideal chunks of every launch
    *bytes = pl.launches == 1 ? (pl.want > 1 ? (size_t)pl.want * pl.per_chunk : 0)
                              : (size_t)pl.launches * (size_t)pl.want * pl.per_chunk;
    return GCONV_OK;
}

GCONV_API int gconv_bwd_weight(const gconv_desc *d, const void *x, const void *dy, void *dw,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    return run_bwd_weight(d, x, dy, dw, workspace, workspace_bytes, stream);
}

GCONV_API int gconv_bwd_weight_noalloc(const gconv_desc *d, const void *x, const void *dy, void *dw,
                                       void *stream)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    if (!x || !dy || !dw) return GCONV_ERR_NULL_PTR;
    // the sizes are checked against the fixed scratch before any HIP call
    BwdwPlan pl;
    rc = bwdw_plan(d, out, kScratchBytes, true, pl);
    if (rc == GCONV_ERR_TOO_LARGE) return GCONV_ERR_SCRATCH;   // the only refusal left after check_desc
    if (rc != GCONV_OK) return rc;
    void *ws = scratch_ptr();
    if (!ws) return GCONV_ERR_LAUNCH;
    return run_bwd_weight(d, x, dy, dw, ws, kScratchBytes, stream);
}

GCONV_API const char *gconv_status_str(int status)
{
    switch (status) {
    case GCONV_OK: return "ok";
    case GCONV_ERR_BAD_DESC: return "bad descriptor";
    case GCONV_ERR_BAD_OUT_DIMS: return "empty output (an output extent is <= 0)";
    case GCONV_ERR_NULL_PTR: return "null pointer";
    case GCONV_ERR_TOO_LARGE: return "tensor too large (>= 2^31 elements)";
    case GCONV_ERR_MISALIGNED: return "misaligned pointer";
    case GCONV_ERR_BAD_PATH: return "unknown path";
    case GCONV_ERR_PATH_UNSUPPORTED: return "path cannot run this problem";
    case GCONV_ERR_LAUNCH: return "kernel launch failed";
    case GCONV_ERR_SCRATCH: return "needs more than the fixed device scratch of the no-allocation entry point";
    default: return "unknown status";
    }
}

GCONV_API const char *gconv_path_name(int path)
{
    switch (path) {
    case GCONV_PATH_AUTO: return "auto";
    case GCONV_PATH_GENERIC: return "generic";
    case GCONV_PATH_DEPTHWISE: return "depthwise";
    case GCONV_PATH_SMALLG: return "smallg_mfma";
    case GCONV_PATH_IGEMM: return "igemm_mfma";
    case GCONV_PATH_IGHALO: return "ighalo_mfma";
    case GCONV_PATH_DIRECT: return "direct_valu";
    default: return "unknown";
    }
}

GCONV_API int gconv_abi_version(void) { return GCONV_ABI_VERSION; }

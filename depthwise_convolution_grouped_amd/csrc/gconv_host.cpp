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

#include "gconv_internal.h"

#define GCONV_API extern "C" __attribute__((visibility("default")))

namespace gconv {
namespace {

constexpr int64_t kMaxElems = (int64_t)INT32_MAX;  // tensors must have < 2^31 elements

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
    // x and y may exceed 2^31 elements as a batch: calls then split the batch
    // into launches of whole images (every launch indexes in 32 bits), so
    // only one image of each, and w, must stay below
    const int64_t x_img = x_el / d->N, y_img = y_el / d->N;
    if (x_img >= kMaxElems || y_img >= kMaxElems || w_el >= kMaxElems || span >= kMaxElems ||
        d->K >= kMaxElems || d->C >= kMaxElems || Kpg >= kMaxElems || d->N >= kMaxElems || x_el >= INT64_MAX / 4 ||
        y_el >= INT64_MAX / 4)
        return GCONV_ERR_TOO_LARGE;
    return GCONV_OK;
}

// Images per launch: the whole batch when x and y each span < 2^31 bytes,
// else the most whole images that keep both below (at least one).  The
// vector paths address a launch's tensors with 32-bit byte offsets, so a
// byte limit keeps every launch on the path the dispatcher would pick for
// its shape; the generic path indexes elements in 32 bits, which a launch
// of one image below 2^31 elements also satisfies.
int64_t images_per_launch(const gconv_desc *d, const int64_t out[3])
{
    const int64_t es = elem_size(d->dtype);
    const int64_t x_img = d->in[0] * d->in[1] * d->in[2] * d->C * es;
    const int64_t y_img = out[0] * out[1] * out[2] * d->K * es;
    const int64_t nx = kMaxElems / x_img, ny = kMaxElems / y_img;
    int64_t n = nx < ny ? nx : ny;
    if (n < 1) n = 1;
    return n < d->N ? n : d->N;
}

// The descriptor of one launch: d with a batch of n images.
gconv_desc with_batch(const gconv_desc *d, int64_t n)
{
    gconv_desc t = *d;
    t.N = n;
    return t;
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

bool path_ok(const Problem &p, int path)
{
    switch (path) {
    case GCONV_PATH_GENERIC: return generic::supported(p);
    case GCONV_PATH_DEPTHWISE: return depthwise::supported(p);
    case GCONV_PATH_SMALLG: return smallg::supported(p);
    case GCONV_PATH_IGEMM: return igemm::supported(p);
    case GCONV_PATH_IGHALO: return ighalo::supported(p);
    default: return false;
    }
}

// Channels-per-group dispatcher.  Depthwise (Cpg = Kpg = 1) goes to the VALU
// direct kernel; large per-group contractions (Cpg, Kpg >= 32, half types)
// are a real GEMM per group and go to the implicit-GEMM MFMA kernel; small
// groups in half types merge several groups into one block-diagonal MFMA
// tile; everything else takes the generic kernel.
int select(const Problem &p)
{
    if (depthwise::supported(p)) return GCONV_PATH_DEPTHWISE;
    if (p.dtype != GCONV_F32 && p.Cpg >= 32 && p.Kpg >= 32) {
        if (ighalo::supported(p)) return GCONV_PATH_IGHALO;
        if (igemm::supported(p)) return GCONV_PATH_IGEMM;
    }
    if (smallg::supported(p)) return GCONV_PATH_SMALLG;
    if (ighalo::supported(p)) return GCONV_PATH_IGHALO;
    if (igemm::supported(p)) return GCONV_PATH_IGEMM;
    return GCONV_PATH_GENERIC;
}

gconv_plan plan_of(const Problem &p, int path)
{
    switch (path) {
    case GCONV_PATH_DEPTHWISE: return depthwise::plan(p);
    case GCONV_PATH_SMALLG: return smallg::plan(p);
    case GCONV_PATH_IGEMM: return igemm::plan(p);
    case GCONV_PATH_IGHALO: return ighalo::plan(p);
    default: return generic::plan(p);
    }
}

bool aligned(const void *ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

int run(const gconv_desc *d, int path, const void *x, const void *w, const void *bias,
        void *y, void *stream, void *ev_start = nullptr, void *ev_stop = nullptr)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    if (!x || !w || !y) return GCONV_ERR_NULL_PTR;
    const int64_t nl = images_per_launch(d, out);
    if (nl < d->N) {
        // a batch of >= 2^31 elements: consecutive launches of nl whole images,
        // the start event bound to the first and the stop event to the last
        const size_t es = (size_t)elem_size(d->dtype);
        const size_t x_img = (size_t)(d->in[0] * d->in[1] * d->in[2] * d->C) * es;
        const size_t y_img = (size_t)(out[0] * out[1] * out[2] * d->K) * es;
        for (int64_t n0 = 0; n0 < d->N; n0 += nl) {
            const int64_t n = d->N - n0 < nl ? d->N - n0 : nl;
            const gconv_desc t = with_batch(d, n);
            rc = run(&t, path, (const char *)x + (size_t)n0 * x_img, w, bias, (char *)y + (size_t)n0 * y_img,
                     stream, n0 == 0 ? ev_start : nullptr, n0 + n >= d->N ? ev_stop : nullptr);
            if (rc != GCONV_OK) return rc;
        }
        return GCONV_OK;
    }
    Problem p = to_problem(d, out);
    const uintptr_t es = (uintptr_t)elem_size(p.dtype);
    if (!aligned(x, es) || !aligned(w, es) || !aligned(y, es) || (bias && !aligned(bias, es)))
        return GCONV_ERR_MISALIGNED;
    // The vector paths load and store 16-byte channel vectors; automatic
    // dispatch falls back to the generic kernel for other pointers.
    const bool vec_ok = aligned(x, 16) && aligned(w, 16) && aligned(y, 16) &&
                        (!bias || aligned(bias, 16));
    if (path == GCONV_PATH_AUTO) {
        path = select(p);
        if (!vec_ok) path = GCONV_PATH_GENERIC;
    } else {
        if (path < 0 || path >= GCONV_NUM_PATHS) return GCONV_ERR_BAD_PATH;
        if (!path_ok(p, path)) return GCONV_ERR_PATH_UNSUPPORTED;
        if (path != GCONV_PATH_GENERIC && !vec_ok) return GCONV_ERR_MISALIGNED;
    }
    Args a{x, w, bias, y, (hipEvent_t)ev_start, (hipEvent_t)ev_stop};
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (path) {
    case GCONV_PATH_DEPTHWISE: e = depthwise::launch(p, a, s); break;
    case GCONV_PATH_SMALLG: e = smallg::launch(p, a, s); break;
    case GCONV_PATH_IGEMM: e = igemm::launch(p, a, s); break;
    case GCONV_PATH_IGHALO: e = ighalo::launch(p, a, s); break;
    default: e = generic::launch(p, a, s); break;
    }
    if (e != hipSuccess) return GCONV_ERR_LAUNCH;
    return GCONV_OK;
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

gconv_desc bwd_forward_desc(const gconv_desc *d, const int64_t out[3])
{
    gconv_desc t = *d;
    t.C = d->K;
    t.K = d->C;
    for (int a = 0; a < 3; ++a) {
        t.in[a] = out[a];
        t.stride[a] = 1;
        t.pad[a] = d->dil[a] * (d->filt[a] - 1) - d->pad[a];
    }
    return t;
}

size_t weight_bytes(const gconv_desc *d)
{
    return (size_t)d->K * (size_t)d->filt[0] * (size_t)d->filt[1] * (size_t)d->filt[2] *
           (size_t)(d->C / d->G) * (size_t)elem_size(d->dtype);
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
    const int64_t nl = images_per_launch(d, out);
    if (nl < d->N) {
        // a batch of >= 2^31 elements: launches of nl whole images
        const size_t x_img = (size_t)(d->in[0] * d->in[1] * d->in[2] * d->C) * es;
        const size_t y_img = (size_t)(out[0] * out[1] * out[2] * d->K) * es;
        for (int64_t n0 = 0; n0 < d->N; n0 += nl) {
            const int64_t n = d->N - n0 < nl ? d->N - n0 : nl;
            const gconv_desc t = with_batch(d, n);
            rc = run_bwd_data(&t, (const char *)dy + (size_t)n0 * y_img, w, (char *)dx + (size_t)n0 * x_img, ws,
                              ws_bytes, direct, stream);
            if (rc != GCONV_OK) return rc;
        }
        return GCONV_OK;
    }
    const Problem p = to_problem(d, out);
    hipStream_t s = (hipStream_t)stream;
    if (!direct && bwd_as_forward(d) && ws && ws_bytes >= weight_bytes(d) && aligned(ws, 16)) {
        if (bwd::launch_flip(p, w, ws, s) != hipSuccess) return GCONV_ERR_LAUNCH;
        const gconv_desc t = bwd_forward_desc(d, out);
        return run(&t, GCONV_PATH_AUTO, dy, ws, nullptr, dx, stream);
    }
    if (bwd::launch_direct(p, dy, w, dx, s) != hipSuccess) return GCONV_ERR_LAUNCH;
    return GCONV_OK;
}

size_t bwd_weight_partials_bytes(const Problem &p, int nch)
{
    return nch > 1 ? (size_t)nch * (size_t)p.G * p.Kpg * p.taps() * p.Cpg * sizeof(float) : 0;
}

int run_bwd_weight(const gconv_desc *d, const void *x, const void *dy, void *dw, void *ws,
                   size_t ws_bytes, void *stream)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    // its reduction runs over the whole batch: no split into launches
    const int64_t x_all = d->N * d->in[0] * d->in[1] * d->in[2] * d->C;
    const int64_t y_all = d->N * out[0] * out[1] * out[2] * d->K;
    if (x_all >= kMaxElems || y_all >= kMaxElems) return GCONV_ERR_TOO_LARGE;
    if (!x || !dy || !dw) return GCONV_ERR_NULL_PTR;
    const uintptr_t es = (uintptr_t)elem_size(d->dtype);
    if (!aligned(x, es) || !aligned(dy, es) || !aligned(dw, es)) return GCONV_ERR_MISALIGNED;
    const Problem p = to_problem(d, out);
    int nch = bwdw::ideal_chunks(p);
    const size_t per = bwd_weight_partials_bytes(p, 2) / 2;   // one chunk of partial sums
    if (!ws || !aligned(ws, 4)) nch = 1;
    else if ((size_t)nch * per > ws_bytes) nch = (int)(ws_bytes / per);
    if (nch < 1) nch = 1;
    if (bwdw::launch(p, x, dy, dw, (float *)ws, nch, (hipStream_t)stream) != hipSuccess)
        return GCONV_ERR_LAUNCH;
    return GCONV_OK;
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

// Selection and plans describe one launch (the first, for a split batch).
GCONV_API int gconv_select_path(const gconv_desc *d)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    const gconv_desc t = with_batch(d, images_per_launch(d, out));
    return select(to_problem(&t, out));
}

GCONV_API int gconv_path_supported(const gconv_desc *d, int path)
{
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    if (path < 0 || path >= GCONV_NUM_PATHS) return GCONV_ERR_BAD_PATH;
    const gconv_desc t = with_batch(d, images_per_launch(d, out));
    return path_ok(to_problem(&t, out), path) ? 1 : 0;
}

GCONV_API int gconv_get_plan(const gconv_desc *d, int path, gconv_plan *plan)
{
    if (!plan) return GCONV_ERR_NULL_PTR;
    int64_t out[3];
    int rc = check_desc(d, out);
    if (rc != GCONV_OK) return rc;
    const gconv_desc t = with_batch(d, images_per_launch(d, out));
    Problem p = to_problem(&t, out);
    if (path == GCONV_PATH_AUTO) path = select(p);
    else if (path < 0 || path >= GCONV_NUM_PATHS) return GCONV_ERR_BAD_PATH;
    else if (!path_ok(p, path)) return GCONV_ERR_PATH_UNSUPPORTED;
    *plan = plan_of(p, path);
    return GCONV_OK;
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
    *bytes = bwd_as_forward(d) ? weight_bytes(d) : 0;
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
    const Problem p = to_problem(d, out);
    *bytes = bwd_weight_partials_bytes(p, bwdw::ideal_chunks(p));
    return GCONV_OK;
}

GCONV_API int gconv_bwd_weight(const gconv_desc *d, const void *x, const void *dy, void *dw,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    return run_bwd_weight(d, x, dy, dw, workspace, workspace_bytes, stream);
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
    default: return "unknown";
    }
}

GCONV_API int gconv_abi_version(void) { return GCONV_ABI_VERSION; }

/*
 * gconv.h -- grouped / depthwise convolution forward on AMD Instinct MI355X
 * (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * The operation (all entry points below compute or describe it):
 *
 *   y[n, o, g*Kpg + k] = bias[g*Kpg + k]
 *       + sum over taps t of the filter window and c < Cpg of
 *           x[n, o*stride - pad + t*dil, g*Cpg + c] * w[g*Kpg + k, t, c]
 *
 * for every image n, output position o (2D or 3D), group g < G and output
 * channel k < Kpg, with Cpg = C/G and Kpg = K/G.  Channel mapping as in
 * rocm-libraries PR 10064 (grouped forward conv in the implicit-GEMM conv),
 * Technical Details: the input channel is (group, channel-in-group) embedded
 * as g*Cpg + c, the output channel is g*Kpg + k.  Grouped and depthwise
 * (G == C) forward conv with and without bias, stride, padding and dilation,
 * 2D and 3D, as the TileOPs PR 1568 review (summary) describes its
 * GroupConv2d/GroupConv3d kernels.  The filter is not flipped
 * (cross-correlation).  Taps outside the input read zero; padding is
 * symmetric, one value per spatial axis (CK grouped_conv tile-engine README,
 * Problem Registry field list).  Output extent per axis:
 *   out = floor((in + 2*pad - dil*(filt-1) - 1) / stride) + 1.
 *
 * Memory layouts (packed, last index fastest; the forward NHWGC / GKYXC pair
 * of the CK grouped-conv Python examples README, Examples table, with a depth
 * axis for 3D):
 *   x     [N][D][H][W][G][Cpg]       (2D: D = 1)      NDHWGC
 *   w     [G][Kpg][Z][Y][X][Cpg]     (2D: Z = 1)      GKZYXC
 *   bias  [G*Kpg]  or NULL
 *   y     [N][Do][Ho][Wo][G][Kpg]                     NDHWGK
 * x, w, bias and y share one element type; products are accumulated in fp32
 * and the result is rounded once (to nearest even) to the element type.
 *
 * Ownership: the caller allocates, owns and frees every buffer (device memory
 * for x, w, bias, y, and the optional workspaces of the backward calls).  The
 * library never allocates, frees or keeps a pointer after a call returns.
 * The forward calls need no workspace; gconv_bwd_data and gconv_bwd_weight
 * take an optional caller-owned workspace (sized by their *_workspace
 * queries) that they may overwrite until the stream has passed the call.  The
 * only global state is a per-device record of which kernels had their LDS
 * limit raised (set once, atomically), so calls from several host threads are
 * safe.  Outputs must not overlap inputs or workspaces.
 *
 * Non-finite inputs: the small-group path (GCONV_PATH_SMALLG) merges several
 * groups into one block-diagonal matrix-core tile (the CK grouped-conv Python
 * examples README's num_groups_to_merge option, Config-options harness), whose
 * off-diagonal weights are zero.  An Inf or NaN in one group's input then
 * makes the outputs of the other groups merged into the same tile NaN
 * (0 * Inf), where the definition keeps them finite; the outputs of groups in
 * other tiles, and every output when all inputs are finite, are unaffected.
 * gconv_fwd_path with GCONV_PATH_GENERIC computes each group alone and keeps
 * non-finite values inside their own group.
 *
 * Errors: every function returns GCONV_OK (0) or a negative gconv_status.
 * Validation errors are detected on the host before anything is launched.
 */
#ifndef GCONV_H
#define GCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GCONV_ABI_VERSION 1

/* Element type of x, w, bias and y. */
typedef enum gconv_dtype {
    GCONV_F32 = 0,
    GCONV_F16 = 1,
    GCONV_BF16 = 2
} gconv_dtype;

typedef enum gconv_status {
    GCONV_OK = 0,
    GCONV_ERR_BAD_DESC = -1,        /* ndim/dtype out of range, C%G or K%G != 0,
                                       non-positive size/stride/dilation,
                                       negative pad, 2D with depth entries set */
    GCONV_ERR_BAD_OUT_DIMS = -2,    /* an output extent would be <= 0 */
    GCONV_ERR_NULL_PTR = -3,        /* desc, x, w or y is NULL */
    GCONV_ERR_TOO_LARGE = -4,       /* w has >= 2^31 elements, N or an extent >= 2^31, or
                                       one slice along the outermost spatial axis (a row
                                       in 2D, a plane in 3D) of x or y, with the window it
                                       needs, spans >= 2^31 bytes; backward weight split
                                       into launches: a workspace holding fewer chunks of
                                       partial sums than the call has launches */
    GCONV_ERR_MISALIGNED = -5,      /* a pointer is not aligned as the path needs */
    GCONV_ERR_BAD_PATH = -6,        /* unknown path id */
    GCONV_ERR_PATH_UNSUPPORTED = -7,/* forced path cannot run this problem */
    GCONV_ERR_LAUNCH = -8,          /* the HIP launch reported an error */
    GCONV_ERR_SCRATCH = -9          /* gconv_bwd_weight_noalloc: the problem needs more than
                                       GCONV_NOALLOC_SCRATCH_BYTES of partial sums */
} gconv_status;

/* Kernel paths.  gconv_fwd picks one from the descriptor. */
typedef enum gconv_path {
    GCONV_PATH_AUTO = -1,
    GCONV_PATH_GENERIC = 0,     /* one thread per output, any shape */
    GCONV_PATH_DEPTHWISE = 1,   /* Cpg = Kpg = 1: input rows streamed through registers,
                                   channel vectors, VALU */
    GCONV_PATH_SMALLG = 2,      /* small groups: LDS row ring or halo box, block-diagonal
                                   MFMA (fp16/bf16; the ring also fp32) */
    GCONV_PATH_IGEMM = 3,       /* larger groups: M-tiled implicit GEMM, group on grid z,
                                   MFMA (fp16/bf16/fp32) */
    GCONV_PATH_IGHALO = 4,      /* large groups: implicit GEMM over an LDS input box per
                                   output block, persistent, MFMA (fp16/bf16) */
    GCONV_PATH_DIRECT = 5,      /* register-blocked direct kernels on the vector ALUs
                                   (group widths no matrix-core path takes; any shape) */
    GCONV_NUM_PATHS = 6
} gconv_path;

/* Problem descriptor.  Spatial arrays are (depth, height, width); a 2D
 * problem sets in[0] = filt[0] = stride[0] = dil[0] = 1 and pad[0] = 0.
 * Fields mirror the CK grouped_conv problem dataclass (tile-engine README,
 * Problem Registry): N, C, K, G, input and filter extents, stride, pad,
 * dilation. */
typedef struct gconv_desc {
    int32_t ndim;       /* 2 or 3 */
    int32_t dtype;      /* gconv_dtype */
    int64_t N, G, C, K; /* batch, groups, total input / output channels */
    int64_t in[3];      /* D, H, W */
    int64_t filt[3];    /* Z, Y, X */
    int64_t stride[3];
    int64_t pad[3];
    int64_t dil[3];
} gconv_desc;

/* Launch shape a path would use (for tests and profiling). */
typedef struct gconv_plan {
    int32_t path;
    uint32_t grid[3];
    uint32_t block;
    uint32_t lds_bytes;
    uint32_t groups_per_tile; /* groups merged into one tile (1 if none) */
} gconv_plan;

/* Checks the descriptor alone (no pointers, no HIP call).  Returns GCONV_OK,
 * GCONV_ERR_BAD_DESC, GCONV_ERR_BAD_OUT_DIMS or GCONV_ERR_TOO_LARGE.  The
 * checks are those of rocm-libraries PR 10064 (Technical Details: C % G == 0
 * and K % G == 0 before a grouped problem is accepted), of the TileOPs PR
 * 1568 review (summary: the grouped ops validate the expected weight shape,
 * which here follows from the descriptor) and positive extents, strides and
 * dilations for the problem fields of the CK grouped_conv tile-engine README
 * (Problem Registry). */
int gconv_validate(const gconv_desc *d);

/* Writes (Do, Ho, Wo) to out[0..2] (Do = 1 in 2D) after validating d: the
 * dilation-aware extent formula above, which the TileOPs PR 1568 review
 * (summary) says the grouped kernels keep and whose 3D case gives the
 * review's 802,816 outputs ("The 50x is a baseline artifact"). */
int gconv_out_dims(const gconv_desc *d, int64_t out[3]);

/* Path gconv_fwd would take for d (a gconv_path >= 0), or a negative status.
 * The choice depends on channels per group and dtype only, after the group
 * dispatch of the TileOPs PR 1568 review (summary: grouped problems are
 * routed to dedicated grouped kernels) and the group merging of the CK
 * Python examples README (Config-options harness, num_groups_to_merge). */
int gconv_select_path(const gconv_desc *d);

/* 1 if `path` can run d, 0 if not, or a negative status.  The counterpart of
 * the legality rules of the CK grouped_conv tile-engine README (How It Works,
 * Kernel Enumeration: the kernel pool holds only the configurations those
 * rules accept), applied here per problem. */
int gconv_path_supported(const gconv_desc *d, int path);

/* Fills *plan with the launch shape of `path` (GCONV_PATH_AUTO: the selected
 * one) for d: the grid, with the group on the grid's z axis for the
 * per-group implicit GEMM (rocm-libraries PR 10064, Technical Details: one
 * grid slice per group), and the groups merged per tile (CK grouped-conv
 * Python examples README, num_groups_to_merge). */
int gconv_get_plan(const gconv_desc *d, int path, gconv_plan *plan);

/* Forward convolution, asynchronous on `stream` (a hipStream_t; NULL = the
 * null stream).  x, w, bias (NULL = no bias) and y are device pointers in the
 * layouts above, aligned to the element size.  Exactly one kernel is
 * launched when x and y each span < 2^31 bytes (every launch addresses its
 * tensors with 32-bit offsets).  Larger tensors are split, as the CK Python
 * examples README's split_image option does for large tensors
 * (Config-options harness): a batch into consecutive launches of as many
 * whole images as fit, and an image that alone does not fit into launches
 * of output slices along its outermost spatial axis (rows in 2D, planes in
 * 3D), each reading the input slices its window covers, halo included, from
 * the same x; no data is copied.  gconv_select_path and gconv_get_plan
 * describe the first launch.  The caller synchronises the stream before
 * reading y.  Results are bitwise deterministic from run to run (no
 * atomics). */
int gconv_fwd(const gconv_desc *d, const void *x, const void *w,
              const void *bias, void *y, void *stream);

/* As gconv_fwd, but on a caller-chosen path (GCONV_PATH_AUTO = select).
 * Returns GCONV_ERR_PATH_UNSUPPORTED when that path cannot take d, and
 * GCONV_ERR_MISALIGNED when it is a vector path (every path but
 * GCONV_PATH_GENERIC) and x, w, y or bias is not 16-byte aligned; gconv_fwd
 * itself falls back to the generic path for such pointers.  Used by the tests to run every path on shapes several can take. */
int gconv_fwd_path(const gconv_desc *d, int path, const void *x, const void *w,
                   const void *bias, void *y, void *stream);

/* Tile variants of `path` (GCONV_PATH_AUTO: the selected path) for d: the
 * size of the path's tile menu (>= 1) or a negative status; *picked (may
 * be NULL) receives the index of the path's own analytic pick.  The menus
 * (run lengths, rows per workgroup, kernel variant, output-channel and
 * reduction tiles, threads per output) are the counterpart of the tile
 * sizes and pipeline variants the CK grouped_conv tile-engine README
 * enumerates per problem (How It Works, Kernel Enumeration); measuring each
 * is how the analytic pick is checked against the best. */
int gconv_tile_count(const gconv_desc *d, int path, int *picked);

/* As gconv_fwd_path on a named path (not GCONV_PATH_AUTO) with tile
 * variant `tile` of its menu (0 .. gconv_tile_count - 1; -1 = the path's own
 * pick).  Every variant computes the same result within the tolerance of
 * the fp32 accumulation; for tests and tile sweeps. */
int gconv_fwd_tile(const gconv_desc *d, int path, int tile, const void *x, const void *w,
                   const void *bias, void *y, void *stream);

/* As gconv_fwd_path, and binds two HIP events (hipEvent_t, either may be
 * NULL; created by the caller, with timing enabled) to the kernel dispatch
 * (the start event to the first and the stop event to the last launch of a
 * split call): hipEventElapsedTime(start, stop) is then the kernels'
 * execution time, with no marker packets between the events and the
 * kernels.  For measurement; the result in y is the same as
 * gconv_fwd_path's. */
int gconv_fwd_timed(const gconv_desc *d, int path, const void *x, const void *w,
                    const void *bias, void *y, void *stream, void *ev_start,
                    void *ev_stop);

/* ---- Backward data ----------------------------------------------------
 *
 * dx, the gradient with respect to x, from dy (the gradient with respect to
 * y) and w: the backward-data variant the CK grouped_conv tile-engine README
 * lists next to forward (introduction), whose runner takes dY and W (CK
 * Python examples README, Runner argument contract).  d is the FORWARD
 * problem's descriptor: d->in gives dx's extents, the forward output extents
 * (gconv_out_dims) dy's.  Layouts: dy [N][Do][Ho][Wo][G][Kpg],
 * w [G][Kpg][Z][Y][X][Cpg], dx [N][D][H][W][G][Cpg], all device pointers
 * aligned to the element size, dtype as d->dtype, fp32 accumulation, no bias.
 *
 *   dx[n,i,g,c] = sum over taps t and k with o = (i + pad - t*dil) / stride
 *                 an integer in [0, out) of dy[n,o,g,k] * w[g,k,t,c]   (per axis)
 */

/* Bytes of device workspace gconv_bwd_data can use for d (0 when it has no
 * use for any):
 *  - at stride 1 with dil*(k-1) >= pad on every axis, the size of w: the call
 *    becomes a weight transform plus one forward launch on the fastest
 *    forward path (depthwise needs none: the forward depthwise kernel reads
 *    each window reversed, so 0 is returned and no workspace is used);
 *  - at a stride above 1, for groups other than depthwise, whose tensors fit
 *    one launch: the weights of every residue class of dx (per axis the dx
 *    positions i = r + stride*m receive only the taps t with (t*dil - r - pad)
 *    divisible by the stride, a stride-1 convolution of dy), each rounded up
 *    to 256 bytes, plus a dense buffer for the largest class; the call then
 *    runs per class a weight transform, one forward launch on the fastest
 *    forward path and a scatter into dx (zeros for a class no tap reaches). */
int gconv_bwd_data_workspace(const gconv_desc *d, size_t *bytes);

/* Backward data, asynchronous on `stream`.  `workspace` (device memory the
 * caller owns, 16-byte aligned, may be NULL) of `workspace_bytes`: when it
 * holds gconv_bwd_data_workspace bytes, the workspace route runs (at stride
 * 1 the weight transform and the forward kernel, or for depthwise the
 * forward kernel alone, with or without a workspace; at larger strides three
 * kernels per residue class); otherwise one direct kernel runs.  Tensors too large for one launch are split as in
 * gconv_fwd: whole images, else slices of dx along the outermost spatial
 * axis, each with the dy slices that reach it.  The workspace may be reused
 * once the stream has passed the call.  Deterministic from run to run.
 * Status codes as for gconv_fwd. */
int gconv_bwd_data(const gconv_desc *d, const void *dy, const void *w, void *dx,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Backward data on the direct kernel alone (any shape; one launch unless
 * the tensors must be split as for gconv_bwd_data). */
int gconv_bwd_data_direct(const gconv_desc *d, const void *dy, const void *w, void *dx,
                          void *stream);

/* ---- Backward weight --------------------------------------------------
 *
 * dw, the gradient with respect to w, from x and dy: the backward-weight
 * variant of the CK grouped_conv tile-engine README (introduction), whose
 * runner takes X and dY (CK Python examples README, Runner argument
 * contract).  d is the FORWARD problem's descriptor.  Layouts:
 * x [N][D][H][W][G][Cpg], dy [N][Do][Ho][Wo][G][Kpg], dw [G][Kpg][Z][Y][X][Cpg],
 * device pointers aligned to the element size, dtype as d->dtype, fp32
 * accumulation, rounded once.
 *
 *   dw[g,k,t,c] = sum over output pixels o whose tap t reads an in-bounds
 *                 input i = o*stride - pad + t*dil of dy[n,o,g,k] * x[n,i,g,c]
 *
 * Tensors too large for one launch are split as in gconv_fwd (whole images,
 * else output slices along the outermost spatial axis with the input slices
 * their windows read); each launch then adds its own chunks of partial sums,
 * so the workspace must hold at least one chunk per launch.
 */

/* Bytes of fp32 partial-sum workspace that lets gconv_bwd_weight split the
 * reduction over enough chunks of output rows to fill the GPU (0 when one
 * chunk already does). */
int gconv_bwd_weight_workspace(const gconv_desc *d, size_t *bytes);

/* Backward weight, asynchronous on `stream`.  `workspace` (device memory the
 * caller owns, 4-byte aligned, may be NULL) of `workspace_bytes`: the
 * reduction is split over as many chunks as it holds partial sums for (at
 * most the gconv_bwd_weight_workspace amount), then the chunks are added in
 * order (two kernels); with no room for two chunks one kernel sums each
 * element alone.  No atomics: for a given workspace size the result is
 * bitwise deterministic (the chunking, hence the summation order, depends on
 * that size).  Status codes as for gconv_fwd. */
int gconv_bwd_weight(const gconv_desc *d, const void *x, const void *dy, void *dw,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the device scratch gconv_bwd_weight_noalloc uses (one copy per
 * GPU, held by the library until the process ends). */
#define GCONV_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Backward weight for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): as gconv_bwd_weight with a workspace of
 * GCONV_NOALLOC_SCRATCH_BYTES, except that the workspace is the library's
 * own device array on the current GPU instead of the caller's.  It calls no
 * allocator.  Partial sums are split over as many chunks as the scratch
 * holds (at most the gconv_bwd_weight_workspace amount), so the result is
 * bitwise that of gconv_bwd_weight with a workspace of
 * min(GCONV_NOALLOC_SCRATCH_BYTES, gconv_bwd_weight_workspace) bytes.
 * Returns GCONV_ERR_SCRATCH, before any HIP call, when a call that must be
 * split into launches (a batch or an image too large for one) needs more
 * than the scratch holds (one chunk of partial sums per launch).  Every call on one GPU uses that GPU's one
 * scratch array: calls that overlap on the same GPU (other streams or host
 * threads) race and must be serialised by the caller.  Status codes
 * otherwise as gconv_bwd_weight. */
int gconv_bwd_weight_noalloc(const gconv_desc *d, const void *x, const void *dy, void *dw,
                             void *stream);

/* Static strings; never NULL.  A status string names why a call failed; the
 * CK grouped_conv tile-engine README records a failed launch as a result of
 * its own rather than a latency (Output CSV Schema: latency_ms=N/A). */
const char *gconv_status_str(int status);
const char *gconv_path_name(int path);

/* GCONV_ABI_VERSION of the built library (this header's layout of
 * gconv_desc and gconv_plan and the entry points above). */
int gconv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GCONV_H */

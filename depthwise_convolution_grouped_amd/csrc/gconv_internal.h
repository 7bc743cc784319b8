// Internal interface between the host library (gconv_host.cpp) and the
// kernel translation units.  Not installed; the public ABI is include/gconv.h.
#pragma once

#include <stdint.h>

#include <atomic>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "gconv.h"

namespace gconv {

// A validated problem.  Every tensor has < 2^31 elements, so all sizes and
// flat offsets fit in int32.
struct Problem {
    int ndim, dtype;
    int N, G, Cpg, Kpg;
    int D, H, W;        // input extents
    int Z, Y, X;        // filter extents
    int Do, Ho, Wo;     // output extents
    int sd, sh, sw;     // strides
    int pd, ph, pw;     // paddings
    int dd, dh, dw;     // dilations
    int C() const { return G * Cpg; }
    int K() const { return G * Kpg; }
    int taps() const { return Z * Y * X; }
    long long y_elems() const { return (long long)N * Do * Ho * Wo * G * Kpg; }
};

struct Args {
    const void *x;
    const void *w;
    const void *bias;   // may be null
    void *y;
    hipEvent_t ev_start = nullptr;   // optional, bound to the kernel dispatch
    hipEvent_t ev_stop = nullptr;
};

template <class T> struct exactly { using type = T; };

// Enqueues kernel `k` on `s` with arguments converted to exactly its own
// parameter types.  Events in `a` (either may be null) are bound to this
// dispatch by hipExtLaunchKernel, so their elapsed time is the kernel's own
// execution time, with no marker packets around it.
template <typename... KP>
hipError_t enqueue(void (*k)(KP...), dim3 grid, dim3 block, unsigned lds, hipStream_t s,
                   const Args &a, typename exactly<KP>::type... args)
{
    void *argv[] = {(void *)&args...};
    return hipExtLaunchKernel((const void *)k, grid, block, argv, lds, s, a.ev_start, a.ev_stop, 0);
}

// Raises kernel `k`'s dynamic LDS limit to `bytes` on the current device,
// once per device and kernel instance (`done` holds one bit per device, so
// concurrent callers at worst repeat the idempotent attribute call).
inline hipError_t allow_lds(const void *k, std::atomic<unsigned long long> &done, unsigned bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// The tile choice of the current call on this host thread: -1 = each
// path's own pick, k >= 0 = entry k of the path's tile menu (set for the
// length of one gconv_fwd_tile call).  Each path's `tiles` returns the size
// of its menu for a problem (>= 1) and stores its own pick in *picked.
int &tile_choice();

// Per-path hooks.  `supported` and `plan` are pure host functions (no HIP
// call); `launch` enqueues exactly one kernel on `stream`.
namespace generic {
int tiles(const Problem &p, int *picked);
bool supported(const Problem &p);
gconv_plan plan(const Problem &p);
hipError_t launch(const Problem &p, const Args &a, hipStream_t s);
}
namespace depthwise {
int tiles(const Problem &p, int *picked);
bool supported(const Problem &p);
gconv_plan plan(const Problem &p);
hipError_t launch(const Problem &p, const Args &a, hipStream_t s);
// The same convolution with each channel's window reversed (weight tap t
// read as tap taps-1-t): backward data at stride 1 without a transformed
// weight copy.
hipError_t launch_flipped(const Problem &p, const Args &a, hipStream_t s);
}
namespace smallg {
int tiles(const Problem &p, int *picked);
bool supported(const Problem &p);
// whether a row-walking variant (LDS ring or row streaming) takes the problem
bool streams(const Problem &p);
gconv_plan plan(const Problem &p);
hipError_t launch(const Problem &p, const Args &a, hipStream_t s);
}
namespace igemm {
int tiles(const Problem &p, int *picked);
bool supported(const Problem &p);
gconv_plan plan(const Problem &p);
hipError_t launch(const Problem &p, const Args &a, hipStream_t s);
}
// Register-blocked VALU direct kernel (k_direct.hip); `preferred` says
// whether it beats the generic kernel for the problem (enough work).
namespace direct {
int tiles(const Problem &p, int *picked);
bool supported(const Problem &p);
bool preferred(const Problem &p);
gconv_plan plan(const Problem &p);
hipError_t launch(const Problem &p, const Args &a, hipStream_t s);
}
// The halo path's variant with the whole input box resident in LDS; the
// halo path runs it whenever it takes the problem.
namespace ighalo_box {
bool supported(const Problem &p);
gconv_plan plan(const Problem &p);
hipError_t launch(const Problem &p, const Args &a, hipStream_t s);
}
namespace ighalo {
int tiles(const Problem &p, int *picked);
bool supported(const Problem &p);
gconv_plan plan(const Problem &p);
hipError_t launch(const Problem &p, const Args &a, hipStream_t s);
}

// Backward data (k_bwd_data.hip).  `p` is the forward problem (its x extents
// are dx's, its y extents dy's).
namespace bwd {
hipError_t launch_direct(const Problem &p, const void *dy, const void *w, void *dx, hipStream_t s);
hipError_t launch_flip(const Problem &p, const void *w, void *wt, hipStream_t s);
// One residue class of a strided backward data: per axis the taps
// t0 + j st (j < J) of the original filter.
struct PhaseTaps {
    int t0[3], st[3], J[3];
};
// Its placement in dx: dx extents D, H, W; class extents M; residues r;
// strides s; channels per pixel cv (the launcher turns it into units);
// zero: write zeros instead of the class's values.
struct PhaseScatter {
    int N, D, H, W;
    int M[3], r[3], s[3];
    int cv, zero;
    long long total;
};
hipError_t launch_phase_flip(const Problem &p, const PhaseTaps &ph, const void *w, void *wt, hipStream_t s);
hipError_t launch_phase_scatter(PhaseScatter q, int elem, const void *src, void *dx, hipStream_t s);
}

// Backward weight (k_bwd_weight.hip).  `p` is the forward problem of one
// launch.  stage1 picks the route (depthwise channel vectors, the MFMA
// implicit GEMM, register tiles, plain) and writes the partial sums of at
// most nch chunks to ws[chunk][f] (*used of them), or, with dw non-null and
// nch == 1, dw itself; stage2 adds nch chunks in order and rounds once.
namespace bwdw {
int ideal_chunks(const Problem &p);
hipError_t stage1(const Problem &p, const void *x, const void *dy, float *ws, void *dw, int nch, int *used,
                  hipStream_t s);
hipError_t stage2(const Problem &p, const float *ws, void *dw, int nch, hipStream_t s);
}

// Backward weight, stage 1 on the matrix cores (k_bwd_weight_mfma.hip):
// half types whose groups merge into super-groups of 16-multiple channel
// counts, windows of 1, 9, 25 or 27 taps.  stage1 writes the partial sums
// of at most nch chunks of output pixels to ws[chunk][f] (*used of them),
// or, with dw non-null and nch == 1, dw itself (rounded once).
namespace bwdw_mfma {
bool supported(const Problem &p);
int chunks(const Problem &p);
hipError_t stage1(const Problem &p, const void *x, const void *dy, float *ws, void *dw, int nch, int *used,
                  hipStream_t s);
}

inline int elem_size(int dtype) { return dtype == GCONV_F32 ? 4 : 2; }

}  // namespace gconv

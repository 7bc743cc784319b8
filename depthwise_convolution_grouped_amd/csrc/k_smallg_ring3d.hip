// Instances of the LDS-ring small-group kernel (smallg_ring.h) for 3D 3x3x3
// windows at stride 1: a ring row holds the three input planes' row
// segments, so each step folds 3 planes x 3 window rows into the output rows.
#include "smallg_ring.h"

namespace gconv {
namespace smallg {
namespace {

template <typename T, int R>
hipError_t ring3d_go(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    constexpr int PF = kRingPF3d;
    if (c.CH8 == 4) return ring_go4<T, 1, R, 4, 1, 3, PF>(p, c, a, s);
    if (c.CH8 == 1)
        return c.NTW == 4 ? ring_go4<T, 1, R, 1, 4, 3, PF>(p, c, a, s) : ring_go4<T, 1, R, 1, 2, 3, PF>(p, c, a, s);
    return c.NTW == 2 ? ring_go4<T, 1, R, 2, 2, 3, PF>(p, c, a, s) : ring_go4<T, 1, R, 2, 1, 3, PF>(p, c, a, s);
}

// 7-row runs, or 2-row runs for small grids
template <typename T>
hipError_t ring3d_launch_t(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    return c.R == 2 ? ring3d_go<T, 2>(p, c, a, s) : ring3d_go<T, 7>(p, c, a, s);
}

}  // namespace

hipError_t ring3d_launch(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    if (p.dtype == GCONV_F32) return ring3d_launch_t<float>(p, c, a, s);
    return p.dtype == GCONV_F16 ? ring3d_launch_t<_Float16>(p, c, a, s) : ring3d_launch_t<__bf16>(p, c, a, s);
}

}  // namespace smallg
}  // namespace gconv

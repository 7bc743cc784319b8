// Instances of the LDS-ring small-group kernel (smallg_ring.h) for 2D 3x3
// windows, and the ring variant's configuration for 2D and 3D.
#include "smallg_ring.h"

namespace gconv {
namespace smallg {
namespace {

template <typename T, int S, int R>
hipError_t ring_go3(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    // tiles of 4 chunks (fp32 16/16, or 32 input channels per 16 outputs)
    if (c.CH8 == 4) return ring_go4<T, S, R, 4, 1, 1, kRingPF2d>(p, c, a, s);
    return c.CH8 == 1 ? ring_go4<T, S, R, 1, 4, 1, kRingPF2d>(p, c, a, s)
                      : ring_go4<T, S, R, 2, 2, 1, kRingPF2d>(p, c, a, s);
}

template <typename T>
hipError_t ring_launch_t(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    if (p.sh == 1) return c.R == 28 ? ring_go3<T, 1, 28>(p, c, a, s) : ring_go3<T, 1, 14>(p, c, a, s);
    return ring_go3<T, 2, 14>(p, c, a, s);
}

}  // namespace

bool ring_configure(const Problem &p, RingConfig &c)
{
    const bool is3 = p.ndim == 3;
    if (p.Y != 3 || p.X != 3 || p.dh != 1 || p.dw != 1) return false;
    if (is3) {
        if (p.Z != 3 || p.sd != 1 || p.dd != 1 || p.sh != 1 || p.sw != 1) return false;
    } else if (p.ndim != 2 || p.sh != p.sw || (p.sh != 1 && p.sh != 2)) {
        return false;
    }
    if (p.dtype != GCONV_F16 && p.dtype != GCONV_BF16 && p.dtype != GCONV_F32) return false;
    const bool f32 = p.dtype == GCONV_F32;
    const int epc = f32 ? 4 : 8;                           // channels per 16-byte chunk
    if (p.Kpg < 1 || p.Kpg > 16 || 16 % p.Kpg != 0) return false;
    c.GN = 16 / p.Kpg;
    if (p.G % c.GN != 0 || (c.GN * p.Cpg) % epc != 0) return false;
    // a chunk holds whole groups or lies inside one group
    if (!(p.Cpg == 1 || p.Cpg == 2 || p.Cpg == 4 || p.Cpg % epc == 0)) return false;
    c.CH8 = c.GN * p.Cpg / epc;
    if (c.CH8 != 1 && c.CH8 != 2 && c.CH8 != 4) return false;
    c.NT = p.G / c.GN;
    // ring pixels of 16 chunks (the 2D swizzle's period): NTW = 16 / (4 CH8)
    // tiles per wave; 3D falls back to pixels of 8 chunks when the tiles do
    // not fill 16
    c.NTW = 16 / (kWaves * c.CH8);
    if (c.NT % (kWaves * c.NTW) != 0) {
        if (!is3 || c.NTW == 1) return false;
        c.NTW /= 2;
        if (c.NT % (kWaves * c.NTW) != 0) return false;
    }
    c.TPB = kWaves * c.NTW;
    c.ntb = c.NT / c.TPB;
    c.DZ = is3 ? 3 : 1;
    const long long es = f32 ? 4 : 2;
    if ((long long)p.D * p.H * p.W * p.C() * es >= (1LL << 31) ||
        (long long)p.Do * p.Ho * p.Wo * p.K() * es >= (1LL << 31))
        return false;
    c.CV = c.TPB * c.CH8;
    c.IW = 15 * p.sw + 3;
    c.RS = (c.DZ * c.IW * c.CV + 63) / 64 * 64;
    c.NINS = c.RS / 64;
    if (c.NINS > 8 * kWaves) return false;
    // PF + 1 ring rows, the zero slot, two staging rows of 16 padded pixels
    const int nr = (is3 ? kRingPF3d : kRingPF2d) + 1;
    c.lds = (int)(nr * c.RS * 16 + 16 + 2 * 16 * (c.TPB * es * 16 + 16));
    c.nmt = (p.Wo + 15) / 16;
    if (is3) {
        // short runs: 3D grids are small; 2-row runs when 7-row ones would
        // leave fewer workgroups than CUs
        c.R = 7;
        if ((long long)c.nmt * ((p.Ho + 6) / 7) * c.ntb * p.Do * p.N < 256) c.R = 2;
    } else {
        // rows per workgroup from {14, 28}: the longer run while the grid still
        // gives every CU two workgroups (long runs amortise the two halo rows);
        // stride 2 keeps 14 (its runs read twice the rows)
        c.R = 14;
        if (p.sh == 1 && (long long)c.nmt * ((p.Ho + 27) / 28) * c.ntb * p.N >= 512) c.R = 28;
    }
    c.nchunk = (p.Ho + c.R - 1) / c.R;
    const long long blocks = (long long)c.nmt * c.nchunk * c.ntb * p.Do * p.N;
    c.blocks = (int)blocks;
    // a 3D grid of fewer than 128 workgroups is left to the halo boxes
    if (is3 && blocks < 128) return false;
    return blocks < (1LL << 31);
}

void ring_set_rows(const Problem &p, RingConfig &c, int R)
{
    const bool ok = p.ndim == 2 ? p.sh == 1 && (R == 14 || R == 28) : (R == 2 || R == 7);
    if (!ok) return;
    c.R = R;
    c.nchunk = (p.Ho + c.R - 1) / c.R;
    c.blocks = (int)((long long)c.nmt * c.nchunk * c.ntb * p.Do * p.N);
}

hipError_t ring_launch(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s)
{
    if (c.DZ == 3) return ring3d_launch(p, c, a, s);
    if (p.dtype == GCONV_F32) return ring_launch_t<float>(p, c, a, s);
    return p.dtype == GCONV_F16 ? ring_launch_t<_Float16>(p, c, a, s) : ring_launch_t<__bf16>(p, c, a, s);
}

}  // namespace smallg
}  // namespace gconv

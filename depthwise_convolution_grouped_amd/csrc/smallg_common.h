// Pieces shared by the small-group MFMA kernels (halo box, row streaming,
// LDS ring): launch shape, buffer descriptors, the direct-to-LDS load, the
// MFMA per element type (16x16x32 for fp16/bf16, four chained 16x16x4 for
// fp32) and the block-diagonal weight slice, plus the host entry points of
// the two row-walking variants.
#pragma once

#include <utility>

#include "device_common.h"
#include "gconv_internal.h"

namespace gconv {
namespace smallg {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr unsigned kOob = 0x80000000u;

typedef int rsrc_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    const unsigned long long a = (unsigned long long)base;
    rsrc_t r;
    r.x = (int)(unsigned)(a & 0xffffffffull);
    r.y = (int)(unsigned)((a >> 32) & 0xffffull);
    r.z = (int)bytes;
    r.w = 0x00020000;
    return r;
}

__device__ __forceinline__ void dma16(unsigned voffset, unsigned lds_byte, rsrc_t r)
{
    asm volatile("s_mov_b32 m0, %1\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voffset), "s"(lds_byte), "s"(r)
                 : "memory", "m0");
}

template <typename T> struct Mfma;
template <> struct Mfma<_Float16> {
    typedef f16x8 V;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<__bf16> {
    typedef bf16x8 V;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
// fp32: a 16-byte slice holds 4 channels, and a 16x16x4 MFMA takes one
// value per lane (row or column lane % 16, k = lane / 16).  Element e of
// both operands' slices goes to the e-th of four MFMAs, so the four MFMAs
// together cover the 16 channels of the four lane groups' slices: the K
// order inside one slice group is permuted the same way on both sides,
// which leaves the sum unchanged.
template <> struct Mfma<float> {
    typedef f32x4 V;
    static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    }
};

// elements of T in one 16-byte slice
template <typename T> constexpr int kSliceElems = 16 / (int)sizeof(T);

// The 8 weights of one K slice (8 input channels at one tap) for the output
// channel of merged-tile row nn: the weight operand is block diagonal, so the
// slice is zero unless its channels belong to nn's group gout.  wk points at
// w[(g0 + gout) * Kpg + kout][tap 0][channel 0] ([g][k][tap][c] order); c8 is
// the slice's 8-channel chunk among the tile's GN * Cpg input channels.  The
// loads are unconditional (callers pass tap = c8 = 0 for a dead slice), so
// they issue together; the zeroing happens afterwards.
template <typename T, int CPGC>
__device__ __forceinline__ uint4 wslice(const T *wk, int tap, int c8, int gout, Div dCpg, bool live)
{
    uint4 raw = make_uint4(0, 0, 0, 0);
    if constexpr (CPGC == 8) {
        // all 8 channels of the slice belong to group (8 c8) / Cpg
        const int Cpg = dCpg.d;
        const int gs = fdiv(8 * c8, dCpg);
        const bool hit = live && gs == gout;
        const uint4 v = *reinterpret_cast<const uint4 *>(wk + tap * Cpg + (8 * c8 - gs * Cpg));
        raw.x = hit ? v.x : 0u; raw.y = hit ? v.y : 0u;
        raw.z = hit ? v.z : 0u; raw.w = hit ? v.w : 0u;
    } else {
        // group gout's CPGC channels sit at e0 = gout * CPGC - 8 c8 of the slice
        const int e0 = gout * CPGC - 8 * c8;
        const bool hit = live && e0 >= 0 && e0 < 8;
        const T *src = wk + tap * CPGC;
        unsigned d0, d1 = 0u;
        if constexpr (CPGC == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(src);
            d0 = v.x; d1 = v.y;
        } else if constexpr (CPGC == 2) {
            d0 = *reinterpret_cast<const unsigned *>(src);
        } else {
            d0 = *reinterpret_cast<const unsigned short *>(src);
        }
        const int dwi = e0 >> 1;                        // dword holding element e0
        const unsigned lo = hit ? ((e0 & 1) ? (d0 << 16) : d0) : 0u;
        const unsigned hi = hit ? d1 : 0u;
        raw.x = dwi == 0 ? lo : 0u;
        raw.y = dwi == 1 ? lo : (dwi == 0 ? hi : 0u);
        raw.z = dwi == 2 ? lo : 0u;
        raw.w = dwi == 3 ? lo : (dwi == 2 ? hi : 0u);
    }
    return raw;
}

// fp32: the 4 weights of one K slice (4 input channels at one tap), zero
// unless they belong to the group gout of the output channel (as above,
// with 4-channel chunks c4).
template <int CPGC>
__device__ __forceinline__ uint4 wslice_f32(const float *wk, int tap, int c4, int gout, Div dCpg, bool live)
{
    uint4 raw = make_uint4(0, 0, 0, 0);
    if constexpr (CPGC >= 4) {
        // Cpg is a multiple of 4: all 4 channels belong to group (4 c4) / Cpg
        const int Cpg = dCpg.d;
        const int gs = fdiv(4 * c4, dCpg);
        const bool hit = live && gs == gout;
        const uint4 v = *reinterpret_cast<const uint4 *>(wk + tap * Cpg + (4 * c4 - gs * Cpg));
        raw.x = hit ? v.x : 0u; raw.y = hit ? v.y : 0u;
        raw.z = hit ? v.z : 0u; raw.w = hit ? v.w : 0u;
    } else {
        // group gout's CPGC (1 or 2) channels sit at e0 = gout * CPGC - 4 c4
        const int e0 = gout * CPGC - 4 * c4;
        const bool hit = live && e0 >= 0 && e0 < 4;
        const unsigned *src = reinterpret_cast<const unsigned *>(wk + tap * CPGC);
        const unsigned d0 = src[0], d1 = CPGC == 2 ? src[1] : 0u;
        const unsigned v0 = hit ? d0 : 0u, v1 = hit ? d1 : 0u;
        raw.x = e0 == 0 ? v0 : 0u;
        raw.y = e0 == 1 ? v0 : (e0 == 0 ? v1 : 0u);
        raw.z = e0 == 2 ? v0 : (e0 == 1 ? v1 : 0u);
        raw.w = e0 == 3 ? v0 : (e0 == 2 ? v1 : 0u);
    }
    return raw;
}

template <typename T, int CPGC>
__device__ __forceinline__ uint4 weight_slice(const T *wk, int tap, int c, int gout, Div dCpg, bool live)
{
    if constexpr (sizeof(T) == 4) return wslice_f32<CPGC>(wk, tap, c, gout, dCpg, live);
    else return wslice<T, CPGC>(wk, tap, c, gout, dCpg, live);
}

template <int... Is, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Is...>, F &&f)
{
    (f(std::integral_constant<int, Is>{}), ...);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Row-streaming variant (k_smallg_rows.hip): 2D 3x3, stride 1 or 2, no dilation.
struct RowConfig {
    int GN, CH8, NT, R, NTW, nchunk, nmt, ntb;
};
bool rows_configure(const Problem &p, RowConfig &c);
hipError_t rows_launch(const Problem &p, const RowConfig &c, const Args &a, hipStream_t s);

// LDS-ring variant (smallg_ring.h): 2D 3x3 windows (stride 1 or 2) and 3D
// 3x3x3 windows (stride 1), no dilation, when the channel tiles group into
// ring pixels of 16 (or, in 3D, 8) chunks.  The 2D instances live in
// k_smallg_ring.hip, the 3D ones in k_smallg_ring3d.hip.
struct RingConfig {
    int GN, CH8, NT, NTW, TPB, ntb, DZ, R, CV, IW, RS, NINS, nmt, nchunk, blocks, lds;
};
bool ring_configure(const Problem &p, RingConfig &c);
// Rows per workgroup of a configured ring: 14 or 28 for 2D stride 1 (the
// tile menu), the configured value otherwise.
void ring_set_rows(const Problem &p, RingConfig &c, int R);
hipError_t ring_launch(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s);
hipError_t ring3d_launch(const Problem &p, const RingConfig &c, const Args &a, hipStream_t s);

}  // namespace smallg
}  // namespace gconv

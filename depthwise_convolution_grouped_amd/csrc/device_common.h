// Device-side element types, conversions and the fused epilogue shared by
// every kernel: fp32 accumulator + bias[g*Kpg + k] -> one round-to-nearest-even
// conversion to the element type -> store.  The output channel index
// g*Kpg + k follows rocm-libraries PR 10064, Technical Details (the epilogue
// folds the group into the output channel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gconv.h"

namespace gconv {

template <int DT> struct Elem;
template <> struct Elem<GCONV_F32> {
    using T = float;
    static constexpr int bytes = 4;
};
template <> struct Elem<GCONV_F16> {
    using T = _Float16;
    static constexpr int bytes = 2;
};
template <> struct Elem<GCONV_BF16> {
    using T = __bf16;
    static constexpr int bytes = 2;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }

// Round-to-nearest-even conversion from the fp32 accumulator.
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

// s_waitcnt vmcnt(n) for a wave-uniform n computed at run time.  The counter
// is an immediate of s_waitcnt, so the wait jumps into a table of
// "s_waitcnt vmcnt(k); s_branch end" pairs (8 bytes each) at k * 8 past the
// table start: a handful of scalar instructions and one indirect jump
// instead of a compare-and-branch tree.  n outside [0, 63] waits for
// vmcnt(0), which is always safe.  s[96:98] are scratch for the address.
__device__ __forceinline__ void vm_wait(int n)
{
    const unsigned u = (unsigned)__builtin_amdgcn_readfirstlane(n);
    const unsigned k = u < 64u ? u : 0u;
    asm volatile(
        "s_getpc_b64 s[96:97]\n"
        ".Lvmw_base%=:\n"
        "s_lshl_b32 s98, %0, 3\n"
        "s_add_u32 s96, s96, s98\n"
        "s_addc_u32 s97, s97, 0\n"
        "s_add_u32 s96, s96, .Lvmw_tab%= - .Lvmw_base%=\n"
        "s_addc_u32 s97, s97, 0\n"
        "s_setpc_b64 s[96:97]\n"
        ".Lvmw_tab%=:\n"
        "s_waitcnt vmcnt(0)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(1)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(2)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(3)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(4)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(5)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(6)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(7)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(8)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(9)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(10)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(11)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(12)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(13)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(14)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(15)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(16)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(17)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(18)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(19)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(20)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(21)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(22)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(23)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(24)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(25)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(26)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(27)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(28)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(29)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(30)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(31)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(32)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(33)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(34)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(35)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(36)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(37)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(38)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(39)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(40)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(41)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(42)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(43)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(44)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(45)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(46)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(47)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(48)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(49)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(50)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(51)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(52)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(53)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(54)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(55)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(56)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(57)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(58)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(59)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(60)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(61)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(62)\n s_branch .Lvmw_end%=\n"
        "s_waitcnt vmcnt(63)\n s_branch .Lvmw_end%=\n"
        ".Lvmw_end%=:\n"
        :
        : "s"(k)
        : "s96", "s97", "s98", "scc", "memory");
}

// n / d for 0 <= n < 2^16 and 1 <= d < 2^16 as umulhi(n, m) with
// m = ceil(2^32 / d): the rounding error n * (m - 2^32 / d) / 2^32 stays below
// 1 / d when n * d < 2^32, so the floor is exact.  d = 1 would need m = 2^32
// and is passed through unchanged.
struct Div {
    unsigned m;
    int d;
};
inline Div make_div(int d)
{
    Div r;
    r.d = d;
    r.m = d > 1 ? (unsigned)((0x100000000ull + (unsigned long long)d - 1) / (unsigned long long)d) : 0u;
    return r;
}
__device__ __forceinline__ int fdiv(int n, Div v)
{
    return v.d == 1 ? n : (int)__umulhi((unsigned)n, v.m);
}

// Epilogue for one output element: optional bias of output channel `ch`.
template <typename T>
__device__ __forceinline__ T finish(float acc, const T *__restrict__ bias, int ch)
{
    if (bias) acc += to_f32(bias[ch]);
    return from_f32<T>(acc);
}

// Block index remap so that consecutive logical tiles land on the same XCD.
// The hardware deals workgroups round-robin over the 8 XCDs of an MI355X
// (workgroup i runs on XCD i % 8); tile t = xcd * per_xcd + i / 8 gives each
// XCD a contiguous run of tiles, which share halo rows in that XCD's L2.
__device__ __forceinline__ int xcd_tile(int bid, int nblocks)
{
    constexpr int kXcd = 8;
    int per = nblocks / kXcd;          // blocks each XCD gets in full rounds
    int xcd = bid % kXcd, i = bid / kXcd;
    if (i >= per) return bid;          // the last partial round keeps its order
    return xcd * per + i;              // a bijection on [0, 8 * per)
}

}  // namespace gconv

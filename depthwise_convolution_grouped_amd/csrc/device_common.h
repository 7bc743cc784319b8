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

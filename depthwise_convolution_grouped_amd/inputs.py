"""Seeded synthetic inputs for the grouped-convolution workloads.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It holds problem shapes and random-number recipes only -- none of
the convolution's arithmetic -- and imports neither the HIP binding nor the
oracle.

Workloads stand in for the cases the pages benchmark: the MobileNetV2-style
depthwise and ResNeXt-style grouped conv2d cases of the TileOPs PR 1568
review (summary), its 3D grouped ResNeXt case (section "The 50x is a baseline
artifact", N=1, C 64->128, 8x28x28, 3x3x3, 32 groups) and a batch-8 version of
it (final review), plus a compute-bound large-channels-per-group case that the
same review asks for (Requested changes, item 3).  The small 2D grouped case
matches the test size of the CK Python examples README (Config-options
harness: N=1, G=2, C=K=64, 8x8, 3x3).

Recipe: values are drawn with numpy's PCG64 from ``seed`` in float32, then
rounded to nearest-even to the workload dtype; the rounded values are what
both the GPU path and the oracle consume.  Seeds are
``1000*workload_index + 10*variant`` (+0 for x, +1 for w, +2 for bias).
"N(0, v)" below gives the variance v (= 1/fan-in).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Problem:
    """A grouped conv forward problem (2D when ndim == 2: D = Z = 1)."""
    ndim: int
    dtype: str
    N: int
    G: int
    C: int
    K: int
    spatial: Tuple[int, int, int]          # (D, H, W)
    filt: Tuple[int, int, int]             # (Z, Y, X)
    stride: Tuple[int, int, int] = (1, 1, 1)
    pad: Tuple[int, int, int] = (0, 0, 0)
    dil: Tuple[int, int, int] = (1, 1, 1)
    bias: bool = True

    @property
    def Cpg(self) -> int:
        return self.C // self.G

    @property
    def Kpg(self) -> int:
        return self.K // self.G

    def x_shape(self):
        D, H, W = self.spatial
        return (self.N, H, W, self.C) if self.ndim == 2 else (self.N, D, H, W, self.C)

    def w_shape(self):
        Z, Y, X = self.filt
        return (self.K, Y, X, self.Cpg) if self.ndim == 2 else (self.K, Z, Y, X, self.Cpg)

    def spatial_args(self):
        """(stride, pad, dil) trimmed to ndim entries."""
        s = slice(1, 3) if self.ndim == 2 else slice(0, 3)
        return self.stride[s], self.pad[s], self.dil[s]


def conv2d(dtype, N, G, C, K, H, W, Y, X, stride=1, pad=0, dil=1, bias=True) -> Problem:
    return Problem(2, dtype, N, G, C, K, (1, H, W), (1, Y, X),
                   (1, stride, stride), (0, pad, pad), (1, dil, dil), bias)


def conv3d(dtype, N, G, C, K, D, H, W, Z, Y, X, stride=1, pad=0, dil=1, bias=True) -> Problem:
    return Problem(3, dtype, N, G, C, K, (D, H, W), (Z, Y, X),
                   (stride,) * 3, (pad,) * 3, (dil,) * 3, bias)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed base = 1000 * index
    variant: int        # seed += 10 * variant
    problem: Problem
    x_dist: Tuple[str, float]     # ("uniform", a) -> U[-a, a]; ("normal", var)
    w_dist: Tuple[str, float]
    b_dist: Tuple[str, float] = ("uniform", 1.0)
    about: str = ""

    @property
    def seed(self) -> int:
        return 1000 * self.index + 10 * self.variant


WORKLOADS = {
    "grouped2d_small_f32": Workload(
        "grouped2d_small_f32", 0, 0,
        conv2d("f32", N=1, G=2, C=64, K=64, H=8, W=8, Y=3, X=3, stride=1, pad=1, dil=1, bias=True),
        ("uniform", 1.0), ("uniform", 1.0),
        about="2D grouped fp32, N=1 G=2 32/32 ch per group, 8x8, 3x3 s1 p1, bias"),
    "depthwise2d_f16": Workload(
        "depthwise2d_f16", 1, 0,
        conv2d("f16", N=32, G=144, C=144, K=144, H=56, W=56, Y=3, X=3, stride=1, pad=1, bias=True),
        ("normal", 1.0), ("normal", 1.0 / 9),
        about="2D depthwise fp16 (MobileNetV2-style), N=32 C=144 56x56 3x3 s1 p1, bias"),
    "depthwise2d_s2_f16": Workload(
        "depthwise2d_s2_f16", 1, 1,
        conv2d("f16", N=32, G=144, C=144, K=144, H=56, W=56, Y=3, X=3, stride=2, pad=1, bias=True),
        ("normal", 1.0), ("normal", 1.0 / 9),
        about="2D depthwise fp16, stride-2 variant -> 28x28, bias"),
    "grouped2d_resnext_bf16": Workload(
        "grouped2d_resnext_bf16", 2, 0,
        conv2d("bf16", N=32, G=32, C=256, K=256, H=56, W=56, Y=3, X=3, stride=1, pad=1, bias=False),
        ("normal", 1.0), ("normal", 1.0 / 72),
        about="2D grouped bf16 (ResNeXt-style), N=32 C=K=256 G=32 (8/group) 56x56 3x3 s1 p1, no bias"),
    "grouped3d_f16_n1": Workload(
        "grouped3d_f16_n1", 3, 0,
        conv3d("f16", N=1, G=32, C=64, K=128, D=8, H=28, W=28, Z=3, Y=3, X=3, stride=1, pad=1, bias=True),
        ("normal", 1.0), ("normal", 1.0 / 54),
        about="3D grouped fp16, C 64->128 G=32 (2 in/4 out per group), 8x28x28, 3x3x3 p1, bias, N=1"),
    "grouped3d_f16_n8": Workload(
        "grouped3d_f16_n8", 3, 1,
        conv3d("f16", N=8, G=32, C=64, K=128, D=8, H=28, W=28, Z=3, Y=3, X=3, stride=1, pad=1, bias=True),
        ("normal", 1.0), ("normal", 1.0 / 54),
        about="same 3D grouped fp16 case at N=8"),
    "grouped2d_large_bf16": Workload(
        "grouped2d_large_bf16", 4, 0,
        conv2d("bf16", N=64, G=8, C=1024, K=1024, H=14, W=14, Y=3, X=3, stride=1, pad=1, bias=True),
        ("normal", 1.0), ("normal", 1.0 / 1152),
        about="2D grouped bf16, compute-bound: N=64 C=K=1024 G=8 (128/group) 14x14 3x3 p1, bias"),
    "grouped2d_large_dil2_bf16": Workload(
        "grouped2d_large_dil2_bf16", 4, 1,
        conv2d("bf16", N=64, G=8, C=1024, K=1024, H=14, W=14, Y=3, X=3, stride=1, pad=2, dil=2, bias=True),
        ("normal", 1.0), ("normal", 1.0 / 1152),
        about="same with dilation 2 / pad 2"),
}


# ---------------------------------------------------------------- rounding

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> the array that holds them in `dtype` (bf16 as uint16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(a32, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError("unknown dtype %r" % dtype)


def storage_to_f64(s: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a storage array to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(s).astype(np.float64)
    return np.asarray(s).astype(np.float64)


def element_size(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


# ---------------------------------------------------------------- drawing

def _draw(rng: np.random.Generator, shape, dist) -> np.ndarray:
    kind, p = dist
    if kind == "uniform":
        return rng.uniform(-p, p, size=shape).astype(np.float32)
    if kind == "normal":
        return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(np.sqrt(p))).astype(np.float32)
    if kind == "int":          # small integers in [-p, p]: exact in every dtype
        return rng.integers(-int(p), int(p) + 1, size=shape).astype(np.float32)
    if kind == "ones":
        return np.ones(shape, dtype=np.float32)
    raise ValueError(kind)


@dataclasses.dataclass
class Tensors:
    """Storage arrays in the problem dtype (bf16 as uint16 bits)."""
    x: np.ndarray
    w: np.ndarray
    bias: Optional[np.ndarray]


def make_tensors(p: Problem, seed: int, x_dist=("normal", 1.0), w_dist=None,
                 b_dist=("uniform", 1.0)) -> Tensors:
    """Seeded tensors for problem p: x in N[D]HWC, w in K[Z]YXC (= G Kpg [Z]YX Cpg), bias [K]."""
    if w_dist is None:
        taps = p.filt[0] * p.filt[1] * p.filt[2]
        w_dist = ("normal", 1.0 / (p.Cpg * taps))
    x = _draw(np.random.default_rng(seed), p.x_shape(), x_dist)
    w = _draw(np.random.default_rng(seed + 1), p.w_shape(), w_dist)
    b = _draw(np.random.default_rng(seed + 2), (p.K,), b_dist) if p.bias else None
    return Tensors(to_storage(x, p.dtype), to_storage(w, p.dtype),
                   to_storage(b, p.dtype) if b is not None else None)


def make_array(shape, dtype: str, seed: int, dist=("normal", 1.0)) -> np.ndarray:
    """A seeded storage array of any shape (e.g. an output gradient dy for backward data)."""
    return to_storage(_draw(np.random.default_rng(seed), tuple(shape), dist), dtype)


def workload_tensors(wl: Workload) -> Tensors:
    return make_tensors(wl.problem, wl.seed, wl.x_dist, wl.w_dist, wl.b_dist)


def random_problem(rng: np.random.Generator, dtype: str, ndim: int) -> Problem:
    """A small random problem for sweeps: odd sizes, strides, pads and dilations."""
    G = int(rng.choice([1, 2, 3, 4, 8]))
    Cpg = int(rng.choice([1, 1, 2, 3, 4, 8, 16]))
    Kpg = int(rng.choice([1, 1, 2, 4, 8, 16]))
    N = int(rng.integers(1, 3))
    sp = [int(rng.integers(3, 12)) for _ in range(3)]
    fl = [int(rng.choice([1, 3, 3, 5])) for _ in range(3)]
    st = int(rng.integers(1, 3))
    dl = int(rng.integers(1, 3))
    pd = int(rng.integers(0, 3))
    if ndim == 2:
        sp[0], fl[0] = 1, 1
    for a in range(3):
        while sp[a] + 2 * pd < dl * (fl[a] - 1) + 1:
            sp[a] += 2
    bias = bool(rng.integers(0, 2))
    if ndim == 2:
        return Problem(2, dtype, N, G, G * Cpg, G * Kpg, (1, sp[1], sp[2]), (1, fl[1], fl[2]),
                       (1, st, st), (0, pd, pd), (1, dl, dl), bias)
    return Problem(3, dtype, N, G, G * Cpg, G * Kpg, tuple(sp), tuple(fl),
                   (st,) * 3, (pd,) * 3, (dl,) * 3, bias)

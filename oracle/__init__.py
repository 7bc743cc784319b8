"""Plain CPU oracle for grouped / depthwise convolution forward, backward data and backward weight.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``depthwise_convolution_grouped_amd``) never imports it and shares no code
with it.

The arithmetic lives in ``gconv_ref.c`` (fp64 direct grouped cross-correlation,
written from the definition; see that file's header for the readings it takes
of the pages).  This module only builds that file with gcc, loads it with
ctypes and marshals numpy arrays:

* ``conv_fwd``        -- every output element plus its error scale
* ``conv_fwd_points`` -- selected output elements (full-size spot checks)
* ``conv_bwd_data``   -- backward data: the gradient w.r.t. x from dy and w
* ``conv_bwd_weight`` -- backward weight: the gradient w.r.t. w from x and dy
* ``out_extent``      -- output length along one axis

Arrays use the oracle's layouts: x ``[N][D][H][W][G][Cpg]``,
w ``[G][Kpg][Z][Y][X][Cpg]``, y ``[N][Do][Ho][Wo][G][Kpg]``, bias ``[G*Kpg]``;
a 2D problem passes D = Z = 1.  Inputs are float64 holding the exact values of
the (possibly fp16/bf16) tensors.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gconv_ref.c")
_LIB = os.path.join(_HERE, "_build", "libgconv_ref.so")

_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile gconv_ref.c (or another source `src`) with gcc -O2 -fopenmp into `out`."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = bind(_LIB)
    return _lib


def bind(path: str):
    """Open a build of gconv_ref.c at `path` and declare its entry points."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    p64 = ctypes.POINTER(ctypes.c_int64)
    pd = ctypes.POINTER(ctypes.c_double)
    lib.gref_out_extent.argtypes = [i64, i64, i64, i64, i64]
    lib.gref_out_extent.restype = i64
    lib.gref_conv_fwd.argtypes = [i64, i64, i64, i64, p64, p64, p64, p64, p64,
                                  pd, pd, pd, pd, pd]
    lib.gref_conv_fwd.restype = ctypes.c_int
    lib.gref_conv_fwd_points.argtypes = [i64, i64, i64, i64, p64, p64, p64, p64, p64,
                                         pd, pd, pd, p64, i64, pd, pd]
    lib.gref_conv_fwd_points.restype = ctypes.c_int
    lib.gref_conv_bwd_data.argtypes = [i64, i64, i64, i64, p64, p64, p64, p64, p64, pd, pd, pd, pd]
    lib.gref_conv_bwd_data.restype = ctypes.c_int
    lib.gref_conv_bwd_weight.argtypes = [i64, i64, i64, i64, p64, p64, p64, p64, p64, pd, pd, pd, pd]
    lib.gref_conv_bwd_weight.restype = ctypes.c_int
    lib.gref_num_threads.argtypes = []
    lib.gref_num_threads.restype = ctypes.c_int
    return lib


def _triple(v, fill):
    v = tuple(int(a) for a in v)
    if len(v) == 2:
        v = (fill,) + v
    if len(v) != 3:
        raise ValueError("expected 2 or 3 spatial values, got %r" % (v,))
    return (ctypes.c_int64 * 3)(*v)


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def out_extent(n: int, k: int, stride: int, pad: int, dil: int, lib=None) -> int:
    return int((lib or _load()).gref_out_extent(n, k, stride, pad, dil))


def _prepare(x, w, bias, groups, stride, pad, dil):
    """Shapes: x (N, D, H, W, C) or (N, H, W, C); w (K, Z, Y, X, Cpg) or (K, Y, X, Cpg)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    if x.ndim == 4:
        x = x[:, None]
    if w.ndim == 4:
        w = w[:, None]
    if x.ndim != 5 or w.ndim != 5:
        raise ValueError("x must be N[D]HWC and w K[Z]YXC")
    N, D, H, W, C = x.shape
    K, Z, Y, X, Cpg = w.shape
    G = int(groups)
    if G <= 0 or C % G or K % G or C // G != Cpg:
        raise ValueError("inconsistent channels: C=%d K=%d G=%d Cpg=%d" % (C, K, G, Cpg))
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float64).reshape(K)
    dims = dict(N=N, G=G, C=C, K=K,
                in_=_triple((D, H, W), 1), filt=_triple((Z, Y, X), 1),
                stride=_triple(stride, 1), pad=_triple(pad, 0), dil=_triple(dil, 1))
    return x, w, bias, dims


def _outs(dims, lib):
    return [out_extent(dims["in_"][a], dims["filt"][a], dims["stride"][a],
                       dims["pad"][a], dims["dil"][a], lib) for a in range(3)]


def conv_fwd(x, w, bias, groups, stride, pad, dil, lib=None):
    """Grouped forward conv, fp64.  Returns (y, scale), both N,[Do,]Ho,Wo,K.

    `lib` selects another build of gconv_ref.c (see `bind`); default: the oracle.
    """
    lib = lib or _load()
    spatial3 = np.ndim(x) == 5
    x, w, bias, d = _prepare(x, w, bias, groups, stride, pad, dil)
    Do, Ho, Wo = _outs(d, lib)
    if min(Do, Ho, Wo) <= 0:
        raise ValueError("empty output")
    y = np.empty((d["N"], Do, Ho, Wo, d["K"]), dtype=np.float64)
    s = np.empty_like(y)
    rc = lib.gref_conv_fwd(d["N"], d["G"], d["C"], d["K"], d["in_"], d["filt"],
                               d["stride"], d["pad"], d["dil"], _dptr(x), _dptr(w),
                               _dptr(bias) if bias is not None else None,
                               _dptr(y), _dptr(s))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    if not spatial3:
        y, s = y[:, 0], s[:, 0]
    return y, s


def conv_fwd_points(x, w, bias, groups, stride, pad, dil, flat_idx):
    """Outputs at flat indices of y's N[Do]HoWoK layout.  Returns (y_pts, scale_pts)."""
    x, w, bias, d = _prepare(x, w, bias, groups, stride, pad, dil)
    idx = np.ascontiguousarray(flat_idx, dtype=np.int64)
    yp = np.empty(idx.shape[0], dtype=np.float64)
    sp = np.empty_like(yp)
    rc = _load().gref_conv_fwd_points(
        d["N"], d["G"], d["C"], d["K"], d["in_"], d["filt"], d["stride"], d["pad"], d["dil"],
        _dptr(x), _dptr(w), _dptr(bias) if bias is not None else None,
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), idx.shape[0],
        _dptr(yp), _dptr(sp))
    if rc != 0:
        raise ValueError("oracle rejected the problem or an index")
    return yp, sp


def conv_bwd_data(dy, w, groups, in_spatial, stride, pad, dil, lib=None):
    """Backward data (the gradient w.r.t. x), fp64.  Returns (dx, scale), both N,[D,]H,W,C.

    dy is N[Do]HoWoK, w K[Z]YXCpg; in_spatial gives the input extents ((H, W) or
    (D, H, W)), which a strided forward does not determine from dy.
    """
    lib = lib or _load()
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    spatial3 = dy.ndim == 5
    if dy.ndim == 4:
        dy = dy[:, None]
    if w.ndim == 4:
        w = w[:, None]
    if dy.ndim != 5 or w.ndim != 5:
        raise ValueError("dy must be N[Do]HoWoK and w K[Z]YXCpg")
    N, K = dy.shape[0], dy.shape[4]
    G = int(groups)
    Cpg = w.shape[4]
    if G <= 0 or K % G or w.shape[0] != K:
        raise ValueError("inconsistent channels")
    C = G * Cpg
    in_ = _triple(in_spatial, 1)
    d = dict(in_=in_, filt=_triple(w.shape[1:4], 1), stride=_triple(stride, 1),
             pad=_triple(pad, 0), dil=_triple(dil, 1))
    outs = _outs(d, lib)
    if tuple(outs) != tuple(dy.shape[1:4]):
        raise ValueError("dy extents %r do not match the forward output %r" % (dy.shape[1:4], tuple(outs)))
    dx = np.empty((N, in_[0], in_[1], in_[2], C), dtype=np.float64)
    s = np.empty_like(dx)
    rc = lib.gref_conv_bwd_data(N, G, C, K, in_, d["filt"], d["stride"], d["pad"], d["dil"],
                                _dptr(dy), _dptr(w), _dptr(dx), _dptr(s))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    if not spatial3:
        dx, s = dx[:, 0], s[:, 0]
    return dx, s


def conv_bwd_weight(x, dy, groups, filt, stride, pad, dil, lib=None):
    """Backward weight (the gradient w.r.t. w), fp64.  Returns (dw, scale), both K,[Z,]Y,X,Cpg.

    x is N[D]HWC, dy N[Do]HoWoK; filt gives the filter extents ((Y, X) or (Z, Y, X)).
    """
    lib = lib or _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    spatial3 = x.ndim == 5
    if x.ndim == 4:
        x = x[:, None]
    if dy.ndim == 4:
        dy = dy[:, None]
    if x.ndim != 5 or dy.ndim != 5:
        raise ValueError("x must be N[D]HWC and dy N[Do]HoWoK")
    N, C, K = x.shape[0], x.shape[4], dy.shape[4]
    G = int(groups)
    if G <= 0 or C % G or K % G or dy.shape[0] != N:
        raise ValueError("inconsistent channels or batch")
    d = dict(in_=_triple(x.shape[1:4], 1), filt=_triple(filt, 1), stride=_triple(stride, 1),
             pad=_triple(pad, 0), dil=_triple(dil, 1))
    outs = _outs(d, lib)
    if tuple(outs) != tuple(dy.shape[1:4]):
        raise ValueError("dy extents %r do not match the forward output %r" % (dy.shape[1:4], tuple(outs)))
    f = d["filt"]
    dw = np.empty((K, f[0], f[1], f[2], C // G), dtype=np.float64)
    s = np.empty_like(dw)
    rc = lib.gref_conv_bwd_weight(N, G, C, K, d["in_"], f, d["stride"], d["pad"], d["dil"],
                                  _dptr(x), _dptr(dy), _dptr(dw), _dptr(s))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    if not spatial3:
        dw, s = dw[:, 0], s[:, 0]
    return dw, s


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().gref_num_threads())

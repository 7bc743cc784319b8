"""Thin ctypes binding of libgconv.so (include/gconv.h), same names as the C ABI.

Argument marshalling only: every step of the convolution runs in the HIP
kernels behind ``gconv_fwd``.  There is no fallback; if the library has not
been built, the first call raises ``GconvUnavailable``.

``conv_fwd`` is a convenience for PyTorch device tensors (PyTorch provides the
device memory and the stream, nothing else):

    y = conv_fwd(x, w, bias, groups=G, stride=(1, 1), pad=(1, 1), dil=(1, 1))

with x in N[D]HWC = N[D]HW(G Cpg) order and w in K[Z]YXC = (G Kpg)[Z]YX Cpg
order, both contiguous, and y returned in N[Do]HoWoK order.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libgconv.so")

GCONV_F32, GCONV_F16, GCONV_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": GCONV_F32, "f16": GCONV_F16, "bf16": GCONV_BF16}

GCONV_OK = 0
GCONV_ERR_BAD_DESC = -1
GCONV_ERR_BAD_OUT_DIMS = -2
GCONV_ERR_NULL_PTR = -3
GCONV_ERR_TOO_LARGE = -4
GCONV_ERR_MISALIGNED = -5
GCONV_ERR_BAD_PATH = -6
GCONV_ERR_PATH_UNSUPPORTED = -7
GCONV_ERR_LAUNCH = -8
GCONV_ERR_SCRATCH = -9
GCONV_NOALLOC_SCRATCH_BYTES = 32 << 20

GCONV_PATH_AUTO = -1
GCONV_PATH_GENERIC = 0
GCONV_PATH_DEPTHWISE = 1
GCONV_PATH_SMALLG = 2
GCONV_PATH_IGEMM = 3
GCONV_PATH_IGHALO = 4
GCONV_PATH_DIRECT = 5
GCONV_NUM_PATHS = 6
PATHS = {"generic": 0, "depthwise": 1, "smallg_mfma": 2, "igemm_mfma": 3, "ighalo_mfma": 4, "direct_valu": 5}

EXPORTS = ("gconv_validate", "gconv_out_dims", "gconv_select_path", "gconv_path_supported",
           "gconv_get_plan", "gconv_fwd", "gconv_fwd_path", "gconv_fwd_timed",
           "gconv_tile_count", "gconv_fwd_tile",
           "gconv_bwd_data_workspace", "gconv_bwd_data", "gconv_bwd_data_direct",
           "gconv_bwd_weight_workspace", "gconv_bwd_weight", "gconv_bwd_weight_noalloc",
           "gconv_status_str", "gconv_path_name", "gconv_abi_version")


class GconvUnavailable(RuntimeError):
    pass


class GconvError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what or "gconv", gconv_status_str(status), status))


class gconv_desc(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("N", ctypes.c_int64), ("G", ctypes.c_int64),
                ("C", ctypes.c_int64), ("K", ctypes.c_int64),
                ("in_", ctypes.c_int64 * 3), ("filt", ctypes.c_int64 * 3),
                ("stride", ctypes.c_int64 * 3), ("pad", ctypes.c_int64 * 3),
                ("dil", ctypes.c_int64 * 3)]


class gconv_plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("grid", ctypes.c_uint32 * 3),
                ("block", ctypes.c_uint32), ("lds_bytes", ctypes.c_uint32),
                ("groups_per_tile", ctypes.c_uint32)]

    def as_dict(self):
        return {"path": self.path, "grid": tuple(self.grid), "block": self.block,
                "lds_bytes": self.lds_bytes, "groups_per_tile": self.groups_per_tile}


_lib = None


def lib():
    """The loaded libgconv.so (raises GconvUnavailable if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise GconvUnavailable(
            "libgconv.so is not built (%s); run python -m depthwise_convolution_grouped_amd.build"
            % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    pd = ctypes.POINTER(gconv_desc)
    vp = ctypes.c_void_p
    L.gconv_validate.argtypes = [pd]
    L.gconv_out_dims.argtypes = [pd, ctypes.POINTER(ctypes.c_int64)]
    L.gconv_select_path.argtypes = [pd]
    L.gconv_path_supported.argtypes = [pd, ctypes.c_int]
    L.gconv_get_plan.argtypes = [pd, ctypes.c_int, ctypes.POINTER(gconv_plan)]
    L.gconv_fwd.argtypes = [pd, vp, vp, vp, vp, vp]
    L.gconv_fwd_path.argtypes = [pd, ctypes.c_int, vp, vp, vp, vp, vp]
    L.gconv_fwd_timed.argtypes = [pd, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
    L.gconv_tile_count.argtypes = [pd, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.gconv_fwd_tile.argtypes = [pd, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
    L.gconv_bwd_data_workspace.argtypes = [pd, ctypes.POINTER(ctypes.c_size_t)]
    L.gconv_bwd_data.argtypes = [pd, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gconv_bwd_data_direct.argtypes = [pd, vp, vp, vp, vp]
    L.gconv_bwd_weight_workspace.argtypes = [pd, ctypes.POINTER(ctypes.c_size_t)]
    L.gconv_bwd_weight.argtypes = [pd, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gconv_bwd_weight_noalloc.argtypes = [pd, vp, vp, vp, vp]
    L.gconv_status_str.argtypes = [ctypes.c_int]
    L.gconv_status_str.restype = ctypes.c_char_p
    L.gconv_path_name.argtypes = [ctypes.c_int]
    L.gconv_path_name.restype = ctypes.c_char_p
    L.gconv_abi_version.argtypes = []
    for name in ("gconv_validate", "gconv_out_dims", "gconv_select_path", "gconv_path_supported",
                 "gconv_get_plan", "gconv_fwd", "gconv_fwd_path", "gconv_fwd_timed",
                 "gconv_tile_count", "gconv_fwd_tile", "gconv_bwd_data_workspace", "gconv_bwd_data", "gconv_bwd_data_direct",
                 "gconv_bwd_weight_workspace", "gconv_bwd_weight", "gconv_bwd_weight_noalloc", "gconv_abi_version"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _t3(v: Sequence[int], fill: int):
    v = tuple(int(a) for a in v)
    if len(v) == 2:
        v = (fill,) + v
    if len(v) != 3:
        raise ValueError("expected 2 or 3 spatial values, got %r" % (v,))
    return (ctypes.c_int64 * 3)(*v)


def make_desc(ndim, dtype, N, G, C, K, spatial, filt, stride, pad, dil) -> gconv_desc:
    """Descriptor from sizes; spatial/filt/stride/pad/dil take 2 (2D) or 3 values."""
    d = gconv_desc()
    d.ndim = int(ndim)
    d.dtype = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    d.N, d.G, d.C, d.K = int(N), int(G), int(C), int(K)
    d.in_ = _t3(spatial, 1)
    d.filt = _t3(filt, 1)
    d.stride = _t3(stride, 1)
    d.pad = _t3(pad, 0)
    d.dil = _t3(dil, 1)
    return d


def desc_from_problem(p) -> gconv_desc:
    """Descriptor of an ``inputs.Problem``."""
    return make_desc(p.ndim, p.dtype, p.N, p.G, p.C, p.K, p.spatial, p.filt, p.stride, p.pad, p.dil)


def gconv_validate(d: gconv_desc) -> int:
    return lib().gconv_validate(ctypes.byref(d))


def gconv_out_dims(d: gconv_desc):
    out = (ctypes.c_int64 * 3)()
    rc = lib().gconv_out_dims(ctypes.byref(d), out)
    if rc != GCONV_OK:
        raise GconvError(rc, "gconv_out_dims")
    return tuple(out)


def gconv_select_path(d: gconv_desc) -> int:
    return lib().gconv_select_path(ctypes.byref(d))


def gconv_path_supported(d: gconv_desc, path: int) -> int:
    return lib().gconv_path_supported(ctypes.byref(d), int(path))


def gconv_get_plan(d: gconv_desc, path: int = GCONV_PATH_AUTO) -> dict:
    pl = gconv_plan()
    rc = lib().gconv_get_plan(ctypes.byref(d), int(path), ctypes.byref(pl))
    if rc != GCONV_OK:
        raise GconvError(rc, "gconv_get_plan")
    return pl.as_dict()


def gconv_fwd(d: gconv_desc, x: int, w: int, bias: Optional[int], y: int, stream: int = 0) -> int:
    """Raw call with device addresses (ints); returns the status code."""
    return lib().gconv_fwd(ctypes.byref(d), x, w, bias or None, y, stream or None)


def gconv_fwd_path(d: gconv_desc, path: int, x: int, w: int, bias: Optional[int], y: int,
                   stream: int = 0) -> int:
    return lib().gconv_fwd_path(ctypes.byref(d), int(path), x, w, bias or None, y, stream or None)


def gconv_fwd_timed(d: gconv_desc, path: int, x: int, w: int, bias: Optional[int], y: int,
                    stream: int, ev_start: int, ev_stop: int) -> int:
    """gconv_fwd_path with two hipEvent_t handles bound to the kernel dispatch."""
    return lib().gconv_fwd_timed(ctypes.byref(d), int(path), x, w, bias or None, y,
                                 stream or None, ev_start or None, ev_stop or None)


def gconv_bwd_data_workspace(d: gconv_desc) -> int:
    """Workspace bytes gconv_bwd_data can use for the forward descriptor d."""
    n = ctypes.c_size_t()
    rc = lib().gconv_bwd_data_workspace(ctypes.byref(d), ctypes.byref(n))
    if rc != GCONV_OK:
        raise GconvError(rc, "gconv_bwd_data_workspace")
    return int(n.value)


def gconv_bwd_data(d: gconv_desc, dy: int, w: int, dx: int, workspace: Optional[int],
                   workspace_bytes: int, stream: int = 0) -> int:
    """Raw call with device addresses (ints); returns the status code."""
    return lib().gconv_bwd_data(ctypes.byref(d), dy, w, dx, workspace or None, int(workspace_bytes),
                                stream or None)


def gconv_bwd_data_direct(d: gconv_desc, dy: int, w: int, dx: int, stream: int = 0) -> int:
    return lib().gconv_bwd_data_direct(ctypes.byref(d), dy, w, dx, stream or None)


def gconv_bwd_weight_workspace(d: gconv_desc) -> int:
    """Partial-sum workspace bytes gconv_bwd_weight can use for the forward descriptor d."""
    n = ctypes.c_size_t()
    rc = lib().gconv_bwd_weight_workspace(ctypes.byref(d), ctypes.byref(n))
    if rc != GCONV_OK:
        raise GconvError(rc, "gconv_bwd_weight_workspace")
    return int(n.value)


def gconv_bwd_weight(d: gconv_desc, x: int, dy: int, dw: int, workspace: Optional[int],
                     workspace_bytes: int, stream: int = 0) -> int:
    """Raw call with device addresses (ints); returns the status code."""
    return lib().gconv_bwd_weight(ctypes.byref(d), x, dy, dw, workspace or None, int(workspace_bytes),
                                  stream or None)


def gconv_bwd_weight_noalloc(d: gconv_desc, x: int, dy: int, dw: int, stream: int = 0) -> int:
    """Raw call with device addresses (ints); the library's own device scratch
    holds the partial sums.  Returns the status code."""
    return lib().gconv_bwd_weight_noalloc(ctypes.byref(d), x, dy, dw, stream or None)


def gconv_tile_count(d: gconv_desc, path: int = GCONV_PATH_AUTO):
    """(menu size, the path's own pick) for d on `path`; raises GconvError on a bad descriptor or path."""
    picked = ctypes.c_int(-1)
    n = lib().gconv_tile_count(ctypes.byref(d), int(path), ctypes.byref(picked))
    if n < 0:
        raise GconvError(n, "gconv_tile_count")
    return n, picked.value


def gconv_fwd_tile(d: gconv_desc, path: int, tile: int, x: int, w: int, bias: Optional[int], y: int,
                   stream: int = 0) -> int:
    """Raw call with device addresses (ints); returns the status code."""
    return lib().gconv_fwd_tile(ctypes.byref(d), int(path), int(tile), x, w, bias or None, y, stream or None)


def gconv_status_str(status: int) -> str:
    try:
        return lib().gconv_status_str(int(status)).decode()
    except GconvUnavailable:
        return "status %d" % status


def gconv_path_name(path: int) -> str:
    return lib().gconv_path_name(int(path)).decode()


def gconv_abi_version() -> int:
    return lib().gconv_abi_version()


# ------------------------------------------------------------ torch helper

def _torch_dtype_code(t):
    import torch
    m = {torch.float32: GCONV_F32, torch.float16: GCONV_F16, torch.bfloat16: GCONV_BF16}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return m[t.dtype]


def conv_fwd(x, w, bias=None, groups: int = 1, stride=None, pad=None, dil=None,
             out=None, path: int = GCONV_PATH_AUTO, stream=None):
    """Grouped conv forward on PyTorch device tensors (channels-last, see module doc)."""
    import torch
    nd = x.dim() - 2
    if nd not in (2, 3) or w.dim() != x.dim():
        raise ValueError("x must be N[D]HWC and w K[Z]YXC")
    if not (x.is_contiguous() and w.is_contiguous()) or (bias is not None and not bias.is_contiguous()):
        raise ValueError("x, w and bias must be contiguous")
    if w.dtype != x.dtype or (bias is not None and bias.dtype != x.dtype):
        raise TypeError("x, w and bias must share one dtype")
    stride = stride or (1,) * nd
    pad = pad or (0,) * nd
    dil = dil or (1,) * nd
    N, C = x.shape[0], x.shape[-1]
    K = w.shape[0]
    if w.shape[-1] * groups != C:
        raise ValueError("w's last extent must be C / groups")
    d = make_desc(nd, _torch_dtype_code(x), N, groups, C, K, tuple(x.shape[1:-1]),
                  tuple(w.shape[1:-1]), stride, pad, dil)
    o = gconv_out_dims(d)
    oshape = (N,) + (o if nd == 3 else o[1:]) + (K,)
    if out is None:
        out = torch.empty(oshape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != oshape or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError("out must be a contiguous %s tensor of shape %s" % (x.dtype, oshape))
    s = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
    rc = gconv_fwd_path(d, path, x.data_ptr(), w.data_ptr(),
                        bias.data_ptr() if bias is not None else None, out.data_ptr(), s)
    if rc != GCONV_OK:
        raise GconvError(rc, "gconv_fwd")
    return out


def conv_bwd_data(dy, w, groups: int, in_spatial, stride=None, pad=None, dil=None, out=None,
                  direct: bool = False, workspace=None, stream=None):
    """Backward data on PyTorch device tensors: dx (N[D]HWC) from dy (N[Do]HoWoK) and w (K[Z]YXCpg).

    in_spatial is dx's (H, W) or (D, H, W).  A workspace of
    gconv_bwd_data_workspace bytes is allocated here unless one is passed
    (a uint8 device tensor) or `direct` asks for the direct kernel.
    """
    import torch
    nd = dy.dim() - 2
    if nd not in (2, 3) or w.dim() != dy.dim():
        raise ValueError("dy must be N[Do]HoWoK and w K[Z]YXCpg")
    if not (dy.is_contiguous() and w.is_contiguous()):
        raise ValueError("dy and w must be contiguous")
    if w.dtype != dy.dtype:
        raise TypeError("dy and w must share one dtype")
    stride = stride or (1,) * nd
    pad = pad or (0,) * nd
    dil = dil or (1,) * nd
    N, K = dy.shape[0], dy.shape[-1]
    C = w.shape[-1] * groups
    d = make_desc(nd, _torch_dtype_code(dy), N, groups, C, K, tuple(in_spatial),
                  tuple(w.shape[1:-1]), stride, pad, dil)
    o = gconv_out_dims(d)
    if tuple(dy.shape[1:-1]) != (o if nd == 3 else o[1:]):
        raise ValueError("dy's extents %r are not the forward output %r" % (tuple(dy.shape[1:-1]), o))
    xshape = (N,) + tuple(in_spatial) + (C,)
    if out is None:
        out = torch.empty(xshape, dtype=dy.dtype, device=dy.device)
    elif tuple(out.shape) != xshape or not out.is_contiguous() or out.dtype != dy.dtype:
        raise ValueError("out must be a contiguous %s tensor of shape %s" % (dy.dtype, xshape))
    s = stream if stream is not None else torch.cuda.current_stream(dy.device).cuda_stream
    if direct:
        rc = gconv_bwd_data_direct(d, dy.data_ptr(), w.data_ptr(), out.data_ptr(), s)
    else:
        need = gconv_bwd_data_workspace(d)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dy.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        rc = gconv_bwd_data(d, dy.data_ptr(), w.data_ptr(), out.data_ptr(), ws_ptr, ws_bytes, s)
    if rc != GCONV_OK:
        raise GconvError(rc, "gconv_bwd_data")
    return out


def conv_bwd_weight(x, dy, groups: int, filt, stride=None, pad=None, dil=None, out=None,
                    workspace=None, use_workspace: bool = True, stream=None):
    """Backward weight on PyTorch device tensors: dw (K[Z]YXCpg) from x (N[D]HWC) and dy (N[Do]HoWoK).

    filt is (Y, X) or (Z, Y, X).  A workspace of gconv_bwd_weight_workspace
    bytes is allocated here unless one is passed (a device tensor) or
    use_workspace is False (one kernel, one chunk).
    """
    import torch
    nd = x.dim() - 2
    if nd not in (2, 3) or dy.dim() != x.dim():
        raise ValueError("x must be N[D]HWC and dy N[Do]HoWoK")
    if not (x.is_contiguous() and dy.is_contiguous()):
        raise ValueError("x and dy must be contiguous")
    if dy.dtype != x.dtype:
        raise TypeError("x and dy must share one dtype")
    stride = stride or (1,) * nd
    pad = pad or (0,) * nd
    dil = dil or (1,) * nd
    N, C, K = x.shape[0], x.shape[-1], dy.shape[-1]
    d = make_desc(nd, _torch_dtype_code(x), N, groups, C, K, tuple(x.shape[1:-1]), tuple(filt),
                  stride, pad, dil)
    o = gconv_out_dims(d)
    if tuple(dy.shape[1:-1]) != (o if nd == 3 else o[1:]) or dy.shape[0] != N:
        raise ValueError("dy's shape %r is not the forward output" % (tuple(dy.shape),))
    wshape = (K,) + tuple(filt) + (C // groups,)
    if out is None:
        out = torch.empty(wshape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != wshape or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError("out must be a contiguous %s tensor of shape %s" % (x.dtype, wshape))
    s = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
    ws_ptr, ws_bytes = None, 0
    if use_workspace:
        need = gconv_bwd_weight_workspace(d)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        if workspace is not None:
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = gconv_bwd_weight(d, x.data_ptr(), dy.data_ptr(), out.data_ptr(), ws_ptr, ws_bytes, s)
    if rc != GCONV_OK:
        raise GconvError(rc, "gconv_bwd_weight")
    return out

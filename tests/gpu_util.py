"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP library through its C ABI, and compare with the oracle to the tolerance
of the grouped-conv forward contract:

    fp32:       |y_gpu - y| <= 1e-5 * scale
    fp16/bf16:  |y_gpu - y| <= 4e-3 * scale + 1e-6

where y is the oracle's unrounded fp64 result and scale = sum |x*w| (+ |bias|)
over the taps of that output.
"""
from __future__ import annotations

import numpy as np
import torch

from depthwise_convolution_grouped_amd import gconv as G
from depthwise_convolution_grouped_amd import inputs

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def tolerance(scale: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return 1e-5 * scale
    return 4e-3 * scale + 1e-6


def to_device(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def device_tensors(p: inputs.Problem, t: inputs.Tensors):
    x = to_device(t.x, p.dtype)
    w = to_device(t.w, p.dtype)
    b = to_device(t.bias, p.dtype) if t.bias is not None else None
    return x, w, b


def run(p: inputs.Problem, x, w, b, path=G.GCONV_PATH_AUTO, out=None, stream=None):
    st, pd, dl = p.spatial_args()
    y = G.conv_fwd(x, w, b, groups=p.G, stride=st, pad=pd, dil=dl, out=out, path=path,
                   stream=stream)
    return y


def oracle_inputs(p: inputs.Problem, t: inputs.Tensors):
    x = inputs.storage_to_f64(t.x, p.dtype)
    w = inputs.storage_to_f64(t.w, p.dtype)
    b = inputs.storage_to_f64(t.bias, p.dtype) if t.bias is not None else None
    return x, w, b


def check(y_gpu: np.ndarray, y_ref: np.ndarray, scale: np.ndarray, dtype: str, what: str) -> float:
    """Assert parity element by element; returns max |err| / tol."""
    assert y_gpu.shape == y_ref.shape, (what, y_gpu.shape, y_ref.shape)
    tol = tolerance(scale, dtype)
    err = np.abs(y_gpu - y_ref)
    ok = err <= tol          # False for NaN
    if not ok.all():
        bad = np.argwhere(~ok)
        lines = []
        for idx in bad[:8]:
            i = tuple(idx)
            lines.append("  at %s: gpu=%r ref=%r tol=%r" % (i, y_gpu[i], y_ref[i], tol[i]))
        raise AssertionError("%s: %d of %d outputs out of tolerance\n%s"
                             % (what, len(bad), y_ref.size, "\n".join(lines)))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(tol > 0, err / tol, 0.0)
    return float(r.max()) if r.size else 0.0

"""GPU parity of backward data (gconv_bwd_data, gconv_bwd_data_direct) against
the oracle's fp64 gradient, through the C ABI, to the tolerance of the
forward contract with scale = sum |dy * w| over the terms of each dx element:

    fp32:       |dx_gpu - dx| <= 1e-5 * scale
    fp16/bf16:  |dx_gpu - dx| <= 4e-3 * scale + 1e-6

Both routes are checked on every case: the workspace route (at stride 1 a
weight transform and the forward dispatcher on the transposed problem; at
larger strides, for groups other than depthwise, one stride-1 forward launch
per residue class of dx on its reversed sub-kernel, scattered into dx) and
the direct kernel.  Inputs are seeded and synthetic: w as the forward
workloads draw it, dy ~ N(0, 1).
"""
import numpy as np
import pytest
import torch

import oracle
from depthwise_convolution_grouped_amd import gconv as G
from depthwise_convolution_grouped_amd import inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()


def dy_shape(p):
    o = [oracle.out_extent(p.spatial[a], p.filt[a], p.stride[a], p.pad[a], p.dil[a]) for a in range(3)]
    return (p.N,) + (tuple(o) if p.ndim == 3 else tuple(o[1:])) + (p.K,)


def run_case(p, seed, what):
    t = inputs.make_tensors(p, seed)
    dy_s = inputs.make_array(dy_shape(p), p.dtype, seed + 5)
    st, pd, dl = p.spatial_args()
    in_sp = p.x_shape()[1:-1]
    dy64 = inputs.storage_to_f64(dy_s, p.dtype)
    w64 = inputs.storage_to_f64(t.w, p.dtype)
    ref, scale = oracle.conv_bwd_data(dy64, w64, p.G, in_sp, st, pd, dl)
    dy = U.to_device(dy_s, p.dtype)
    w = U.to_device(t.w, p.dtype)
    ratios = {}
    for direct in (False, True):
        out = torch.full(p.x_shape(), float("nan"), dtype=U.TORCH_DTYPE[p.dtype], device="cuda")
        G.conv_bwd_data(dy, w, p.G, in_sp, st, pd, dl, out=out, direct=direct)
        torch.cuda.synchronize()
        ratios[direct] = U.check(U.to_f64(out), ref, scale, p.dtype,
                                 "%s %s" % (what, "direct" if direct else "auto"))
    print("%s max err/tol auto %.3f direct %.3f" % (what, ratios[False], ratios[True]))


CASES = [
    # (ndim, dtype, N, G, C, K, spatial, filt, stride, pad, dil)
    (2, "f16", 2, 16, 16, 16, (13, 17), (3, 3), 1, 1, 1),       # depthwise, stride 1
    (2, "f16", 2, 16, 16, 16, (13, 17), (3, 3), 2, 1, 1),       # depthwise, stride 2
    (2, "bf16", 1, 8, 64, 64, (9, 11), (3, 3), 1, 1, 1),        # ResNeXt-like small groups
    (2, "bf16", 1, 2, 256, 256, (7, 7), (3, 3), 1, 1, 1),       # large groups
    (2, "bf16", 1, 2, 256, 256, (7, 7), (3, 3), 1, 2, 2),       # large groups, dilation 2
    (2, "f32", 1, 2, 64, 64, (8, 8), (3, 3), 1, 1, 1),          # fp32 grouped
    (3, "f16", 1, 8, 16, 32, (4, 7, 9), (3, 3, 3), 1, 1, 1),    # 3D grouped, 2 in / 4 out
    (3, "f16", 2, 4, 8, 12, (5, 6, 7), (3, 3, 3), 2, 1, 1),     # 3D, stride 2
    (2, "bf16", 2, 3, 6, 9, (10, 9), (5, 3), 1, (2, 1), 1),     # 5x3 window, C != K
    (2, "f16", 1, 1, 8, 8, (9, 9), (3, 3), 1, 3, 1),            # pad beyond the filter: direct only
    (2, "bf16", 1, 4, 32, 64, (12, 10), (1, 1), 1, 0, 1),       # 1x1
    (2, "f32", 3, 5, 15, 10, (7, 8), (3, 2), (2, 1), (1, 0), (1, 2)),   # mixed strides and dilations
    (2, "f32", 2, 12, 12, 12, (11, 10), (3, 3), 2, 1, 2),       # depthwise fp32, channel vectors of 4
    (3, "bf16", 1, 24, 24, 24, (5, 9, 8), (3, 3, 3), 2, 1, 1),  # depthwise 3D stride 2, vectors of 8
    (2, "f16", 1, 20, 20, 20, (9, 9), (3, 3), 2, 1, 1),         # depthwise, C not a multiple of 8: scalar
    # depthwise 3x3 stride 2 on 2 x 2 dx blocks: both pad parities per axis, odd extents
    (2, "f16", 2, 24, 24, 24, (12, 16), (3, 3), 2, 0, 1),       # pad 0, even extents
    (2, "bf16", 1, 16, 16, 16, (15, 9), (3, 3), 2, 2, 1),       # pad 2, odd extents (half blocks)
    (2, "f32", 2, 8, 8, 8, (10, 7), (3, 3), 2, (3, 0), 1),      # pad 3 rows (past the window), 0 columns
    (2, "bf16", 3, 40, 40, 40, (5, 6), (3, 3), 2, (0, 1), 1),   # mixed parities, tiny image
    # strided, grouped: residue classes of dx on the forward kernels
    (2, "bf16", 2, 4, 512, 512, (14, 13), (3, 3), 2, 1, 1),     # large groups: the classes on the halo / M-tiled GEMMs
    (2, "bf16", 2, 32, 256, 256, (15, 14), (3, 3), 2, 1, 1),    # ResNeXt-like 8/8 groups, stride 2
    (2, "bf16", 1, 8, 64, 64, (13, 11), (3, 3), 2, 2, 2),       # stride 2 with dilation 2: one class per axis takes every tap
    (2, "f16", 1, 2, 32, 32, (17, 15), (3, 3), 4, 0, 1),        # stride 4 > window: classes no tap reaches are zero
    (2, "f16", 2, 8, 128, 64, (12, 13), (5, 5), 3, 2, 1),       # stride 3, 5x5
    (3, "bf16", 1, 4, 64, 128, (5, 7, 6), (3, 3, 3), 2, 1, 1),  # 3D stride 2: 8 classes
]


def problem(case):
    nd, dt, N, Gr, C, K, sp, fl, s, pd, dl = case
    tr = lambda v, n: v if isinstance(v, tuple) else (v,) * n
    st, pa, di = tr(s, nd), tr(pd, nd), tr(dl, nd)
    if nd == 2:
        return inputs.Problem(2, dt, N, Gr, C, K, (1,) + sp, (1,) + fl, (1,) + st, (0,) + pa, (1,) + di, False)
    return inputs.Problem(3, dt, N, Gr, C, K, sp, fl, st, pa, di, False)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bwd_data_shapes(case):
    run_case(problem(CASES[case]), 8000 + 10 * case, "bwd_data %r" % (CASES[case],))


SWEEP = [(dt, nd, i) for dt in ("f32", "f16", "bf16") for nd in (2, 3) for i in range(6)]


@pytest.mark.parametrize("case", range(len(SWEEP)), ids=["%s-%dd-%d" % c for c in SWEEP])
def test_bwd_data_random_small(case):
    dt, nd, i = SWEEP[case]
    rng = np.random.default_rng(8500 + case)
    p = inputs.random_problem(rng, dt, nd)
    p = inputs.Problem(p.ndim, p.dtype, p.N, p.G, p.C, p.K, p.spatial, p.filt, p.stride, p.pad, p.dil, False)
    run_case(p, 8600 + 10 * case, "bwd_data random %s" % (p,))


@pytest.mark.parametrize("name,N", [("depthwise2d_f16", 2), ("depthwise2d_s2_f16", 2), ("grouped2d_resnext_bf16", 1),
                                    ("grouped3d_f16_n1", 1), ("grouped2d_large_bf16", 1)])
def test_bwd_data_reduced_workloads(name, N):
    wl = inputs.WORKLOADS[name].problem
    p = inputs.Problem(wl.ndim, wl.dtype, N, wl.G, wl.C, wl.K, wl.spatial, wl.filt, wl.stride, wl.pad,
                       wl.dil, False)
    run_case(p, 8900, "bwd_data %s N=%d" % (name, N))


def test_bwd_data_deterministic():
    p = problem(CASES[2])
    t = inputs.make_tensors(p, 9100)
    dy = U.to_device(inputs.make_array(dy_shape(p), p.dtype, 9105), p.dtype)
    w = U.to_device(t.w, p.dtype)
    st, pd, dl = p.spatial_args()
    a = G.conv_bwd_data(dy, w, p.G, p.x_shape()[1:-1], st, pd, dl)
    b = G.conv_bwd_data(dy, w, p.G, p.x_shape()[1:-1], st, pd, dl)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))

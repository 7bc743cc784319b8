"""GPU parity of backward weight (gconv_bwd_weight) against the oracle's fp64
gradient, through the C ABI, to the tolerance of the forward contract with
scale = sum |dy * x| over the terms of each dw element:

    fp32:       |dw_gpu - dw| <= 1e-5 * scale
    fp16/bf16:  |dw_gpu - dw| <= 4e-3 * scale + 1e-6

Every case runs three ways: with the full partial-sum workspace (two-stage
reduction), with room for only a few chunks, and with no workspace (one
chunk, one kernel).  Inputs are seeded and synthetic: x as the forward
workloads draw it, dy ~ N(0, 1).
"""
import numpy as np
import pytest
import torch

import oracle
from depthwise_convolution_grouped_amd import gconv as G
from depthwise_convolution_grouped_amd import inputs
from tests import gpu_util as U
from tests.test_gpu_bwd_data import CASES, dy_shape, problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()


def run_case(p, seed, what):
    t = inputs.make_tensors(p, seed)
    dy_s = inputs.make_array(dy_shape(p), p.dtype, seed + 5)
    st, pd, dl = p.spatial_args()
    filt = p.w_shape()[1:-1]
    x64 = inputs.storage_to_f64(t.x, p.dtype)
    dy64 = inputs.storage_to_f64(dy_s, p.dtype)
    ref, scale = oracle.conv_bwd_weight(x64, dy64, p.G, filt, st, pd, dl)
    x = U.to_device(t.x, p.dtype)
    dy = U.to_device(dy_s, p.dtype)
    d = G.desc_from_problem(p)
    need = G.gconv_bwd_weight_workspace(d)
    ratios = []
    for mode in ("full", "small", "none"):
        out = torch.full(p.w_shape(), float("nan"), dtype=U.TORCH_DTYPE[p.dtype], device="cuda")
        if mode == "full":
            G.conv_bwd_weight(x, dy, p.G, filt, st, pd, dl, out=out)
        elif mode == "small":
            ws = torch.empty(max(need // 7, 4), dtype=torch.uint8, device="cuda")
            G.conv_bwd_weight(x, dy, p.G, filt, st, pd, dl, out=out, workspace=ws)
        else:
            G.conv_bwd_weight(x, dy, p.G, filt, st, pd, dl, out=out, use_workspace=False)
        torch.cuda.synchronize()
        ratios.append(U.check(U.to_f64(out), ref, scale, p.dtype, "%s %s" % (what, mode)))
    print("%s workspace %d B, max err/tol full %.3f small %.3f none %.3f" % (what, need, *ratios))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bwd_weight_shapes(case):
    run_case(problem(CASES[case]), 9300 + 10 * case, "bwd_weight %r" % (CASES[case],))


SWEEP = [(dt, nd, i) for dt in ("f32", "f16", "bf16") for nd in (2, 3) for i in range(5)]


@pytest.mark.parametrize("case", range(len(SWEEP)), ids=["%s-%dd-%d" % c for c in SWEEP])
def test_bwd_weight_random_small(case):
    dt, nd, i = SWEEP[case]
    rng = np.random.default_rng(9500 + case)
    p = inputs.random_problem(rng, dt, nd)
    p = inputs.Problem(p.ndim, p.dtype, p.N, p.G, p.C, p.K, p.spatial, p.filt, p.stride, p.pad, p.dil, False)
    run_case(p, 9600 + 10 * case, "bwd_weight random %s" % (p,))


@pytest.mark.parametrize("name,N", [("depthwise2d_f16", 2), ("depthwise2d_s2_f16", 2), ("grouped2d_resnext_bf16", 1),
                                    ("grouped3d_f16_n1", 1)])
def test_bwd_weight_reduced_workloads(name, N):
    wl = inputs.WORKLOADS[name].problem
    p = inputs.Problem(wl.ndim, wl.dtype, N, wl.G, wl.C, wl.K, wl.spatial, wl.filt, wl.stride, wl.pad,
                       wl.dil, False)
    run_case(p, 9900, "bwd_weight %s N=%d" % (name, N))


def test_bwd_weight_deterministic():
    p = problem(CASES[2])
    t = inputs.make_tensors(p, 9910)
    x = U.to_device(t.x, p.dtype)
    dy = U.to_device(inputs.make_array(dy_shape(p), p.dtype, 9915), p.dtype)
    st, pd, dl = p.spatial_args()
    filt = p.w_shape()[1:-1]
    a = G.conv_bwd_weight(x, dy, p.G, filt, st, pd, dl)
    b = G.conv_bwd_weight(x, dy, p.G, filt, st, pd, dl)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))

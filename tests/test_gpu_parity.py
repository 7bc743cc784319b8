"""GPU parity of the HIP library (called through its C ABI) against the oracle.

* every workload at full size: element by element where the oracle finishes
  in seconds, else at sampled outputs (random positions plus every corner);
* reduced-batch versions of the large workloads element by element;
* every kernel path forced on shapes it can take, including random small
  2D/3D problems with odd channel counts, strides, paddings and dilations,
  and every tile of each path's menu on the workloads and on group widths
  off the 32-channel grid;
* output poisoned with NaN before the call (every element must be written),
  canary elements after y (nothing written past the end), bitwise run-to-run
  determinism, and a non-default stream.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from depthwise_convolution_grouped_amd import gconv as G
from depthwise_convolution_grouped_amd import inputs, metrics
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()   # fail loudly if the library is missing


def poisoned_out(p):
    shape = (p.N,) + (metrics.out_spatial(p) if p.ndim == 3 else metrics.out_spatial(p)[1:]) + (p.K,)
    return torch.full(shape, float("nan"), dtype=U.TORCH_DTYPE[p.dtype], device="cuda")


def run_and_fetch(p, t, path=G.GCONV_PATH_AUTO):
    x, w, b = U.device_tensors(p, t)
    y = U.run(p, x, w, b, path=path, out=poisoned_out(p))
    torch.cuda.synchronize()
    return U.to_f64(y)


def reduced(p: inputs.Problem, N: int) -> inputs.Problem:
    return inputs.Problem(p.ndim, p.dtype, N, p.G, p.C, p.K, p.spatial, p.filt, p.stride,
                          p.pad, p.dil, p.bias)


FULL = ["grouped2d_small_f32", "depthwise2d_f16", "depthwise2d_s2_f16",
        "grouped3d_f16_n1", "grouped3d_f16_n8"]
SAMPLED = ["grouped2d_resnext_bf16", "grouped2d_large_bf16", "grouped2d_large_dil2_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_elementwise(name):
    wl = inputs.WORKLOADS[name]
    p, t = wl.problem, inputs.workload_tensors(wl)
    y = run_and_fetch(p, t)
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    r = U.check(y, ref, scale, p.dtype, name)
    print("%s path=%s max err/tol=%.3f" % (name, G.gconv_path_name(G.gconv_select_path(G.desc_from_problem(p))), r))


def corner_indices(p):
    Do, Ho, Wo = metrics.out_spatial(p)
    dims = (p.N, Do, Ho, Wo, p.K)
    idx = []
    for n, od, oh, ow, k in itertools.product({0, p.N - 1}, {0, Do - 1}, {0, Ho - 1}, {0, Wo - 1},
                                             {0, p.Kpg - 1, p.K - p.Kpg, p.K - 1}):
        idx.append(np.ravel_multi_index((n, od, oh, ow, k), dims))
    return np.array(sorted(set(idx)), dtype=np.int64)


@pytest.mark.parametrize("name", SAMPLED)
def test_workload_full_sampled(name):
    wl = inputs.WORKLOADS[name]
    p, t = wl.problem, inputs.workload_tensors(wl)
    y = run_and_fetch(p, t)
    assert np.isfinite(y).all(), "some outputs were not written"
    total = y.size
    rng = np.random.default_rng(wl.seed + 5)
    idx = np.unique(np.concatenate([rng.integers(0, total, 6000), corner_indices(p)]))
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd_points(*U.oracle_inputs(p, t), p.G, st, pd, dl, idx)
    r = U.check(y.reshape(-1)[idx], ref, scale, p.dtype, name)
    print("%s sampled %d max err/tol=%.3f" % (name, idx.size, r))


REDUCED = [("grouped2d_resnext_bf16", 2), ("grouped2d_large_bf16", 2),
           ("grouped2d_large_dil2_bf16", 1), ("depthwise2d_f16", 3), ("depthwise2d_s2_f16", 3),
           ("grouped3d_f16_n8", 2), ("grouped2d_small_f32", 1)]


@pytest.mark.parametrize("name,N", REDUCED)
@pytest.mark.parametrize("path", list(G.PATHS))
def test_reduced_workload_every_path(name, N, path):
    wl = inputs.WORKLOADS[name]
    p = reduced(wl.problem, N)
    d = G.desc_from_problem(p)
    pid = G.PATHS[path]
    if G.gconv_path_supported(d, pid) != 1:
        pytest.skip("%s cannot run %s" % (path, name))
    t = inputs.make_tensors(p, wl.seed + 7, wl.x_dist, wl.w_dist, wl.b_dist)
    y = run_and_fetch(p, t, pid)
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    r = U.check(y, ref, scale, p.dtype, "%s N=%d path=%s" % (name, N, path))
    print("%s N=%d path=%s max err/tol=%.3f" % (name, N, path, r))


def sweep_cases():
    cases = []
    for dtype, ndim in itertools.product(["f32", "f16", "bf16"], [2, 3]):
        rng = np.random.default_rng({"f32": 1, "f16": 2, "bf16": 3}[dtype] * 10 + ndim)
        for i in range(12):
            cases.append((dtype, ndim, i, inputs.random_problem(rng, dtype, ndim)))
    return cases


SWEEP = sweep_cases()


@pytest.mark.parametrize("case", range(len(SWEEP)),
                         ids=["%s-%dd-%d" % c[:3] for c in SWEEP])
def test_random_small_every_path(case):
    dtype, ndim, i, p = SWEEP[case]
    t = inputs.make_tensors(p, 90000 + case)
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    d = G.desc_from_problem(p)
    ran = []
    for path, pid in G.PATHS.items():
        if G.gconv_path_supported(d, pid) != 1:
            continue
        y = run_and_fetch(p, t, pid)
        U.check(y, ref, scale, p.dtype, "%s path=%s" % (p, path))
        ran.append(path)
    assert "generic" in ran


@pytest.mark.parametrize("name", ["depthwise2d_f16", "grouped2d_resnext_bf16", "grouped3d_f16_n1",
                                  "grouped2d_large_bf16", "grouped2d_small_f32"])
def test_deterministic_and_no_overrun(name):
    wl = inputs.WORKLOADS[name]
    p = wl.problem if name != "grouped2d_resnext_bf16" else reduced(wl.problem, 4)
    t = inputs.workload_tensors(wl) if p is wl.problem else inputs.make_tensors(p, wl.seed, wl.x_dist, wl.w_dist)
    x, w, b = U.device_tensors(p, t)
    shape = tuple(poisoned_out(p).shape)
    n = int(np.prod(shape))
    canary = 4096
    buf = torch.full((n + canary,), 7.0, dtype=U.TORCH_DTYPE[p.dtype], device="cuda")
    y1 = U.run(p, x, w, b, out=buf[:n].view(shape))
    torch.cuda.synchronize()
    first = y1.clone()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y2 = U.run(p, x, w, b, out=buf[:n].view(shape), stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(first.view(torch.int16 if p.dtype != "f32" else torch.int32),
                       y2.view(torch.int16 if p.dtype != "f32" else torch.int32)), "not bitwise deterministic"
    assert torch.all(buf[n:] == 7.0).item(), "kernel wrote past the end of y"


@pytest.mark.parametrize("name", ["depthwise2d_f16", "grouped3d_f16_n1"])
def test_timed_entry_matches_and_times_the_kernel(name):
    """gconv_fwd_timed writes the same bits as gconv_fwd_path and its events
    span the kernel (positive, and within the stream time around it)."""
    import ctypes
    wl = inputs.WORKLOADS[name]
    p = wl.problem
    t = inputs.workload_tensors(wl)
    x, w, b = U.device_tensors(p, t)
    y_ref = U.run(p, x, w, b, out=poisoned_out(p))
    y = poisoned_out(p)
    d = G.desc_from_problem(p)
    path = G.gconv_select_path(d)
    hip = ctypes.CDLL(next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64.so" in l))
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    s = torch.cuda.current_stream()
    outer0 = torch.cuda.Event(enable_timing=True)
    outer1 = torch.cuda.Event(enable_timing=True)
    outer0.record(s)
    rc = G.gconv_fwd_timed(d, path, x.data_ptr(), w.data_ptr(), b.data_ptr() if b is not None else None,
                           y.data_ptr(), s.cuda_stream, ev[0].value, ev[1].value)
    outer1.record(s)
    assert rc == G.GCONV_OK
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    for e in ev:
        hip.hipEventDestroy(e)
    assert 0.0 < ms.value <= outer0.elapsed_time(outer1) + 1e-3
    iv = torch.int16 if p.dtype != "f32" else torch.int32
    assert torch.equal(y.view(iv), y_ref.view(iv))


def test_misaligned_falls_back_or_errors():
    p = reduced(inputs.WORKLOADS["depthwise2d_f16"].problem, 1)
    t = inputs.make_tensors(p, 123)
    x, w, b = U.device_tensors(p, t)
    # x shifted by one element: 2-byte aligned, not 16-byte aligned
    xs = torch.empty(x.numel() + 1, dtype=x.dtype, device="cuda")
    xs[1:].copy_(x.view(-1))
    xv = xs[1:].view(x.shape)
    y = U.run(p, xv, w, b, out=poisoned_out(p))       # auto: falls back to a path that accepts it
    torch.cuda.synchronize()
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    U.check(U.to_f64(y), ref, scale, p.dtype, "misaligned x")
    d = G.desc_from_problem(p)
    sel = G.gconv_select_path(d)
    if sel != G.GCONV_PATH_GENERIC:
        rc = G.gconv_fwd_path(d, sel, xv.data_ptr(), w.data_ptr(), b.data_ptr(), y.data_ptr(), 0)
        assert rc == G.GCONV_ERR_MISALIGNED


DW_CASES = [
    # dtype, N, C, H, W, stride, pad, dil
    ("f16", 1, 8, 5, 7, 1, 1, 1),
    ("f16", 2, 24, 17, 13, 2, 1, 1),
    ("bf16", 1, 40, 9, 31, 1, 2, 2),
    ("bf16", 3, 144, 11, 57, 2, 1, 2),
    ("f32", 2, 12, 19, 23, 1, 0, 1),
    ("f32", 1, 100, 6, 6, 2, 2, 1),
    ("f16", 1, 520, 7, 9, 1, 1, 1),     # more channel vectors than one slab holds
    ("bf16", 2, 264, 30, 3, 1, 1, 2),
    ("f16", 1, 16, 64, 1, 1, 1, 1),     # one column
    ("f16", 1, 16, 1, 64, 2, 1, 1),     # one row
    ("f16", 1, 1024, 82, 82, 1, 1, 1),  # 14-row runs
    ("bf16", 1, 1024, 118, 118, 1, 2, 2),  # 28-row runs, dilation 2
    ("f32", 1, 512, 164, 164, 2, 1, 1),  # 14-row runs at stride 2
]


@pytest.mark.parametrize("case", range(len(DW_CASES)))
def test_depthwise_shapes(case):
    dtype, N, C, H, W, s, pd, dl = DW_CASES[case]
    p = inputs.conv2d(dtype, N=N, G=C, C=C, K=C, H=H, W=W, Y=3, X=3, stride=s, pad=pd, dil=dl,
                      bias=case % 2 == 0)
    d = G.desc_from_problem(p)
    assert G.gconv_path_supported(d, G.GCONV_PATH_DEPTHWISE) == 1, "depthwise path should take %r" % (p,)
    t = inputs.make_tensors(p, 5000 + case)
    st, pad, dil = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pad, dil)
    y = run_and_fetch(p, t, G.GCONV_PATH_DEPTHWISE)
    U.check(y, ref, scale, p.dtype, "depthwise %r" % (DW_CASES[case],))


SMALLG_CASES = [
    # ndim, dtype, N, G, Cpg, Kpg, spatial (D,H,W), filt (Z,Y,X), stride, pad, dil, bias
    (2, "bf16", 2, 32, 8, 8, (1, 13, 17), (1, 3, 3), 1, 1, 1, False),   # ResNeXt-like, ragged tiles
    (3, "f16", 2, 32, 4, 2, (5, 9, 11), (3, 3, 3), 1, 1, 1, True),     # 27 x 4 K slices: the 28-fragment instance
    (3, "bf16", 1, 16, 4, 2, (4, 7, 6), (3, 3, 3), 1, 1, 1, False),
    (2, "f16", 1, 8, 8, 8, (1, 9, 30), (1, 3, 3), 2, 1, 1, True),
    (2, "bf16", 1, 16, 4, 4, (1, 11, 11), (1, 3, 3), 1, 2, 2, True),     # dilation 2
    (2, "f16", 2, 4, 16, 16, (1, 7, 9), (1, 3, 3), 1, 1, 1, True),      # one group per tile
    (2, "bf16", 1, 16, 4, 8, (1, 6, 40), (1, 5, 5), 1, 2, 1, True),     # 5x5
    (2, "f16", 1, 64, 1, 2, (1, 10, 10), (1, 3, 3), 1, 1, 1, False),    # 8 groups per tile
    (3, "f16", 1, 32, 2, 4, (8, 28, 28), (3, 3, 3), 1, 1, 1, True),     # the 3D workload at N=1
    (3, "bf16", 2, 8, 2, 4, (5, 7, 9), (3, 3, 3), 1, 1, 1, True),
    (3, "f16", 1, 16, 4, 4, (6, 5, 7), (3, 3, 3), 2, 1, 1, True),       # 14 MFMAs per tile
    (2, "bf16", 2, 32, 4, 2, (1, 20, 21), (1, 3, 3), 1, 1, 1, True),    # ring tiles of 4 chunks (32 in / 16 out)
    (3, "f16", 16, 32, 4, 2, (8, 14, 14), (3, 3, 3), 1, 1, 1, False),   # the same in 3D (the 3D N=8 shape transposed)
    (3, "bf16", 1, 8, 8, 8, (4, 6, 6), (3, 1, 3), 1, (1, 0, 1), 1, False),
    (3, "f16", 1, 4, 4, 4, (7, 7, 7), (3, 3, 3), 1, 2, 2, True),
]


@pytest.mark.parametrize("case", range(len(SMALLG_CASES)))
def test_smallg_shapes(case):
    nd, dt, N, Gr, Cpg, Kpg, sp, fl, s, pd, dl, bias = SMALLG_CASES[case]
    pad = pd if isinstance(pd, tuple) else (pd, pd, pd)
    if nd == 2:
        pad = (0, pad[1], pad[2])
    p = inputs.Problem(nd, dt, N, Gr, Gr * Cpg, Gr * Kpg, sp, fl,
                       (1, s, s) if nd == 2 else (s, s, s), pad,
                       (1, dl, dl) if nd == 2 else (dl, dl, dl), bias)
    d = G.desc_from_problem(p)
    assert G.gconv_path_supported(d, G.GCONV_PATH_SMALLG) == 1, "small-group path should take %r" % (p,)
    t = inputs.make_tensors(p, 6000 + case)
    st, pa, di = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pa, di)
    y = run_and_fetch(p, t, G.GCONV_PATH_SMALLG)
    r = U.check(y, ref, scale, p.dtype, "smallg %r" % (SMALLG_CASES[case],))
    print("smallg case %d max err/tol %.3f plan %s" % (case, r, G.gconv_get_plan(d, G.GCONV_PATH_SMALLG)))


IGEMM_CASES = [
    # ndim, dtype, N, G, Cpg, Kpg, spatial (D,H,W), filt (Z,Y,X), stride, pad, dil, bias
    (2, "bf16", 1, 2, 128, 128, (1, 14, 14), (1, 3, 3), 1, 1, 1, True),     # the large-group case, small batch
    (2, "bf16", 1, 2, 128, 128, (1, 14, 14), (1, 3, 3), 1, 2, 2, True),     # its dilation-2 variant
    (2, "f16", 2, 3, 64, 64, (1, 9, 11), (1, 3, 3), 2, 1, 1, False),        # stride 2, ragged M
    (2, "bf16", 1, 1, 32, 192, (1, 7, 13), (1, 1, 1), 1, 0, 1, True),       # 1x1, KT=32, BN=64 tiles
    (2, "f16", 1, 4, 96, 64, (1, 10, 10), (1, 5, 3), 1, (0, 2, 1), 1, True),  # 5x3 filter, Cpg=96
    (3, "bf16", 1, 2, 64, 128, (4, 6, 7), (3, 3, 3), 1, 1, 1, True),
    (3, "f16", 2, 2, 32, 64, (5, 5, 5), (3, 1, 3), (2, 1, 1), 1, (1, 2, 1), False),
    (2, "bf16", 8, 2, 128, 128, (1, 14, 14), (1, 3, 3), 1, 1, 1, True),     # 16 items, XCD-split ranges
    (2, "f16", 33, 8, 64, 64, (1, 14, 14), (1, 3, 3), 1, 1, 1, True),       # 264 items: some workgroups take 2
    (2, "bf16", 1, 1, 64, 64, (1, 30, 29), (1, 3, 3), 1, 1, 1, True),       # row blocks, ragged last block
    (2, "bf16", 1, 1, 64, 128, (1, 3, 300), (1, 3, 3), 1, 1, 1, False),     # column blocks (Wo > 224)
    (2, "f16", 2, 1, 256, 256, (1, 6, 6), (1, 3, 3), 1, 1, 1, True),        # 4 channel chunks, 2 channel blocks
    (2, "f16", 70, 8, 64, 64, (1, 14, 14), (1, 3, 3), 1, 1, 1, True),       # 560 items: next box loads under the stores
    (3, "bf16", 1, 2, 128, 64, (5, 6, 7), (3, 3, 3), 1, 1, (2, 1, 1), True),  # depth dilation, one workgroup per CU
    (2, "bf16", 3, 2, 128, 128, (1, 17, 15), (1, 3, 3), 2, 1, 1, False),    # stride 2, whole-box variant
    (2, "bf16", 1, 2, 192, 64, (1, 9, 10), (1, 3, 3), 1, 1, 1, True),       # three 64-channel box chunks
    (3, "f16", 1, 1, 256, 128, (3, 5, 6), (3, 3, 3), 1, 1, 1, True),        # two 128-channel chunks, 3D
    (2, "bf16", 2, 4, 128, 128, (1, 14, 14), (1, 3, 3), 1, 2, 2, True),     # dilation 2: two 64-channel chunks
]


@pytest.mark.parametrize("path", ["igemm_mfma", "ighalo_mfma"])
@pytest.mark.parametrize("case", range(len(IGEMM_CASES)))
def test_igemm_shapes(case, path):
    nd, dt, N, Gr, Cpg, Kpg, sp, fl, s, pd, dl, bias = IGEMM_CASES[case]
    tr = lambda v, fill: (v if isinstance(v, tuple) else (v, v, v))
    st, pad, dil = tr(s, 1), tr(pd, 0), tr(dl, 1)
    if nd == 2:
        st, pad, dil = (1, st[1], st[2]), (0, pad[1], pad[2]), (1, dil[1], dil[2])
    p = inputs.Problem(nd, dt, N, Gr, Gr * Cpg, Gr * Kpg, sp, fl, st, pad, dil, bias)
    d = G.desc_from_problem(p)
    pid = G.PATHS[path]
    assert G.gconv_path_supported(d, pid) == 1, "%s should take %r" % (path, p)
    t = inputs.make_tensors(p, 7000 + case)
    sa, pa, da = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, sa, pa, da)
    y = run_and_fetch(p, t, pid)
    r = U.check(y, ref, scale, p.dtype, "%s %r" % (path, IGEMM_CASES[case]))
    print("%s case %d max err/tol %.3f plan %s" % (path, case, r, G.gconv_get_plan(d, pid)))


@pytest.mark.parametrize("case", range(len(IGEMM_CASES)))
def test_halo_every_variant(case):
    """Every variant of the halo implicit GEMM's menu (whole box, chunk
    streaming, warp-specialised whole box) that takes the shape matches the
    oracle element by element."""
    nd, dt, N, Gr, Cpg, Kpg, sp, fl, s, pd, dl, bias = IGEMM_CASES[case]
    tr = lambda v: (v if isinstance(v, tuple) else (v, v, v))
    st, pad, dil = tr(s), tr(pd), tr(dl)
    if nd == 2:
        st, pad, dil = (1, st[1], st[2]), (0, pad[1], pad[2]), (1, dil[1], dil[2])
    p = inputs.Problem(nd, dt, N, Gr, Gr * Cpg, Gr * Kpg, sp, fl, st, pad, dil, bias)
    d = G.desc_from_problem(p)
    if G.gconv_path_supported(d, G.GCONV_PATH_IGHALO) != 1:
        pytest.skip("the halo path does not take this shape")
    t = inputs.make_tensors(p, 7000 + case)
    sa, pa, da = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, sa, pa, da)
    x, w, b = U.device_tensors(p, t)
    n, _ = G.gconv_tile_count(d, G.GCONV_PATH_IGHALO)
    for tile in range(n):
        y = poisoned_out(p)
        rc = G.gconv_fwd_tile(d, G.GCONV_PATH_IGHALO, tile, x.data_ptr(), w.data_ptr(),
                              b.data_ptr() if b is not None else None, y.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0, G.gconv_status_str(rc)
        torch.cuda.synchronize()
        r = U.check(U.to_f64(y), ref, scale, p.dtype, "halo case %d tile %d" % (case, tile))
        print("halo case %d tile %d/%d max err/tol %.3f" % (case, tile, n, r))


IGEMM_ONLY_CASES = [
    # groups of 32 output channels: only the M-tiled implicit GEMM takes them (32-channel tiles)
    (2, "bf16", 4, 8, 32, 32, (1, 28, 28), (1, 3, 3), 1, 1, 1, True),
    (2, "f16", 2, 3, 64, 96, (1, 13, 11), (1, 3, 3), 2, 1, 1, False),      # Kpg = 96: three 32-channel tiles
    (3, "bf16", 1, 2, 32, 32, (4, 6, 7), (3, 3, 3), 1, 1, (1, 2, 1), True),
]


@pytest.mark.parametrize("case", range(len(IGEMM_ONLY_CASES)))
def test_igemm_32_channel_tiles(case):
    nd, dt, N, Gr, Cpg, Kpg, sp, fl, s, pd, dl, bias = IGEMM_ONLY_CASES[case]
    tr = lambda v: (v if isinstance(v, tuple) else (v, v, v))
    st, pad, dil = tr(s), tr(pd), tr(dl)
    if nd == 2:
        st, pad, dil = (1, st[1], st[2]), (0, pad[1], pad[2]), (1, dil[1], dil[2])
    p = inputs.Problem(nd, dt, N, Gr, Gr * Cpg, Gr * Kpg, sp, fl, st, pad, dil, bias)
    d = G.desc_from_problem(p)
    assert G.gconv_select_path(d) == G.GCONV_PATH_IGEMM
    t = inputs.make_tensors(p, 7500 + case)
    sa, pa, da = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, sa, pa, da)
    y = run_and_fetch(p, t, G.GCONV_PATH_IGEMM)
    r = U.check(y, ref, scale, p.dtype, "igemm %r" % (IGEMM_ONLY_CASES[case],))
    print("igemm 32-channel case %d max err/tol %.3f plan %s" % (case, r, G.gconv_get_plan(d)))


CHUNKED_CASES = [
    # groups of 8k input channels that are not 32k, or more than 16 output
    # channels over narrow inputs: the M-tiled implicit GEMM walks K in
    # 8-channel chunks across taps
    (3, "bf16", 1, 4, 16, 32, (4, 6, 7), (3, 3, 3), 1, 1, 1, True),          # 16 in / 32 out, 3D
    (2, "f16", 2, 3, 24, 24, (1, 13, 11), (1, 3, 3), 2, 1, 1, True),         # 24-channel groups, stride 2
    (2, "bf16", 3, 5, 8, 32, (1, 9, 10), (1, 1, 1), 2, 0, 1, False),         # 1x1 stride 2, one chunk per tap
    (2, "f16", 1, 2, 40, 48, (1, 10, 9), (1, 5, 3), 1, (0, 2, 2), (1, 1, 2), True),  # 5x3, width dilation
    (3, "f16", 1, 2, 56, 112, (3, 5, 6), (3, 3, 3), 1, 1, (2, 1, 1), True),  # 112 of a 128-channel tile
    (2, "bf16", 2, 7, 16, 12, (1, 8, 8), (1, 3, 3), 1, 1, 1, True),          # 12 output channels, odd G
    (2, "bf16", 3, 4, 24, 24, (1, 28, 28), (1, 3, 3), 1, 1, 1, False),       # many M tiles, ragged tail
]


@pytest.mark.parametrize("case", range(len(CHUNKED_CASES)))
def test_igemm_chunked_k_every_tile(case):
    """Every tile of the implicit GEMM's menu on group widths outside the
    32-channel grid, element by element against the oracle."""
    nd, dt, N, Gr, Cpg, Kpg, sp, fl, s, pd, dl, bias = CHUNKED_CASES[case]
    tr = lambda v: (v if isinstance(v, tuple) else (v, v, v))
    st, pad, dil = tr(s), tr(pd), tr(dl)
    if nd == 2:
        st, pad, dil = (1, st[1], st[2]), (0, pad[1], pad[2]), (1, dil[1], dil[2])
    p = inputs.Problem(nd, dt, N, Gr, Gr * Cpg, Gr * Kpg, sp, fl, st, pad, dil, bias)
    d = G.desc_from_problem(p)
    assert G.gconv_select_path(d) == G.GCONV_PATH_IGEMM
    t = inputs.make_tensors(p, 7700 + case)
    sa, pa, da = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, sa, pa, da)
    x, w, b = U.device_tensors(p, t)
    n, picked = G.gconv_tile_count(d, G.GCONV_PATH_IGEMM)
    assert n >= 2
    for tile in range(n):
        y = poisoned_out(p)
        rc = G.gconv_fwd_tile(d, G.GCONV_PATH_IGEMM, tile, x.data_ptr(), w.data_ptr(),
                              b.data_ptr() if b is not None else None, y.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0, G.gconv_status_str(rc)
        torch.cuda.synchronize()
        r = U.check(U.to_f64(y), ref, scale, p.dtype, "chunked case %d tile %d" % (case, tile))
    y = run_and_fetch(p, t)
    U.check(y, ref, scale, p.dtype, "chunked case %d auto" % case)
    print("igemm chunked case %d: %d tiles (own %d), last max err/tol %.3f plan %s"
          % (case, n, picked, r, G.gconv_get_plan(d)))


def test_ring_3d_with_fewer_stores_than_lanes():
    """3D ring of 8-chunk pixels (2 merged 8/8 groups per tile, one tile per
    wave): a staged output row is 128 stores for 256 threads, so two waves
    issue none.  Their wait for a ring row must not count stores they did
    not issue (it once let them pass the barrier with their row loads in
    flight).  Several launches, each element by element."""
    p = inputs.conv3d("bf16", 4, 8, 64, 64, 8, 40, 56, 3, 3, 3, 1, 1)
    d = G.desc_from_problem(p)
    assert G.gconv_select_path(d) == G.GCONV_PATH_SMALLG
    assert G.gconv_get_plan(d)["groups_per_tile"] == 2
    t = inputs.make_tensors(p, 7900)
    sa, pa, da = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, sa, pa, da)
    x, w, b = U.device_tensors(p, t)
    for rep in range(6):
        y = U.run(p, x, w, b, out=poisoned_out(p))
        torch.cuda.synchronize()
        r = U.check(U.to_f64(y), ref, scale, p.dtype, "3D ring launch %d" % rep)
    print("3D ring, 8-chunk pixels: 6 launches, last max err/tol %.3f, plan %s" % (r, G.gconv_get_plan(d)))


@pytest.mark.parametrize("name,N", [("grouped2d_resnext_bf16", 1), ("grouped3d_f16_n1", 1)])
def test_nonfinite_input_stays_in_its_merged_tile(name, N):
    """One Inf in one group's input.  The generic path keeps it inside that
    group; the small-group path, whose block-diagonal tiles merge
    groups_per_tile consecutive groups, may also turn the other groups of
    that tile NaN (0 * Inf), and nothing else.  Every other output matches
    the oracle."""
    wl = inputs.WORKLOADS[name]
    p = reduced(wl.problem, N)
    t = inputs.workload_tensors(wl)
    t = inputs.Tensors(t.x[:N].copy(), t.w, t.bias)
    g_bad, c_bad = 5, p.Cpg - 1
    pos = (0,) + tuple(s // 2 for s in t.x.shape[1:-1])
    inf = inputs.to_storage(np.array([np.inf], dtype=np.float32), p.dtype)[0]
    t.x[pos + (g_bad * p.Cpg + c_bad,)] = inf
    st, pd, dl = p.spatial_args()
    xo, wo, bo = U.oracle_inputs(p, t)
    ref, scale = oracle.conv_fwd(xo, wo, bo, p.G, st, pd, dl)
    ref_bad = ~np.isfinite(ref)
    assert ref_bad.any()
    grp = np.arange(p.K) // p.Kpg
    d = G.desc_from_problem(p)
    for path in (G.GCONV_PATH_GENERIC, G.GCONV_PATH_SMALLG):
        assert G.gconv_path_supported(d, path) == 1
        y = run_and_fetch(p, t, path)
        gpt = G.gconv_get_plan(d, path)["groups_per_tile"] if path == G.GCONV_PATH_SMALLG else 1
        tile = (grp // gpt) == (g_bad // gpt)
        pix_bad = ref_bad.any(axis=-1, keepdims=True)       # pixels whose window reads the Inf
        may_differ = pix_bad & tile                         # outputs the tile merge may turn NaN
        assert not np.isfinite(y[ref_bad]).any(), "non-finite outputs of the Inf's group must stay non-finite"
        keep = ~ref_bad & ~may_differ
        U.check(y[keep], ref[keep], scale[keep], p.dtype, "%s path %d finite outputs" % (name, path))
        if path == G.GCONV_PATH_GENERIC:
            assert np.isfinite(y[~ref_bad]).all()
        print("%s path=%s groups_per_tile=%d NaN outside the Inf's group: %d of %d allowed"
              % (name, G.gconv_path_name(path), gpt, int((~np.isfinite(y) & ~ref_bad).sum()),
                 int((may_differ & ~ref_bad).sum())))


FP32_GROUPED = [
    inputs.conv2d("f32", N=4, G=32, C=256, K=256, H=56, W=56, Y=3, X=3, stride=1, pad=1, bias=False),
    inputs.conv2d("f32", N=2, G=8, C=1024, K=1024, H=14, W=14, Y=3, X=3, stride=1, pad=2, dil=2, bias=True),
    inputs.conv3d("f32", N=2, G=32, C=64, K=128, D=8, H=28, W=28, Z=3, Y=3, X=3, stride=1, pad=1, bias=True),
    inputs.Problem(2, "f32", 3, 6, 18, 30, (1, 23, 37), (1, 5, 3), (1, 2, 2), (0, 2, 1), (1, 1, 1), True),
]


@pytest.mark.parametrize("case", range(len(FP32_GROUPED)))
def test_fp32_grouped_register_blocked_kernel(case):
    """fp32 grouped problems on the VALU direct path, element by element, on
    every entry of its tile menu: the per-thread register-blocked kernel and
    the wave-uniform-weight kernel, each with every channel block
    (ResNeXt-style, large groups with dilation 2, 3D, and a ragged one with
    3 channels per group, 5 per output group, stride 2)."""
    p = FP32_GROUPED[case]
    d = G.desc_from_problem(p)
    assert G.gconv_path_supported(d, G.GCONV_PATH_DIRECT) == 1
    t = inputs.make_tensors(p, 77000 + case)
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    y = run_and_fetch(p, t, G.GCONV_PATH_DIRECT)
    r = U.check(y, ref, scale, p.dtype, "direct_valu case %d" % case)
    print("direct_valu case %d (auto path %s) max err/tol %.3f"
          % (case, G.gconv_path_name(G.gconv_select_path(d)), r))
    x, w, b = U.device_tensors(p, t)
    n, _ = G.gconv_tile_count(d, G.GCONV_PATH_DIRECT)
    assert n >= 2
    for tile in range(n):
        yt = poisoned_out(p)
        rc = G.gconv_fwd_tile(d, G.GCONV_PATH_DIRECT, tile, x.data_ptr(), w.data_ptr(),
                              b.data_ptr() if b is not None else None, yt.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0, G.gconv_status_str(rc)
        torch.cuda.synchronize()
        r = U.check(U.to_f64(yt), ref, scale, p.dtype, "direct_valu case %d tile %d" % (case, tile))
        print("direct_valu case %d tile %d/%d max err/tol %.3f" % (case, tile, n, r))


FP32_RING = [
    # ndim, N, G, Cpg, Kpg, spatial (D,H,W), stride, bias: fp32 small groups on the LDS ring
    (2, 2, 32, 8, 8, (1, 56, 56), 1, False),     # ResNeXt-style: 16-channel tiles of 4 fp32 chunks
    (2, 1, 16, 4, 4, (1, 30, 29), 2, True),      # stride 2, four groups per tile
    (2, 1, 64, 2, 2, (1, 17, 19), 1, True),      # 2-channel groups, eight per tile
    (2, 1, 64, 1, 4, (1, 20, 21), 1, False),     # one input channel per group: 1 chunk per tile
    (2, 2, 8, 8, 16, (1, 14, 14), 1, True),      # one group per tile, two chunks
    (3, 8, 32, 2, 4, (8, 28, 28), 1, True),      # the 3D grouped shape at N=8, in fp32
]


@pytest.mark.parametrize("case", range(len(FP32_RING)))
def test_fp32_small_groups_on_the_ring(case):
    """fp32 small groups on the LDS-ring kernel with 16x16x4 fp32 MFMAs,
    element by element against the oracle, on every entry of the small-group
    path's menu."""
    nd, N, Gr, Cpg, Kpg, sp, s, bias = FP32_RING[case]
    st = (1, s, s) if nd == 2 else (s, s, s)
    filt = (1, 3, 3) if nd == 2 else (3, 3, 3)
    pad = (0, 1, 1) if nd == 2 else (1, 1, 1)
    p = inputs.Problem(nd, "f32", N, Gr, Gr * Cpg, Gr * Kpg, sp, filt, st, pad, (1, 1, 1), bias)
    d = G.desc_from_problem(p)
    assert G.gconv_path_supported(d, G.GCONV_PATH_SMALLG) == 1, "the ring should take %r" % (p,)
    assert G.gconv_path_name(G.gconv_select_path(d)) == "smallg_mfma"
    t = inputs.make_tensors(p, 91000 + case)
    sa, pa, da = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, sa, pa, da)
    x, w, b = U.device_tensors(p, t)
    n, _ = G.gconv_tile_count(d, G.GCONV_PATH_SMALLG)
    for tile in range(n):
        y = poisoned_out(p)
        rc = G.gconv_fwd_tile(d, G.GCONV_PATH_SMALLG, tile, x.data_ptr(), w.data_ptr(),
                              b.data_ptr() if b is not None else None, y.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0, G.gconv_status_str(rc)
        torch.cuda.synchronize()
        r = U.check(U.to_f64(y), ref, scale, p.dtype, "fp32 ring case %d tile %d" % (case, tile))
        print("fp32 ring case %d tile %d/%d max err/tol %.3f plan %s" % (case, tile, n, r, G.gconv_get_plan(d)))


FP32_IGEMM = [
    # ndim, N, G, Cpg, Kpg, spatial (D,H,W), filt (Z,Y,X), stride, pad, dil, bias
    (2, 2, 8, 128, 128, (1, 14, 14), (1, 3, 3), 1, 1, 1, True),    # large groups: one tap per stage
    (2, 3, 4, 64, 64, (1, 28, 27), (1, 3, 3), 2, 1, 1, False),     # stride 2, ragged M
    (2, 2, 2, 24, 20, (1, 13, 11), (1, 5, 3), 1, (0, 2, 1), 1, True),  # 4-channel chunks across taps, partial N tile
    (3, 1, 2, 32, 32, (4, 6, 7), (3, 3, 3), 1, 1, 1, True),        # 3D
    (2, 2, 4, 64, 64, (1, 14, 14), (1, 3, 3), 1, 2, 2, True),      # dilation 2
    (2, 1, 3, 36, 44, (1, 9, 10), (1, 1, 1), 1, 0, 1, False),      # 1x1, odd widths
]


@pytest.mark.parametrize("case", range(len(FP32_IGEMM)))
def test_fp32_implicit_gemm_every_tile(case):
    """fp32 groups of 4k input and output channels on the M-tiled implicit
    GEMM with 16x16x4 fp32 MFMAs, element by element, on every tile."""
    nd, N, Gr, Cpg, Kpg, sp, fl, s, pd, dl, bias = FP32_IGEMM[case]
    tr = lambda v: (v if isinstance(v, tuple) else (v, v, v))
    st, pad, dil = tr(s), tr(pd), tr(dl)
    if nd == 2:
        st, pad, dil = (1, st[1], st[2]), (0, pad[1], pad[2]), (1, dil[1], dil[2])
    p = inputs.Problem(nd, "f32", N, Gr, Gr * Cpg, Gr * Kpg, sp, fl, st, pad, dil, bias)
    d = G.desc_from_problem(p)
    assert G.gconv_path_supported(d, G.GCONV_PATH_IGEMM) == 1, "the implicit GEMM should take %r" % (p,)
    t = inputs.make_tensors(p, 93000 + case)
    sa, pa, da = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, sa, pa, da)
    x, w, b = U.device_tensors(p, t)
    n, _ = G.gconv_tile_count(d, G.GCONV_PATH_IGEMM)
    for tile in range(n):
        y = poisoned_out(p)
        rc = G.gconv_fwd_tile(d, G.GCONV_PATH_IGEMM, tile, x.data_ptr(), w.data_ptr(),
                              b.data_ptr() if b is not None else None, y.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0, G.gconv_status_str(rc)
        torch.cuda.synchronize()
        r = U.check(U.to_f64(y), ref, scale, p.dtype, "fp32 igemm case %d tile %d" % (case, tile))
        print("fp32 igemm case %d tile %d/%d max err/tol %.3f" % (case, tile, n, r))


TILE_CASES = [("depthwise2d_f16", 2), ("depthwise2d_s2_f16", 2), ("grouped2d_resnext_bf16", 2),
              ("grouped3d_f16_n8", 1), ("grouped2d_large_bf16", 2), ("grouped2d_large_dil2_bf16", 1)]


@pytest.mark.parametrize("name,N", TILE_CASES)
def test_every_tile_of_every_path(name, N):
    """Every entry of every path's tile menu (gconv_fwd_tile) matches the oracle."""
    wl = inputs.WORKLOADS[name]
    p = reduced(wl.problem, N)
    t = inputs.make_tensors(p, wl.seed + 11, wl.x_dist, wl.w_dist, wl.b_dist)
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    d = G.desc_from_problem(p)
    x, w, b = U.device_tensors(p, t)
    ran = 0
    for path, pid in G.PATHS.items():
        if path == "generic" or G.gconv_path_supported(d, pid) != 1:
            continue
        n, _ = G.gconv_tile_count(d, pid)
        for tile in range(n):
            y = poisoned_out(p)
            rc = G.gconv_fwd_tile(d, pid, tile, x.data_ptr(), w.data_ptr(),
                                  b.data_ptr() if b is not None else None, y.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
            assert rc == 0, G.gconv_status_str(rc)
            torch.cuda.synchronize()
            U.check(U.to_f64(y), ref, scale, p.dtype, "%s path=%s tile=%d" % (name, path, tile))
            ran += 1
    assert ran >= 2
    print("%s N=%d: %d tile variants checked" % (name, N, ran))


GENERIC_CASES = [
    # problem, then what it exercises
    (inputs.conv2d("f32", 1, 2, 64, 64, 8, 8, 3, 3, 1, 1), "the small fp32 config: flat at 8 and 16 threads"),
    (inputs.conv2d("f16", 2, 3, 15, 6, 9, 11, 3, 1, 2, 1), "5 channels per group, 3 taps, stride 2"),
    (inputs.conv2d("bf16", 1, 4, 16, 8, 13, 10, 3, 3, 1, 2, 2), "dilation 2"),
    (inputs.conv2d("f32", 3, 1, 3, 7, 7, 5, 1, 1, 2, 1), "1x1 window, stride 2, padding"),
    (inputs.Problem(3, "f16", 1, 2, 8, 4, (5, 6, 7), (3, 3, 3), (1, 1, 1), (1, 1, 1)), "27 taps: loop form"),
    (inputs.conv2d("f32", 1, 2, 80, 4, 6, 6, 3, 3, 1, 1), "40 channels: loop form below 16 threads"),
]


@pytest.mark.parametrize("case", range(len(GENERIC_CASES)), ids=[c[1] for c in GENERIC_CASES])
def test_generic_every_tile(case):
    """Every generic tile (1, 2, 4, 8, 16 threads per output), in its flat
    form (windows of <= 9 taps, <= 4 channels per thread) and its loop form."""
    p, what = GENERIC_CASES[case]
    t = inputs.make_tensors(p, 5100 + case)
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    d = G.desc_from_problem(p)
    x, w, b = U.device_tensors(p, t)
    taps = p.filt[0] * p.filt[1] * p.filt[2]
    forms = []
    for tile in range(5):
        y = poisoned_out(p)
        rc = G.gconv_fwd_tile(d, G.GCONV_PATH_GENERIC, tile, x.data_ptr(), w.data_ptr(),
                              b.data_ptr() if b is not None else None, y.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0, G.gconv_status_str(rc)
        torch.cuda.synchronize()
        U.check(U.to_f64(y), ref, scale, p.dtype, "%s generic tile=%d" % (what, tile))
        forms.append("flat" if taps <= 9 and -(-p.Cpg // (1 << tile)) <= 4 else "loop")
    print("%s: generic tiles %s" % (what, forms))


def test_generic_inf_weight_beside_the_padding():
    """An Inf weight at tap (0, 0) of one output channel: outputs whose
    window puts that tap in the padding have no such product in the sum and
    stay finite (the flat form drops a product, it never multiplies the
    weight by zero); the others are infinite, as in the oracle."""
    p = inputs.conv2d("f32", 1, 2, 64, 64, 8, 8, 3, 3, 1, 1)
    t = inputs.make_tensors(p, 5200)
    t.w[5, 0, 0, 3] = np.inf
    st, pd, dl = p.spatial_args()
    ref, scale = oracle.conv_fwd(*U.oracle_inputs(p, t), p.G, st, pd, dl)
    fin = np.isfinite(ref)
    assert fin[0, 0, :, 5].all() and fin[0, :, 0, 5].all() and not fin[0, 1:, 1:, 5].any()
    d = G.desc_from_problem(p)
    x, w, b = U.device_tensors(p, t)
    for tile in range(5):
        y = poisoned_out(p)
        rc = G.gconv_fwd_tile(d, G.GCONV_PATH_GENERIC, tile, x.data_ptr(), w.data_ptr(), b.data_ptr(),
                              y.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0, G.gconv_status_str(rc)
        torch.cuda.synchronize()
        got = U.to_f64(y)
        U.check(got[fin], ref[fin], scale[fin], p.dtype, "Inf weight, finite outputs, tile=%d" % tile)
        assert np.isinf(got[~fin]).all(), "tile=%d" % tile

"""Pins of the oracle's backward data (the gradient of the forward with respect to x).

The pages name backward data as the second grouped-convolution variant (CK
grouped_conv tile-engine README, introduction; CK Python examples README,
Examples table and Runner argument contract: it takes dY and W).  They print
no values for it, so it is pinned by what the mathematics fixes:

* the adjoint identity <conv_fwd(x, w), dy> = <x, bwd_data(dy, w)>, exact on
  small integers, against the forward oracle (itself pinned in
  test_oracle_pins);
* PyTorch's own input gradient (torch.nn.grad.conv2d_input / conv3d_input)
  in fp64, dense and grouped;
* a scatter-form brute force (loops over dy, adding dy * w into every input
  the forward tap read), written here separately, exact on integers;
* the error scale equals the gradient of |dy| through |w|.
A mutation test plants mistakes in a copy of the C source and checks that
these pins reject each one.  CPU only.
"""
import itertools
import os
import shutil

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import small_int_problem


def scatter_bwd_data(dy, w, G, in_spatial, stride, pad, dil):
    """dx by scattering every dy element through the taps it was produced by."""
    dy = dy if dy.ndim == 5 else dy[:, None]
    w = w if w.ndim == 5 else w[:, None]
    N, Do, Ho, Wo, K = dy.shape
    _, Z, Y, X, Cpg = w.shape
    D, H, W = in_spatial if len(in_spatial) == 3 else (1, *in_spatial)
    st = stride if len(stride) == 3 else (1, *stride)
    pd = pad if len(pad) == 3 else (0, *pad)
    dl = dil if len(dil) == 3 else (1, *dil)
    Kpg = K // G
    dx = np.zeros((N, D, H, W, G * Cpg))
    sc = np.zeros_like(dx)
    for n, od, oh, ow, kk in itertools.product(range(N), range(Do), range(Ho), range(Wo), range(K)):
        g, v = kk // Kpg, dy[n, od, oh, ow, kk]
        for z, yy, xx in itertools.product(range(Z), range(Y), range(X)):
            i0 = od * st[0] - pd[0] + z * dl[0]
            i1 = oh * st[1] - pd[1] + yy * dl[1]
            i2 = ow * st[2] - pd[2] + xx * dl[2]
            if 0 <= i0 < D and 0 <= i1 < H and 0 <= i2 < W:
                t = v * w[kk, z, yy, xx, :]
                dx[n, i0, i1, i2, g * Cpg:(g + 1) * Cpg] += t
                sc[n, i0, i1, i2, g * Cpg:(g + 1) * Cpg] += np.abs(t)
    return dx, sc


def problem_with_dy(rng, ndim):
    x, w, _, G, st, pd, dl = small_int_problem(rng, ndim)
    y, _ = oracle.conv_fwd(x, w, None, G, st, pd, dl)
    dy = rng.integers(-3, 4, size=y.shape).astype(np.float64)
    in_sp = x.shape[1:-1]
    if ndim == 2:
        x, y, dy = x[:, 0], y[:, 0], dy[:, 0]
        w = w[:, 0]
        in_sp = in_sp[1:]
        st, pd, dl = st[1:], pd[1:], dl[1:]
    return x, w, G, st, pd, dl, y, dy, in_sp


@pytest.mark.parametrize("case", range(24))
def test_adjoint_identity_exact(case):
    rng = np.random.default_rng(5100 + case)
    nd = 2 if case % 2 else 3
    x, w, G, st, pd, dl, y, dy, in_sp = problem_with_dy(rng, nd)
    dx, _ = oracle.conv_bwd_data(dy, w, G, in_sp, st, pd, dl)
    assert dx.shape == x.shape
    assert float(np.sum(y * dy)) == float(np.sum(x * dx))


@pytest.mark.parametrize("case", range(16))
def test_scatter_bruteforce_exact(case):
    rng = np.random.default_rng(5200 + case)
    nd = 2 if case % 2 else 3
    x, w, G, st, pd, dl, y, dy, in_sp = problem_with_dy(rng, nd)
    dx, sc = oracle.conv_bwd_data(dy, w, G, in_sp, st, pd, dl)
    dx_ref, sc_ref = scatter_bwd_data(dy, w, G, in_sp, st, pd, dl)
    if nd == 2:
        dx_ref, sc_ref = dx_ref[:, 0], sc_ref[:, 0]
    assert np.array_equal(dx, dx_ref)
    assert np.array_equal(sc, sc_ref)


@pytest.mark.parametrize("ndim,case", [(2, i) for i in range(6)] + [(3, i) for i in range(4)])
def test_matches_torch_input_grad(ndim, case):
    rng = np.random.default_rng(5300 + 10 * ndim + case)
    G = int(rng.integers(1, 4))
    Cpg, Kpg = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    k = [int(rng.integers(1, 4)) for _ in range(ndim)]
    st = [int(rng.integers(1, 3)) for _ in range(ndim)]
    pd = [int(rng.integers(0, 3)) for _ in range(ndim)]
    dl = [int(rng.integers(1, 3)) for _ in range(ndim)]
    sp = [max(int(rng.integers(3, 9)), dl[a] * (k[a] - 1) + 1 - 2 * pd[a]) for a in range(ndim)]
    N = 2
    w = rng.standard_normal((G * Kpg, *k, Cpg))
    outs = [(sp[a] + 2 * pd[a] - dl[a] * (k[a] - 1) - 1) // st[a] + 1 for a in range(ndim)]
    dy = rng.standard_normal((N, *outs, G * Kpg))
    dx, _ = oracle.conv_bwd_data(dy, w, G, tuple(sp), tuple(st), tuple(pd), tuple(dl))
    perm_x = (0, ndim + 1) + tuple(range(1, ndim + 1))          # N..C -> N C ..
    wt = torch.from_numpy(np.ascontiguousarray(np.moveaxis(w, -1, 1)))   # K Cpg ..
    dyt = torch.from_numpy(np.ascontiguousarray(np.transpose(dy, perm_x)))
    f = torch.nn.grad.conv2d_input if ndim == 2 else torch.nn.grad.conv3d_input
    ref = f((N, G * Cpg, *sp), wt, dyt, stride=st, padding=pd, dilation=dl, groups=G).numpy()
    ref = np.moveaxis(ref, 1, -1)
    np.testing.assert_allclose(dx, ref, rtol=1e-12, atol=1e-12)


def test_scale_is_gradient_of_magnitudes():
    rng = np.random.default_rng(5400)
    x, w, G, st, pd, dl, y, dy, in_sp = problem_with_dy(rng, 3)
    dx, sc = oracle.conv_bwd_data(dy * 0.5, w, G, in_sp, st, pd, dl)
    mag, _ = oracle.conv_bwd_data(np.abs(dy * 0.5), np.abs(w), G, in_sp, st, pd, dl)
    assert np.array_equal(sc, mag)
    assert np.all(np.abs(dx) <= sc)


def test_rejects_mismatched_dy():
    dy = np.zeros((1, 4, 4, 2))
    w = np.zeros((2, 3, 3, 1))
    with pytest.raises(ValueError):
        oracle.conv_bwd_data(dy, w, 2, (7, 7), (1, 1), (1, 1), (1, 1))   # forward output is 7x7


SRC = os.path.join(os.path.dirname(oracle.__file__), "gconv_ref.c")
MUTANTS = {
    "ignores_stride_divisibility": ("if (th < 0 || th % stride[1] != 0 || th / stride[1] >= Ho) continue;",
                                    "if (th < 0 || th / stride[1] >= Ho) continue;"),
    "pad_sign": ("const int64_t tw = iw + pad[2] - xx * dil[2];", "const int64_t tw = iw - pad[2] - xx * dil[2];"),
    "flipped_taps": ("const int64_t td = id + pad[0] - z * dil[0];",
                     "const int64_t td = id + pad[0] - (Z - 1 - z) * dil[0];"),
    "wrong_group_of_dy": ("const double t = dy[yi] * w[wi];",
                          "const double t = dy[yi + (G - 1 - 2 * g) * Kpg] * w[wi];"),
    "extent_bound_off_by_one": ("td / stride[0] >= Do) continue;", "td / stride[0] > Do) continue;"),
}


def _caught(lib) -> bool:
    for case in range(16):
        rng = np.random.default_rng(5500 + case)
        x, w, G, st, pd, dl, y, dy, in_sp = problem_with_dy(rng, 2 if case % 2 else 3)
        try:
            dx, _ = oracle.conv_bwd_data(dy, w, G, in_sp, st, pd, dl, lib=lib)
        except ValueError:
            return True
        if float(np.sum(y * dy)) != float(np.sum(x * dx)):
            return True
    return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site missing or ambiguous: %s" % name
    mutated = tmp_path / ("gconv_ref_%s.c" % name)
    mutated.write_text(src.replace(old, new, 1))
    lib = oracle.bind(oracle.build(src=str(mutated), out=str(tmp_path / ("lib_%s.so" % name))))
    assert _caught(lib), "pins did not catch mutant %s" % name


def test_unmutated_passes():
    assert not _caught(oracle._load())

"""Pins of the oracle's backward weight (the gradient of the forward with respect to w).

The pages name backward weight as the third grouped-convolution variant (CK
grouped_conv tile-engine README, introduction; CK Python examples README,
Runner argument contract: it takes X and dY).  They print no values for it,
so it is pinned by what the mathematics fixes:

* the adjoint identity <conv_fwd(x, w), dy> = <w, bwd_weight(x, dy)>, exact
  on small integers, against the pinned forward oracle;
* PyTorch's own weight gradient (torch.nn.grad.conv2d_weight /
  conv3d_weight) in fp64, dense and grouped;
* a scatter-form brute force written here, exact on integers;
* the error scale equals the gradient through |x| and |dy|.
A mutation test plants mistakes in a copy of the C source.  CPU only.
"""
import itertools
import os
import shutil

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import small_int_problem


def scatter_bwd_weight(x, dy, G, filt, stride, pad, dil):
    x = x if x.ndim == 5 else x[:, None]
    dy = dy if dy.ndim == 5 else dy[:, None]
    N, D, H, W, C = x.shape
    _, Do, Ho, Wo, K = dy.shape
    Z, Y, X = filt if len(filt) == 3 else (1, *filt)
    st = stride if len(stride) == 3 else (1, *stride)
    pd = pad if len(pad) == 3 else (0, *pad)
    dl = dil if len(dil) == 3 else (1, *dil)
    Cpg, Kpg = C // G, K // G
    dw = np.zeros((K, Z, Y, X, Cpg))
    sc = np.zeros_like(dw)
    for n, od, oh, ow, kk in itertools.product(range(N), range(Do), range(Ho), range(Wo), range(K)):
        g, v = kk // Kpg, dy[n, od, oh, ow, kk]
        for z, yy, xx in itertools.product(range(Z), range(Y), range(X)):
            i0 = od * st[0] - pd[0] + z * dl[0]
            i1 = oh * st[1] - pd[1] + yy * dl[1]
            i2 = ow * st[2] - pd[2] + xx * dl[2]
            if 0 <= i0 < D and 0 <= i1 < H and 0 <= i2 < W:
                t = v * x[n, i0, i1, i2, g * Cpg:(g + 1) * Cpg]
                dw[kk, z, yy, xx] += t
                sc[kk, z, yy, xx] += np.abs(t)
    return dw, sc


def problem_with_dy(rng, ndim):
    x, w, _, G, st, pd, dl = small_int_problem(rng, ndim)
    y, _ = oracle.conv_fwd(x, w, None, G, st, pd, dl)
    dy = rng.integers(-3, 4, size=y.shape).astype(np.float64)
    filt = w.shape[1:4]
    if ndim == 2:
        x, y, dy, w = x[:, 0], y[:, 0], dy[:, 0], w[:, 0]
        filt = filt[1:]
        st, pd, dl = st[1:], pd[1:], dl[1:]
    return x, w, G, st, pd, dl, y, dy, filt


@pytest.mark.parametrize("case", range(24))
def test_adjoint_identity_exact(case):
    rng = np.random.default_rng(6100 + case)
    x, w, G, st, pd, dl, y, dy, filt = problem_with_dy(rng, 2 if case % 2 else 3)
    dw, _ = oracle.conv_bwd_weight(x, dy, G, filt, st, pd, dl)
    assert dw.shape == w.shape
    assert float(np.sum(y * dy)) == float(np.sum(w * dw))


@pytest.mark.parametrize("case", range(12))
def test_scatter_bruteforce_exact(case):
    rng = np.random.default_rng(6200 + case)
    nd = 2 if case % 2 else 3
    x, w, G, st, pd, dl, y, dy, filt = problem_with_dy(rng, nd)
    dw, sc = oracle.conv_bwd_weight(x, dy, G, filt, st, pd, dl)
    dw_ref, sc_ref = scatter_bwd_weight(x, dy, G, filt, st, pd, dl)
    if nd == 2:
        dw_ref, sc_ref = dw_ref[:, 0], sc_ref[:, 0]
    assert np.array_equal(dw, dw_ref)
    assert np.array_equal(sc, sc_ref)


@pytest.mark.parametrize("ndim,case", [(2, i) for i in range(6)] + [(3, i) for i in range(4)])
def test_matches_torch_weight_grad(ndim, case):
    rng = np.random.default_rng(6300 + 10 * ndim + case)
    G = int(rng.integers(1, 4))
    Cpg, Kpg = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    k = [int(rng.integers(1, 4)) for _ in range(ndim)]
    st = [int(rng.integers(1, 3)) for _ in range(ndim)]
    pd = [int(rng.integers(0, 3)) for _ in range(ndim)]
    dl = [int(rng.integers(1, 3)) for _ in range(ndim)]
    sp = [max(int(rng.integers(3, 9)), dl[a] * (k[a] - 1) + 1 - 2 * pd[a]) for a in range(ndim)]
    N = 2
    x = rng.standard_normal((N, *sp, G * Cpg))
    outs = [(sp[a] + 2 * pd[a] - dl[a] * (k[a] - 1) - 1) // st[a] + 1 for a in range(ndim)]
    dy = rng.standard_normal((N, *outs, G * Kpg))
    dw, _ = oracle.conv_bwd_weight(x, dy, G, tuple(k), tuple(st), tuple(pd), tuple(dl))
    perm = (0, ndim + 1) + tuple(range(1, ndim + 1))
    xt = torch.from_numpy(np.ascontiguousarray(np.transpose(x, perm)))
    dyt = torch.from_numpy(np.ascontiguousarray(np.transpose(dy, perm)))
    f = torch.nn.grad.conv2d_weight if ndim == 2 else torch.nn.grad.conv3d_weight
    ref = f(xt, (G * Kpg, Cpg, *k), dyt, stride=st, padding=pd, dilation=dl, groups=G).numpy()
    ref = np.moveaxis(ref, 1, -1)          # K Cpg .. -> K .. Cpg
    np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-11)


def test_scale_is_gradient_of_magnitudes():
    rng = np.random.default_rng(6400)
    x, w, G, st, pd, dl, y, dy, filt = problem_with_dy(rng, 3)
    dw, sc = oracle.conv_bwd_weight(x * 0.5, dy, G, filt, st, pd, dl)
    mag, _ = oracle.conv_bwd_weight(np.abs(x * 0.5), np.abs(dy), G, filt, st, pd, dl)
    assert np.array_equal(sc, mag)
    assert np.all(np.abs(dw) <= sc)


SRC = os.path.join(os.path.dirname(oracle.__file__), "gconv_ref.c")
MUTANTS = {
    "flipped_taps": ("const int64_t ih = oh * stride[1] - pad[1] + yy * dil[1];\n                                    if (ih < 0 || ih >= H) continue;\n                                    for (int64_t ow",
                     "const int64_t ih = oh * stride[1] - pad[1] + (Y - 1 - yy) * dil[1];\n                                    if (ih < 0 || ih >= H) continue;\n                                    for (int64_t ow"),
    "wrong_input_group": ("const int64_t xi = ((((n * D + id) * H + ih) * W + iw) * G + g) * Cpg + c;\n                                        const double t = dy[yi] * x[xi];",
                          "const int64_t xi = ((((n * D + id) * H + ih) * W + iw) * G + (G - 1 - g)) * Cpg + c;\n                                        const double t = dy[yi] * x[xi];"),
    "drops_last_image": ("for (int64_t n = 0; n < N; ++n)\n                            for (int64_t od",
                         "for (int64_t n = 0; n + 1 < N; ++n)\n                            for (int64_t od"),
    "pad_sign": ("const int64_t iw = ow * stride[2] - pad[2] + xx * dil[2];\n                                        if (iw < 0 || iw >= W) continue;\n                                        const int64_t yi",
                 "const int64_t iw = ow * stride[2] + pad[2] + xx * dil[2];\n                                        if (iw < 0 || iw >= W) continue;\n                                        const int64_t yi"),
}


def _caught(lib) -> bool:
    for case in range(16):
        rng = np.random.default_rng(6500 + case)
        x, w, G, st, pd, dl, y, dy, filt = problem_with_dy(rng, 2 if case % 2 else 3)
        try:
            dw, _ = oracle.conv_bwd_weight(x, dy, G, filt, st, pd, dl, lib=lib)
        except ValueError:
            return True
        if float(np.sum(y * dy)) != float(np.sum(w * dw)):
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

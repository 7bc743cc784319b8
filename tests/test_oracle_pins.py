"""Pins for the CPU oracle against facts other than itself.

Each check fixes a part of the definition of the grouped cross-correlation
(channel mapping of rocm-libraries PR 10064, Technical Details; the
cross-correlation the TileOPs PR 1568 review compares against PyTorch; the
output count of that review's 3D case) from an independent route:

* a scatter-form brute force written here (loops over inputs, not outputs),
  on small-integer data where fp64 sums are exact -> exact equality;
* PyTorch's CPU convolution in float64 (library routine), dense and grouped;
* closed forms: all-ones input gives filter sums; a one-hot input gives the
  filter taps back; linearity;
* output extents counted by enumeration of window positions.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from depthwise_convolution_grouped_amd import inputs

pytestmark = pytest.mark.filterwarnings("ignore")


# ------------------------------------------------------------------ helpers

def brute_extent(n, k, s, p, d):
    """Count window starts o*s - p whose last tap (k-1)*d lands inside the padded input."""
    cnt = 0
    for o in range(0, n + 2 * p + 1):
        first = o * s - p
        last = first + (k - 1) * d
        if first >= -p and last <= n - 1 + p:
            cnt += 1
    return cnt


def scatter_conv(x, w, b, G, stride, pad, dil):
    """Independent scatter form: every input element pushes x*w into each output it reaches.

    x: (N, D, H, W, C), w: (K, Z, Y, X, Cpg), b: (K,) or None.  Returns (y, scale).
    """
    N, D, H, W, C = x.shape
    K, Z, Y, X, Cpg = w.shape
    Kpg = K // G
    outs = [brute_extent(n, k, s, p, d) for n, k, s, p, d in
            zip((D, H, W), (Z, Y, X), stride, pad, dil)]
    y = np.zeros((N, *outs, K))
    sc = np.zeros_like(y)
    for n, i0, i1, i2 in itertools.product(range(N), range(D), range(H), range(W)):
        for t0, t1, t2 in itertools.product(range(Z), range(Y), range(X)):
            o = []
            ok = True
            for i, t, s, p, d, lim in zip((i0, i1, i2), (t0, t1, t2), stride, pad, dil, outs):
                num = i + p - t * d
                if num % s != 0 or not (0 <= num // s < lim):
                    ok = False
                    break
                o.append(num // s)
            if not ok:
                continue
            for g in range(G):
                xv = x[n, i0, i1, i2, g * Cpg:(g + 1) * Cpg]          # (Cpg,)
                wv = w[g * Kpg:(g + 1) * Kpg, t0, t1, t2, :]           # (Kpg, Cpg)
                prod = wv * xv[None, :]
                y[n, o[0], o[1], o[2], g * Kpg:(g + 1) * Kpg] += prod.sum(axis=1)
                sc[n, o[0], o[1], o[2], g * Kpg:(g + 1) * Kpg] += np.abs(prod).sum(axis=1)
    if b is not None:
        y += b
        sc += np.abs(b)
    return y, sc


def small_int_problem(rng, ndim):
    G = int(rng.integers(1, 4))
    Cpg = int(rng.integers(1, 4))
    Kpg = int(rng.integers(1, 4))
    N = int(rng.integers(1, 3))
    sp = [int(rng.integers(1, 6)) for _ in range(3)]
    fl = [int(rng.integers(1, 4)) for _ in range(3)]
    st = [int(rng.integers(1, 3)) for _ in range(3)]
    pd = [int(rng.integers(0, 3)) for _ in range(3)]
    dl = [int(rng.integers(1, 3)) for _ in range(3)]
    if ndim == 2:
        sp[0], fl[0], st[0], pd[0], dl[0] = 1, 1, 1, 0, 1
    for a in range(3):
        while sp[a] + 2 * pd[a] < dl[a] * (fl[a] - 1) + 1:
            sp[a] += 1
    x = rng.integers(-3, 4, size=(N, *sp, G * Cpg)).astype(np.float64)
    w = rng.integers(-3, 4, size=(G * Kpg, *fl, Cpg)).astype(np.float64)
    b = rng.integers(-3, 4, size=(G * Kpg,)).astype(np.float64) if rng.integers(0, 2) else None
    return x, w, b, G, tuple(st), tuple(pd), tuple(dl)


def to_torch_layout(x, w):
    """N D H W C -> N C D H W;  K Z Y X Cpg -> K Cpg Z Y X."""
    xt = torch.from_numpy(np.ascontiguousarray(np.moveaxis(x, -1, 1)))
    wt = torch.from_numpy(np.ascontiguousarray(np.moveaxis(w, -1, 1)))
    return xt, wt


def torch_conv(x, w, b, G, stride, pad, dil):
    xt, wt = to_torch_layout(x, w)
    bt = torch.from_numpy(b) if b is not None else None
    yt = torch.nn.functional.conv3d(xt, wt, bt, stride=stride, padding=pad, dilation=dil, groups=G)
    return np.moveaxis(yt.numpy(), 1, -1)


# ------------------------------------------------------------------ pins

@pytest.mark.parametrize("case", range(40))
def test_scatter_bruteforce_exact(case):
    rng = np.random.default_rng(7000 + case)
    x, w, b, G, st, pd, dl = small_int_problem(rng, 2 if case % 2 else 3)
    y, s = oracle.conv_fwd(x, w, b, G, st, pd, dl)
    y_ref, s_ref = scatter_conv(x, w, b, G, st, pd, dl)
    assert y.shape == y_ref.shape
    np.testing.assert_array_equal(y, y_ref)
    np.testing.assert_array_equal(s, s_ref)


def test_extent_matches_enumeration():
    for n, k, s, p, d in itertools.product(range(1, 9), range(1, 5), range(1, 4), range(0, 3), range(1, 3)):
        assert oracle.out_extent(n, k, s, p, d) == brute_extent(n, k, s, p, d), (n, k, s, p, d)


def test_extent_of_the_reviewed_3d_case():
    # TileOPs PR 1568 review, "The 50x is a baseline artifact": 8x28x28 input,
    # 3x3x3 filter, 128 output channels -> 802,816 output elements.
    D, H, W = 8, 28, 28
    outs = [oracle.out_extent(v, 3, 1, 1, 1) for v in (D, H, W)]
    assert outs[0] * outs[1] * outs[2] * 128 == 802816


@pytest.mark.parametrize("ndim,case", [(2, i) for i in range(4)] + [(3, i) for i in range(3)])
def test_dense_groups1_matches_torch(ndim, case):
    rng = np.random.default_rng(100 + 10 * ndim + case)
    C, K = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    sp = (1 if ndim == 2 else 5, 7, 6)
    fl = (1 if ndim == 2 else 3, 3, 2)
    st = (1, 1 + case % 2, 1)
    pd = (0 if ndim == 2 else 1, 1, case % 3)
    dl = (1, 1, 1 + case % 2)
    x = rng.standard_normal((2, *sp, C))
    w = rng.standard_normal((K, *fl, C))
    b = rng.standard_normal(K)
    y, _ = oracle.conv_fwd(x, w, b, 1, st, pd, dl)
    y_t = torch_conv(x, w, b, 1, st, pd, dl)
    np.testing.assert_allclose(y, y_t, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", range(6))
def test_grouped_matches_torch_groups(case):
    rng = np.random.default_rng(300 + case)
    G = [2, 3, 4, 8, 6, 5][case]
    Cpg, Kpg = [(1, 1), (2, 3), (3, 1), (1, 2), (4, 4), (2, 1)][case]
    ndim = 3 if case % 3 == 0 else 2
    sp = (4 if ndim == 3 else 1, 9, 8)
    fl = (3 if ndim == 3 else 1, 3, 3)
    st = (1, 2 if case == 1 else 1, 1)
    pd = (1 if ndim == 3 else 0, 1, 2)
    dl = (1, 1, 2 if case in (2, 4) else 1)
    x = rng.standard_normal((2, *sp, G * Cpg))
    w = rng.standard_normal((G * Kpg, *fl, Cpg))
    b = rng.standard_normal(G * Kpg) if case % 2 else None
    y, _ = oracle.conv_fwd(x, w, b, G, st, pd, dl)
    y_t = torch_conv(x, w, b, G, st, pd, dl)
    np.testing.assert_allclose(y, y_t, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", range(4))
def test_grouped_is_concat_of_dense(case):
    rng = np.random.default_rng(400 + case)
    G, Cpg, Kpg = [(4, 2, 3), (3, 1, 1), (2, 5, 2), (6, 2, 1)][case]
    x = rng.standard_normal((2, 3, 7, 6, G * Cpg))
    w = rng.standard_normal((G * Kpg, 3, 3, 3, Cpg))
    b = rng.standard_normal(G * Kpg)
    st, pd, dl = (1, 2, 1), (1, 1, 0), (1, 1, 2)
    y, _ = oracle.conv_fwd(x, w, b, G, st, pd, dl)
    parts = []
    for g in range(G):
        yg, _ = oracle.conv_fwd(x[..., g * Cpg:(g + 1) * Cpg], w[g * Kpg:(g + 1) * Kpg],
                                b[g * Kpg:(g + 1) * Kpg], 1, st, pd, dl)
        parts.append(yg)
    np.testing.assert_array_equal(y, np.concatenate(parts, axis=-1))


@pytest.mark.parametrize("ndim", [2, 3])
def test_all_ones_gives_filter_sums(ndim):
    rng = np.random.default_rng(500 + ndim)
    G, Cpg, Kpg = 4, 3, 2
    sp = (1 if ndim == 2 else 6, 9, 10)
    fl = (1 if ndim == 2 else 3, 3, 5)
    st, pd, dl = (1, 1, 2), (0 if ndim == 2 else 1, 2, 1), (1, 2, 1)
    x = np.ones((1, *sp, G * Cpg))
    w = rng.standard_normal((G * Kpg, *fl, Cpg))
    b = rng.standard_normal(G * Kpg)
    y, _ = oracle.conv_fwd(x, w, b, G, st, pd, dl)
    outs = y.shape[1:4]
    # Sum of the weights over the in-bounds taps of each output position.
    for o in itertools.product(*[range(v) for v in outs]):
        mask = np.ones(fl, dtype=bool)
        for a in range(3):
            coords = o[a] * st[a] - pd[a] + np.arange(fl[a]) * dl[a]
            inside = (coords >= 0) & (coords < sp[a])
            shape = [1, 1, 1]
            shape[a] = fl[a]
            mask &= inside.reshape(shape)
        expect = (w * mask[None, :, :, :, None]).sum(axis=(1, 2, 3, 4)) + b
        np.testing.assert_allclose(y[0][o], expect, rtol=1e-13, atol=1e-13)
    # interior points (whole window inside) see the plain weight sums
    full = w.sum(axis=(1, 2, 3, 4)) + b
    interior = [o for o in itertools.product(*[range(v) for v in outs])
                if all(o[a] * st[a] - pd[a] >= 0 and o[a] * st[a] - pd[a] + (fl[a] - 1) * dl[a] < sp[a]
                       for a in range(3))]
    assert interior, "test shape must have interior points"
    for o in interior:
        np.testing.assert_allclose(y[0][o], full, rtol=1e-13, atol=1e-13)


def test_impulse_returns_filter_taps():
    rng = np.random.default_rng(600)
    G, Cpg, Kpg = 3, 2, 2
    sp, fl = (5, 7, 8), (3, 3, 2)
    st, pd, dl = (1, 2, 1), (1, 1, 1), (2, 1, 3)
    w = rng.standard_normal((G * Kpg, *fl, Cpg))
    for (i0, i1, i2, g, c) in [(2, 3, 4, 1, 0), (0, 0, 0, 0, 1), (4, 6, 7, 2, 1)]:
        x = np.zeros((1, *sp, G * Cpg))
        x[0, i0, i1, i2, g * Cpg + c] = 1.0
        y, _ = oracle.conv_fwd(x, w, None, G, st, pd, dl)
        expect = np.zeros_like(y)
        outs = y.shape[1:4]
        for o in itertools.product(*[range(v) for v in outs]):
            for t in itertools.product(*[range(v) for v in fl]):
                if all(o[a] * st[a] - pd[a] + t[a] * dl[a] == (i0, i1, i2)[a] for a in range(3)):
                    expect[0, o[0], o[1], o[2], g * Kpg:(g + 1) * Kpg] = w[g * Kpg:(g + 1) * Kpg, t[0], t[1], t[2], c]
        assert np.count_nonzero(expect) > 0
        np.testing.assert_array_equal(y, expect)


def test_linearity():
    rng = np.random.default_rng(700)
    G, Cpg, Kpg = 2, 3, 2
    x1 = rng.integers(-4, 5, size=(2, 6, 7, G * Cpg)).astype(np.float64)
    x2 = rng.integers(-4, 5, size=(2, 6, 7, G * Cpg)).astype(np.float64)
    w = rng.integers(-4, 5, size=(G * Kpg, 3, 3, Cpg)).astype(np.float64)
    args = (G, (2, 1), (1, 2), (1, 2))
    y1, _ = oracle.conv_fwd(x1, w, None, *args)
    y2, _ = oracle.conv_fwd(x2, w, None, *args)
    y12, _ = oracle.conv_fwd(3 * x1 + x2, w, None, *args)
    np.testing.assert_array_equal(y12, 3 * y1 + y2)


def test_points_match_full():
    rng = np.random.default_rng(800)
    p = inputs.conv3d("f32", N=2, G=4, C=8, K=12, D=4, H=6, W=5, Z=3, Y=3, X=3, stride=1, pad=1)
    t = inputs.make_tensors(p, 800)
    st, pd, dl = p.spatial_args()
    y, s = oracle.conv_fwd(t.x, t.w, t.bias, p.G, st, pd, dl)
    idx = rng.integers(0, y.size, size=200)
    yp, sp = oracle.conv_fwd_points(t.x, t.w, t.bias, p.G, st, pd, dl, idx)
    np.testing.assert_array_equal(yp, y.reshape(-1)[idx])
    np.testing.assert_array_equal(sp, s.reshape(-1)[idx])


def test_scale_bounds_output():
    # |y| <= scale always; scale >= 0; scale == 0 only where y == 0.
    rng = np.random.default_rng(900)
    x = rng.standard_normal((1, 5, 6, 6))
    w = rng.standard_normal((6, 3, 3, 2))
    b = rng.standard_normal(6)
    y, s = oracle.conv_fwd(x, w, b, 3, (1, 1), (1, 1), (1, 1))
    assert np.all(s >= 0)
    assert np.all(np.abs(y) <= s * (1 + 1e-15))


def test_rejects_bad_sizes():
    x = np.zeros((1, 4, 4, 6))
    w = np.zeros((4, 3, 3, 3))
    with pytest.raises(ValueError):
        oracle.conv_fwd(x, w, None, 4, (1, 1), (0, 0), (1, 1))       # C % G != 0
    with pytest.raises(ValueError):
        oracle.conv_fwd(x, np.zeros((4, 5, 5, 3)), None, 2, (1, 1), (0, 0), (1, 1))   # empty output

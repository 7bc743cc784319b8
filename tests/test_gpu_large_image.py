"""One image too large for a single launch (>= 2^31 elements) is split into
launches of output slices along its outermost spatial axis (rows in 2D,
planes in 3D), each with the halo its window needs (gconv_fwd,
gconv_bwd_data, gconv_bwd_weight).  Checked against the oracle on bands of slices around
every launch boundary and at both ends of the image: the oracle runs on the
band of input slices the band's outputs read (its outputs depend on nothing
else), so the comparison is exact in its extent.  Inputs are seeded N(0, 1)
drawn on the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from depthwise_convolution_grouped_amd import gconv as G
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

LIM = (1 << 31) - 1      # bytes one launch's tensor may span


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    if torch.cuda.get_device_properties(0).total_memory < 64 << 30:
        pytest.skip("needs a GPU with >= 64 GB")


def fwd_slices(slice_in, slice_out, reach, stride):
    """Output slices per launch: the input window and the output each < 2^31 bytes."""
    return min(LIM // slice_out, (LIM // slice_in - reach) // stride + 1)


def bwd_slices(slice_in, slice_out, reach0, stride):
    """dx slices per launch for backward data (reach0 = dil (k - 1))."""
    return min(LIM // slice_in, (LIM // slice_out - 2) * stride + 1 - reach0)


def bands(extent, per):
    """Slice ranges [a, b) around every launch boundary and at both ends."""
    out = [(0, 3), (extent - 3, extent)]
    for b in range(per, extent, per):
        out.append((b - 3, b + 3))
    return out


def test_forward_2d_image_split_into_row_slices():
    H = W = 6000
    C = 64
    gen = torch.Generator(device="cuda").manual_seed(21)
    x = torch.randn((1, H, W, C), device="cuda", generator=gen, dtype=torch.float32).to(torch.float16)
    w = (torch.randn((C, 3, 3, 1), device="cuda", generator=gen) / 3).to(torch.float16)
    b = torch.rand((C,), device="cuda", generator=gen).to(torch.float16)
    assert x.numel() >= 1 << 31
    y = G.conv_fwd(x, w, b, groups=C, stride=(1, 1), pad=(1, 1), dil=(1, 1))
    torch.cuda.synchronize()
    w64, b64 = w.to("cpu", torch.float64).numpy(), b.to("cpu", torch.float64).numpy()
    per = fwd_slices(W * C * 2, W * C * 2, 3, 1)
    assert per < H
    for r0, r1 in bands(H, per):
        lo, hi = max(r0 - 1, 0), min(r1 + 1, H)
        ref, scale = oracle.conv_fwd(x[:, lo:hi].to("cpu", torch.float64).numpy(), w64, b64, C, (1, 1), (1, 1), (1, 1))
        ref, scale = ref[:, r0 - lo:r1 - lo], scale[:, r0 - lo:r1 - lo]
        got = y[:, r0:r1].to("cpu", torch.float64).numpy()
        r = U.check(got, ref, scale, "f16", "forward rows %d..%d" % (r0, r1))
        print("forward rows %d..%d (launch boundary every %d rows) max err/tol %.3f" % (r0, r1, per, r))
    del x, y


@pytest.mark.parametrize("direct", [False, True])
def test_bwd_data_2d_image_split_into_row_slices(direct):
    H = W = 6000
    C = 64
    gen = torch.Generator(device="cuda").manual_seed(22)
    dy = torch.randn((1, H, W, C), device="cuda", generator=gen, dtype=torch.float32).to(torch.float16)
    w = (torch.randn((C, 3, 3, 1), device="cuda", generator=gen) / 3).to(torch.float16)
    dx = G.conv_bwd_data(dy, w, C, (H, W), (1, 1), (1, 1), (1, 1), direct=direct)
    torch.cuda.synchronize()
    w64 = w.to("cpu", torch.float64).numpy()
    per = bwd_slices(W * C * 2, W * C * 2, 2, 1)
    assert per < H
    for r0, r1 in bands(H, per):
        lo, hi = max(r0 - 1, 0), min(r1 + 1, H)
        ref, scale = oracle.conv_bwd_data(dy[:, lo:hi].to("cpu", torch.float64).numpy(), w64, C, (hi - lo, W),
                                          (1, 1), (1, 1), (1, 1))
        ref, scale = ref[:, r0 - lo:r1 - lo], scale[:, r0 - lo:r1 - lo]
        got = dx[:, r0:r1].to("cpu", torch.float64).numpy()
        r = U.check(got, ref, scale, "f16", "bwd_data rows %d..%d" % (r0, r1))
        print("bwd_data (%s) rows %d..%d (boundary every %d rows) max err/tol %.3f"
              % ("direct" if direct else "auto", r0, r1, per, r))
    del dy, dx


def test_forward_3d_image_split_into_plane_slices():
    D, H, W = 600, 240, 240
    G8, C = 8, 64
    gen = torch.Generator(device="cuda").manual_seed(23)
    x = torch.randn((1, D, H, W, C), device="cuda", generator=gen, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((C, 3, 3, 3, C // G8), device="cuda", generator=gen) / 15).to(torch.bfloat16)
    assert x.numel() >= 1 << 31
    y = G.conv_fwd(x, w, None, groups=G8, stride=(1, 1, 1), pad=(1, 1, 1), dil=(1, 1, 1))
    torch.cuda.synchronize()
    w64 = w.to("cpu", torch.float64).numpy()
    per = fwd_slices(H * W * C * 2, H * W * C * 2, 3, 1)
    assert per < D
    for p0, p1 in bands(D, per):
        lo, hi = max(p0 - 1, 0), min(p1 + 1, D)
        ref, scale = oracle.conv_fwd(x[:, lo:hi].to("cpu", torch.float64).numpy(), w64, None, G8,
                                     (1, 1, 1), (1, 1, 1), (1, 1, 1))
        ref, scale = ref[:, p0 - lo:p1 - lo], scale[:, p0 - lo:p1 - lo]
        got = y[:, p0:p1].to("cpu", torch.float64).numpy()
        r = U.check(got, ref, scale, "bf16", "forward planes %d..%d" % (p0, p1))
        print("3D forward planes %d..%d (boundary every %d planes) max err/tol %.3f" % (p0, p1, per, r))
    del x, y


def _bwd_weight_bands(x, dy, groups, filt, per, extent, dtype, what):
    """dw of the whole image against the sum of the bands' contributions:
    dy is zero outside the bands (which are apart), so each band's share is
    the oracle's dw on the band's dy slices and the input slices they read
    (one slice of halo each side; the slices next to a band hold zero dy,
    so the halo's own padding in the band's problem adds nothing).  Inputs
    are uniform in [0, 0.5): the products share one sign, so the tolerance,
    which scales with the sum of |products|, stays small against every
    band's share."""
    nd = len(filt)
    dw = G.conv_bwd_weight(x, dy, groups, filt, (1,) * nd, (1,) * nd, (1,) * nd)
    torch.cuda.synchronize()
    got = dw.to("cpu", torch.float64).numpy()
    ref, scale, shares = 0.0, 0.0, []
    for a0, a1 in bands(extent, per):
        lo, hi = max(a0 - 1, 0), min(a1 + 1, extent)
        r, s = oracle.conv_bwd_weight(x[:, lo:hi].to("cpu", torch.float64).numpy(),
                                      dy[:, lo:hi].to("cpu", torch.float64).numpy(),
                                      groups, filt, (1,) * nd, (1,) * nd, (1,) * nd)
        ref, scale = ref + r, scale + s
        shares.append(r)
    r = U.check(got, ref, scale, dtype, what)
    print("%s (boundary every %d slices) max err/tol %.3f" % (what, per, r))
    # every band's share is far above the tolerance, so a launch dropped or
    # counted twice (or a halo slice lost) cannot pass
    tol = U.tolerance(scale, dtype)
    for sh in shares:
        assert (np.abs(sh) > 4 * tol).any()


@pytest.mark.parametrize("groups", [64, 8])
def test_bwd_weight_2d_image_split_into_row_slices(groups):
    """Depthwise (channel-vector kernel) and 8-channel groups (matrix-core
    kernel) over one 4.6 GB image: three launches of row slices."""
    H = W = 6000
    C = 64
    gen = torch.Generator(device="cuda").manual_seed(24)
    x = (torch.rand((1, H, W, C), device="cuda", generator=gen, dtype=torch.float32) / 2).to(torch.float16)
    assert x.numel() >= 1 << 31
    per = fwd_slices(W * C * 2, W * C * 2, 3, 1)
    assert per < H
    dy = torch.zeros((1, H, W, C), device="cuda", dtype=torch.float16)
    for r0, r1 in bands(H, per):
        dy[:, r0:r1] = (torch.rand((1, r1 - r0, W, C), device="cuda", generator=gen) / 2).to(torch.float16)
    _bwd_weight_bands(x, dy, groups, (3, 3), per, H, "f16", "bwd_weight G=%d rows" % groups)
    del x, dy


def test_bwd_weight_3d_image_split_into_plane_slices():
    """2-channel groups over one 4.4 GB 3D image: three launches of plane
    slices (16 channels keep the oracle's bands to seconds)."""
    D, H, W = 600, 480, 480
    G8, C = 8, 16
    gen = torch.Generator(device="cuda").manual_seed(25)
    x = (torch.rand((1, D, H, W, C), device="cuda", generator=gen, dtype=torch.float32) / 2).to(torch.bfloat16)
    assert x.numel() >= 1 << 31
    per = fwd_slices(H * W * C * 2, H * W * C * 2, 3, 1)
    assert per < D
    dy = torch.zeros((1, D, H, W, C), device="cuda", dtype=torch.bfloat16)
    for p0, p1 in bands(D, per):
        dy[:, p0:p1] = (torch.rand((1, p1 - p0, H, W, C), device="cuda", generator=gen) / 2).to(torch.bfloat16)
    _bwd_weight_bands(x, dy, G8, (3, 3, 3), per, D, "bf16", "3D bwd_weight planes")
    del x, dy

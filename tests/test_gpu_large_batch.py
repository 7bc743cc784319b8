"""Batches whose x and y have >= 2^31 elements run as launches of whole
images (gconv_fwd, gconv_bwd_data).  A depthwise fp16 problem with
33 x 1024 x 1024 x 64 = 2.2 G elements per tensor (4.4 GB each) is run
through the C ABI and checked against the oracle on sampled outputs of
images on both sides of the launch boundary (31 images per launch) and of
the last image, each image's oracle run on that image alone (its outputs
depend on no other image).  Inputs are seeded N(0, 1) drawn on the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from depthwise_convolution_grouped_amd import gconv as G
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

N, HW, C = 33, 1024, 64


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    if torch.cuda.get_device_properties(0).total_memory < 64 << 30:
        pytest.skip("needs a GPU with >= 64 GB")


def _sample_check(out, ref_fn, images, what):
    rng = np.random.default_rng(77)
    for n in images:
        ref, scale = ref_fn(n)
        got = out[n].to("cpu", torch.float64).numpy()
        idx = rng.integers(0, got.size, size=4000)
        g, r, s = got.reshape(-1)[idx], ref.reshape(-1)[idx], scale.reshape(-1)[idx]
        U.check(g, r, s, "f16", "%s image %d" % (what, n))


def test_forward_large_batch():
    gen = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((N, HW, HW, C), device="cuda", generator=gen, dtype=torch.float32).to(torch.float16)
    w = (torch.randn((C, 3, 3, 1), device="cuda", generator=gen) / 3).to(torch.float16)
    b = torch.rand((C,), device="cuda", generator=gen).to(torch.float16)
    assert x.numel() >= 1 << 31
    y = G.conv_fwd(x, w, b, groups=C, stride=(1, 1), pad=(1, 1), dil=(1, 1))
    torch.cuda.synchronize()
    w64 = w.to("cpu", torch.float64).numpy()
    b64 = b.to("cpu", torch.float64).numpy()

    def ref(n):
        r, s = oracle.conv_fwd(x[n:n + 1].to("cpu", torch.float64).numpy(), w64, b64, C, (1, 1), (1, 1), (1, 1))
        return r[0], s[0]
    _sample_check(y, ref, [0, 30, 31, 32], "forward")
    del x, y


def test_bwd_data_large_batch():
    gen = torch.Generator(device="cuda").manual_seed(12)
    dy = torch.randn((N, HW, HW, C), device="cuda", generator=gen, dtype=torch.float32).to(torch.float16)
    w = (torch.randn((C, 3, 3, 1), device="cuda", generator=gen) / 3).to(torch.float16)
    dx = G.conv_bwd_data(dy, w, C, (HW, HW), (1, 1), (1, 1), (1, 1))
    torch.cuda.synchronize()
    w64 = w.to("cpu", torch.float64).numpy()

    def ref(n):
        r, s = oracle.conv_bwd_data(dy[n:n + 1].to("cpu", torch.float64).numpy(), w64, C, (HW, HW),
                                    (1, 1), (1, 1), (1, 1))
        return r[0], s[0]
    _sample_check(dx, ref, [0, 30, 31, 32], "bwd_data")


def test_bwd_weight_large_batch_accumulates_every_launch():
    """Backward weight on a batch split into launches (15 + 15 + 3 images):
    every launch's partial sums enter the one reduction exactly once.
    Images alternate between two seeded patterns A and B, so the result is
    17 dw(A) + 16 dw(B), each term from the oracle on one image."""
    gen = torch.Generator(device="cuda").manual_seed(13)
    # N(0, 1/16^2) inputs keep sums over 33 M pixels inside fp16's range
    xa, xb = ((torch.randn((1, HW, HW, C), device="cuda", generator=gen) / 16).to(torch.float16) for _ in range(2))
    da, db = ((torch.randn((1, HW, HW, C), device="cuda", generator=gen) / 16).to(torch.float16) for _ in range(2))
    x = torch.cat([xa if n % 2 == 0 else xb for n in range(N)]).contiguous()
    dy = torch.cat([da if n % 2 == 0 else db for n in range(N)]).contiguous()
    assert x.numel() >= 1 << 31
    dw = G.conv_bwd_weight(x, dy, C, (3, 3), (1, 1), (1, 1), (1, 1))
    torch.cuda.synchronize()
    got = dw.to("cpu", torch.float64).numpy()
    del x, dy

    def one(xi, di):
        return oracle.conv_bwd_weight(xi.to("cpu", torch.float64).numpy(), di.to("cpu", torch.float64).numpy(),
                                      C, (3, 3), (1, 1), (1, 1), (1, 1))
    ra, sa = one(xa, da)
    rb, sb = one(xb, db)
    r = U.check(got, 17 * ra + 16 * rb, 17 * sa + 16 * sb, "f16", "bwd_weight split batch")
    # one launch dropped or counted twice moves every element by a whole image's share
    assert np.abs(got - (17 * ra + 15 * rb)).max() > 0.1
    print("bwd_weight over 3 launches: max err/tol %.3f" % r)

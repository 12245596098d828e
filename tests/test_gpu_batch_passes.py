"""Batches above the 32-bit buffer range run as passes over consecutive samples.

A conv whose input or output exceeds 2 GiB (H3 L0 at N = 8: 2.28 GB each way)
is run by the library as passes over as many samples as fit. Every output
element's fp32 sum runs over the same taps in the same order whatever the
batch around it, so each sample of a batched call must equal, bit for bit, a
call on that sample alone; the single-sample layers are compared with the
oracle on every element in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import convolution_video_vae_amd as cv
import workloads
from convolution_video_vae_amd.layer import Conv3d

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cv.lib()
    yield
    torch.cuda.empty_cache()


def seeded(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name,kernel", [("h3_l0_128", "ns=-2"), ("h3_l0_128_s122", "ns=-3")])
def test_h3_l0_batch_of_8_in_passes(name, kernel):
    """Passes of 7 samples: slot indices up to 7.9 M (the float-reciprocal
    row split is exact below 2^24), the pixel-pair view's frame order over
    samples with their own leading frames."""
    L = workloads.LAYERS[name]
    t = workloads.make_tensors(L)
    n = 8
    xs = (n,) + L.x_shape[1:]
    geo = dict(stride=L.stride, pad_lo=L.pad_lo, pad_hi=L.pad_hi)
    big = Conv3d(t.w.cuda(), xs, **geo)
    plan = cv.conv3d_plan_describe(big.desc)
    print(f"[batch] {name} n={n}: {plan}", flush=True)
    assert "passes=2 samples_per_pass=7" in plan and kernel in plan, plan
    x = seeded(xs, 5)
    y = big.new_output()
    y.fill_(float("nan"))
    big(x, y=y)
    one = Conv3d(t.w.cuda(), (1,) + L.x_shape[1:], **geo)
    ys = one.new_output()
    for i in range(n):
        one(x[i:i + 1], y=ys)
        torch.cuda.synchronize()
        assert same_bits(y[i:i + 1], ys), f"sample {i} differs"


@pytest.mark.parametrize("layout", [cv.NDHWC, cv.NCDHW], ids=["ndhwc", "ncdhw"])
def test_fused_layer_batch_above_2gib_in_passes(layout):
    """Bias, residual, saved residual sum and the fused norm, in NDHWC and
    through the NCDHW boundary transposes."""
    L = workloads.LAYERS["wan_fused_160to320"]
    t = workloads.make_tensors(L)
    n = 120                                   # y: 120 x 24.6 MB = 2.95 GB
    _, d, h, w, c = L.x_shape
    xs = (n, d, h, w, c) if layout == cv.NDHWC else (n, c, d, h, w)
    kw = dict(layout=layout, bias=t.bias, gamma=t.gamma, norm_silu=True, residual=True,
              residual_out=True)
    big = Conv3d(t.w.cuda(), xs, **kw)
    e = cv.make_epilogue(bias=big.bias, gamma=big.gamma, norm_silu=True)
    e.flags |= cv.EPI_RESIDUAL | cv.EPI_RESIDUAL_OUT
    plan = cv.conv3d_plan_describe(big.desc, e)
    print(f"[batch] wan_fused n={n} layout={layout}: {plan}", flush=True)
    assert "passes=2" in plan, plan
    x = seeded(xs, 7)
    res = seeded(big.out_shape, 8)
    y = big.new_output()
    ro = torch.empty_like(y)
    big(x, residual=res, y=y, residual_out=ro)
    one = Conv3d(t.w.cuda(), (1,) + xs[1:], **kw)
    y1 = one.new_output()
    r1 = torch.empty_like(y1)
    for i in range(n):
        one(x[i:i + 1], residual=res[i:i + 1], y=y1, residual_out=r1)
        torch.cuda.synchronize()
        assert same_bits(y[i:i + 1], y1), f"sample {i}: y differs"
        assert same_bits(ro[i:i + 1], r1), f"sample {i}: residual_out differs"

"""GPU parity of reflect spatial padding (the H3 encoder's convs: reflect in
H and W, causal zeros in time) across the kernel families that compile it:
the slot kernel (stride 1 along W), the K-split halo kernel with its
fragment-order reduction, the plain kernel (stride 2, odd channel counts)
and the fused-norm epilogue. Integer data makes every sum exact, so results
are compared bit for bit with oracle.conv3d_reflect; random-data cases use
the parity rule.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import convolution_video_vae_amd as cv
from convolution_video_vae_amd.layer import Conv3d
from parity import check, check_every_element, oracle_every_pixel

pytestmark = pytest.mark.gpu

R = cv.PAD_REFLECT


def bits(t):
    return workloads.bf16_bits(t.cpu())


CASES = [
    # label, x shape, cout, stride, pad_lo, pad_hi, split_k, expected kernel (plan substring)
    ("slot_causal_128", (1, 4, 12, 40, 128), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1, "ns=-2"),
    ("slot_96_rows_straddle", (1, 3, 9, 37, 32), 96, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1, "ns=-2"),
    ("halo_split_256", (1, 3, 8, 16, 256), 256, (1, 1, 1), (2, 1, 1), (0, 1, 1), 0, "ns=-1"),
    ("plain_split_512", (1, 3, 6, 6, 512), 512, (1, 1, 1), (2, 1, 1), (0, 1, 1), 0, "mode=partial"),
    ("plain_stride222_odd_h", (1, 9, 13, 12, 64), 64, (2, 2, 2), (2, 1, 1), (0, 1, 1), 1, "ns=3"),
    ("plain_stride122", (1, 3, 12, 15, 64), 128, (1, 2, 2), (2, 1, 1), (0, 1, 1), 1, "ns=3"),
    ("plain_cout_48", (1, 3, 7, 9, 32), 48, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1, ""),
    ("two_by_two_frames", (2, 3, 2, 2, 32), 64, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1, ""),
]


@pytest.mark.parametrize("label,xs,cout,st,lo,hi,sk,kern", CASES, ids=[c[0] for c in CASES])
def test_reflect_integer_exact(label, xs, cout, st, lo, hi, sk, kern):
    x, w, b = workloads.integer_tensors(xs, cout, seed=11, bias=True)
    conv = Conv3d(w.cuda(), xs, stride=st, pad_lo=lo, pad_hi=hi, split_k=sk, bias=b, pad_mode=R)
    plan = cv.conv3d_plan_describe(conv.desc, cv.make_epilogue(bias=conv.bias))
    print(f"[reflect] {label} x={xs} cout={cout} stride={st} plan: {plan}", flush=True)
    assert kern in plan
    y = conv(x.cuda())
    torch.cuda.synchronize()
    ref = oracle.conv3d_reflect(bits(x), bits(w), stride=st, pad_lo=lo, pad_hi=hi, bias=b.numpy())
    assert np.array_equal(bits(y), ref)


def test_reflect_differs_from_zero_padding_only_on_the_border():
    x, w, _ = workloads.integer_tensors((1, 3, 8, 10, 32), 32, seed=12)
    yr = Conv3d(w.cuda(), tuple(x.shape), pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), pad_mode=R)(x.cuda())
    yz = Conv3d(w.cuda(), tuple(x.shape), pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))(x.cuda())
    torch.cuda.synchronize()
    a, z = bits(yr), bits(yz)
    assert np.array_equal(a[:, :, 1:-1, 1:-1], z[:, :, 1:-1, 1:-1])
    assert not np.array_equal(a[:, :, 0], z[:, :, 0])


def test_reflect_fused_norm_random():
    L = workloads.LAYERS["wan_fused_160to320"]
    xs = (1, 4, 9, 14, 160)
    t = workloads.make_tensors(L, x_shape=xs)
    lo, hi = (2, 1, 1), (0, 1, 1)
    res = torch.from_numpy(np.random.default_rng(13).standard_normal((1, 4, 9, 14, 320))
                           .astype(np.float32)).to(torch.bfloat16)
    conv = Conv3d(t.w.cuda(), xs, pad_lo=lo, pad_hi=hi, bias=t.bias, gamma=t.gamma,
                  norm_silu=True, residual=True, pad_mode=R)
    y = conv(t.x.cuda(), residual=res.cuda())
    torch.cuda.synchronize()
    ref = oracle.conv3d_reflect(bits(t.x), bits(t.w), pad_lo=lo, pad_hi=hi, bias=t.bias.numpy(),
                                residual=bits(res), gamma=bits(t.gamma), norm_silu=True,
                                intermediates=True)
    check(bits(y), ref, fused=True, gamma_bits=bits(t.gamma), what="reflect fused")


def test_reflect_h3_l0_every_element():
    """H3 L0 at full size with its own padding (reflect spatial, causal time)
    in the launch configuration the benchmark times, against the oracle on
    every output element (the reflected border rows and columns included)."""
    L = workloads.LAYERS["h3_l0_128_reflect"]
    t = workloads.make_tensors(L)
    conv = Conv3d(t.w.cuda(), L.x_shape, pad_lo=L.pad_lo, pad_hi=L.pad_hi, pad_mode=R)
    y = conv(t.x.cuda())
    torch.cuda.synchronize()
    got = bits(y).reshape(-1, L.cout)
    xr = oracle.reflect_pad_hw(bits(t.x), (1, 1), (1, 1))
    wb = bits(t.w)
    chunk = 1 << 16
    ref = oracle_every_pixel(
        lambda pix: oracle.conv3d(xr, wb, pad_lo=(2, 0, 0), pad_hi=(0, 0, 0), pixels=pix,
                                  intermediates=True), L.m, chunk, what="h3 l0 reflect")
    diag = check_every_element(got, ref, chunk=chunk, what="h3 l0 reflect")
    print("[reflect] h3 l0 every element:", diag, flush=True)
    assert diag["bit_identical"] > 0.97

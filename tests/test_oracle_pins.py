"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each test targets a mistake the oracle could plausibly make (orientation of
the cross-correlation, causal direction, stride/pad offsets, a dropped tap,
summation, bf16 rounding ties, post-operation order and constants), using a
formulation that shares nothing with the oracle's loops: numpy im2col over an
explicitly padded tensor, PyTorch's F.conv3d/F.conv2d in fp64, exact integer
arithmetic, impulses, and hand-worked epilogue values.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_to_bits(a):
    """bf16 bits of fp32 values via PyTorch's cast (a library RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return workloads.bf16_bits(t)


def rand_bf16(rng, shape, scale=1.0):
    return f32_to_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def b2f(bits):
    return oracle.bf16_to_f32(bits)


def ref_im2col(x_bits, w_bits, stride, pad_lo, pad_hi):
    """fp64 reference: explicit zero pad, gather every patch, one matmul."""
    x = b2f(x_bits).astype(np.float64)
    w = b2f(w_bits).astype(np.float64)
    N, D, H, W, Ci = x.shape
    Co, _, KD, KH, KW = w.shape
    xp = np.pad(x, ((0, 0), (pad_lo[0], pad_hi[0]), (pad_lo[1], pad_hi[1]),
                    (pad_lo[2], pad_hi[2]), (0, 0)))
    Do = (xp.shape[1] - KD) // stride[0] + 1
    Ho = (xp.shape[2] - KH) // stride[1] + 1
    Wo = (xp.shape[3] - KW) // stride[2] + 1
    cols = np.empty((N, Do, Ho, Wo, KD, KH, KW, Ci))
    for kd, kh, kw in itertools.product(range(KD), range(KH), range(KW)):
        cols[:, :, :, :, kd, kh, kw, :] = xp[:, kd:kd + stride[0] * Do:stride[0],
                                             kh:kh + stride[1] * Ho:stride[1],
                                             kw:kw + stride[2] * Wo:stride[2], :]
    wm = w.transpose(2, 3, 4, 1, 0).reshape(-1, Co)       # [(kd,kh,kw,ci), co]
    return cols.reshape(-1, wm.shape[0]) @ wm, (N, Do, Ho, Wo, Co)


def ref_torch(x_bits, w_bits, stride, pad_lo, pad_hi):
    """fp64 reference through PyTorch's own conv3d (after an explicit F.pad)."""
    x = torch.from_numpy(b2f(x_bits).astype(np.float64)).permute(0, 4, 1, 2, 3)
    w = torch.from_numpy(b2f(w_bits).astype(np.float64))
    x = F.pad(x, (pad_lo[2], pad_hi[2], pad_lo[1], pad_hi[1], pad_lo[0], pad_hi[0]))
    y = F.conv3d(x, w, stride=stride)
    return y.permute(0, 2, 3, 4, 1).numpy()


def assert_acc_matches(acc32, ref64):
    """The oracle's fp32 accumulator is the exact sum rounded once to fp32:
    equal to fp32(ref) up to the (vanishing) chance that two fp64 sums land on
    opposite sides of an fp32 rounding boundary (allow one fp32 ulp)."""
    want = ref64.astype(np.float32)
    diff = np.abs(acc32.astype(np.float64) - want.astype(np.float64))
    ulp = np.spacing(np.abs(want)).astype(np.float64)
    assert np.all(diff <= ulp), float(np.max(diff / np.maximum(ulp, 1e-45)))
    assert np.mean(acc32 == want) > 0.999


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_ties_to_even():
    cases = {257.0: 256.0, 259.0: 260.0, -257.0: -256.0, 1.0 + 2.0 ** -8: 1.0,
             1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6, 0.73105857: 0.73046875,
             17.888544: 17.875, 3.0e38: 3.0040553e38, 3.4028235e38: float("inf")}
    got = b2f(oracle.bf16_round(list(cases.keys())))
    np.testing.assert_array_equal(got, np.array(list(cases.values()), dtype=np.float32))


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 100,
        # exact ties and near-ties: bf16 values plus half an ulp (+-1 fp32 ulp)
        (b2f(f32_to_bits(rng.standard_normal(5000).astype(np.float32))).view(np.uint32)
         + np.uint32(0x8000) + rng.integers(-1, 2, 5000).astype(np.uint32)).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40], dtype=np.float32),
    ])
    np.testing.assert_array_equal(oracle.bf16_round(v), f32_to_bits(v))


# ---------------------------------------------------------------- brute force

SHAPES = [
    # (N, D, H, W, Ci, Co, stride, pad_lo, pad_hi)
    (1, 1, 1, 1, 8, 8, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    (2, 2, 3, 7, 8, 16, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    (1, 5, 7, 3, 16, 8, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    (1, 3, 7, 7, 8, 8, (1, 1, 1), (0, 0, 0), (0, 0, 0)),
    (2, 5, 3, 7, 16, 16, (1, 1, 1), (0, 0, 0), (0, 0, 0)),
    (1, 5, 7, 7, 8, 16, (1, 2, 2), (2, 0, 0), (0, 1, 1)),
    (1, 3, 2, 7, 16, 8, (1, 2, 2), (2, 0, 0), (0, 1, 1)),
    (2, 5, 7, 7, 8, 8, (2, 2, 2), (2, 1, 1), (0, 1, 1)),
    (1, 2, 1, 3, 8, 8, (2, 1, 2), (2, 1, 1), (0, 1, 1)),
    (1, 5, 7, 3, 16, 16, (1, 1, 2), (1, 1, 1), (1, 1, 1)),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_brute_force_against_im2col_and_torch(shape):
    N, D, H, W, Ci, Co, st, lo, hi = shape
    rng = np.random.default_rng(100 + SHAPES.index(shape))
    x = rand_bf16(rng, (N, D, H, W, Ci))
    w = rand_bf16(rng, (Co, Ci, 3, 3, 3), 0.2)
    got = oracle.conv3d(x, w, stride=st, pad_lo=lo, pad_hi=hi, intermediates=True)
    ref, oshape = ref_im2col(x, w, st, lo, hi)
    ref = ref.reshape(oshape)
    assert got["y"].shape == oshape
    np.testing.assert_allclose(ref, ref_torch(x, w, st, lo, hi), rtol=1e-12, atol=1e-12)
    assert_acc_matches(got["acc"], ref)
    # y = B(acc) with no bias and no post-operations.
    np.testing.assert_array_equal(got["y"], f32_to_bits(got["acc"]))


def test_output_dims_follow_pytorch():
    for (N, D, H, W, Ci, Co, st, lo, hi) in SHAPES:
        x = torch.zeros(1, 1, D + lo[0] + hi[0], H + lo[1] + hi[1], W + lo[2] + hi[2])
        want = F.conv3d(x, torch.zeros(1, 1, 3, 3, 3), stride=st).shape[2:]
        got, ok = oracle.output_dims((D, H, W), (3, 3, 3), st, lo, hi)
        assert ok and got == tuple(want)
    _, ok = oracle.output_dims((2, 5, 5), (3, 3, 3), (1, 1, 1), (0, 0, 0), (0, 0, 0))
    assert not ok   # a valid conv needs T/H/W >= 3


# ---------------------------------------------------------------- identities

def test_t1_causal_equals_2d_slice():
    """Causal 3x3x3 on T=1 equals Conv2d with weight[:, :, 2] and padding 1
    (Qwen-Image PR page, "T=1 degeneration")."""
    rng = np.random.default_rng(11)
    x = rand_bf16(rng, (2, 1, 9, 13, 16))
    w = rand_bf16(rng, (8, 16, 3, 3, 3), 0.2)
    got = oracle.conv3d(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), intermediates=True)
    x2 = torch.from_numpy(b2f(x)[:, 0].astype(np.float64)).permute(0, 3, 1, 2)
    w3 = torch.from_numpy(b2f(w).astype(np.float64))
    ref = F.conv2d(x2, w3[:, :, 2], padding=1).permute(0, 2, 3, 1).numpy()[:, None]
    assert_acc_matches(got["acc"], ref)
    np.testing.assert_array_equal(got["y"], f32_to_bits(ref.astype(np.float32)))
    # The front-padded slice is the live one: slice 0 would be a different conv.
    wrong = F.conv2d(x2, w3[:, :, 0], padding=1).permute(0, 2, 3, 1).numpy()[:, None]
    assert np.mean(np.abs(wrong - ref)) > 0.1


def test_symmetric_time_padding_is_not_causal():
    """Padding time on both sides changes the result (Qwen-Image PR page warns
    against symmetric padding=1 for the causal conv)."""
    rng = np.random.default_rng(12)
    x = rand_bf16(rng, (1, 4, 5, 5, 8))
    w = rand_bf16(rng, (8, 8, 3, 3, 3), 0.2)
    causal = oracle.conv3d(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    sym = oracle.conv3d(x, w, pad_lo=(1, 1, 1), pad_hi=(1, 1, 1))
    assert causal.shape == sym.shape
    assert np.mean(causal != sym) > 0.5


def test_one_by_one_conv_is_a_matmul():
    rng = np.random.default_rng(13)
    x = rand_bf16(rng, (2, 3, 4, 5, 32))
    w = rand_bf16(rng, (24, 32, 1, 1, 1), 0.2)
    got = oracle.conv3d(x, w, intermediates=True)
    ref = b2f(x).astype(np.float64).reshape(-1, 32) @ b2f(w).astype(np.float64).reshape(24, 32).T
    assert_acc_matches(got["acc"].reshape(-1, 24), ref)


def test_zero_weight_gives_bias_everywhere():
    rng = np.random.default_rng(14)
    x = rand_bf16(rng, (1, 3, 5, 6, 16))
    w = np.zeros((16, 16, 3, 3, 3), np.uint16)
    bias = rng.standard_normal(16).astype(np.float32)
    y = oracle.conv3d(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), bias=bias)
    np.testing.assert_array_equal(y, np.broadcast_to(f32_to_bits(bias), y.shape))


def test_causality():
    """Changing input frame t leaves every output frame before t unchanged."""
    rng = np.random.default_rng(15)
    x = rand_bf16(rng, (1, 6, 5, 5, 8))
    w = rand_bf16(rng, (8, 8, 3, 3, 3), 0.3)
    y0 = oracle.conv3d(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    for t in range(6):
        x2 = x.copy()
        x2[:, t] = rand_bf16(rng, x2[:, t].shape)
        y1 = oracle.conv3d(x2, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
        np.testing.assert_array_equal(y1[:, :t], y0[:, :t])
        assert np.any(y1[:, t] != y0[:, t])


# ---------------------------------------------------------------- exact integer data

@pytest.mark.parametrize("stride,lo,hi", [((1, 1, 1), (2, 1, 1), (0, 1, 1)),
                                         ((1, 2, 2), (2, 0, 0), (0, 1, 1)),
                                         ((1, 1, 1), (0, 0, 0), (0, 0, 0))])
def test_integer_data_is_exact_and_rounds_ties_to_even(stride, lo, hi):
    rng = np.random.default_rng(16)
    xi = rng.integers(1, 3, size=(1, 4, 6, 7, 64))        # mostly-positive sums > 256
    wi = rng.integers(0, 2, size=(16, 64, 3, 3, 3))
    bias = rng.integers(-3, 4, size=16).astype(np.float32)
    x = f32_to_bits(xi.astype(np.float32))
    w = f32_to_bits(wi.astype(np.float32))
    got = oracle.conv3d(x, w, stride=stride, pad_lo=lo, pad_hi=hi, bias=bias, intermediates=True)
    # exact integer convolution on an explicitly padded int64 tensor
    xp = np.pad(xi, ((0, 0), (lo[0], hi[0]), (lo[1], hi[1]), (lo[2], hi[2]), (0, 0)))
    Do, Ho, Wo = got["y"].shape[1:4]
    exact = np.zeros((1, Do, Ho, Wo, 16), np.int64)
    for kd, kh, kw in itertools.product(range(3), range(3), range(3)):
        patch = xp[:, kd:kd + stride[0] * Do:stride[0], kh:kh + stride[1] * Ho:stride[1],
                   kw:kw + stride[2] * Wo:stride[2], :]
        exact += np.einsum("ndhwc,oc->ndhwo", patch, wi[:, :, kd, kh, kw])
    np.testing.assert_array_equal(got["acc"], exact.astype(np.float32))
    conv = f32_to_bits(exact.astype(np.float32))
    np.testing.assert_array_equal(got["conv"], conv)
    # ties at odd integers above 256 really occur and round to even
    assert np.mean((np.abs(exact) > 256) & (exact % 2 == 1)) > 0.05
    main = f32_to_bits(b2f(conv) + bias)
    np.testing.assert_array_equal(got["y"], main)


# ---------------------------------------------------------------- impulses

@pytest.mark.parametrize("stride,lo,hi", [((1, 1, 1), (2, 1, 1), (0, 1, 1)),
                                         ((1, 2, 2), (2, 0, 0), (0, 1, 1)),
                                         ((2, 2, 1), (2, 1, 1), (0, 1, 1))])
def test_input_impulse_maps_to_weight_taps(stride, lo, hi):
    rng = np.random.default_rng(17)
    shape = (1, 5, 6, 7, 8)
    w = rand_bf16(rng, (8, 8, 3, 3, 3))
    wf = b2f(w)
    for (d, h, ww, ci) in [(0, 0, 0, 0), (4, 5, 6, 7), (2, 3, 1, 5), (1, 0, 6, 2)]:
        x = np.zeros(shape, np.uint16)
        x[0, d, h, ww, ci] = f32_to_bits(np.float32(1.0)).item()
        y = b2f(oracle.conv3d(x, w, stride=stride, pad_lo=lo, pad_hi=hi))
        want = np.zeros_like(y)
        for do, ho, wo in itertools.product(*(range(s) for s in y.shape[1:4])):
            kd = d - (do * stride[0] - lo[0])
            kh = h - (ho * stride[1] - lo[1])
            kw = ww - (wo * stride[2] - lo[2])
            if 0 <= kd < 3 and 0 <= kh < 3 and 0 <= kw < 3:
                want[0, do, ho, wo, :] = wf[:, ci, kd, kh, kw]
        np.testing.assert_array_equal(y, want)


def test_weight_impulse_shifts_the_input():
    rng = np.random.default_rng(18)
    x = rand_bf16(rng, (1, 4, 5, 6, 8))
    xf = b2f(x)
    for (co, ci, kd, kh, kw) in [(0, 0, 0, 0, 0), (3, 5, 2, 1, 0), (7, 7, 1, 2, 2)]:
        w = np.zeros((8, 8, 3, 3, 3), np.uint16)
        w[co, ci, kd, kh, kw] = f32_to_bits(np.float32(1.0)).item()
        y = b2f(oracle.conv3d(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1)))
        want = np.zeros_like(y)
        xp = np.pad(xf, ((0, 0), (2, 0), (1, 1), (1, 1), (0, 0)))
        want[..., co] = xp[:, kd:kd + 4, kh:kh + 5, kw:kw + 6, ci]
        np.testing.assert_array_equal(y, want)


# ---------------------------------------------------------------- post-operations

def _closed_forms():
    with open(os.path.join(GOLDEN, "epilogue_closed_forms.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _closed_forms(), ids=lambda c: c["name"])
def test_epilogue_closed_forms(case):
    C = 320
    rng = np.random.default_rng(19)
    x = rand_bf16(rng, (1, 3, 4, 4, 16))
    w = np.zeros((C, 16, 3, 3, 3), np.uint16)            # conv result is exactly 0
    bias = np.full(C, case["bias"], np.float32)
    if "bias_channel0" in case:
        bias[0] = case["bias_channel0"]
    gamma = np.full(C, case["gamma"], np.float32)
    if "gamma_channel0" in case:
        gamma[0] = case["gamma_channel0"]
    residual = None
    if case["residual"] is not None:
        residual = f32_to_bits(np.full((1, 1, 2, 2, C), case["residual"], np.float32))
    got = oracle.conv3d(x, w, bias=bias, residual=residual, gamma=f32_to_bits(gamma),
                        norm_silu=True, intermediates=True)
    y = b2f(got["y"]).reshape(-1, C)
    np.testing.assert_array_equal(y[:, 0], np.float32(case["out_channel0"]))
    np.testing.assert_array_equal(y[:, 1:], np.float32(case["out"]))
    np.testing.assert_allclose(got["den"], case["den"], rtol=1e-6)
    v = b2f(got["value"]).reshape(-1, C)
    np.testing.assert_array_equal(v[:, 1:], np.float32(case["value"]))


def test_epilogue_sqrt_c_is_output_channels():
    """The norm scales by sqrt(Co) of the layer, here Co=64, not a fixed 320:
    constant row 1 gives normalized=B(1/8)=0.125, scaled=1, out=0.73046875."""
    w = np.zeros((64, 8, 3, 3, 3), np.uint16)
    x = np.zeros((1, 3, 3, 3, 8), np.uint16)
    got = oracle.conv3d(x, w, bias=np.ones(64, np.float32), gamma=f32_to_bits(np.ones(64, np.float32)),
                        norm_silu=True, intermediates=True)
    np.testing.assert_allclose(got["den"], 8.0)
    np.testing.assert_array_equal(b2f(got["y"]), np.float32(0.73046875))


# ---------------------------------------------------------------- reflect padding

def test_reflect_pad_matches_torch():
    rng = np.random.default_rng(51)
    x = rand_bf16(rng, (2, 3, 5, 6, 8))
    got = oracle.reflect_pad_hw(x, (1, 1), (1, 0))
    xt = torch.from_numpy(b2f(x).astype(np.float64)).permute(0, 4, 1, 2, 3)   # N, C, D, H, W
    want = F.pad(xt, (1, 0, 1, 1, 0, 0), mode="reflect").permute(0, 2, 3, 4, 1).numpy()
    assert np.array_equal(b2f(got).astype(np.float64), want)


def test_reflect_pad_hand_example():
    x = np.arange(3 * 4, dtype=np.uint16).reshape(1, 1, 3, 4, 1)
    got = oracle.reflect_pad_hw(x, (1, 1), (1, 1))[0, 0, :, :, 0]
    want = np.array([[5, 4, 5, 6, 7, 6],
                     [1, 0, 1, 2, 3, 2],
                     [5, 4, 5, 6, 7, 6],
                     [9, 8, 9, 10, 11, 10],
                     [5, 4, 5, 6, 7, 6]])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("stride", [(1, 1, 1), (2, 2, 2), (1, 2, 2)])
def test_reflect_conv_matches_torch(stride):
    """Causal time pad (zeros) + reflect spatial pad, as the H3 encoder's convs."""
    rng = np.random.default_rng(52)
    x = rand_bf16(rng, (1, 5, 6, 7, 8))
    w = rand_bf16(rng, (16, 8, 3, 3, 3), 0.2)
    got = oracle.conv3d_reflect(x, w, stride=stride, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1),
                                intermediates=True)
    xt = torch.from_numpy(b2f(x).astype(np.float64)).permute(0, 4, 1, 2, 3)
    xt = F.pad(xt, (1, 1, 1, 1, 0, 0), mode="reflect")
    xt = F.pad(xt, (0, 0, 0, 0, 2, 0))
    ref = F.conv3d(xt, torch.from_numpy(b2f(w).astype(np.float64)), stride=stride)
    assert_acc_matches(got["acc"], ref.permute(0, 2, 3, 4, 1).numpy())
    with pytest.raises(ValueError):
        oracle.reflect_pad_hw(rand_bf16(rng, (1, 1, 1, 4, 8)), (1, 1), (1, 1))

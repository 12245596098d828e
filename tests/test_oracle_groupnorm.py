"""Pins for the channels-last GroupNorm (+ SiLU) oracle.

What the norm computes is fixed by the FlyDSL issue page (MiniMax H3 comment,
the GroupNorm argument): statistics per frame once time is folded into the
batch, groups of C/G consecutive channels, then SiLU; GroupNorm itself is the
textbook definition (population variance, eps inside the square root, per-
channel affine). Each test below targets a mistake the oracle could make:

  - the fold or the group->channel mapping: PyTorch's F.group_norm in fp64 on
    the NCHW tensor made by an explicit permute + reshape,
  - frames not isolated (or isolated when they should not be): editing one
    frame,
  - unbiased instead of population variance, eps outside the root: the +-v
    closed form,
  - consecutive vs strided groups: per-channel constants with a closed form,
  - a dropped mean or a lost shift: x + c gives the same output,
  - a wrong SiLU or a missing rounding point: SiLU written as a * expit(a)
    through scipy, and constant groups where the output is B(silu(B(beta))).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import oracle
from oracle.groupnorm import bf16_rne, bf16_value


def torch_bits(a):
    """bf16 bits through PyTorch's own fp32 -> bf16 cast (a library RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_x(rng, shape, scale=1.0, offset=0.0):
    return torch_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
                      + np.float32(offset))


def affine_params(rng, c):
    gamma = rng.uniform(0.5, 1.5, size=c).astype(np.float32)
    beta = (0.2 * rng.standard_normal(c)).astype(np.float32)
    return gamma, beta


def ref_torch(x_bits, groups, gamma, beta, eps, t_isolated):
    """fp64 F.group_norm on the channels-first tensor: [N*D, C, H, W] (frames
    folded into the batch) or [N, C, D, H, W]; returned NDHWC."""
    x = torch.from_numpy(bf16_value(x_bits))
    N, D, H, W, C = x.shape
    if t_isolated:
        xc = x.reshape(N * D, H, W, C).permute(0, 3, 1, 2)
    else:
        xc = x.permute(0, 4, 1, 2, 3)
    y = F.group_norm(xc, groups, torch.from_numpy(gamma.astype(np.float64)),
                     torch.from_numpy(beta.astype(np.float64)), eps)
    if t_isolated:
        return y.permute(0, 2, 3, 1).reshape(N, D, H, W, C).numpy()
    return y.permute(0, 2, 3, 4, 1).numpy()


# ------------------------------------------------------------ library check

@pytest.mark.parametrize("t_isolated", [True, False])
@pytest.mark.parametrize("shape,groups", [((2, 3, 5, 7, 64), 32), ((1, 4, 6, 5, 96), 32),
                                          ((1, 2, 3, 4, 48), 8)])
def test_matches_torch_group_norm(shape, groups, t_isolated):
    rng = np.random.default_rng(11)
    x = rand_x(rng, shape, scale=2.0, offset=0.5)
    gamma, beta = affine_params(rng, shape[-1])
    out = oracle.group_norm(x, groups, gamma, beta, eps=1e-5, t_isolated=t_isolated,
                            intermediates=True)
    ref = ref_torch(x, groups, gamma, beta, 1e-5, t_isolated)
    np.testing.assert_allclose(out["affine"], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out["a"], torch_bits(ref.astype(np.float32)))


def test_silu_is_a_times_sigmoid_of_rounded_a():
    rng = np.random.default_rng(12)
    x = rand_x(rng, (1, 3, 4, 6, 64), scale=1.5)
    gamma, beta = affine_params(rng, 64)
    gamma *= 3.0                           # reach the SiLU's flat and linear parts
    out = oracle.group_norm(x, 32, gamma, beta, silu=True, intermediates=True)
    a = bf16_value(out["a"])
    assert np.array_equal(out["y"], torch_bits((a * expit(a)).astype(np.float32)))
    plain = oracle.group_norm(x, 32, gamma, beta, silu=False)
    assert np.array_equal(plain, out["a"])


# ------------------------------------------------------------ frame isolation

def test_time_isolated_statistics_are_per_frame():
    rng = np.random.default_rng(13)
    x = rand_x(rng, (1, 3, 4, 4, 32))
    gamma, beta = affine_params(rng, 32)
    x2 = x.copy()
    x2[0, 1] = rand_x(rng, (4, 4, 32), scale=5.0, offset=3.0)    # rewrite frame 1
    y1 = oracle.group_norm(x, 8, gamma, beta, silu=True)
    y2 = oracle.group_norm(x2, 8, gamma, beta, silu=True)
    assert np.array_equal(y1[0, 0], y2[0, 0]) and np.array_equal(y1[0, 2], y2[0, 2])
    assert not np.array_equal(y1[0, 1], y2[0, 1])
    # over the whole clip the edit reaches every frame
    z1 = oracle.group_norm(x, 8, gamma, beta, t_isolated=False)
    z2 = oracle.group_norm(x2, 8, gamma, beta, t_isolated=False)
    assert not np.array_equal(z1[0, 0], z2[0, 0])


def test_single_frame_clip_is_the_same_either_way():
    rng = np.random.default_rng(14)
    x = rand_x(rng, (2, 1, 5, 6, 32))
    gamma, beta = affine_params(rng, 32)
    assert np.array_equal(oracle.group_norm(x, 32, gamma, beta, t_isolated=True),
                          oracle.group_norm(x, 32, gamma, beta, t_isolated=False))


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("eps", [0.25, 1.0])
def test_plus_minus_v_group(eps):
    """Half of each group at +v, half at -v: mean 0, population variance v^2,
    so the norm is +-v / sqrt(v^2 + eps) (not v*sqrt(n/(n-1)), not v/(v+eps))."""
    v = 2.0
    x = np.zeros((1, 2, 2, 2, 16), dtype=np.float32)
    x[..., 0::2] = v
    x[..., 1::2] = -v
    xb = torch_bits(x)
    ones, zeros = np.ones(16, np.float32), np.zeros(16, np.float32)
    out = oracle.group_norm(xb, 4, ones, zeros, eps=eps, intermediates=True)
    want = v / math.sqrt(v * v + eps)
    assert np.allclose(out["affine"][..., 0::2], want, rtol=1e-14)
    assert np.allclose(out["affine"][..., 1::2], -want, rtol=1e-14)
    assert np.allclose(out["mean"], 0.0) and np.allclose(out["rstd"], 1 / math.sqrt(v * v + eps))


def test_groups_are_consecutive_channels():
    """x[..., c] = c everywhere: group g holds channels 4g..4g+3 with values
    4g + {0,1,2,3}, so every group has mean 4g+1.5 and variance 1.25 and the
    output depends only on c % 4. Strided groups {g, g+G, ...} would not."""
    C, G = 32, 8
    x = np.broadcast_to(np.arange(C, dtype=np.float32), (1, 2, 3, 3, C)).copy()
    ones, zeros = np.ones(C, np.float32), np.zeros(C, np.float32)
    out = oracle.group_norm(torch_bits(x), G, ones, zeros, eps=0.0, intermediates=True)
    k = np.arange(C) % 4
    want = (k - 1.5) / math.sqrt(1.25)
    assert np.allclose(out["affine"], np.broadcast_to(want, out["affine"].shape), rtol=1e-14)
    assert np.allclose(out["mean"], 4 * np.arange(G) + 1.5)


def test_constant_group_gives_silu_of_beta():
    """var = 0: the norm is 0 (eps keeps it finite), a = B(beta), y = B(silu(a))."""
    C = 16
    x = torch_bits(np.full((1, 2, 3, 3, C), 0.75, np.float32))
    beta = np.array([0.0, 1.0, -1.0, 2.0] * 4, np.float32)
    gamma = np.full(C, 3.0, np.float32)
    out = oracle.group_norm(x, 4, gamma, beta, silu=True, intermediates=True)
    silu = {0.0: 0.0, 1.0: 1.0 / (1.0 + math.exp(-1.0)), -1.0: -1.0 / (1.0 + math.exp(1.0)),
            2.0: 2.0 / (1.0 + math.exp(-2.0))}
    # bf16 by hand: 0.7310586 -> 187/256, -0.2689414 -> -138/512, 1.7615942 -> 225/128
    by_hand = {0.0: 0.0, 1.0: 187 / 256, -1.0: -138 / 512, 2.0: 225 / 128}
    for c in range(C):
        b = float(beta[c])
        assert np.all(bf16_value(out["a"][..., c]) == b)
        assert np.all(bf16_value(out["y"][..., c]) == by_hand[b])
        assert abs(by_hand[b] - silu[b]) <= 2.0 ** -8 * max(abs(silu[b]), 2 ** -126)


def test_shift_invariance():
    """Integer data plus 64 is exact in bf16; mean moves by 64, nothing else."""
    rng = np.random.default_rng(15)
    xi = rng.integers(-3, 4, size=(1, 2, 4, 5, 32)).astype(np.float32)
    gamma, beta = affine_params(rng, 32)
    a = oracle.group_norm(torch_bits(xi), 8, gamma, beta, intermediates=True)
    b = oracle.group_norm(torch_bits(xi + 64), 8, gamma, beta, intermediates=True)
    assert np.allclose(b["mean"], a["mean"] + 64, rtol=0, atol=1e-12)
    assert np.allclose(b["affine"], a["affine"], rtol=0, atol=1e-12)


def test_bf16_helpers_round_to_nearest_even():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3e-39], np.float32)
    assert np.array_equal(bf16_rne(v), torch_bits(v))
    # 1 + 2^-8 and 1 + 3 * 2^-8 are ties: both go to the even neighbour
    assert np.array_equal(bf16_value(bf16_rne(v))[:4], [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5])


def test_rejects_channels_not_divisible_by_groups():
    x = np.zeros((1, 1, 1, 1, 12), np.uint16)
    with pytest.raises(ValueError):
        oracle.group_norm(x, 8, np.ones(12, np.float32), np.zeros(12, np.float32))

"""GPU checks of 2D and 1x3x3 layers run through the 3x3x3 kernels.

A 2D weight packed by conv3d_pack_weight_2d sits in the last temporal slice;
a causal conv on single frames then computes each frame's 2D conv (Qwen PR,
"T=1 degeneration"), and a 1x3x3 conv over d frames is the same call on the
[n*d][1][h][w][c] view. Integer data keeps every sum exact, so results are
compared bit for bit with the oracle's conv using the zero-extended 3x3x3
weight (whose T=1 identity with F.conv2d is pinned in test_oracle_pins.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from convolution_video_vae_amd.layer import Conv3d

pytestmark = pytest.mark.gpu


def bits(t):
    return workloads.bf16_bits(t.cpu())


def int_weight_2d(rng, cout, cin):
    return torch.from_numpy(rng.integers(-1, 2, size=(cout, cin, 3, 3)).astype(np.float32)).to(torch.bfloat16)


def extend(w2d):
    """[cout][cin][3][3] -> [cout][cin][3][3][3] with the 2D taps at kd = 2."""
    w3 = torch.zeros(w2d.shape[:2] + (3, 3, 3), dtype=torch.bfloat16)
    w3[:, :, 2] = w2d
    return w3


CASES = [
    # label, x shape (NDHWC, D = 1), cout, stride, pad_lo, pad_hi
    ("qwen_2d_96", (1, 1, 40, 56, 96), 96, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("qwen_2d_96_downsample", (1, 1, 40, 56, 96), 96, (1, 2, 2), (2, 0, 0), (0, 1, 1)),
    ("batch2_2d_64_to_128", (2, 1, 17, 23, 64), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
]


@pytest.mark.parametrize("label,xs,cout,st,lo,hi", CASES, ids=[c[0] for c in CASES])
def test_2d_conv_from_packed_2d_weight(label, xs, cout, st, lo, hi):
    rng = np.random.default_rng(41)
    print(f"[conv2d] {label} x={xs} cout={cout}", flush=True)
    x = torch.from_numpy(rng.integers(-2, 3, size=xs).astype(np.float32)).to(torch.bfloat16)
    w2 = int_weight_2d(rng, cout, xs[4])
    conv = Conv3d(w2.cuda(), xs, stride=st, pad_lo=lo, pad_hi=hi)
    y = conv(x.cuda())
    # the same layer with the zero-extended 3x3x3 weight
    y3 = Conv3d(extend(w2).cuda(), xs, stride=st, pad_lo=lo, pad_hi=hi)(x.cuda())
    torch.cuda.synchronize()
    ref = oracle.conv3d(bits(x), bits(extend(w2)), stride=st, pad_lo=lo, pad_hi=hi)
    assert np.array_equal(bits(y), ref)
    assert np.array_equal(bits(y3), ref)


def test_1x3x3_over_frames_is_the_frame_batched_2d_conv():
    rng = np.random.default_rng(42)
    n, d, h, w, c, cout = 2, 5, 12, 18, 64, 64
    x = torch.from_numpy(rng.integers(-2, 3, size=(n, d, h, w, c)).astype(np.float32)).to(torch.bfloat16)
    w2 = int_weight_2d(rng, cout, c)
    view = x.cuda().view(n * d, 1, h, w, c)                      # no copy in NDHWC
    conv = Conv3d(w2.cuda(), tuple(view.shape), pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    y = conv(view).view(n, d, h, w, cout)
    torch.cuda.synchronize()
    got = bits(y)
    for k in range(d):                                           # per frame, its own 2D conv
        ref = oracle.conv3d(bits(x[:, k:k + 1]), bits(extend(w2)), pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
        assert np.array_equal(got[:, k:k + 1], ref), k

"""Pins for the streaming oracle (padded outputs, history planes, caches).

The property that fixes the cuDNN page's streaming scheme ("Causal Conv3D
with Cache", "Normalization and Padding Variant") is that running a causal
encoder chunk by chunk, each chunk's input padded with the previous chunk's
last two frames, gives exactly what the whole clip gives at once. These tests
check the oracle's packing, padding and caches against that property with the
oracle's own direct conv (whose result does not depend on where zero
operands come from), plus the spatial-padding variant against the stride-2
conv's own zero pad (Qwen PR, "Test shapes" table 2).
"""
import numpy as np
import pytest

import oracle
from oracle.stream import cache_tail, pack_stream_input, pad_output

CAUSAL = dict(pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))


def bits(rng, shape, scale=1.0):
    return oracle.bf16_round(rng.standard_normal(int(np.prod(shape))).astype(np.float32)
                             * np.float32(scale)).reshape(shape)


def widen(w, cin_pad):
    """OIDHW weight with zero input channels up to cin_pad."""
    out = np.zeros((w.shape[0], cin_pad) + w.shape[2:], dtype=np.uint16)
    out[:, :w.shape[1]] = w
    return out


@pytest.mark.parametrize("chunks", [[1, 4, 4], [3, 1, 2, 3], [9]])
def test_streamed_first_layer_equals_whole_clip(chunks):
    rng = np.random.default_rng(21)
    T = sum(chunks)
    video = bits(rng, (1, 12, T, 5, 7))                       # NCTHW, 12 channels
    w = bits(rng, (16, 12, 3, 3, 3), 0.1)
    whole = oracle.conv3d(np.transpose(video, (0, 2, 3, 4, 1)), w, **CAUSAL)
    outs, cache, t0 = [], None, 0
    for t in chunks:
        padded, cache_new = pack_stream_input(video[:, :, t0:t0 + t], history=cache, c_pad=16)
        assert padded.shape == (1, t + 2, 7, 9, 16)
        outs.append(oracle.conv3d(padded, widen(w, 16)))       # valid conv
        seen = np.transpose(video[:, :, :t0 + t], (0, 2, 3, 4, 1))
        assert np.array_equal(cache_new, seen[:, -min(2, t0 + t):])
        cache, t0 = cache_new, t0 + t
    assert np.array_equal(np.concatenate(outs, axis=1), whole)


def test_pack_zeros_border_channels_and_missing_history():
    rng = np.random.default_rng(22)
    chunk = bits(rng, (2, 12, 3, 4, 5))
    for P in (0, 1, 2):
        hist = bits(rng, (2, P, 4, 5, 12)) if P else None
        padded, cache = pack_stream_input(chunk, history=hist, c_pad=16)
        assert not padded[:, :2 - P].any()
        assert not padded[:, :, 0].any() and not padded[:, :, -1].any()
        assert not padded[:, :, :, 0].any() and not padded[:, :, :, -1].any()
        assert not padded[..., 12:].any()
        assert np.array_equal(padded[:, 2:, 1:-1, 1:-1, :12], np.transpose(chunk, (0, 2, 3, 4, 1)))
        if P:
            assert np.array_equal(padded[:, 2 - P:2, 1:-1, 1:-1, :12], hist)
        assert cache.shape == (2, min(2, 3 + P), 4, 5, 12)


@pytest.mark.parametrize("chunks", [[2, 3], [1, 1, 3]])
def test_streamed_two_layer_chain_equals_whole_clip(chunks):
    """Layer 1: conv + bias + residual + L2 norm + SiLU, output written padded
    with the previous chunk's last two activated frames as history; layer 2:
    valid conv on that buffer. Equal to the causal chain over the whole clip."""
    rng = np.random.default_rng(23)
    T, H, W, C1, C2, C3 = sum(chunks), 4, 6, 16, 32, 16
    x = bits(rng, (1, T, H, W, C1))
    w1 = bits(rng, (C2, C1, 3, 3, 3), 0.1)
    w2 = bits(rng, (C3, C2, 3, 3, 3), 0.1)
    b1 = (0.1 * rng.standard_normal(C2)).astype(np.float32)
    g1 = oracle.bf16_round(rng.uniform(0.5, 1.5, C2).astype(np.float32))
    res = bits(rng, (1, T, H, W, C2))
    a_whole = oracle.conv3d(x, w1, bias=b1, residual=res, gamma=g1, norm_silu=True, **CAUSAL)
    y_whole = oracle.conv3d(a_whole, w2, **CAUSAL)
    xcache = acache = None
    ys, t0 = [], 0
    for t in chunks:
        xp = pad_output(x[:, t0:t0 + t], (2, 1, 1), (0, 1, 1), history=xcache)
        a = oracle.conv3d(xp, w1, bias=b1, residual=res[:, t0:t0 + t], gamma=g1, norm_silu=True)
        ap = pad_output(a, (2, 1, 1), (0, 1, 1), history=acache)
        ys.append(oracle.conv3d(ap, w2))
        xcache = cache_tail(x[:, t0:t0 + t], min(2, t0 + t), previous=xcache)
        acache = cache_tail(a, min(2, t0 + t), previous=acache)
        t0 += t
    assert np.array_equal(np.concatenate(ys, axis=1), y_whole)


def test_bottom_right_pad_feeds_stride_two_conv():
    """Spatial-padding variant: a zero bottom row and right column written by
    the producer equal the stride-2 conv's own (0, 1) zero pad."""
    rng = np.random.default_rng(24)
    x = bits(rng, (1, 5, 7, 9, 16))
    w1 = bits(rng, (16, 16, 3, 3, 3), 0.1)
    w2 = bits(rng, (32, 16, 3, 3, 3), 0.1)
    b1 = (0.1 * rng.standard_normal(16)).astype(np.float32)
    res = bits(rng, (1, 3, 5, 7, 16))
    a = oracle.conv3d(x, w1, bias=b1, residual=res)            # valid: [1,3,5,7,16]
    ap = pad_output(a, (0, 0, 0), (0, 1, 1))                   # [1,3,6,8,16]
    assert ap.shape == (1, 3, 6, 8, 16)
    y_padded = oracle.conv3d(ap, w2, stride=(1, 2, 2), pad_lo=(2, 0, 0), pad_hi=(0, 0, 0))
    y_direct = oracle.conv3d(a, w2, stride=(1, 2, 2), pad_lo=(2, 0, 0), pad_hi=(0, 1, 1))
    assert np.array_equal(y_padded, y_direct)


def test_cache_tail_and_history_edge_cases():
    rng = np.random.default_rng(25)
    cur = bits(rng, (1, 1, 2, 2, 8))
    prev = bits(rng, (1, 2, 2, 2, 8))
    assert np.array_equal(cache_tail(cur, 2, previous=prev), np.concatenate([prev[:, 1:], cur], 1))
    assert np.array_equal(cache_tail(cur, 1), cur)
    with pytest.raises(ValueError):
        cache_tail(cur, 2)
    with pytest.raises(ValueError):
        pad_output(cur, (1, 1, 1), (0, 1, 1), history=prev)
    with pytest.raises(ValueError):
        pack_stream_input(bits(rng, (1, 12, 1, 2, 2)), c_pad=8)


@pytest.mark.parametrize("with_bias,with_res", [(False, False), (True, False), (True, True)])
def test_standalone_norm_silu_equals_the_fused_contract(with_bias, with_res):
    """Post-operations on a raw conv output equal the oracle's own fused conv
    (its C implementation of the same contract), bit for bit."""
    from oracle.stream import norm_silu
    rng = np.random.default_rng(26)
    x = bits(rng, (1, 3, 4, 5, 32))
    w = bits(rng, (64, 32, 3, 3, 3), 0.05)
    b = (0.1 * rng.standard_normal(64)).astype(np.float32) if with_bias else None
    res = bits(rng, (1, 3, 4, 5, 64)) if with_res else None
    g = oracle.bf16_round(rng.uniform(0.5, 1.5, 64).astype(np.float32))
    raw = oracle.conv3d(x, w, **CAUSAL)
    fused = oracle.conv3d(x, w, bias=b, residual=res, gamma=g, norm_silu=True, intermediates=True,
                          **CAUSAL)
    got = norm_silu(raw, g, bias=b, residual=res, intermediates=True)
    assert np.array_equal(got["y"], fused["y"])
    assert np.array_equal(got["value"], fused["value"])


def test_standalone_norm_silu_closed_forms():
    """A pixel whose row is (v, 0, ..., 0): den = |v|, the first channel's
    norm is sign(v), scaled by sqrt(C); C = 64, gamma 0.5 gives a = 4."""
    from oracle.stream import norm_silu
    raw = np.zeros((1, 64), np.uint16)
    raw[0, 0] = oracle.bf16_round(np.float32([-3.0]))[0]
    g = oracle.bf16_round(np.full(64, 0.5, np.float32))
    y = oracle.bf16_to_f32(norm_silu(raw, g))
    silu = lambda a: a / (1 + np.exp(-a))
    # a = B(B(-1 * 8) * 0.5) = -4; B(silu(-4)) = B(-0.0719...) = -0.07177734375 (RNE by hand:
    # -0.0719448 / 2^-11 = -147.34 -> -147 * 2^-11)
    assert y[0, 0] == np.float32(-147 * 2.0 ** -11)
    assert abs(y[0, 0] - silu(-4.0)) < 2.0 ** -11
    assert np.all(y[0, 1:] == 0)

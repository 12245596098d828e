"""GPU parity of the streaming pieces: padded outputs with history planes and
frame caches (conv3d_fwd_padded), first-layer chunk packing
(conv3d_stream_pack_input), and chunked runs against whole clips.

Placement, zero fill, history and caches are data movement: they are checked
bit for bit (integer conv data makes the whole padded output exact). Float
outputs use the parity rule of tests/parity.py against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import convolution_video_vae_amd as cv
import workloads
from convolution_video_vae_amd.layer import Conv3d, stream_pack_input
from oracle.stream import cache_tail, pack_stream_input, pad_output
from guard import Guarded
from parity import check

pytestmark = pytest.mark.gpu


def bits(t):
    return workloads.bf16_bits(t.cpu())


def from_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def noise_bits(rng, shape):
    """Arbitrary finite bf16 patterns (a sentinel for untouched memory)."""
    return (rng.integers(0, 0x7f00, size=shape) | (rng.integers(0, 2, size=shape) << 15)).astype(np.uint16)


VALID = ((1, 1, 1), (0, 0, 0), (0, 0, 0))
CAUSAL = ((1, 1, 1), (2, 1, 1), (0, 1, 1))

PAD_CASES = [
    # name, x shape, cout, history frames, cache frames, (stride, pad_lo, pad_hi),
    # split_k, plan
    ("slot_path_128", (1, 5, 10, 20, 32), 128, 1, 2, VALID, 0, None),
    ("generic_path_160", (1, 4, 6, 9, 64), 160, 2, 2, VALID, 0, None),
    ("split_k_512", (1, 3, 5, 5, 512), 512, 0, 1, VALID, 0, None),
    ("one_output_frame", (1, 3, 7, 11, 32), 64, 2, 2, VALID, 0, None),
    # slot kernels write the padded output in place (the placement pass then
    # writes only the border, history and cache)
    ("in_place_slot_512x128", (1, 5, 10, 40, 32), 128, 2, 2, CAUSAL, 1, "ns=-2"),
    ("in_place_slot_512x128_nobias", (1, 5, 10, 40, 32), 128, 0, 1, CAUSAL, 1, "ns=-2"),
    ("in_place_slot_384x160_batch2", (2, 4, 9, 21, 64), 160, 1, 2, CAUSAL, 1, "ns=-2"),
    ("in_place_pair_view", (1, 4, 10, 24, 64), 128, 2, 2, ((1, 2, 2), (2, 0, 0), (0, 1, 1)), 1,
     "ns=-3"),
    # 289 tiles on 256 persistent work-groups: tiles whose epilogue (the
    # generic one, padded output, no post-operations) precedes the next
    # tile's main loop
    ("in_place_slot_persistent_nobias", (1, 9, 64, 254, 32), 128, 0, 1, CAUSAL, 1,
     "persistent=1"),
]


@pytest.mark.parametrize("name,xs,cout,P,cf,geo,split_k,plan_has", PAD_CASES,
                         ids=[c[0] for c in PAD_CASES])
def test_padded_output_integer_exact(name, xs, cout, P, cf, geo, split_k, plan_has):
    print(f"[stream] padded {name} x={xs} cout={cout} P={P} cache={cf}", flush=True)
    rng = np.random.default_rng(31)
    x, w, b = workloads.integer_tensors(xs, cout, seed=5, bias=True)
    if name.endswith("_nobias"):   # the plain store path of the kernel
        b = None
    stride, lo, hi = geo
    conv = Conv3d(w.cuda(), xs, stride=stride, pad_lo=lo, pad_hi=hi, split_k=split_k, bias=b,
                  out_pad_lo=(2, 1, 1), out_pad_hi=(0, 1, 1), history_frames=P, cache_frames=cf)
    if plan_has:
        e = cv.make_epilogue(bias=conv.bias)
        plan = cv.conv3d_plan_describe(conv.desc, e if e.flags else None)
        assert plan_has in plan and "reduce=0" in plan, plan
    Do, Ho, Wo = conv.out_dhw
    y0 = noise_bits(rng, conv.out_shape)
    hist = noise_bits(rng, (xs[0], P, Ho, Wo, cout))
    y0[:, 2 - P:2, 1:1 + Ho, 1:1 + Wo] = hist
    c0 = noise_bits(rng, conv.cache_shape)
    yg = Guarded(y0.shape, fill=y0)
    cg = Guarded(c0.shape, fill=c0)
    y, cache = yg.t, cg.t
    conv(x.cuda(), y=y, cache=cache)
    torch.cuda.synchronize()
    yg.assert_intact(name + " padded y")
    cg.assert_intact(name + " cache")
    ref = oracle.conv3d(bits(x), bits(w), bias=None if b is None else b.numpy(), stride=stride,
                        pad_lo=lo, pad_hi=hi)
    want = pad_output(ref, (2, 1, 1), (0, 1, 1), history=hist if P else None)
    assert np.array_equal(bits(y), want)
    k = min(cf, Do)
    got_cache = bits(cache)
    assert np.array_equal(got_cache[:, cf - k:], ref[:, Do - k:])
    assert np.array_equal(got_cache[:, :cf - k], c0[:, :cf - k])      # caller's frames kept


def test_padded_fused_norm_layer():
    """Wan fused 160->320 (bias, residual, L2 norm, SiLU) at a small frame
    size, output padded for the next causal conv, two history frames."""
    L = workloads.LAYERS["wan_fused_160to320"]
    xs = (1, 7, 10, 18, 160)
    t = workloads.make_tensors(L, x_shape=xs)
    conv = Conv3d(t.w.cuda(), xs, bias=t.bias, gamma=t.gamma, norm_silu=True, residual=True,
                  out_pad_lo=(2, 1, 1), out_pad_hi=(0, 1, 1), history_frames=2, cache_frames=2)
    Do, Ho, Wo = conv.out_dhw
    rng = np.random.default_rng(32)
    y0 = noise_bits(rng, conv.out_shape)
    hist = noise_bits(rng, (1, 2, Ho, Wo, 320))
    y0[:, 0:2, 1:1 + Ho, 1:1 + Wo] = hist
    y = from_bits(y0).cuda()
    cache = torch.empty(conv.cache_shape, dtype=torch.bfloat16, device="cuda")
    conv(t.x.cuda(), residual=t.residual.cuda(), y=y, cache=cache)
    torch.cuda.synchronize()
    got = bits(y)
    ref = oracle.conv3d(bits(t.x), bits(t.w), bias=t.bias.numpy(), residual=bits(t.residual),
                        gamma=bits(t.gamma), norm_silu=True, intermediates=True)
    check(got[:, 2:, 1:-1, 1:-1], ref, fused=True, gamma_bits=bits(t.gamma), what="padded fused")
    border = pad_output(np.zeros((1, Do, Ho, Wo, 320), np.uint16), (2, 1, 1), (0, 1, 1), history=hist)
    mask = np.ones(got.shape, bool)
    mask[:, 2:, 1:-1, 1:-1] = False
    assert np.array_equal(got[mask], border[mask])                    # zeros and history
    assert np.array_equal(bits(cache), got[:, -2:, 1:-1, 1:-1])       # cache = last frames


def test_bottom_right_pad_feeds_stride_two_conv():
    """Spatial-padding variant: bias + residual written with a zero bottom row
    and right column, then a stride-(1,2,2) valid conv on it."""
    rng = np.random.default_rng(33)
    x, w1, b1 = workloads.integer_tensors((1, 5, 9, 13, 64), 64, seed=6, bias=True)
    res = torch.from_numpy(rng.integers(-3, 4, size=(1, 3, 7, 11, 64)).astype(np.float32)).to(torch.bfloat16)
    _, w2, _ = workloads.integer_tensors((1, 3, 8, 12, 64), 128, seed=7)
    c1 = Conv3d(w1.cuda(), x.shape, bias=b1, residual=True, out_pad_lo=(0, 0, 0),
                out_pad_hi=(0, 1, 1))
    a = c1(x.cuda(), residual=res.cuda())
    assert tuple(a.shape) == (1, 3, 8, 12, 64)
    c2 = Conv3d(w2.cuda(), tuple(a.shape), stride=(1, 2, 2), pad_lo=(2, 0, 0))
    y = c2(a)
    torch.cuda.synchronize()
    a_ref = oracle.conv3d(bits(x), bits(w1), bias=b1.numpy(), residual=bits(res))
    assert np.array_equal(bits(a), pad_output(a_ref, (0, 0, 0), (0, 1, 1)))
    y_ref = oracle.conv3d(a_ref, bits(w2), stride=(1, 2, 2), pad_lo=(2, 0, 0), pad_hi=(0, 1, 1))
    assert np.array_equal(bits(y), y_ref)


@pytest.mark.parametrize("P", [0, 1, 2])
def test_stream_pack_strided_chunk(P):
    rng = np.random.default_rng(34 + P)
    video = from_bits(noise_bits(rng, (2, 12, 9, 6, 11))).cuda()      # NCTHW
    chunk = video[:, :, 3:7]                                           # strided view, T = 4
    hist = from_bits(noise_bits(rng, (2, P, 6, 11, 12))).cuda() if P else None
    print(f"[stream] pack P={P} strides={chunk.stride()}", flush=True)
    padded, cache = stream_pack_input(chunk, hist, c_pad=16)
    torch.cuda.synchronize()
    want_p, want_c = pack_stream_input(bits(chunk.contiguous()), None if hist is None else bits(hist),
                                       c_pad=16)
    assert np.array_equal(bits(padded), want_p)
    assert np.array_equal(bits(cache), want_c)


def test_streamed_first_layer_equals_whole_clip():
    """Wan's 12-channel first layer over chunks of 1, 4 and 4 frames: chunk
    packing with the previous raw frames, then a valid conv; the outputs
    joined equal the causal conv of the whole clip."""
    rng = np.random.default_rng(35)
    H, W, T = 12, 20, 9
    v32 = rng.standard_normal((1, 12, T, H, W)).astype(np.float32)
    video = torch.from_numpy(v32).to(torch.bfloat16)
    w32 = (rng.standard_normal((160, 12, 3, 3, 3)) * np.sqrt(1 / 324)).astype(np.float32)
    w = torch.from_numpy(w32).to(torch.bfloat16)
    wide = torch.zeros((160, 32, 3, 3, 3), dtype=torch.bfloat16)
    wide[:, :12] = w
    vd = video.cuda()
    outs, cache, t0 = [], None, 0
    for t in (1, 4, 4):
        padded, cache = stream_pack_input(vd[:, :, t0:t0 + t], cache, c_pad=32)
        conv = Conv3d(wide.cuda(), tuple(padded.shape))
        outs.append(conv(padded))
        t0 += t
    torch.cuda.synchronize()
    got = bits(torch.cat(outs, dim=1))
    ref = oracle.conv3d(bits(video.permute(0, 2, 3, 4, 1).contiguous()), bits(w), pad_lo=(2, 1, 1),
                        pad_hi=(0, 1, 1), intermediates=True)
    diag = check(got, ref, what="streamed first layer")
    assert diag["bit_identical"] > 0.999, diag


def test_streamed_chain_mechanics():
    """Two streamed layers: a fused layer writes its activations padded, with
    the previous chunk's cached activations as history; the next layer runs a
    valid conv on that buffer. Each step is checked against the oracle on the
    GPU's own inputs, and the caches against the GPU's own activations."""
    L = workloads.LAYERS["wan_fused_160to320"]
    H, W, C1, C2, C3 = 8, 12, 160, 320, 64
    t1 = workloads.make_tensors(L, x_shape=(1, 6, H, W, C1))
    x_all = t1.x
    _, w2, _ = workloads.integer_tensors((1, 3, H, W, C2), C3, seed=8)
    rng = np.random.default_rng(36)
    res_all = torch.from_numpy(rng.standard_normal((1, 6, H, W, C2)).astype(np.float32)).to(torch.bfloat16)
    xcache = acache = None
    t0 = 0
    for t in (2, 1, 3):
        xp = pad_output(bits(x_all[:, t0:t0 + t]), (2, 1, 1), (0, 1, 1),
                        history=None if xcache is None else xcache)
        P = 0 if acache is None else acache.shape[1]
        c1 = Conv3d(t1.w.cuda(), xp.shape, bias=t1.bias, gamma=t1.gamma, norm_silu=True,
                    residual=True, out_pad_lo=(2, 1, 1), out_pad_hi=(0, 1, 1), history_frames=P,
                    cache_frames=min(2, t0 + t))
        ybuf = torch.zeros(c1.out_shape, dtype=torch.bfloat16)
        if P:
            ybuf[:, 2 - P:2, 1:-1, 1:-1] = from_bits(acache)
        ybuf = ybuf.cuda()
        cache_new = np.zeros(c1.cache_shape, np.uint16)
        old = c1.cache_frames - min(c1.cache_frames, t)
        if old:
            cache_new[:, :old] = acache[:, -old:]
        cache_d = from_bits(cache_new).cuda()
        res = res_all[:, t0:t0 + t].contiguous()
        c1(from_bits(xp).cuda(), residual=res.cuda(), y=ybuf, cache=cache_d)
        c2 = Conv3d(w2.cuda(), tuple(ybuf.shape))
        y2 = c2(ybuf)
        torch.cuda.synchronize()
        a = bits(ybuf)
        ref1 = oracle.conv3d(xp, bits(t1.w), bias=t1.bias.numpy(), residual=bits(res),
                             gamma=bits(t1.gamma), norm_silu=True, intermediates=True)
        check(a[:, 2:, 1:-1, 1:-1], ref1, fused=True, gamma_bits=bits(t1.gamma), what=f"chunk {t0}")
        if P:
            assert np.array_equal(a[:, 2 - P:2, 1:-1, 1:-1], acache)
        assert not a[:, :2 - P].any() and not a[:, :, 0].any() and not a[:, :, :, -1].any()
        ref2 = oracle.conv3d(a, bits(w2), intermediates=True)
        check(bits(y2), ref2, what=f"layer 2 chunk {t0}")
        want_cache = cache_tail(a[:, 2:, 1:-1, 1:-1], c1.cache_frames, previous=acache)
        assert np.array_equal(bits(cache_d), want_cache)
        acache = bits(cache_d)
        xcache = cache_tail(bits(x_all[:, t0:t0 + t]), min(2, t0 + t), previous=xcache)
        t0 += t


def _norm_inputs(rng, shape, c):
    raw = from_bits(oracle.bf16_round(rng.standard_normal(int(np.prod(shape)) * c).astype(np.float32))
                    .reshape(shape + (c,)))
    bias = torch.from_numpy((0.1 * rng.standard_normal(c)).astype(np.float32))
    res = from_bits(oracle.bf16_round(rng.standard_normal(int(np.prod(shape)) * c).astype(np.float32))
                    .reshape(shape + (c,)))
    gamma = from_bits(oracle.bf16_round(rng.uniform(0.5, 1.5, c).astype(np.float32)))
    return raw, bias, res, gamma


@pytest.mark.parametrize("P", [1, 2])
def test_standalone_norm_silu_padded_with_history(P):
    """C640 (above the fused tile): raw conv output -> bias, residual, L2 norm,
    SiLU, written padded, history planes and the cache's older frames copied
    from the previous chunk's cache, residual_out saved."""
    from oracle.stream import norm_silu
    rng = np.random.default_rng(40 + P)
    n, d, h, w, c = 1, 3, 6, 10, 640
    raw, bias, res, gamma = _norm_inputs(rng, (n, d, h, w), c)
    prev = from_bits(noise_bits(rng, (n, P, h, w, c)))
    cf = 2
    y = from_bits(noise_bits(rng, (n, d + 2, h + 2, w + 2, c))).cuda()
    cache = from_bits(noise_bits(rng, (n, cf, h, w, c))).cuda()
    rout = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device="cuda")
    # (the epilogue holds raw addresses: keep every device tensor referenced)
    bd, rd, gd, xd, pd = bias.cuda(), res.cuda(), gamma.cuda(), raw.cuda(), prev.cuda()
    epi = cv.make_epilogue(bias=bd, residual=rd, gamma=gd, residual_out=rout, norm_silu=True)
    op = cv.make_out_pad((2, 1, 1), (0, 1, 1), P, cache, cf)
    print(f"[stream] norm_silu C{c} P={P}", flush=True)
    cv.conv3d_norm_silu(xd, n, d, h, w, c, epi, op, pd, y)
    torch.cuda.synchronize()
    ref = norm_silu(bits(raw), bits(gamma), bias=bias.numpy(), residual=bits(res), intermediates=True)
    got = bits(y)
    check(got[:, 2:, 1:-1, 1:-1], ref, fused=True, gamma_bits=bits(gamma), what=f"norm_silu P={P}")
    assert np.array_equal(bits(rout), ref["value"])
    want = pad_output(np.zeros((n, d, h, w, c), np.uint16), (2, 1, 1), (0, 1, 1), history=bits(prev))
    mask = np.ones(got.shape, bool)
    mask[:, 2:, 1:-1, 1:-1] = False
    assert np.array_equal(got[mask], want[mask])                     # zeros and history
    assert np.array_equal(bits(cache), got[:, -2:, 1:-1, 1:-1])      # d >= 2: current frames


def test_standalone_norm_silu_contiguous_and_saved_value():
    from oracle.stream import norm_silu
    rng = np.random.default_rng(44)
    n, d, h, w, c = 2, 2, 5, 7, 320
    raw, bias, _, gamma = _norm_inputs(rng, (n, d, h, w), c)
    y = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device="cuda")
    saved = torch.empty_like(y)
    bd, gd, xd = bias.cuda(), gamma.cuda(), raw.cuda()
    epi = cv.make_epilogue(bias=bd, gamma=gd, residual_out=saved, norm_silu=True)
    cv.conv3d_norm_silu(xd, n, d, h, w, c, epi, None, None, y)
    torch.cuda.synchronize()
    ref = norm_silu(bits(raw), bits(gamma), bias=bias.numpy(), intermediates=True)
    check(bits(y), ref, fused=True, gamma_bits=bits(gamma), what="norm_silu contiguous")
    assert np.array_equal(bits(saved), ref["value"])                  # save_input: B(x + bias)


def test_standalone_norm_silu_one_frame_cache_keeps_previous():
    """d = 1 current frame, cache of 2: the older cache frame is the last
    previous frame (copied by the call), the newer one the current output."""
    from oracle.stream import norm_silu
    rng = np.random.default_rng(45)
    n, d, h, w, c = 1, 1, 4, 6, 640
    raw, _, _, gamma = _norm_inputs(rng, (n, d, h, w), c)
    prev = from_bits(noise_bits(rng, (n, 2, h, w, c)))
    y = torch.empty((n, 3, h + 2, w + 2, c), dtype=torch.bfloat16, device="cuda")
    cache = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device="cuda")
    gd, xd, pd = gamma.cuda(), raw.cuda(), prev.cuda()
    epi = cv.make_epilogue(gamma=gd, norm_silu=True)
    cv.conv3d_norm_silu(xd, n, d, h, w, c, epi, cv.make_out_pad((2, 1, 1), (0, 1, 1), 2, cache, 2),
                        pd, y)
    torch.cuda.synchronize()
    got_cache = bits(cache)
    assert np.array_equal(got_cache[:, 0], bits(prev)[:, 1])
    assert np.array_equal(got_cache[:, 1], bits(y)[:, 2, 1:-1, 1:-1])
    ref = norm_silu(bits(raw), bits(gamma), intermediates=True)
    check(bits(y)[:, 2:, 1:-1, 1:-1], ref, fused=True, gamma_bits=bits(gamma), what="one frame")

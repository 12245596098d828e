"""GroupNorm statistics formed by the conv that produces the normalised tensor
(conv3d_fwd_gn_stats, conv3d_group_norm_from_partials), through the C ABI.

The conv's y must equal conv3d_fwd's bit for bit: the statistics only add
sums. The GroupNorm from the conv's partial sums is checked against the
oracle's GroupNorm of that y on every element under the GroupNorm rule, and
against conv3d_group_norm's own two-pass statistics: per-frame and per-clip
statistics, 4- and 8-channel groups, two channel tiles, zero and reflect
padding, a batch of two, tiles inside one frame and across two, and the
full-size H3 L0 layer in the launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import convolution_video_vae_amd as cv
from convolution_video_vae_amd.layer import Conv3d, GroupNorm
from parity import check_group_norm, rms_of

pytestmark = pytest.mark.gpu

CAUSAL = dict(pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cv.lib()
    yield
    torch.cuda.empty_cache()


def seeded(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * scale).to(
        torch.bfloat16)


def bits(t):
    return workloads.bf16_bits(t.cpu())


def conv_with_stats(x_shape, cout, *, seed, split_k=1, pad_mode=cv.PAD_ZERO):
    """y from conv3d_fwd and from conv3d_fwd_gn_stats (with its partials)."""
    cin = x_shape[-1]
    w = seeded((cout, cin, 3, 3, 3), seed + 1, scale=(27 * cin) ** -0.5)
    layer = Conv3d(w, x_shape, split_k=split_k, pad_mode=pad_mode, **CAUSAL)
    plan = cv.conv3d_plan_describe(layer.desc)
    print(f"[gn-stats] x={x_shape} cout={cout} pad_mode={pad_mode}: {plan}", flush=True)
    assert "ns=-2 bm=512 bn=128" in plan and "order=frame" not in plan, plan
    x = seeded(x_shape, seed)
    y_ref = layer(x)
    nbytes = cv.conv3d_gn_partials_bytes(layer.desc)
    part = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = layer.new_output()
    y.fill_(float("nan"))
    cv.conv3d_fwd_gn_stats(layer.desc, x, layer.w_packed, y, part, layer.workspace)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "y differs from conv3d_fwd"
    assert not torch.isnan(part).any(), "partial sums left unwritten"
    return layer, y, part


def gn_from_partials(layer, y, part, groups, *, silu, t_isolated, eps=1e-5, seed=0):
    shape = tuple(y.shape)
    c = shape[-1]
    g = torch.Generator().manual_seed(100 + seed)
    gamma = (1.0 + 0.1 * torch.randn(c, generator=g)).to(torch.float32)
    beta = (0.1 * torch.randn(c, generator=g)).to(torch.float32)
    gn = GroupNorm(shape, groups, gamma.cuda(), beta.cuda(), eps=eps, silu=silu,
                   t_isolated=t_isolated)
    out = torch.empty_like(y)
    cv.conv3d_group_norm_from_partials(gn.desc, layer.desc, part, y, gn.gamma, gn.beta, out,
                                       gn.workspace)
    two_pass = gn(y)
    torch.cuda.synchronize()
    return out, two_pass, gamma, beta


CASES = [
    # name, x shape (NDHWC), cout, groups, t_isolated, silu, pad_mode
    # (20 x 42 slots per frame: two of every three 510-slot tiles cross a frame)
    ("c128_g32_frames", (1, 3, 20, 40, 128), 128, 32, True, True, cv.PAD_ZERO),
    ("c128_g16_clip_batch2", (2, 3, 20, 40, 64), 128, 16, False, False, cv.PAD_ZERO),
    ("c256_two_channel_tiles", (1, 4, 24, 30, 128), 256, 32, True, True, cv.PAD_ZERO),
    ("c128_reflect", (1, 3, 20, 40, 128), 128, 32, True, True, cv.PAD_REFLECT),
    ("c128_one_group_per_tile", (1, 2, 17, 33, 96), 128, 1, True, False, cv.PAD_ZERO),
]


@pytest.mark.parametrize("name,shape,cout,groups,t_iso,silu,pad_mode", CASES,
                         ids=[c[0] for c in CASES])
def test_group_norm_from_conv_partials(name, shape, cout, groups, t_iso, silu, pad_mode):
    cpg = cout // groups
    if cpg % 4 or 128 % cpg:
        with pytest.raises(cv.Conv3dError):
            layer, y, part = conv_with_stats(shape, cout, seed=11, pad_mode=pad_mode)
            gn_from_partials(layer, y, part, groups, silu=silu, t_isolated=t_iso)
        return
    layer, y, part = conv_with_stats(shape, cout, seed=11, pad_mode=pad_mode)
    out, two_pass, gamma, beta = gn_from_partials(layer, y, part, groups, silu=silu,
                                                  t_isolated=t_iso)
    yb = bits(y)
    ref = oracle.group_norm(yb, groups, gamma.numpy(), beta.numpy(), eps=float(np.float32(1e-5)),
                            silu=silu, t_isolated=t_iso, intermediates=True)
    diag = check_group_norm(bits(out), ref, what=name)
    print(f"[gn-stats] {name}: {diag}", flush=True)
    assert diag["bit_identical"] > 0.99, diag
    # the two statistics paths differ only by fp32 rounding of their sums
    # (both meet the oracle's rule; near zero a tiny shift of the mean can
    # move an output by many of its own ulps, within the rule's RMS floor)
    same = float(np.mean(bits(out) == bits(two_pass)))
    assert same > 0.99, same


def test_partials_match_plain_sums():
    """The partial sums themselves: per (frame, 4-channel subgroup), the sum
    over tiles of a frame equals the float64 sum of y's values (and of their
    squares) up to fp32 accumulation error."""
    shape, cout = (1, 3, 20, 40, 128), 128
    layer, y, part = conv_with_stats(shape, cout, seed=21)
    yf = oracle.bf16_to_f32(bits(y)).astype(np.float64)           # [1, 3, 20, 40, 128]
    p = part.cpu().numpy().reshape(-1, 2, 32, 2)                  # [tile][frame slot][sg][k]
    TS, WP, Ho = 510, 42, 20
    n_frames = shape[1]
    got = np.zeros((n_frames, 32, 2))
    for t in range(p.shape[0]):
        f0 = (t * TS // WP) // Ho
        for fs in range(2):
            if f0 + fs < n_frames:
                got[f0 + fs] += p[t, fs]
    sub = yf.reshape(n_frames, -1, 32, 4)
    want = np.stack([sub.sum(axis=(1, 3)), (sub * sub).sum(axis=(1, 3))], axis=-1)
    err = np.abs(got - want)
    tol = 1e-5 * np.stack([np.abs(sub).sum(axis=(1, 3)), (sub * sub).sum(axis=(1, 3))], axis=-1)
    assert np.all(err <= tol + 1e-6), float(np.max(err - tol))


def test_full_size_h3_l0():
    """H3 L0 in the bench's launch configuration (persistent 512 x 128 slot
    plan): y bit-identical to conv3d_fwd, and the GroupNorm (32 groups,
    per-frame statistics, SiLU) from the conv's partials against the oracle
    on every element, frame by frame."""
    L = workloads.LAYERS["h3_l0_128"]
    t = workloads.make_tensors(L)
    layer = Conv3d(t.w.cuda(), L.x_shape, **CAUSAL)
    plan = cv.conv3d_plan_describe(layer.desc)
    assert "persistent=1" in plan and "ns=-2" in plan, plan
    x = t.x.cuda()
    y_ref = layer(x)
    part = torch.empty(cv.conv3d_gn_partials_bytes(layer.desc) // 4, dtype=torch.float32,
                       device="cuda")
    y = layer.new_output()
    cv.conv3d_fwd_gn_stats(layer.desc, x, layer.w_packed, y, part, layer.workspace)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    del y_ref
    out, two_pass, gamma, beta = gn_from_partials(layer, y, part, 32, silu=True, t_isolated=True)
    yb, ob = bits(y), bits(out)
    refs = []
    for d in range(L.x_shape[1]):
        r = oracle.group_norm(yb[:, d:d + 1], 32, gamma.numpy(), beta.numpy(),
                              eps=float(np.float32(1e-5)), silu=True, t_isolated=True,
                              intermediates=True)
        refs.append({"y": r["y"], "a": r["a"]})
    rms = rms_of(np.concatenate([r["y"].ravel() for r in refs]))
    for d, r in enumerate(refs):
        diag = check_group_norm(ob[:, d:d + 1], r, what=f"frame {d}", rms=rms)
        assert diag["bit_identical"] > 0.99, (d, diag)
    same = float(np.mean(ob == bits(two_pass)))
    print(f"[gn-stats] full size: {same:.6f} of the outputs equal the two-pass path's", flush=True)
    assert same > 0.99, same

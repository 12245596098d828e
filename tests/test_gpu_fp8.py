"""GPU parity of the e4m3fn (fp8) conv: activations and weights in e4m3fn,
fp32 accumulation, bf16 output (Qwen PR, "Test plan": the FP8 suite). Small
e4m3 values keep every sum exact, so those cases, across the slot kernel
(whole 64-channel chunks) and the plain kernel, are bit-exact against the
oracle on the decoded operands; random operands use the raw parity rule plus
the fp8 MFMA's accumulation term (tests/parity.py, check_fp8); and
the pages' own criterion (mean relative error of the fp8 conv against the
bf16 conv of the same operands below 2e-2) is checked on a Qwen-like layer."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import convolution_video_vae_amd as cv
from convolution_video_vae_amd.layer import Conv3d
from oracle.fp8 import conv3d_fp8, e4m3_to_bf16_bits
from parity import check_fp8, rms_of

pytestmark = pytest.mark.gpu

SMALL_CODES = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0, 0x30, 0xB0, 0x3C, 0xBC], np.uint8)  # 0, +-1, +-2, +-0.5, +-1.5


def f8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)


def codes_of(t):
    return t.cpu().view(torch.uint8).numpy()


def bits(t):
    return workloads.bf16_bits(t.cpu())


CASES = [
    # label, x shape, cout, stride, pad_lo, pad_hi, split_k, expected kernel (plan substring)
    ("slot_causal_128", (1, 4, 10, 22, 128), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1, "ns=-2"),
    ("slot_cin_192_rows_straddle", (1, 3, 9, 37, 192), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1,
     "ns=-2"),
    ("slot_cin_64_cout_256_batch_2", (2, 3, 7, 30, 64), 256, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1,
     "ns=-2"),
    ("slot_valid_wide_rows", (1, 4, 5, 150, 64), 128, (1, 1, 1), (0, 0, 0), (0, 0, 0), 1, "ns=-2"),
    ("valid_96_cin_48", (1, 5, 9, 13, 48), 96, (1, 1, 1), (0, 0, 0), (0, 0, 0), 1, "ns=3"),
    ("stride122_64", (1, 3, 12, 15, 64), 64, (1, 2, 2), (2, 0, 0), (0, 1, 1), 1, "ns=3"),
    ("split_k_512", (1, 3, 6, 6, 512), 512, (1, 1, 1), (2, 1, 1), (0, 1, 1), 0, "mode=partial"),
    ("cin_16", (2, 3, 7, 9, 16), 32, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1, ""),
    ("cin_96_not_slot", (1, 3, 8, 20, 96), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1), 1, "ns=3"),
]


@pytest.mark.parametrize("label,xs,cout,st,lo,hi,sk,kern", CASES, ids=[c[0] for c in CASES])
def test_fp8_small_values_bit_exact(label, xs, cout, st, lo, hi, sk, kern):
    rng = np.random.default_rng(71)
    xc = rng.choice(SMALL_CODES, size=xs)
    wc = rng.choice(SMALL_CODES, size=(cout, xs[4], 3, 3, 3))
    b = torch.from_numpy(rng.integers(-8, 9, size=cout).astype(np.float32))
    conv = Conv3d(f8(wc).cuda(), xs, stride=st, pad_lo=lo, pad_hi=hi, split_k=sk, bias=b)
    plan = cv.conv3d_plan_describe(conv.desc, cv.make_epilogue(bias=conv.bias))
    print(f"[fp8] {label} x={xs} cout={cout} plan: {plan}", flush=True)
    assert kern in plan
    y = conv(f8(xc).cuda())
    torch.cuda.synchronize()
    ref = conv3d_fp8(xc, wc, stride=st, pad_lo=lo, pad_hi=hi, bias=b.numpy())
    assert np.array_equal(bits(y), ref)


def test_fp8_slot_kernel_persistent_bit_exact():
    """290 slot tiles on 256 persistent work-groups (a second tile for some,
    its first stages fetched during the last two of the first); small values,
    so exact."""
    rng = np.random.default_rng(76)
    xs, cout = (1, 9, 128, 126, 128), 128
    xc = rng.choice(SMALL_CODES, size=xs)
    wc = rng.choice(SMALL_CODES, size=(cout, xs[4], 3, 3, 3))
    conv = Conv3d(f8(wc).cuda(), xs, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    plan = cv.conv3d_plan_describe(conv.desc, cv.make_epilogue())
    print(f"[fp8] persistent plan: {plan}", flush=True)
    assert "ns=-2" in plan and "persistent=1" in plan
    y = conv(f8(xc).cuda())
    torch.cuda.synchronize()
    ref = conv3d_fp8(xc, wc, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    assert np.array_equal(bits(y), ref)


def test_fp8_random_operands_against_oracle():
    rng = np.random.default_rng(72)
    xs, cout = (1, 5, 12, 20, 96), 96
    x = torch.from_numpy(rng.standard_normal(xs).astype(np.float32)).to(torch.float8_e4m3fn)
    w = torch.from_numpy(rng.standard_normal((cout, 96, 3, 3, 3)).astype(np.float32) * 0.5).to(
        torch.float8_e4m3fn)
    conv = Conv3d(w.cuda(), xs, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    y = conv(x.cuda())
    torch.cuda.synchronize()
    xc, wc = codes_of(x), codes_of(w)
    ref = conv3d_fp8(xc, wc, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), intermediates=True)
    # sum of |x w| per output: the same conv on the magnitudes (sign bit cleared)
    mag = conv3d_fp8(xc & 0x7F, wc & 0x7F, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), intermediates=True)
    diag = check_fp8(bits(y), ref, mag["acc"], what="fp8 random")
    print(f"[fp8] random: {diag}", flush=True)
    assert diag["bit_identical"] > 0.98, diag


def test_fp8_slot_kernel_random_operands_against_oracle():
    """The slot kernel's MFMAs take a whole 64-channel chunk each; random
    operands over several tiles, two chunks and a row that straddles tiles."""
    rng = np.random.default_rng(75)
    xs, cout = (1, 4, 11, 45, 128), 128
    x = torch.from_numpy(rng.standard_normal(xs).astype(np.float32)).to(torch.float8_e4m3fn)
    w = torch.from_numpy(rng.standard_normal((cout, 128, 3, 3, 3)).astype(np.float32) * 0.5).to(
        torch.float8_e4m3fn)
    conv = Conv3d(w.cuda(), xs, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=1)
    plan = cv.conv3d_plan_describe(conv.desc, cv.make_epilogue())
    print(f"[fp8] slot random plan: {plan}", flush=True)
    assert "ns=-2" in plan
    y = conv(x.cuda())
    torch.cuda.synchronize()
    xc, wc = codes_of(x), codes_of(w)
    ref = conv3d_fp8(xc, wc, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), intermediates=True)
    mag = conv3d_fp8(xc & 0x7F, wc & 0x7F, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), intermediates=True)
    diag = check_fp8(bits(y), ref, mag["acc"], what="fp8 slot random")
    print(f"[fp8] slot random: {diag}", flush=True)
    assert diag["bit_identical"] > 0.98, diag


def test_fp8_error_against_bf16_conv_is_within_the_pages_bound():
    """Qwen PR, "Test plan": mean relative error of the FP8 conv against the
    bf16 conv below 2e-2. The bf16 conv runs on the same e4m3 operands,
    decoded (exactly) to bf16: the bound is on the kernel, not on the e4m3
    rounding of the inputs, which alone is about 4% on N(0, 1) data. Operands
    N(0, 1) cast to e4m3fn, a T = 1 Qwen-Image-like 96-channel layer."""
    rng = np.random.default_rng(73)
    xs, cout = (1, 1, 64, 72, 96), 96
    x8 = torch.from_numpy(rng.standard_normal(xs).astype(np.float32)).to(torch.float8_e4m3fn)
    w8 = torch.from_numpy(rng.standard_normal((cout, 96, 3, 3, 3)).astype(np.float32)).to(
        torch.float8_e4m3fn)
    lo, hi = (2, 1, 1), (0, 1, 1)
    y8 = Conv3d(w8.cuda(), xs, pad_lo=lo, pad_hi=hi)(x8.cuda())
    y16 = Conv3d(w8.to(torch.bfloat16).cuda(), xs, pad_lo=lo, pad_hi=hi)(x8.to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    a, r = y8.float().cpu().numpy(), y16.float().cpu().numpy()
    rel = np.mean(np.abs(a - r)) / np.mean(np.abs(r))
    print(f"[fp8] mean relative error vs bf16 conv of the same operands: {rel:.2e}", flush=True)
    assert rel < 2e-2


def test_fp8_full_size_h3_l0_every_element():
    """The benchmark's fp8 layer (H3 L0 with e4m3fn operands cast from the
    seeded bf16 tensors) at full size, against the oracle on every output
    element."""
    L = workloads.LAYERS["h3_l0_128_fp8"]
    t = workloads.make_tensors(L)
    x8 = t.x.float().to(torch.float8_e4m3fn)
    w8 = t.w.float().to(torch.float8_e4m3fn)
    conv = Conv3d(w8.cuda(), L.x_shape, pad_lo=L.pad_lo, pad_hi=L.pad_hi)
    plan = cv.conv3d_plan_describe(conv.desc, cv.make_epilogue())
    print(f"[fp8] h3 l0 plan: {plan}", flush=True)
    assert "ns=-2" in plan
    y = conv(x8.cuda())
    torch.cuda.synchronize()
    got = bits(y).reshape(-1, L.cout)
    xc, wc = codes_of(x8), codes_of(w8)
    # decoded once: conv3d_fp8 is the oracle conv on these bf16 values
    xb, wb = e4m3_to_bf16_bits(xc), e4m3_to_bf16_bits(wc)
    xab, wab = e4m3_to_bf16_bits(xc & 0x7F), e4m3_to_bf16_bits(wc & 0x7F)
    chunk = 1 << 16
    refs, mags = [], []
    for p0 in range(0, L.m, chunk):
        pix = np.arange(p0, min(L.m, p0 + chunk))
        refs.append(oracle.conv3d(xb, wb, pad_lo=L.pad_lo, pad_hi=L.pad_hi, pixels=pix,
                                  intermediates=True))
        mags.append(oracle.conv3d(xab, wab, pad_lo=L.pad_lo, pad_hi=L.pad_hi, pixels=pix,
                                  intermediates=True)["acc"])
        if (p0 // chunk) % 4 == 0:
            print(f"  oracle fp8: {pix[-1] + 1} of {L.m} pixels", flush=True)
    rms = rms_of(np.concatenate([r["y"] for r in refs]))
    same = 0
    for k, p0 in enumerate(range(0, L.m, chunk)):
        sl = slice(p0, min(L.m, p0 + chunk))
        d = check_fp8(got[sl], refs[k], mags[k], what=f"fp8 h3 l0 pixels {sl.start}..", rms=rms)
        same += d["bit_identical"] * d["n"]
    print(f"[fp8] h3 l0 every element: bit-identical {same / got.size:.4f}", flush=True)

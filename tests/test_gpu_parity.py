"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Integer-valued data, impulses, packing and transposes must match bit for bit;
random data must satisfy the ulp rule in tests/parity.py. Small cases span
several tiles and a ragged tail; the full-size layers run in the launch
configuration the benchmark times. Every case is compared on every output
element, and outputs are pre-filled with NaN so an unwritten element fails.
"""
import numpy as np
import pytest
import torch

import convolution_video_vae_amd as cv
import oracle
import workloads
from guard import Guarded
from parity import b2f, check, check_every_element, oracle_every_pixel

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cv.lib()          # fail loudly if the HIP library is missing
    yield


def bits(t):
    return workloads.bf16_bits(t.cpu())


def from_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def poisoned(shape):
    return torch.full(shape, NAN_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def run_gpu(x, w, *, stride=(1, 1, 1), pad_lo=(0, 0, 0), pad_hi=(0, 0, 0), bias=None,
            residual=None, gamma=None, norm=False, split_k=0, want_residual_out=False,
            layout=cv.NDHWC, out_layout=None, label="", reflect=False):
    """x (NDHWC or NCDHW per layout), w OIDHW: CPU tensors. Returns CPU outputs."""
    print(f"[gpu] {label} x={tuple(x.shape)} w={tuple(w.shape)} stride={stride} "
          f"pad={pad_lo}/{pad_hi} split_k={split_k} norm={norm}", flush=True)
    out_layout = layout if out_layout is None else out_layout
    cout, cin = w.shape[:2]
    xd = x.cuda().contiguous()
    wd = w.cuda().contiguous()
    wp = torch.empty(cv.conv3d_packed_weight_bytes(cout, cin) // 2, dtype=torch.bfloat16, device="cuda")
    cv.conv3d_pack_weight(wd, wp, cout, cin)
    desc = cv.make_desc(tuple(x.shape), cout, stride=stride, pad_lo=pad_lo, pad_hi=pad_hi,
                        layout=layout, out_layout=out_layout, split_k=split_k,
                        pad_mode=cv.PAD_REFLECT if reflect else cv.PAD_ZERO)
    od = cv.conv3d_output_dims(desc)
    n = x.shape[0]
    yshape = (n,) + od + (cout,) if out_layout == cv.NDHWC else (n, cout) + od
    yg = Guarded(yshape)
    y = yg.t
    bd = bias.cuda() if bias is not None else None
    rd = residual.cuda().contiguous() if residual is not None else None
    gd = gamma.cuda() if gamma is not None else None
    rog = Guarded(yshape) if want_residual_out else None
    ro = rog.t if rog is not None else None
    epi = cv.make_epilogue(bias=bd, residual=rd, gamma=gd, residual_out=ro, norm_silu=norm)
    ws_bytes = cv.conv3d_workspace_bytes(desc, epi)
    wsg = Guarded((max(ws_bytes, 16),), dtype=torch.uint8, fill=0)
    cv.conv3d_fwd(desc, xd, wp, epi if epi.flags else None, y, wsg.t, ws_bytes)
    torch.cuda.synchronize()
    yg.assert_intact(label + " y")
    wsg.assert_intact(label + " workspace")
    out = {"y": y.cpu(), "plan": cv.conv3d_plan_describe(desc, epi if epi.flags else None)}
    if ro is not None:
        rog.assert_intact(label + " residual_out")
        out["residual_out"] = ro.cpu()
    return out


def run_oracle(x, w, *, stride=(1, 1, 1), pad_lo=(0, 0, 0), pad_hi=(0, 0, 0), bias=None,
               residual=None, gamma=None, norm=False, pixels=None, reflect=False):
    conv = oracle.conv3d_reflect if reflect else oracle.conv3d
    return conv(bits(x), bits(w), stride=stride, pad_lo=pad_lo, pad_hi=pad_hi,
                         bias=None if bias is None else bias.numpy(),
                         residual=None if residual is None else bits(residual),
                         gamma=None if gamma is None else bits(gamma), norm_silu=norm,
                         pixels=pixels, intermediates=True)


def geom(layer):
    return dict(stride=layer.stride, pad_lo=layer.pad_lo, pad_hi=layer.pad_hi,
                reflect=layer.reflect)


# ------------------------------------------------------------------ pack / transpose

@pytest.mark.parametrize("cout,cin", [(64, 64), (96, 40), (320, 160), (16, 8), (1024, 512)])
def test_pack_weight_matches_documented_layout(cout, cin):
    rng = np.random.default_rng(cout * 7 + cin)
    w = rng.integers(0, 65536, size=(cout, cin, 3, 3, 3), dtype=np.uint16)
    wd = from_bits(w).cuda()
    nb = cv.conv3d_packed_weight_bytes(cout, cin)
    wp = torch.full((nb // 2,), NAN_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    cv.conv3d_pack_weight(wd, wp, cout, cin)
    got = bits(wp)
    cc = (cin + 31) // 32
    # packed[t][c // 32][co][c % 32] = w[co][c][kd][kh][kw], t = kd*9 + kh*3 + kw; 0 for c >= cin
    want = np.zeros((27, cc * 32, cout), np.uint16)
    want[:, :cin, :] = w.reshape(cout, cin, 27).transpose(2, 1, 0)
    want = want.reshape(27, cc, 32, cout).transpose(0, 1, 3, 2)
    np.testing.assert_array_equal(got, want.ravel())


# (A leading extent that is a multiple of 8 takes the 16-byte register-
# transpose kernel: 16-byte loads when the other extent is a multiple of 8
# (320 x 38400, 40 x 64), 8-byte loads for 4 mod 8 (160 x 56364, 16 x 252
# with a ragged last block), element by element otherwise (24 x 105,
# 72 x 234, 8 x 1). Other extents that are multiples of 4 take the
# 8-byte LDS-tile kernel (56364 x 160, 12 x 60, 68 x 180), the rest the
# 2-byte one.)
@pytest.mark.parametrize("shape", [(2, 24, 3, 5, 7), (1, 160, 7, 66, 122), (1, 320, 5, 64, 120),
                                   (3, 8, 1, 1, 1), (1, 72, 2, 9, 13), (2, 12, 3, 4, 5),
                                   (1, 68, 3, 5, 12), (2, 40, 2, 4, 8), (1, 16, 3, 7, 12)])
def test_transpose_round_trip_is_exact(shape):
    n, c, d, h, w = shape
    rng = np.random.default_rng(sum(shape))
    src = from_bits(rng.integers(0, 65536, size=shape, dtype=np.uint16)).cuda()
    mid = poisoned((n, d, h, w, c))
    cv.conv3d_transpose(src, cv.NCDHW, mid, n, c, d, h, w)
    back = poisoned(shape)
    cv.conv3d_transpose(mid, cv.NDHWC, back, n, c, d, h, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(mid), bits(src.cpu().permute(0, 2, 3, 4, 1).contiguous()))
    np.testing.assert_array_equal(bits(back), bits(src.cpu()))


# ------------------------------------------------------------------ exact cases

INT_CASES = [
    # label, x shape, cout, stride, pad_lo, pad_hi, bias
    ("causal64", (1, 5, 16, 16, 64), 64, (1, 1, 1), (2, 1, 1), (0, 1, 1), True),
    ("causal128_ragged", (2, 3, 9, 21, 128), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1), False),
    ("s122_pad01", (1, 4, 17, 23, 128), 128, (1, 2, 2), (2, 0, 0), (0, 1, 1), False),
    ("valid96", (1, 6, 12, 30, 96), 96, (1, 1, 1), (0, 0, 0), (0, 0, 0), False),
    ("t1_96", (1, 1, 33, 40, 96), 96, (1, 1, 1), (2, 1, 1), (0, 1, 1), False),
    ("cin40_cout48", (1, 3, 7, 9, 40), 48, (1, 1, 1), (2, 1, 1), (0, 1, 1), True),
    ("s222", (1, 9, 12, 12, 64), 64, (2, 2, 2), (2, 1, 1), (0, 1, 1), False),
    ("wide512", (1, 3, 6, 6, 512), 1024, (1, 1, 1), (2, 1, 1), (0, 1, 1), True),
    # one 256-pixel tile per frame: the automatic split gives the first two
    # frames' tiles (3 and 6 live (kd, kh) pairs) fewer slices than the rest
    ("wide_live_split", (1, 5, 16, 16, 256), 512, (1, 1, 1), (2, 1, 1), (0, 1, 1), True),
    ("live_split_ragged", (2, 4, 7, 13, 96), 192, (1, 1, 1), (2, 1, 1), (0, 1, 1), True),
]


@pytest.mark.parametrize("case", INT_CASES, ids=[c[0] for c in INT_CASES])
@pytest.mark.parametrize("split_k", [0, 1, 3])
def test_integer_data_bit_exact(case, split_k):
    label, xs, cout, st, lo, hi, has_bias = case
    x, w, b = workloads.integer_tensors(xs, cout, seed=len(label), bias=has_bias)
    g = run_gpu(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b, split_k=split_k, label=label)
    r = run_oracle(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b)
    np.testing.assert_array_equal(bits(g["y"]), r["y"], err_msg=g["plan"])


def test_integer_fused_epilogue_bit_exact_across_splits():
    """Same integer conv, fused norm epilogue: the conv value is exact, so any
    K split must give the same bits as the single-pass fused kernel."""
    xs, cout = (1, 3, 10, 12, 160), 320
    x, w, b = workloads.integer_tensors(xs, cout, seed=3, bias=True)
    rng = np.random.default_rng(3)
    res = torch.from_numpy(rng.integers(-4, 5, size=(1, 1, 8, 10, cout)).astype(np.float32)).to(torch.bfloat16)
    gam = torch.from_numpy(rng.uniform(0.5, 1.5, cout).astype(np.float32)).to(torch.bfloat16)
    outs = [run_gpu(x, w, bias=b, residual=res, gamma=gam, norm=True, split_k=s,
                    want_residual_out=True, label=f"fused_int_s{s}") for s in (1, 2, 0)]
    for o in outs[1:]:
        np.testing.assert_array_equal(bits(o["y"]), bits(outs[0]["y"]))
        np.testing.assert_array_equal(bits(o["residual_out"]), bits(outs[0]["residual_out"]))
    r = run_oracle(x, w, bias=b, residual=res, gamma=gam, norm=True)
    np.testing.assert_array_equal(bits(outs[0]["residual_out"]), r["value"])
    check(bits(outs[0]["y"]), r, fused=True, gamma_bits=bits(gam), what="fused integer")


HALO_CASES = [
    # label, x shape, cout, stride, pad_lo, pad_hi: stride 1 along W, Cin % 32 == 0,
    # run without a K split so the row-halo kernel computes them.
    ("halo_causal128_batch2", (2, 3, 9, 40, 128), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("halo_valid96_wide", (1, 4, 6, 300, 96), 96, (1, 1, 1), (0, 0, 0), (0, 0, 0)),
    ("halo_cin32_cout256", (1, 3, 5, 64, 32), 256, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("halo_wo22_25rows", (1, 2, 30, 22, 64), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("halo_t1", (1, 1, 17, 50, 64), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("halo_asym_wpad", (1, 3, 7, 33, 96), 96, (1, 1, 1), (2, 1, 0), (0, 1, 2)),
    ("halo_stride_dh", (1, 7, 13, 45, 64), 128, (2, 2, 1), (2, 1, 1), (0, 1, 1)),
]


def halo_tile(cout):
    """Tile override selecting the row-halo kernel (the planner prefers the
    slot kernel for the same layers)."""
    return "32,4,1,4,4,9,-1" if cout % 128 == 0 else "32,4,1,4,3,9,-1"


@pytest.mark.parametrize("case", HALO_CASES, ids=[c[0] for c in HALO_CASES])
def test_halo_kernel_integer_bit_exact(case, monkeypatch):
    label, xs, cout, st, lo, hi = case
    monkeypatch.setenv("CONV3D_TILE", halo_tile(cout))
    x, w, b = workloads.integer_tensors(xs, cout, seed=len(label) + 7, bias=True)
    g = run_gpu(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b, split_k=1, label=label)
    assert "ns=-1" in g["plan"], g["plan"]
    r = run_oracle(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b)
    np.testing.assert_array_equal(bits(g["y"]), r["y"], err_msg=g["plan"])


SLOT_CASES = HALO_CASES + [
    # label, x shape, cout, stride, pad_lo, pad_hi: slot kernel (stride 1 along
    # W, Cin % 32 == 0; output rows of Wo + 2 slots, 512-slot tiles).
    ("slot_wo8_many_rows", (1, 3, 20, 8, 64), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("slot_batch3_valid96", (3, 4, 9, 37, 32), 96, (1, 1, 1), (0, 0, 0), (0, 0, 0)),
    ("slot_wo254_tile_straddles_rows", (1, 3, 5, 256, 64), 128, (1, 1, 1), (0, 1, 2), (0, 1, 0)),
    ("slot_160_channel_tile", (1, 4, 10, 30, 32), 160, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("slot_320_two_channel_tiles", (1, 3, 8, 21, 64), 320, (1, 1, 1), (0, 0, 0), (0, 0, 0)),
    # 512 x 128 tiles store through LDS in pairs of adjacent slots; with Wo + 2
    # odd, pairs straddle output rows
    ("slot_staged_store_odd_rows", (1, 3, 7, 37, 64), 128, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
]


@pytest.mark.parametrize("with_bias", [False, True], ids=["plain_store", "bias_epilogue"])
@pytest.mark.parametrize("case", SLOT_CASES, ids=[c[0] for c in SLOT_CASES])
def test_slot_kernel_integer_bit_exact(case, with_bias):
    label, xs, cout, st, lo, hi = case
    x, w, b = workloads.integer_tensors(xs, cout, seed=len(label) + 7, bias=True)
    b = b if with_bias else None
    g = run_gpu(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b, split_k=1, label=label)
    assert "ns=-2" in g["plan"], g["plan"]
    r = run_oracle(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b)
    np.testing.assert_array_equal(bits(g["y"]), r["y"], err_msg=g["plan"])


PAIR_CASES = [
    # label, x shape, cout, stride, pad_lo, pad_hi: stride 2 along W with no
    # leading W pad, even W and Cin % 32 == 0 -> the slot kernel on the
    # pixel-pair view (two taps along W, Wo + 1 slots per output row).
    ("pair_s122", (1, 4, 17, 24, 128), 128, (1, 2, 2), (2, 0, 0), (0, 1, 1)),
    ("pair_cin32_wo15", (1, 3, 9, 30, 32), 128, (1, 2, 2), (2, 0, 0), (0, 1, 1)),
    # no trailing pad: the last input column is read by no output
    ("pair_batch2_no_hi_pad", (2, 3, 10, 40, 64), 128, (1, 2, 2), (2, 0, 0), (0, 0, 0)),
    # a trailing pad of 3: the last output column sees only padding
    ("pair_hi_pad3_two_channel_tiles", (1, 3, 8, 20, 64), 256, (1, 2, 2), (0, 0, 0), (0, 2, 3)),
    ("pair_stride222", (1, 9, 12, 16, 64), 128, (2, 2, 2), (2, 1, 0), (0, 1, 1)),
    ("pair_wo8_many_rows", (1, 3, 30, 16, 32), 128, (1, 2, 2), (2, 1, 0), (0, 1, 1)),
    ("pair_wo256_tiles_straddle_rows", (1, 3, 5, 512, 64), 128, (1, 2, 2), (2, 0, 0), (0, 1, 1)),
    ("pair_cin96_t1", (1, 1, 21, 66, 96), 128, (1, 2, 2), (2, 0, 0), (0, 1, 1)),
]


@pytest.mark.parametrize("with_bias", [False, True], ids=["plain_store", "bias_epilogue"])
@pytest.mark.parametrize("case", PAIR_CASES, ids=[c[0] for c in PAIR_CASES])
def test_pair_view_integer_bit_exact(case, with_bias):
    label, xs, cout, st, lo, hi = case
    x, w, b = workloads.integer_tensors(xs, cout, seed=len(label) + 17, bias=True)
    b = b if with_bias else None
    g = run_gpu(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b, split_k=1, label=label)
    assert "ns=-3" in g["plan"], g["plan"]
    r = run_oracle(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b)
    np.testing.assert_array_equal(bits(g["y"]), r["y"], err_msg=g["plan"])


@pytest.mark.parametrize("case", PAIR_CASES[:3], ids=[c[0] for c in PAIR_CASES[:3]])
def test_pair_view_random_against_oracle(case):
    label, xs, cout, st, lo, hi = case
    rng = np.random.default_rng(len(label) + 5)
    x = torch.from_numpy(rng.standard_normal(xs).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((cout, xs[-1], 3, 3, 3)) / np.sqrt(27 * xs[-1]))
                         .astype(np.float32)).to(torch.bfloat16)
    g = run_gpu(x, w, stride=st, pad_lo=lo, pad_hi=hi, split_k=1, label=label + "_random")
    assert "ns=-3" in g["plan"], g["plan"]
    r = run_oracle(x, w, stride=st, pad_lo=lo, pad_hi=hi)
    check(bits(g["y"]), r, what=label)


PERSIST_CASES = [
    # label, x shape, cout: 290 slot tiles on 256 persistent work-groups, so
    # some work-groups take a second tile from their queue. With Cin = 128
    # every tile's stage count (live (kd, kh) pairs x 4 chunks) is a multiple
    # of six and the next tile's set-up and first two stages go out during
    # the current tile's last two; with Cin = 160 (5 chunks) only tiles with
    # six live pairs have such a count, the rest start the plain way.
    ("slot_persistent_cin128", (1, 9, 128, 126, 128), 128),
    ("slot_persistent_cin160_mixed", (1, 9, 128, 126, 160), 128),
]


@pytest.mark.parametrize("with_bias", [False, True], ids=["plain_store", "bias_epilogue"])
@pytest.mark.parametrize("case", PERSIST_CASES, ids=[c[0] for c in PERSIST_CASES])
def test_slot_kernel_persistent_integer_bit_exact(case, with_bias):
    """(Without an epilogue the 512 x 128 tiles store through LDS in rounds.)"""
    label, xs, cout = case
    x, w, b = workloads.integer_tensors(xs, cout, seed=len(label) + 13, bias=True)
    b = b if with_bias else None
    g = run_gpu(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), bias=b, split_k=0, label=label)
    assert "ns=-2" in g["plan"] and "persistent=1" in g["plan"], g["plan"]
    r = run_oracle(x, w, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), bias=b)
    np.testing.assert_array_equal(bits(g["y"]), r["y"], err_msg=g["plan"])


HALO_SPLIT_CASES = [
    # label, x shape, cout, stride, pad_lo, pad_hi: K-split halo kernel (fp32
    # partials summed in fixed order by the reduce kernel).
    ("halo_split_cout256", (1, 3, 6, 40, 64), 256, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("halo_split_cout192_w16", (1, 2, 9, 16, 96), 192, (1, 1, 1), (2, 1, 1), (0, 1, 1)),
    ("halo_split_cout128_valid", (2, 3, 5, 70, 32), 128, (1, 1, 1), (0, 0, 0), (0, 0, 0)),
]


@pytest.mark.parametrize("case", HALO_SPLIT_CASES, ids=[c[0] for c in HALO_SPLIT_CASES])
@pytest.mark.parametrize("split_k", [2, 5])
def test_halo_kernel_split_k_integer_bit_exact(case, split_k):
    label, xs, cout, st, lo, hi = case
    x, w, b = workloads.integer_tensors(xs, cout, seed=len(label) + 11, bias=True)
    g = run_gpu(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b, split_k=split_k, label=label)
    assert "ns=-1" in g["plan"] and "mode=partial" in g["plan"], g["plan"]
    r = run_oracle(x, w, stride=st, pad_lo=lo, pad_hi=hi, bias=b)
    np.testing.assert_array_equal(bits(g["y"]), r["y"], err_msg=g["plan"])


@pytest.mark.parametrize("kernel", ["halo", "slot"])
@pytest.mark.parametrize("case", HALO_CASES[:2], ids=[c[0] for c in HALO_CASES[:2]])
def test_row_kernels_random_against_oracle(case, kernel, monkeypatch):
    label, xs, cout, st, lo, hi = case
    if kernel == "halo":
        monkeypatch.setenv("CONV3D_TILE", halo_tile(cout))
    rng = np.random.default_rng(len(label))
    x = torch.from_numpy(rng.standard_normal(xs).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((cout, xs[-1], 3, 3, 3)) / np.sqrt(27 * xs[-1]))
                         .astype(np.float32)).to(torch.bfloat16)
    g = run_gpu(x, w, stride=st, pad_lo=lo, pad_hi=hi, split_k=1, label=label + "_random")
    assert ("ns=-1" if kernel == "halo" else "ns=-2") in g["plan"], g["plan"]
    r = run_oracle(x, w, stride=st, pad_lo=lo, pad_hi=hi)
    check(bits(g["y"]), r, what=label)


@pytest.mark.parametrize("stride,lo,hi", [((1, 1, 1), (2, 1, 1), (0, 1, 1)),
                                         ((1, 2, 2), (2, 0, 0), (0, 1, 1)),
                                         ((1, 1, 1), (0, 0, 0), (0, 0, 0))])
def test_input_impulses_bit_exact(stride, lo, hi):
    rng = np.random.default_rng(21)
    xs = (1, 5, 9, 11, 32)
    w = torch.from_numpy(rng.standard_normal((32, 32, 3, 3, 3)).astype(np.float32)).to(torch.bfloat16)
    x = np.zeros(xs, np.float32)
    for (d, h, ww, ci) in [(0, 0, 0, 0), (4, 8, 10, 31), (2, 3, 1, 5), (1, 0, 10, 17)]:
        x[0, d, h, ww, ci] = 1.0
    x = torch.from_numpy(x).to(torch.bfloat16)
    g = run_gpu(x, w, stride=stride, pad_lo=lo, pad_hi=hi, label="impulse")
    r = run_oracle(x, w, stride=stride, pad_lo=lo, pad_hi=hi)
    np.testing.assert_array_equal(bits(g["y"]), r["y"])


# ------------------------------------------------------------------ random data, small

SMALL = [
    # name, layer family it scales down, x shape, cout
    ("tiny_causal_64", "tiny_causal_64", (1, 5, 16, 16, 64), 64),
    ("causal_128", "h3_l0_128", (1, 5, 24, 40, 128), 128),
    ("s122_128", "h3_l0_128_s122", (1, 5, 23, 41, 128), 128),
    ("valid_96", "wan_valid_96", (1, 6, 20, 42, 96), 96),
    ("valid_384", "wan_valid_384", (1, 3, 14, 22, 384), 384),
    ("t1_96", "qwen_t1_96", (1, 1, 64, 72, 96), 96),
    ("wide_1024", "h3_l5_1024", (1, 3, 8, 8, 1024), 1024),
    ("wide_512to1024", "h3_l5_512to1024", (1, 5, 8, 8, 512), 1024),
    ("fused_160to320", "wan_fused_160to320", (1, 5, 14, 22, 160), 320),
    ("fused_160to160", "wan_fused_160to320", (1, 5, 14, 22, 160), 160),
    ("valid_160", "wan_valid_96", (1, 6, 20, 42, 64), 160),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_random_small_against_oracle(case):
    name, fam, xs, cout = case
    L = workloads.LAYERS[fam]
    t = workloads.make_tensors(L, x_shape=xs, cout=cout)
    kw = dict(bias=t.bias, residual=t.residual, gamma=t.gamma, norm=L.norm_silu, **geom(L))
    g = run_gpu(t.x, t.w, want_residual_out=L.residual, label=name, **kw)
    r = run_oracle(t.x, t.w, **kw)
    diag = check(bits(g["y"]), r, fused=L.norm_silu,
                 gamma_bits=None if t.gamma is None else bits(t.gamma), what=name)
    print(name, g["plan"], diag)
    if L.residual:
        check(bits(g["residual_out"]), dict(r, y=r["value"]), what=name + " residual_out",
              through=("conv", "main"))


def test_fused_reduce_path_matches_fused_kernel():
    """The split-K route (partials + reducing epilogue) and the single-pass
    fused kernel both satisfy the rule on the same random layer."""
    L = workloads.LAYERS["wan_fused_160to320"]
    t = workloads.make_tensors(L, x_shape=(1, 4, 10, 19, 160))
    kw = dict(bias=t.bias, residual=t.residual, gamma=t.gamma, norm=True)
    r = run_oracle(t.x, t.w, **kw)
    for s in (1, 4):
        g = run_gpu(t.x, t.w, split_k=s, label=f"fused_s{s}", **kw)
        check(bits(g["y"]), r, fused=True, gamma_bits=bits(t.gamma), what=f"split_k={s}")


def test_bias_residual_without_norm():
    """bias -> residual, stopping at `value` (the cuDNN page's bias/residual
    variant, without its padding)."""
    L = workloads.LAYERS["wan_fused_160to320"]
    t = workloads.make_tensors(L, x_shape=(1, 4, 9, 13, 160))
    g = run_gpu(t.x, t.w, bias=t.bias, residual=t.residual, want_residual_out=True, label="bias_res")
    r = run_oracle(t.x, t.w, bias=t.bias, residual=t.residual)
    check(bits(g["y"]), r, what="bias+residual", through=("conv", "main"))
    np.testing.assert_array_equal(bits(g["residual_out"]), bits(g["y"]))


# ------------------------------------------------------------------ full-size layers

FULL = [n for n, L in workloads.LAYERS.items() if not L.fp8]   # fp8: tests/test_gpu_fp8.py


def oracle_chunk(layer):
    """Output pixels per oracle call: about 50 GFLOP of direct convolution."""
    per_pixel = 2.0 * layer.cout * layer.cin * layer.live_taps
    return int(max(1024, min(layer.m, 5e10 // per_pixel)))


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer_every_element(name):
    """The layer at its full size, in the launch configuration the benchmark
    times, against the oracle on every output element (and, for the fused
    layer, every element of the saved residual sum)."""
    L = workloads.LAYERS[name]
    t = workloads.make_tensors(L)
    kw = dict(bias=t.bias, residual=t.residual, gamma=t.gamma, norm=L.norm_silu, **geom(L))
    g = run_gpu(t.x, t.w, want_residual_out=L.residual, label=name, **kw)
    y = bits(g["y"]).reshape(-1, L.cout)
    assert not np.any(y == NAN_BF16), "unwritten output elements"
    chunk = oracle_chunk(L)
    ref = oracle_every_pixel(lambda pix: run_oracle(t.x, t.w, pixels=pix, **kw), L.m, chunk,
                             what=name)
    diag = check_every_element(y, ref, chunk=chunk, fused=L.norm_silu,
                               gamma_bits=None if t.gamma is None else bits(t.gamma), what=name)
    print(name, g["plan"], diag, flush=True)
    assert diag["bit_identical"] > 0.97
    if L.residual:
        ro = bits(g["residual_out"]).reshape(-1, L.cout)
        assert not np.any(ro == NAN_BF16), "unwritten residual_out elements"
        dv = check_every_element(ro, dict(ref, y=ref["value"]), chunk=chunk,
                                 what=name + " residual_out", through=("conv", "main"))
        print(name, "residual_out", dv, flush=True)


def test_fused_layer_ncdhw_boundary_variants_are_bit_identical():
    """NCDHW input (and NCDHW output with an NCDHW residual) gives exactly the
    NDHWC result, transposed: a transpose is exact."""
    L = workloads.LAYERS["wan_fused_160to320"]
    t = workloads.make_tensors(L)
    kw = dict(bias=t.bias, gamma=t.gamma, norm=True, **geom(L))
    ref = run_gpu(t.x, t.w, residual=t.residual, want_residual_out=True, label="ndhwc", **kw)
    x_ncdhw = t.x.permute(0, 4, 1, 2, 3).contiguous()
    a = run_gpu(x_ncdhw, t.w, residual=t.residual, want_residual_out=True, layout=cv.NCDHW,
                out_layout=cv.NDHWC, label="ncdhw_in", **kw)
    np.testing.assert_array_equal(bits(a["y"]), bits(ref["y"]))
    res_ncdhw = t.residual.permute(0, 4, 1, 2, 3).contiguous()
    b = run_gpu(x_ncdhw, t.w, residual=res_ncdhw, want_residual_out=True, layout=cv.NCDHW,
                label="ncdhw_in_out", **kw)
    np.testing.assert_array_equal(bits(b["y"]), bits(ref["y"].permute(0, 4, 1, 2, 3).contiguous()))
    np.testing.assert_array_equal(bits(b["residual_out"]),
                                  bits(ref["residual_out"].permute(0, 4, 1, 2, 3).contiguous()))


@pytest.mark.parametrize("name", ["h3_l5_1024", "tiny_causal_64"])
def test_run_to_run_deterministic(name):
    L = workloads.LAYERS[name]
    t = workloads.make_tensors(L)
    kw = dict(bias=t.bias, **geom(L))
    a = run_gpu(t.x, t.w, label=name + "_a", **kw)
    b = run_gpu(t.x, t.w, label=name + "_b", **kw)
    np.testing.assert_array_equal(bits(a["y"]), bits(b["y"]))


@pytest.mark.parametrize("kind", ["raw", "bias_residual", "norm"])
def test_slot_160_channel_tile_random(kind):
    """The 384-slot x 160-channel slot tile (one wave column holds the whole
    160-channel row), without K split: raw, bias + residual, fused norm."""
    L = workloads.LAYERS["wan_fused_160to320"]
    t = workloads.make_tensors(L, x_shape=(1, 5, 12, 26, 160), cout=160)
    kw = dict(bias=None if kind == "raw" else t.bias,
              residual=None if kind == "raw" else t.residual,
              gamma=t.gamma if kind == "norm" else None, norm=kind == "norm")
    g = run_gpu(t.x, t.w, split_k=1, want_residual_out=kind != "raw", label="slot160_" + kind, **kw)
    assert "pb=3 cb=5 kb=0 ns=-2 bm=384 bn=160" in g["plan"], g["plan"]
    r = run_oracle(t.x, t.w, **kw)
    diag = check(bits(g["y"]), r, fused=kind == "norm",
                 gamma_bits=None if kind != "norm" else bits(t.gamma), what="slot160 " + kind)
    assert diag["bit_identical"] > 0.99, diag
    if kind != "raw":
        check(bits(g["residual_out"]), dict(r, y=r["value"]), what="slot160 residual_out",
              through=("conv", "main"))


# ------------------------------------------------------------------ contract edge cases

def _closed_forms():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "epilogue_closed_forms.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("route", ["fused_slot", "split_reduce"])
@pytest.mark.parametrize("case", _closed_forms(), ids=lambda c: c["name"])
def test_contract_closed_forms_on_the_gpu(case, route):
    """The hand-worked rows of the contract (cuDNN page, "Operation
    Contract"; tests/golden) through the HIP epilogues: a zero weight makes
    the conv exactly 0, so bias, residual and gamma fix every value. Both the
    single-pass fused kernel (the whole 320-channel row in one work-group)
    and the split-K route (fp32 partials, then the reducing norm epilogue)
    must give the golden numbers bit for bit, and the saved residual sum."""
    C = 320
    rng = np.random.default_rng(23)
    x = torch.from_numpy(rng.standard_normal((1, 3, 6, 9, 32)).astype(np.float32)).to(torch.bfloat16)
    w = torch.zeros((C, 32, 3, 3, 3), dtype=torch.bfloat16)
    bias = torch.full((C,), case["bias"], dtype=torch.float32)
    if "bias_channel0" in case:
        bias[0] = case["bias_channel0"]
    gamma = torch.full((C,), case["gamma"], dtype=torch.float32)
    if "gamma_channel0" in case:
        gamma[0] = case["gamma_channel0"]
    gamma = gamma.to(torch.bfloat16)
    out_shape = (1, 1, 4, 7, C)
    residual = None
    if case["residual"] is not None:
        residual = torch.full(out_shape, case["residual"], dtype=torch.bfloat16)
    g = run_gpu(x, w, bias=bias, residual=residual, gamma=gamma, norm=True,
                split_k=1 if route == "fused_slot" else 3, want_residual_out=residual is not None,
                label=f"golden_{case['name']}_{route}")
    want_plan = "mode=norm" if route == "fused_slot" else "mode=partial"
    assert want_plan in g["plan"], g["plan"]
    y = b2f(bits(g["y"])).reshape(-1, C)
    np.testing.assert_array_equal(y[:, 0], np.float32(case["out_channel0"]))
    np.testing.assert_array_equal(y[:, 1:], np.float32(case["out"]))
    r = run_oracle(x, w, bias=bias, residual=residual, gamma=gamma, norm=True)
    np.testing.assert_array_equal(bits(g["y"]), r["y"])
    if residual is not None:
        v = b2f(bits(g["residual_out"])).reshape(-1, C)
        np.testing.assert_array_equal(v[:, 1:], np.float32(case["value"]))
        np.testing.assert_array_equal(bits(g["residual_out"]), r["value"])

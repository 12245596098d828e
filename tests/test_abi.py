"""Host-side tests of the C-ABI library: it loads, exports what include/conv3d.h
declares, and rejects bad calls before any GPU work.

No test here launches a kernel: every conv3d_fwd / pack / transpose call is
built to fail an argument check (the checks run on the host before anything
is enqueued), using fake but aligned addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import convolution_video_vae_amd as cv
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv3d.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(conv3d_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = cv.lib()
    names = header_functions()
    assert set(names) == set(cv.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_desc_struct_matches_header_layout():
    # 6 ints, 3x3 ints, layout, out_layout, split_k, pad_mode, dtype = 20 ints
    assert ctypes.sizeof(cv.conv3d_desc) == 20 * 4
    assert ctypes.sizeof(cv.conv3d_epilogue) == 8 + 4 * 8


def test_status_strings():
    for code in range(8):
        assert cv.status_str(code)
    assert cv.status_str(0) == "ok"


def test_packed_weight_bytes():
    assert cv.conv3d_packed_weight_bytes(128, 128) == 27 * 128 * 128 * 2
    assert cv.conv3d_packed_weight_bytes(320, 160) == 27 * 160 * 320 * 2
    assert cv.conv3d_packed_weight_bytes(64, 40) == 27 * 64 * 64 * 2   # cin padded to 64
    assert cv.conv3d_packed_weight_bytes(0, 8) == 0


@pytest.mark.parametrize("name", list(workloads.LAYERS))
def test_output_dims_match_layer_table(name):
    L = workloads.LAYERS[name]
    d = cv.make_desc(L.x_shape, L.cout, stride=L.stride, pad_lo=L.pad_lo, pad_hi=L.pad_hi)
    assert cv.conv3d_output_dims(d) == L.out_dhw()


def test_output_shapes_from_the_pages():
    # valid conv: [N,T,H,W,Ci] -> [N,T-2,H-2,W-2,Co] (cuDNN page, "Raw Conv3D Variant")
    d = cv.make_desc((1, 7, 66, 122, 160), 320)
    assert cv.conv3d_output_dims(d) == (5, 64, 120)
    # stride-2 downsample after a (0,1,0,1) zero pad: 1024 -> 512 (Qwen-Image PR, table 2)
    d = cv.make_desc((1, 1, 1024, 1024, 96), 96, stride=(1, 2, 2), pad_lo=(2, 0, 0), pad_hi=(0, 1, 1))
    assert cv.conv3d_output_dims(d) == (1, 512, 512)
    # causal conv keeps T, H, W
    d = cv.make_desc((1, 17, 256, 256, 128), 128, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    assert cv.conv3d_output_dims(d) == (17, 256, 256)


def test_workspace_and_plans():
    big = workloads.LAYERS["h3_l0_128"]
    d = cv.make_desc(big.x_shape, big.cout, pad_lo=big.pad_lo, pad_hi=big.pad_hi)
    plan = cv.conv3d_plan_describe(d)
    assert "splits=1" in plan
    # many more tiles than CUs: persistent work-groups, whose tile queues are
    # the only workspace
    assert "persistent=1" in plan
    assert 0 < cv.conv3d_workspace_bytes(d) <= 4096
    wide = workloads.LAYERS["h3_l5_1024"]
    d = cv.make_desc(wide.x_shape, wide.cout, pad_lo=wide.pad_lo, pad_hi=wide.pad_hi)
    plan = cv.conv3d_plan_describe(d)
    splits = int(re.search(r"splits=(\d+)", plan).group(1))
    assert splits > 1
    # one fp32 partial tile per work-group (the halo kernel's fragment order)
    grid, bm, bn = (int(re.search(k + r"=(\d+)", plan).group(1)) for k in ("grid", "bm", "bn"))
    assert grid <= 256 and bm * bn * grid >= wide.m * wide.cout
    assert cv.conv3d_workspace_bytes(d) >= grid * bm * bn * 4
    # the automatic split follows the live taps; an explicit one is uniform
    assert "split=live" in plan
    d.split_k = 4
    assert "split=live" not in cv.conv3d_plan_describe(d)
    assert cv.conv3d_workspace_bytes(d) >= 4 * wide.m * wide.cout * 4
    d.split_k = 1
    assert cv.conv3d_workspace_bytes(d) == 0
    # stride 2 along W, no leading W pad, even W: the pixel-pair view of the
    # slot kernel (Wo + 1 slots per output row, 511 stored per tile), each
    # frame's 128 x 129 slots tiled on their own
    s2 = workloads.LAYERS["h3_l0_128_s122"]
    d = cv.make_desc(s2.x_shape, s2.cout, stride=s2.stride, pad_lo=s2.pad_lo, pad_hi=s2.pad_hi)
    plan = cv.conv3d_plan_describe(d)
    assert "ns=-3" in plan and "persistent=1" in plan and "splits=1" in plan, plan
    assert "order=frame" in plan and f"m_tiles={17 * -(-128 * 129 // 511)}" in plan, plan
    assert cv.conv3d_workspace_bytes(d) <= 4096
    # odd W or a leading W pad: not a whole number of pairs per row
    for shape, lo in (((1, 17, 256, 255, 128), (2, 0, 0)), ((1, 17, 256, 256, 128), (2, 0, 1))):
        d = cv.make_desc(shape, 128, stride=(1, 2, 2), pad_lo=lo, pad_hi=(0, 1, 1))
        assert "ns=-3" not in cv.conv3d_plan_describe(d)
    # a batch above the 32-bit buffer range runs in passes of as many samples
    # as fit (7 of H3 L0's 285 MB), each still on the slot kernel
    d = cv.make_desc((16,) + big.x_shape[1:], big.cout, pad_lo=big.pad_lo, pad_hi=big.pad_hi)
    plan = cv.conv3d_plan_describe(d)
    assert "passes=3 samples_per_pass=7" in plan and "ns=-2" in plan, plan
    # the fused layer's 24.6 MB outputs: passes of 87 samples, NCDHW included
    d = cv.make_desc((120, 160, 7, 66, 122), 320, layout=cv.NCDHW)
    assert "passes=2 samples_per_pass=87" in cv.conv3d_plan_describe(d)
    # NCDHW in and out need NDHWC staging copies
    d = cv.make_desc((1, 160, 7, 66, 122), 320, layout=cv.NCDHW)
    assert cv.conv3d_workspace_bytes(d) >= 1 * 160 * 7 * 66 * 122 * 2 + 5 * 64 * 120 * 320 * 2


# ------------------------------------------------------------------ rejected calls

X, W, Y, WS, R, G, B = (0x10000000 * k for k in range(1, 8))   # aligned, never dereferenced


def fwd(desc, x=X, w=W, epi=None, y=Y, ws=None, ws_bytes=0):
    return cv.lib().conv3d_fwd(ctypes.byref(desc), x, w, ctypes.byref(epi) if epi else None, y,
                               ws, ws_bytes, None)


def small_desc(**kw):
    # split_k=1: no workspace, so each call below fails only on what it probes
    args = dict(pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=1)
    args.update(kw)
    return cv.make_desc((1, 3, 8, 8, 32), 32, **args)


def test_null_pointers_rejected():
    assert fwd(small_desc(), x=None) == 1
    assert fwd(small_desc(), w=None) == 1
    assert fwd(small_desc(), y=None) == 1
    assert cv.lib().conv3d_fwd(None, X, W, None, Y, None, 0, None) == 1
    assert fwd(small_desc(), epi=cv.conv3d_epilogue(cv.EPI_BIAS, None, None, None, None)) == 1
    assert fwd(small_desc(), epi=cv.conv3d_epilogue(cv.EPI_L2NORM_SILU, None, None, None, None)) == 1
    assert cv.lib().conv3d_pack_weight(None, W, 8, 8, None) == 1
    assert cv.lib().conv3d_transpose(None, 0, Y, 1, 8, 1, 1, 1, None) == 1


def test_bad_shapes_rejected():
    assert fwd(cv.make_desc((1, 2, 8, 8, 32), 32)) == 2        # valid conv needs T >= 3
    assert fwd(cv.make_desc((0, 3, 8, 8, 32), 32)) == 2
    assert fwd(small_desc(stride=(0, 1, 1))) == 2
    assert fwd(small_desc(pad_lo=(-1, 0, 0))) == 2
    d = small_desc(); d.layout = 7
    assert fwd(d) == 2
    assert cv.lib().conv3d_transpose(X, 3, Y, 1, 8, 1, 1, 1, None) == 2
    out = (ctypes.c_int * 3)()
    assert cv.lib().conv3d_output_dims(ctypes.byref(cv.make_desc((1, 2, 2, 2, 8), 8)),
                                       ctypes.byref(out)) == 2


def test_alignment_rejected():
    assert fwd(small_desc(), x=X + 2) == 3
    assert fwd(small_desc(), w=W + 8) == 3
    assert fwd(small_desc(), y=Y + 4) == 3
    assert fwd(cv.make_desc((1, 3, 8, 8, 12), 32, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))) == 3
    epi = cv.conv3d_epilogue(cv.EPI_BIAS, B + 4, None, None, None)
    assert fwd(small_desc(), epi=epi) == 3
    assert cv.lib().conv3d_pack_weight(X + 2, W, 8, 8, None) == 3


def test_unsupported_rejected_without_fallback():
    assert fwd(cv.make_desc((1, 3, 8, 8, 32), 24, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))) == 6
    epi = cv.conv3d_epilogue(cv.EPI_RESIDUAL_OUT, None, None, None, R)
    assert fwd(small_desc(), epi=epi) == 6                    # residual_out needs residual
    epi = cv.conv3d_epilogue(64, None, None, None, None)      # unknown flag
    assert fwd(small_desc(), epi=epi) == 6
    huge = cv.make_desc((1, 17, 1024, 1024, 128), 128, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    assert fwd(huge) == 6                                       # > 2 GiB activation
    wide = cv.make_desc((1, 3, 4, 4, 32), 4096)
    epi = cv.conv3d_epilogue(cv.EPI_L2NORM_SILU, None, None, G, None)
    assert fwd(wide, epi=epi) == 6                              # norm row too long


def test_overlap_rejected():
    d = small_desc()
    assert fwd(d, y=X) == 4                                     # y aliases x
    assert fwd(d, y=X + 64) == 4                                # y inside x
    assert fwd(d, y=W) == 4
    epi = cv.conv3d_epilogue(cv.EPI_RESIDUAL | cv.EPI_RESIDUAL_OUT, None, R, None, Y)
    assert fwd(d, epi=epi) == 4                                 # residual_out aliases y
    epi = cv.conv3d_epilogue(cv.EPI_RESIDUAL, None, Y, None, None)
    assert fwd(d, epi=epi) == 4                                 # residual aliases y
    assert cv.lib().conv3d_pack_weight(X, X + 16, 8, 8, None) == 4
    assert cv.lib().conv3d_transpose(X, 0, X + 64, 1, 8, 2, 2, 2, None) == 4


def test_workspace_checked():
    wide = workloads.LAYERS["h3_l5_1024"]
    d = cv.make_desc(wide.x_shape, wide.cout, pad_lo=wide.pad_lo, pad_hi=wide.pad_hi)
    need = cv.conv3d_workspace_bytes(d)
    assert fwd(d) == 5
    assert fwd(d, ws=WS, ws_bytes=need - 1) == 5
    assert fwd(d, ws=WS + 8, ws_bytes=need) == 3
    assert fwd(d, ws=X, ws_bytes=need) == 4                     # workspace aliases x


# ------------------------------------------------------------------ GroupNorm

def gn(desc, x=X, gamma=G, beta=B, y=Y, ws=WS, ws_bytes=1 << 30):
    return cv.lib().conv3d_group_norm(ctypes.byref(desc) if desc is not None else None, x, gamma,
                                      beta, y, ws, ws_bytes, None)


def gn_desc(shape=(1, 3, 8, 8, 64), groups=32, **kw):
    return cv.make_group_norm_desc(shape, groups, **kw)


def test_group_norm_desc_struct_matches_header_layout():
    assert ctypes.sizeof(cv.conv3d_group_norm_desc) == 9 * 4


def test_group_norm_workspace_covers_partials_and_stats():
    for name, L in workloads.NORM_LAYERS.items():
        d = gn_desc(L.x_shape, L.groups)
        need = cv.conv3d_group_norm_workspace_bytes(d)
        units = L.x_shape[0] * L.x_shape[1]
        # at least one chunk partial (two fp64) and one (mean, rstd) pair per group and unit
        assert need >= units * L.groups * (16 + 8), name
        assert need < 64 << 20, name
    # statistics over the whole clip: one unit per sample
    a = cv.conv3d_group_norm_workspace_bytes(gn_desc((2, 5, 4, 4, 64), t_isolated=False))
    assert a >= 2 * 32 * 24


def test_group_norm_rejected_calls():
    assert gn(None) == 1
    assert gn(gn_desc(), x=None) == 1
    assert gn(gn_desc(), gamma=None) == 1
    assert gn(gn_desc(), beta=None) == 1
    assert gn(gn_desc(), y=None) == 1
    assert gn(gn_desc((0, 3, 8, 8, 64))) == 2
    assert gn(gn_desc(groups=0)) == 2
    assert gn(gn_desc(groups=24)) == 2                         # 64 % 24 != 0
    assert gn(gn_desc(eps=0.0)) == 2
    assert gn(gn_desc(eps=float("inf"))) == 2
    assert gn(gn_desc((1, 3, 8, 8, 36), groups=4)) == 3        # c % 8 != 0
    assert gn(gn_desc(), x=X + 2) == 3
    assert gn(gn_desc(), gamma=G + 4) == 3
    assert gn(gn_desc((1, 1, 2, 2, 4096), groups=32)) == 6     # c > 2048
    assert gn(gn_desc((1, 1, 2, 2, 1024), groups=512)) == 6    # groups > 256
    need = cv.conv3d_group_norm_workspace_bytes(gn_desc())
    assert gn(gn_desc(), ws=None) == 5
    assert gn(gn_desc(), ws_bytes=need - 1) == 5
    assert gn(gn_desc(), ws=WS + 8, ws_bytes=need) == 3
    assert gn(gn_desc(), y=X + 64) == 4                        # partial overlap with x
    assert gn(gn_desc(), ws=X, ws_bytes=need) == 4             # workspace inside x
    assert gn(gn_desc(), gamma=Y) == 4                         # gamma inside y
    assert gn(gn_desc(), beta=WS) == 4                         # beta inside the workspace


# ------------------------------------------------------------------ padded outputs, stream packing

def fwd_padded(desc, op, x=X, w=W, epi=None, y=Y, ws=WS, ws_bytes=1 << 30):
    return cv.lib().conv3d_fwd_padded(ctypes.byref(desc), x, w, ctypes.byref(epi) if epi else None,
                                      ctypes.byref(op) if op else None, y, ws, ws_bytes, None)


def test_out_pad_struct_matches_header_layout():
    assert ctypes.sizeof(cv.conv3d_out_pad) == 8 * 4 + 8


def test_padded_workspace_adds_the_staged_output():
    d = small_desc()
    base = cv.conv3d_workspace_bytes(d)
    op = cv.make_out_pad((2, 1, 1), (0, 1, 1), 1, R, 2)
    staged = cv.conv3d_padded_workspace_bytes(d, None, op)
    assert staged >= base + 1 * 3 * 8 * 8 * 32 * 2
    assert cv.conv3d_padded_workspace_bytes(d, None, None) == base
    assert cv.conv3d_padded_workspace_bytes(d, None, cv.make_out_pad()) == base


def test_padded_rejected_calls():
    d = small_desc()
    assert fwd_padded(d, cv.make_out_pad((-1, 0, 0))) == 2
    assert fwd_padded(d, cv.make_out_pad((1, 1, 1), history_frames=2)) == 2   # history > pad
    assert fwd_padded(d, cv.make_out_pad((2, 1, 1), cache=R, cache_frames=0)) == 2
    assert fwd_padded(d, cv.make_out_pad((2, 1, 1), history_frames=1, cache=R,
                                         cache_frames=5)) == 2                 # > Do + history
    assert fwd_padded(d, cv.make_out_pad((2, 1, 1), cache=R + 8, cache_frames=1)) == 3
    dn = small_desc(); dn.out_layout = cv.NCDHW
    assert fwd_padded(dn, cv.make_out_pad((0, 1, 1), (0, 1, 1))) == 6
    need = cv.conv3d_padded_workspace_bytes(d, None, cv.make_out_pad((2, 1, 1), (0, 1, 1)))
    assert fwd_padded(d, cv.make_out_pad((2, 1, 1), (0, 1, 1)), ws=None, ws_bytes=0) == 5
    assert fwd_padded(d, cv.make_out_pad((2, 1, 1), (0, 1, 1)), ws_bytes=need - 1) == 5
    assert fwd_padded(d, cv.make_out_pad((2, 1, 1), (0, 1, 1), cache=Y + 256, cache_frames=1)) == 4
    assert fwd_padded(d, cv.make_out_pad((2, 1, 1), (0, 1, 1)), y=X + 4096) == 4


def pack(chunk=X, strides=(12 * 4 * 6 * 6, 4 * 6 * 6, 6 * 6, 6, 1), n=1, c=12, t=4, h=6, w=6,
         hist=None, P=0, padded=Y, c_pad=16, cache=None, cf=0):
    st = (ctypes.c_longlong * 5)(*strides)
    return cv.lib().conv3d_stream_pack_input(chunk, ctypes.byref(st), n, c, t, h, w, hist, P, padded,
                                             c_pad, cache, cf, None)


def test_stream_pack_rejected_calls():
    assert pack(chunk=None) == 1
    assert pack(padded=None) == 1
    assert pack(P=1) == 1                                         # history missing
    assert pack(t=0) == 2
    assert pack(hist=R, P=3) == 2
    assert pack(c_pad=8) == 2                                     # c_pad < c
    assert pack(c_pad=20) == 3                                    # c_pad % 8
    assert pack(strides=(-1, 1, 1, 1, 1)) == 2
    assert pack(cache=G, cf=5) == 2                               # > t + history
    assert pack(padded=Y + 8) == 3
    assert pack(chunk=X + 1) == 3
    assert pack(padded=X + 64) == 4                               # padded inside the chunk
    assert pack(cache=Y + 64, cf=2) == 4                          # cache inside padded


def test_pack_weight_2d_rejected_calls():
    assert cv.lib().conv3d_pack_weight_2d(None, W, 8, 8, None) == 1
    assert cv.lib().conv3d_pack_weight_2d(X, W, 0, 8, None) == 2
    assert cv.lib().conv3d_pack_weight_2d(X + 2, W, 8, 8, None) == 3
    assert cv.lib().conv3d_pack_weight_2d(X, X + 16, 8, 8, None) == 4


def test_reflect_padding_checks():
    d = small_desc(pad_mode=cv.PAD_REFLECT)
    assert cv.conv3d_output_dims(d) == (3, 8, 8)
    assert fwd(small_desc(pad_mode=2)) == 2
    assert fwd(small_desc(pad_mode=cv.PAD_REFLECT, pad_lo=(2, 2, 1))) == 6   # spatial pad > 1
    thin = cv.make_desc((1, 3, 1, 8, 32), 32, pad_lo=(2, 0, 1), pad_hi=(0, 0, 1), split_k=1,
                        pad_mode=cv.PAD_REFLECT)
    assert fwd(thin) == 2                                                    # h < 2


def norm_silu_call(epi, x=X, y=Y, op=None, prev=None, c=64, shape=(1, 3, 8, 8)):
    n, d, h, w = shape
    return cv.lib().conv3d_norm_silu(x, n, d, h, w, c, ctypes.byref(epi) if epi else None,
                                     ctypes.byref(op) if op else None, prev, y, None)


def test_norm_silu_rejected_calls():
    ok = cv.conv3d_epilogue(cv.EPI_L2NORM_SILU, None, None, G, None)
    assert norm_silu_call(None) == 1
    assert norm_silu_call(ok, x=None) == 1
    assert norm_silu_call(cv.conv3d_epilogue(cv.EPI_L2NORM_SILU, None, None, None, None)) == 1
    assert norm_silu_call(cv.conv3d_epilogue(cv.EPI_BIAS, B, None, G, None)) == 6   # no norm flag
    assert norm_silu_call(cv.conv3d_epilogue(cv.EPI_L2NORM_SILU | 64, None, None, G, None)) == 6
    assert norm_silu_call(ok, c=4100) == 3                                          # c % 8
    assert norm_silu_call(ok, c=4096) == 6                                          # c > 2048
    assert norm_silu_call(ok, c=60) == 3
    assert norm_silu_call(ok, y=Y + 8) == 3
    assert norm_silu_call(ok, prev=R) == 2                                          # no history planes
    op = cv.make_out_pad((2, 1, 1), (0, 1, 1), 1, None, 0)
    assert norm_silu_call(ok, op=op, prev=R + 8) == 3
    op2 = cv.make_out_pad((2, 1, 1), (0, 1, 1), 1, WS, 5)                           # cache 5 > d + 1
    assert norm_silu_call(ok, op=op2) == 2
    assert norm_silu_call(ok, y=X + 64) == 4                                        # y inside x
    assert norm_silu_call(ok, op=op, prev=Y + 256) == 4                             # previous inside y


def test_fp8_checks():
    assert cv.conv3d_packed_weight_bytes_fp8(128, 128) == 27 * 128 * 128
    assert cv.conv3d_packed_weight_bytes_fp8(64, 40) == 27 * 64 * 64        # cin padded to 64
    f8 = dict(dtype=cv.FP8_E4M3)
    assert fwd(small_desc(dtype=2)) == 2
    assert fwd(cv.make_desc((1, 3, 8, 8, 24), 32, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=1,
                            **f8)) == 3                                    # cin % 16
    assert fwd(small_desc(**f8, pad_mode=cv.PAD_REFLECT)) == 6
    d = small_desc(**f8)
    d.layout = cv.NCDHW
    assert fwd(d) == 6
    assert fwd(cv.make_desc((1, 3, 8, 8, 32), 48, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=1,
                            **f8)) == 6                                    # cout % 32
    assert cv.lib().conv3d_pack_weight_fp8(None, W, 8, 8, None) == 1
    assert cv.lib().conv3d_pack_weight_fp8(X, W + 8, 8, 8, None) == 3
    assert cv.lib().conv3d_pack_weight_fp8(X, X + 16, 8, 8, None) == 4


def test_tile_override_keeps_fused_norm_rows_whole(monkeypatch):
    """The development tile override (CONV3D_TILE) may only pick a fused-norm
    tile that holds the whole channel row; a 160-channel tile for the
    320-channel fused layer is ignored. Plan queries launch nothing."""
    L = workloads.LAYERS["wan_fused_160to320"]
    d = cv.make_desc(L.x_shape, L.cout, pad_lo=L.pad_lo, pad_hi=L.pad_hi)
    import torch
    g = torch.ones(L.cout, dtype=torch.bfloat16)
    epi = cv.make_epilogue(gamma=g, norm_silu=True)
    base = cv.conv3d_plan_describe(d, epi)
    assert "mode=norm" in base and "bn=320" in base
    monkeypatch.setenv("CONV3D_TILE", "32,4,1,3,5,0,-2")
    assert cv.conv3d_plan_describe(d, epi) == base
    monkeypatch.setenv("CONV3D_TILE", "32,2,2,3,5,0,-2")
    assert "bn=320" in cv.conv3d_plan_describe(d, epi)


def test_tile_override_never_gives_a_norm_layer_halo_partials(monkeypatch):
    """A split fused-norm layer reduces [S][M][Cout] partials with the norm
    epilogue; the halo kernel's fragment-order partials have a reduction
    without it, so the override may not select a halo tile there."""
    d = cv.make_desc((1, 5, 16, 16, 128), 256, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=4)
    import torch
    g = torch.ones(256, dtype=torch.bfloat16)
    epi = cv.make_epilogue(gamma=g, norm_silu=True)
    base = cv.conv3d_plan_describe(d, epi)
    assert "mode=partial" in base and "ns=-1" not in base
    for tile in ("32,2,2,4,4,5,-1", "32,4,1,4,4,9,-1"):
        monkeypatch.setenv("CONV3D_TILE", tile)
        assert cv.conv3d_plan_describe(d, epi) == base
    # the same tiles are taken for a split layer without the norm
    monkeypatch.setenv("CONV3D_TILE", "32,2,2,4,4,5,-1")
    assert "ns=-1" in cv.conv3d_plan_describe(d, None)


def test_noalloc_rejects_before_touching_the_device():
    """conv3d_fwd_noalloc checks the descriptor, the pointers and the plan's
    scratch need on the host first: a plan above the fixed 96 MiB (here the
    headline layer given NCDHW, whose 285 MB staging copy would not fit)
    is refused with CONV3D_ERR_WORKSPACE and nothing is enqueued."""
    lib = cv.lib()
    L = workloads.LAYERS["h3_l0_128"]
    n, d, h, w, c = L.x_shape
    big = cv.make_desc((n, c, d, h, w), L.cout, pad_lo=L.pad_lo, pad_hi=L.pad_hi, layout=cv.NCDHW)
    assert cv.conv3d_workspace_bytes(big) > 96 << 20
    X = 1 << 32
    assert lib.conv3d_fwd_noalloc(ctypes.byref(big), X, X + (1 << 31), None, X + (1 << 33),
                                  None) == 5
    small = cv.make_desc(L.x_shape, L.cout, pad_lo=L.pad_lo, pad_hi=L.pad_hi)
    assert lib.conv3d_fwd_noalloc(ctypes.byref(small), None, X, None, X + (1 << 33), None) == 1
    bad = cv.make_desc((1, 1, 4, 4, 64), 64)          # empty valid output
    assert lib.conv3d_fwd_noalloc(ctypes.byref(bad), X, X, None, X, None) == 2
    assert lib.conv3d_fwd_noalloc(None, X, X, None, X, None) == 1


def test_gn_partials_plan_rules():
    """conv3d_gn_partials_bytes: 512 bytes per pixel tile and 128-channel tile
    for convs on the 512 x 128 slot plan with a plain store; every other plan
    (split K, another tile, NCDHW, e4m3, the pixel-pair view, frames of fewer
    than 510 slots) is CONV3D_ERR_UNSUPPORTED. Plan queries launch nothing."""
    lib = cv.lib()
    out = ctypes.c_size_t()
    L = workloads.LAYERS["h3_l0_128"]
    d = cv.make_desc(L.x_shape, L.cout, pad_lo=L.pad_lo, pad_hi=L.pad_hi)
    assert lib.conv3d_gn_partials_bytes(ctypes.byref(d), ctypes.byref(out)) == 0
    assert out.value == 512 * 2202
    assert lib.conv3d_gn_partials_bytes(ctypes.byref(d), None) == 1
    assert lib.conv3d_gn_partials_bytes(None, ctypes.byref(out)) == 1
    two = cv.make_desc((1, 4, 24, 30, 128), 256, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=1)
    assert lib.conv3d_gn_partials_bytes(ctypes.byref(two), ctypes.byref(out)) == 0
    assert out.value == 512 * 7 * 2
    unsupported = [
        cv.make_desc((1, 3, 20, 40, 128), 128, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1)),   # split K
        cv.make_desc((1, 3, 10, 16, 128), 128, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1),
                     split_k=1),                                                     # 180-slot frames
        cv.make_desc((1, 3, 20, 40, 128), 96, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=1),
        cv.make_desc(L.x_shape, L.cout, pad_lo=L.pad_lo, pad_hi=L.pad_hi, dtype=cv.FP8_E4M3),
        cv.make_desc(L.x_shape, L.cout, stride=(1, 2, 2), pad_lo=(2, 0, 0), pad_hi=(0, 1, 1)),
    ]
    n, dd, h, w, c = L.x_shape
    unsupported.append(cv.make_desc((n, c, dd, h, w), L.cout, pad_lo=L.pad_lo, pad_hi=L.pad_hi,
                                    layout=cv.NCDHW))
    for u in unsupported:
        assert lib.conv3d_gn_partials_bytes(ctypes.byref(u), ctypes.byref(out)) == 6, \
            cv.conv3d_plan_describe(u)
        assert out.value == 0


def test_gn_stats_calls_reject_before_launching():
    """conv3d_fwd_gn_stats and conv3d_group_norm_from_partials check pointers,
    plans, shapes, group layout, alignment, workspace and overlaps on the host;
    each failing call returns before anything is enqueued."""
    lib = cv.lib()
    X, W, Y, P, WS = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40   # never dereferenced
    conv = cv.make_desc((1, 3, 20, 40, 128), 128, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1), split_k=1)
    fwd = lib.conv3d_fwd_gn_stats
    assert fwd(ctypes.byref(conv), X, W, Y, None, None, 0, None) == 1          # no partials
    assert fwd(ctypes.byref(conv), X, W, Y, P + 4, None, 0, None) == 3         # misaligned
    split = cv.make_desc((1, 3, 20, 40, 128), 128, pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
    assert fwd(ctypes.byref(split), X, W, Y, P, WS, 1 << 30, None) == 6        # split plan
    assert fwd(ctypes.byref(conv), X, W, Y, Y + 16, None, 0, None) == 4        # partials in y
    gn = cv.make_group_norm_desc((1, 3, 20, 40, 128), 32, silu=True)
    ws = ctypes.c_size_t()
    assert lib.conv3d_group_norm_workspace_bytes(ctypes.byref(gn), ctypes.byref(ws)) == 0
    G = 6 << 40
    frm = lib.conv3d_group_norm_from_partials
    args = lambda d, c, p, ws_bytes=ws.value: (ctypes.byref(d), ctypes.byref(c), p, Y, G, G + 512,
                                               X, WS, ws_bytes, None)
    assert frm(*args(gn, conv, None)) == 1
    assert frm(*args(gn, split, P)) == 6                                         # not a stats plan
    wrong = cv.make_group_norm_desc((1, 3, 20, 40, 256), 32)
    assert frm(*args(wrong, conv, P)) == 2                                       # not the conv's output
    g3 = cv.make_group_norm_desc((1, 3, 20, 40, 128), 16)                         # 8 channels: fine
    assert frm(*args(g3, conv, P, 0)) == 5                                       # workspace too small
    g_odd = cv.make_group_norm_desc((1, 3, 20, 40, 128), 64)                      # 2-channel groups
    assert frm(*args(g_odd, conv, P)) == 6
    assert frm(*args(gn, conv, P + 8)) == 3                                      # misaligned partials
    assert frm(*args(gn, conv, WS)) == 4                                         # partials in workspace

"""conv3d_fwd_noalloc against conv3d_fwd, through the C ABI.

The entry point for callers that cannot allocate keeps its split-K
partials, tile queues and NDHWC staging in the library's fixed per-device
scratch instead of a caller workspace; it runs the same plans and kernels,
so its output must equal conv3d_fwd's bit for bit. Each case makes two
calls in a row, the second with a smaller input, so whatever the first
call left in the scratch (partials, queue counters, staged copies) must not
leak into the second."""
import numpy as np
import pytest
import torch

import convolution_video_vae_amd as cv
import workloads

pytestmark = pytest.mark.gpu


def bits(t):
    return workloads.bf16_bits(t.cpu())


CASES = [
    # name, (first x NDHWC, second x NDHWC), cout, pad_lo, pad_hi, layout, epilogue, plan substr
    ("split_k_halo", ((1, 5, 16, 16, 1024), (1, 3, 8, 8, 512)), 1024, (2, 1, 1), (0, 1, 1),
     cv.NDHWC, "bias", "mode=partial"),
    ("persistent_slot", ((1, 9, 128, 126, 128), (1, 9, 120, 126, 128)), 128, (2, 1, 1), (0, 1, 1),
     cv.NDHWC, "none", "persistent=1"),
    ("ncdhw_fused", ((1, 7, 66, 122, 160), (1, 4, 20, 30, 160)), 320, (0, 0, 0), (0, 0, 0),
     cv.NCDHW, "norm", "mode=norm"),
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cv.lib()
    yield


def one_call(xs, cout, lo, hi, layout, epi_kind, seed):
    L = workloads.Layer("noalloc", 5, xs, cout, pad_lo=lo, pad_hi=hi, bias=epi_kind != "none",
                        residual=epi_kind == "norm", norm_silu=epi_kind == "norm")
    t = workloads.make_tensors(L, family=seed)
    x = t.x.cuda()
    res = None if t.residual is None else t.residual.cuda()
    if layout == cv.NCDHW:
        x = x.permute(0, 4, 1, 2, 3).contiguous()
        if res is not None:
            res = res.permute(0, 4, 1, 2, 3).contiguous()
    cin = xs[-1]
    wp = torch.empty(cv.conv3d_packed_weight_bytes(cout, cin) // 2, dtype=torch.bfloat16,
                     device="cuda")
    cv.conv3d_pack_weight(t.w.cuda(), wp, cout, cin)
    desc = cv.make_desc(tuple(x.shape), cout, pad_lo=lo, pad_hi=hi, layout=layout)
    od = cv.conv3d_output_dims(desc)
    shape = (xs[0],) + od + (cout,) if layout == cv.NDHWC else (xs[0], cout) + od
    bias = None if t.bias is None else t.bias.cuda()
    gamma = None if t.gamma is None else t.gamma.cuda()
    outs = []
    for kind in ("workspace", "noalloc"):
        y = torch.full(shape, 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        ro = (torch.full(shape, 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
              if res is not None else None)
        epi = cv.make_epilogue(bias=bias, residual=res, gamma=gamma, residual_out=ro,
                               norm_silu=epi_kind == "norm")
        e = epi if epi.flags else None
        if kind == "workspace":
            ws_bytes = cv.conv3d_workspace_bytes(desc, epi)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
            cv.conv3d_fwd(desc, x, wp, e, y, ws, ws_bytes)
            plan = cv.conv3d_plan_describe(desc, e)
        else:
            cv.conv3d_fwd_noalloc(desc, x, wp, e, y)
        torch.cuda.synchronize()
        outs.append((bits(y), None if ro is None else bits(ro)))
    return outs, plan


@pytest.mark.parametrize("name,shapes,cout,lo,hi,layout,epi_kind,plan_has", CASES,
                         ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_call(name, shapes, cout, lo, hi, layout, epi_kind, plan_has):
    for k, xs in enumerate(shapes):
        print(f"[noalloc] {name} call {k}: x={xs} cout={cout} layout={layout} epi={epi_kind}",
              flush=True)
        (ref, got), plan = one_call(xs, cout, lo, hi, layout, epi_kind, seed=40 + k)
        if k == 0:
            assert plan_has in plan, plan
        assert not np.any(ref[0] == 0x7FC0), "reference output not fully written"
        np.testing.assert_array_equal(got[0], ref[0], err_msg=f"{name} call {k} ({plan})")
        if ref[1] is not None:
            np.testing.assert_array_equal(got[1], ref[1], err_msg=f"{name} call {k} residual_out")

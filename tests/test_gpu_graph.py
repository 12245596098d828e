"""The library's calls under HIP graph capture.

The boundary promises calls that allocate nothing and never synchronise
(cuDNN page, "Requirements": execution does not allocate, so it can be
captured and replayed). Each plan family is captured once in a graph with
torch.cuda.graph on a side stream, replayed several times with the
program's own eager work and synchronisations between replays, and every
replay must reproduce the eager call bit for bit: the persistent slot plan
(with its tile-queue reset kernel), the K-split halo plan (fragment-order
partials and their reduction) and the fused-norm plan.
"""
import numpy as np
import pytest
import torch

import convolution_video_vae_amd as cv
import workloads
from convolution_video_vae_amd.layer import Conv3d

pytestmark = pytest.mark.gpu


def bits(t):
    return workloads.bf16_bits(t.cpu())


CASES = [
    # name, x shape, cout, pad_lo, pad_hi, epilogue, split_k, plan substrings
    ("persistent_slot", (1, 9, 128, 126, 128), 128, (2, 1, 1), (0, 1, 1), "none", 0,
     ("ns=-2", "persistent=1")),
    ("split_k_halo", (1, 5, 16, 16, 512), 1024, (2, 1, 1), (0, 1, 1), "bias", 0,
     ("ns=-1", "mode=partial")),
    ("fused_norm_slot", (1, 5, 14, 22, 160), 320, (0, 0, 0), (0, 0, 0), "norm", 1,
     ("mode=norm", "ns=-2")),
    ("fused_norm_split_reduce", (1, 5, 14, 22, 160), 320, (0, 0, 0), (0, 0, 0), "norm", 0,
     ("mode=partial", "reduce=1")),
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cv.lib()
    yield


@pytest.mark.parametrize("name,xs,cout,lo,hi,epi,split_k,plan_has", CASES,
                         ids=[c[0] for c in CASES])
def test_graph_replay_is_bit_identical(name, xs, cout, lo, hi, epi, split_k, plan_has):
    _check_graph(name, xs, cout, lo, hi, epi, split_k, plan_has)


def test_graph_replay_pair_view_frame_order():
    """Stride 2 along W: the persistent pixel-pair plan in frame order (297
    tiles on 256 work-groups, tile-queue reset captured with it)."""
    _check_graph("pair_view_persistent", (1, 9, 256, 256, 128), 128, (2, 0, 0), (0, 1, 1),
                 "none", 0, ("ns=-3", "persistent=1", "order=frame"), stride=(1, 2, 2))


def _check_graph(name, xs, cout, lo, hi, epi, split_k, plan_has, stride=(1, 1, 1)):
    print(f"[graph] {name} x={xs} cout={cout} stride={stride} epilogue={epi}", flush=True)
    L = workloads.Layer(name, 5, xs, cout, stride=stride, pad_lo=lo, pad_hi=hi,
                        bias=epi != "none", residual=epi == "norm", norm_silu=epi == "norm")
    t = workloads.make_tensors(L)
    conv = Conv3d(t.w.cuda(), xs, stride=stride, pad_lo=lo, pad_hi=hi, bias=t.bias,
                  gamma=t.gamma, norm_silu=L.norm_silu, residual=L.residual, split_k=split_k)
    probe = cv.make_epilogue(bias=conv.bias, gamma=conv.gamma, norm_silu=conv.norm_silu)
    probe.flags |= cv.EPI_RESIDUAL if L.residual else 0
    plan = cv.conv3d_plan_describe(conv.desc, probe if probe.flags else None)
    for p in plan_has:
        assert p in plan, plan
    x = t.x.cuda()
    res = None if t.residual is None else t.residual.cuda()
    eager = conv(x, residual=res)
    torch.cuda.synchronize()
    want = bits(eager)

    y = conv.new_output()
    y.fill_(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # one eager call on the capture stream first
        conv(x, residual=res, y=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        conv(x, residual=res, y=y)
    for k in range(4):
        y.fill_(0)                       # eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bits(y)
        assert np.array_equal(got, want), f"{name}: replay {k} differs ({plan})"
        del junk
    # the captured graph still works after an eager call of the same layer
    conv(x, residual=res)
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), want)

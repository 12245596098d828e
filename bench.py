"""Benchmark of the MI355X bf16 3x3x3 Conv3D library on the pages' layer shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-layers]
                    [--no-cpu-baseline]

One step is one conv3d_fwd call on the headline layer (H3 L0: x NDHWC
[1,17,256,256,128] bf16, w [128,128,3,3,3], causal time pad 2, spatial pad 1,
about 1 TFLOP) with its inputs already resident in HBM and the weight packed
once beforehand. The K timed steps run back to back on one stream between
HIP events, bracketed by device synchronisation, after W untimed warm-up
steps (default 60, about 45 ms of this layer: the chip's clocks settle over
the first 40 or so back-to-back calls). `value` is TFLOP/s at the layer's
algorithmic FLOP count 2*M*Cout*27*Cin (only live taps for the T=1 layer).
Every other layer shape is timed the same way, after at least 50 ms of
warm-up, and reported under "per_layer". One JSON line is printed on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published 2.5 PFLOP/s)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (published 5.0 PFLOP/s)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# HBM traffic of the headline layer's main kernel, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch), each divided by what
# the same counter read per byte for an elementwise kernel that reads and
# writes a known number of bytes (the --calibrate-copy pass). Valid only for
# the kernel source it was taken on: reported as null once the source hash
# differs.
TRAFFIC = {"workload": "h3_l0_128", "kernel_hash": "01530ac0d47950b7",
           "bytes": 1403356160}   # 1117.8 MB fetched (FETCH_SIZE x 2.000) + 285.6 MB written
# conv layer -> the GroupNorm of its output, timed with and without the
# statistics summed in the conv's epilogue
CONV_GN_PAIRS = {"conv_gn_h3_l0_128": ("h3_l0_128", "gn_h3_l0_128")}
KERNEL_SOURCES = ("convolution_video_vae_amd/csrc/conv3d_igemm.hip",
                  "convolution_video_vae_amd/csrc/conv3d_device.h")


def kernel_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=60)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-layers", action="store_true", help="time only the headline layer")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--layers", default=None,
                   help="comma-separated per_layer entries to time (default: all)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a 1 GiB read + 1 GiB write elementwise kernel 3 times (the "
                        "byte-counter calibration for rocprofv3 --pmc passes)")
    p.add_argument("--sweep", default=None,
                   help="development: time the headline layer under each CONV3D_TILE value in "
                        "this ';'-separated list and print one line per tile to stderr")
    return p.parse_args()


def describe(L):
    return (f"{L.name}: x NDHWC {list(L.x_shape)} bf16, w [{L.cout},{L.cin},3,3,3], "
            f"stride {list(L.stride)}, pad lo {list(L.pad_lo)} hi {list(L.pad_hi)}, "
            f"out {list(L.out_shape())}"
            + (", fp32 bias" if L.bias else "") + (", residual" if L.residual else "")
            + (", L2-norm*sqrt(C)*gamma+SiLU epilogue" if L.norm_silu else "")
            + (", reflect spatial padding" if L.reflect else "")
            + (", e4m3fn x and w (peak 5 PFLOP/s)" if L.fp8 else ""))


class Case:
    """Device buffers and a bound launch for one layer."""

    def __init__(self, L, torch, cv, layout=None):
        from convolution_video_vae_amd.layer import Conv3d
        import workloads
        t = workloads.make_tensors(L)
        self.L = L
        lay = cv.NDHWC if layout is None else layout
        if L.fp8:   # e4m3fn operands: the same seeded tensors, cast
            t.x = t.x.float().to(torch.float8_e4m3fn)
            t.w = t.w.float().to(torch.float8_e4m3fn)
        x = t.x.cuda()
        if lay == cv.NCDHW:
            x = x.permute(0, 4, 1, 2, 3).contiguous()
        self.x = x
        self.layer = Conv3d(t.w.cuda(), tuple(x.shape), stride=L.stride, pad_lo=L.pad_lo,
                            pad_hi=L.pad_hi, layout=lay, bias=t.bias, gamma=t.gamma,
                            norm_silu=L.norm_silu, residual=L.residual,
                            pad_mode=cv.PAD_REFLECT if L.reflect else cv.PAD_ZERO)
        self.res = None if t.residual is None else t.residual.cuda()
        if lay == cv.NCDHW and self.res is not None:
            self.res = self.res.permute(0, 4, 1, 2, 3).contiguous()
        self.y = self.layer.new_output()
        probe = cv.make_epilogue(bias=self.layer.bias, gamma=self.layer.gamma,
                                 norm_silu=L.norm_silu)
        probe.flags |= cv.EPI_RESIDUAL if L.residual else 0
        self.plan = cv.conv3d_plan_describe(self.layer.desc, probe if probe.flags else None)

    def __call__(self):
        self.layer(self.x, residual=self.res, y=self.y)


# Per-layer entries warm up for at least this much GPU time: under sustained
# launches the chip takes some tens of milliseconds to settle (the headline
# layer's back-to-back time falls from about 850 to about 750 us over its
# first 40 calls, then stays there for hundreds of calls).
LAYER_WARM_MS = 50.0


def warm_up(case, warmup, torch, warm_ms=0.0):
    """`warmup` calls, then (warm_ms > 0) batches of 5 more until the
    warm-up has taken at least warm_ms of GPU time."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(warmup):
        case()
    stop.record()
    torch.cuda.synchronize()
    spent = start.elapsed_time(stop)
    while spent < warm_ms:
        start.record()
        for _ in range(5):
            case()
        stop.record()
        torch.cuda.synchronize()
        spent += start.elapsed_time(stop)


def time_case(case, steps, warmup, torch, warm_ms=0.0):
    """Mean ms per call over `steps` back-to-back calls between two events,
    after warm_up(case, warmup, torch, warm_ms)."""
    warm_up(case, warmup, torch, warm_ms)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        case()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


SCRUB_BYTES = 512 << 20     # twice the 256 MB memory-side cache


class Scrubber:
    """Writes 512 MB between timed calls, so the L2s and the memory-side
    cache hold none of the layer's operands when a cold call starts."""

    def __init__(self, torch):
        self.buf = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda")
        self.k = 0

    def __call__(self):
        self.k += 1
        self.buf.fill_(float(self.k))


def time_each(case, n, torch, scrub=None):
    """Median ms of n calls, each between its own pair of events; with a
    scrubber, 512 MB are written (outside the events) before every call."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        if scrub is not None:
            scrub()
        a.record()
        case()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def time_layer(case, steps, warmup, torch, scrub):
    """Back-to-back mean (the stepped figure, after a warm-up of at least
    LAYER_WARM_MS), warm per-call median and cold per-call median, all in
    ms."""
    mean, wall = time_case(case, steps, warmup, torch, LAYER_WARM_MS)
    warm = time_each(case, max(50, steps), torch)
    cold = time_each(case, 20, torch, scrub)
    return mean, warm, cold, wall


def host_enqueue_us(torch, cv, workloads, n=200):
    """Host time per conv3d_fwd call (µs): through the Conv3d layer wrapper
    (Python argument checks and marshalling included), and as a bare ctypes
    call of the C entry point with prepared arguments. Measured on the tiny
    causal layer, whose kernels finish faster than they are enqueued, so the
    launch queue never blocks the host."""
    import ctypes
    from convolution_video_vae_amd.layer import Conv3d
    L = workloads.LAYERS["tiny_causal_64"]
    t = workloads.make_tensors(L)
    conv = Conv3d(t.w.cuda(), L.x_shape, stride=L.stride, pad_lo=L.pad_lo, pad_hi=L.pad_hi,
                  bias=t.bias)
    x = t.x.cuda()
    y = conv.new_output()
    for _ in range(20):
        conv(x, y=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        conv(x, y=y)
    layer_us = (time.perf_counter() - t0) / n * 1e6
    torch.cuda.synchronize()
    lib = cv.lib()
    epi = cv.make_epilogue(bias=conv.bias)
    args = (ctypes.byref(conv.desc), x.data_ptr(), conv.w_packed.data_ptr(), ctypes.byref(epi),
            y.data_ptr(), conv.workspace.data_ptr(), conv.workspace_bytes,
            torch.cuda.current_stream().cuda_stream)
    fn = lib.conv3d_fwd
    t0 = time.perf_counter()
    for _ in range(n):
        rc = fn(*args)
    c_us = (time.perf_counter() - t0) / n * 1e6
    torch.cuda.synchronize()
    assert rc == 0
    return {"layer_call_us": round(layer_us, 2), "c_call_us": round(c_us, 2), "calls": n,
            "layer": L.name, "plan": cv.conv3d_plan_describe(conv.desc, epi)}


def host_cpu():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(L, seconds):
    """The oracle, untuned, on a bounded sample of the same layer's output pixels."""
    import oracle
    import workloads
    t = workloads.make_tensors(L)
    x, w = workloads.bf16_bits(t.x), workloads.bf16_bits(t.w)
    per_pixel = 2.0 * L.cout * L.cin * L.live_taps
    chunk = max(256, int(2e10 / per_pixel))            # ~20 GFLOP per call
    rng = np.random.default_rng(0)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        start = int(rng.integers(0, max(1, L.m - chunk)))
        pix = np.arange(start, min(L.m, start + chunk))
        oracle.conv3d(x, w, stride=L.stride, pad_lo=L.pad_lo, pad_hi=L.pad_hi,
                      bias=None if t.bias is None else t.bias.numpy(), pixels=pix)
        done += pix.size
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(done * per_pixel / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "host_cpu": host_cpu(), "host_logical_cpus": os.cpu_count(),
            "sample": f"{done} output pixels (all {L.cout} channels each) of {L.name} "
                      f"({L.m} in the layer), in random contiguous runs of {chunk}, "
                      f"{dt:.1f} s wall"}


def stream_cases(args, per_layer, wanted, torch, cv, workloads):
    """Streaming variants: padded outputs with history and cache, and the
    first layer's chunk packing (timed together with its conv)."""
    from convolution_video_vae_amd.layer import Conv3d, stream_pack_input
    for name, S in workloads.STREAM_LAYERS.items():
        if wanted is not None and name not in wanted:
            continue
        if "norm" in S:
            n, d, h, w, c = S["norm"]
            rng = np.random.default_rng(np.random.SeedSequence([1008, 0]))
            mk = lambda shape: torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(
                torch.bfloat16).cuda()
            x, res = mk((n, d, h, w, c)), mk((n, d, h, w, c))
            prev = mk((n, S["history"], h, w, c))
            bias = torch.from_numpy(rng.standard_normal(c, dtype=np.float32) * np.float32(0.3)).cuda()
            gamma = torch.from_numpy(rng.uniform(0.5, 1.5, c).astype(np.float32)).to(torch.bfloat16).cuda()
            y = torch.empty((n, d + 2, h + 2, w + 2, c), dtype=torch.bfloat16, device="cuda")
            cache = torch.empty((n, S["cache"], h, w, c), dtype=torch.bfloat16, device="cuda")
            rout = torch.empty_like(x)
            epi = cv.make_epilogue(bias=bias, residual=res, gamma=gamma, residual_out=rout,
                                   norm_silu=True)
            op = cv.make_out_pad(S["pad_lo"], S["pad_hi"], S["history"], cache, S["cache"])

            def step():
                cv.conv3d_norm_silu(x, n, d, h, w, c, epi, op, prev, y)
            nms, _ = time_case(step, max(5, args.steps), 3, torch, LAYER_WARM_MS)
            moved = 2 * (3 * x.numel() + y.numel() + prev.numel() + cache.numel())
            per_layer[name] = {
                "us": round(nms * 1e3, 2), "gbs": round(moved / (nms * 1e-3) / 1e9, 1),
                "pct_hbm": round(100 * moved / (nms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                "config": f"raw NDHWC {list(S['norm'])} + bias + residual -> L2 norm, SiLU; "
                          f"written padded {list(y.shape)} with {S['history']} history frames "
                          f"copied in, {S['cache']}-frame cache, value saved"}
            continue
        if "video" in S:
            rng = np.random.default_rng(np.random.SeedSequence([1007, 0]))
            video = torch.from_numpy(rng.standard_normal(S["video"], dtype=np.float32)).to(
                torch.bfloat16).cuda()
            n, c, T, h, w = S["video"]
            chunk = video[:, :, S["t0"]:S["t0"] + S["t"]]
            hist = video[:, :, S["t0"] - S["history"]:S["t0"]].permute(0, 2, 3, 4, 1).contiguous()
            wt = torch.zeros((S["cout"], S["c_pad"], 3, 3, 3), dtype=torch.bfloat16)
            wt[:, :c] = torch.from_numpy(rng.standard_normal((S["cout"], c, 3, 3, 3), dtype=np.float32)
                                         * np.float32(np.sqrt(1 / (27 * c)))).to(torch.bfloat16)
            padded = torch.empty((n, S["t"] + 2, h + 2, w + 2, S["c_pad"]), dtype=torch.bfloat16,
                                 device="cuda")
            cache = torch.empty((n, 2, h, w, c), dtype=torch.bfloat16, device="cuda")
            conv = Conv3d(wt.cuda(), tuple(padded.shape))
            y = conv.new_output()

            def step():
                stream_pack_input(chunk, hist, S["c_pad"], padded=padded, cache=cache)
                conv(padded, y=y)
            m = n * S["t"] * h * w
            flops = 2.0 * m * S["cout"] * 27 * c
            plan = cv.conv3d_plan_describe(conv.desc)
            config = (f"chunk NCTHW [{n}, {c}, {S['t']}, {h}, {w}] (strided view of a {T}-frame "
                      f"clip) + {S['history']} history frames -> padded [{n}, {S['t'] + 2}, {h + 2}, "
                      f"{w + 2}, {S['c_pad']}] -> valid conv to {S['cout']} channels")
        else:
            if "layer" in S:
                L = workloads.LAYERS[S["layer"]]
                t = workloads.make_tensors(L)
                xs, cout = L.x_shape, L.cout
                kw = dict(bias=t.bias, gamma=t.gamma, norm_silu=L.norm_silu, residual=L.residual)
                res = None if t.residual is None else t.residual.cuda()
                x, w = t.x.cuda(), t.w.cuda()
            else:
                xs, cout = S["x"], S["cout"]
                L = workloads.Layer(name, 5, xs, cout, bias=True, residual=True)
                t = workloads.make_tensors(L)
                kw = dict(bias=t.bias, residual=True)
                res, x, w = t.residual.cuda(), t.x.cuda(), t.w.cuda()
            conv = Conv3d(w, xs, out_pad_lo=S["pad_lo"], out_pad_hi=S["pad_hi"],
                          history_frames=S.get("history", 0), cache_frames=S.get("cache", 0), **kw)
            y = torch.zeros(conv.out_shape, dtype=torch.bfloat16, device="cuda")
            cache = (torch.empty(conv.cache_shape, dtype=torch.bfloat16, device="cuda")
                     if S.get("cache") else None)

            def step():
                conv(x, residual=res, y=y, cache=cache)
            flops = L.flops()
            probe = cv.make_epilogue(bias=conv.bias, gamma=conv.gamma, norm_silu=conv.norm_silu)
            probe.flags |= cv.EPI_RESIDUAL if conv.has_residual else 0
            plan = cv.conv3d_plan_describe(conv.desc, probe)
            config = (f"x NDHWC {list(xs)} -> {cout} channels, output written padded "
                      f"{list(S['pad_lo'])}/{list(S['pad_hi'])} into {list(conv.out_shape)}"
                      f"{', history ' + str(S['history']) if S.get('history') else ''}"
                      f"{', cache ' + str(S['cache']) if S.get('cache') else ''}")
        sms, _ = time_case(step, max(5, args.steps), 3, torch, LAYER_WARM_MS)
        assert torch.isfinite(y.float()).all().item()
        tf = flops / (sms * 1e-3) / 1e12
        per_layer[name] = {"us": round(sms * 1e3, 2), "tflops": round(tf, 2),
                           "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                           "gflop": round(flops / 1e9, 3), "config": config, "plan": plan}
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the kernel "
              "is measured at one GPU's share of the work, at its real shape)", file=sys.stderr)
        sys.exit(2)
    import torch
    import convolution_video_vae_amd as cv
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cv.lib()
    head = workloads.LAYERS[args.workload or workloads.HEADLINE]

    if args.sweep:
        for tile in args.sweep.split(";"):
            os.environ["CONV3D_TILE"] = tile
            c = Case(head, torch, cv)
            sms, _ = time_case(c, args.steps, args.warmup, torch)
            print(f"sweep {head.name} tile={tile} {c.plan}: {sms * 1e3:.1f} us "
                  f"{head.flops() / (sms * 1e-3) / 1e12:.1f} TFLOP/s", file=sys.stderr, flush=True)
            del c
        os.environ.pop("CONV3D_TILE", None)
        torch.cuda.empty_cache()

    case = Case(head, torch, cv)
    ms, wall = time_case(case, args.steps, args.warmup, torch)
    flops = head.flops(live=True)
    tflops = flops / (ms * 1e-3) / 1e12
    assert torch.isfinite(case.y.float()).all().item()
    head_scrub = Scrubber(torch)
    head_warm = time_each(case, max(20, args.steps), torch)
    head_cold = time_each(case, 10, torch, head_scrub)
    del case, head_scrub
    torch.cuda.empty_cache()

    per_layer = {}
    scrub = Scrubber(torch)
    if not args.no_layers:
        wanted = None if args.layers is None else set(args.layers.split(","))
        for name, L in workloads.LAYERS.items():
            if wanted is not None and name not in wanted:
                continue
            variants = [(name, None)]
            if L.norm_silu:
                variants.append((name + "_ncdhw", cv.NCDHW))
            for vname, lay in variants:
                c = Case(L, torch, cv, layout=lay)
                lms, warm, cold, _ = time_layer(c, max(5, args.steps), 3, torch, scrub)
                lt = L.flops(live=True) / (lms * 1e-3) / 1e12
                peak = PEAK_FP8_TFLOPS if L.fp8 else PEAK_BF16_TFLOPS
                io = (L.m * L.cin * 0 + np.prod(L.x_shape) + L.m * L.cout
                      + 27 * L.cin * L.cout + (L.m * L.cout if L.residual else 0)) * 2
                per_layer[vname] = {
                    "us": round(lms * 1e3, 2), "tflops": round(lt, 2),
                    "pct_peak": round(100 * lt / peak, 2),
                    "us_warm_median": round(warm * 1e3, 2), "us_cold": round(cold * 1e3, 2),
                    "pct_peak_cold": round(100 * L.flops(live=True) / (cold * 1e-3) / 1e12 / peak, 2),
                    "algorithmic_gbs": round(io / (lms * 1e-3) / 1e9, 1),
                    "algorithmic_gbs_cold": round(io / (cold * 1e-3) / 1e9, 1),
                    "gflop": round(L.flops(live=True) / 1e9, 3), "plan": c.plan}
                del c
                torch.cuda.empty_cache()
        # boundary transpose on its own (NCDHW -> NDHWC of the fused layer's input)
        L = workloads.LAYERS["wan_fused_160to320"]
        n, d, h, w, c = L.x_shape
        src = torch.zeros((n, c, d, h, w), dtype=torch.bfloat16, device="cuda")
        dst = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device="cuda")
        tcase = lambda: cv.conv3d_transpose(src, cv.NCDHW, dst, n, c, d, h, w)
        tms, twarm, tcold, _ = time_layer(tcase, max(5, args.steps), 3, torch, scrub)
        moved = 2 * src.numel() * 2
        per_layer["transpose_ncdhw_to_ndhwc_" + L.name] = {
            "us": round(tms * 1e3, 2), "gbs": round(moved / (tms * 1e-3) / 1e9, 1),
            "pct_hbm": round(100 * moved / (tms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
            "us_warm_median": round(twarm * 1e3, 2), "us_cold": round(tcold * 1e3, 2),
            "gbs_cold": round(moved / (tcold * 1e-3) / 1e9, 1)}
        # and back: the conv's NDHWC output to NCDHW at the network's edge
        n2, d2, h2, w2, c2 = L.out_shape()
        src2 = torch.zeros((n2, d2, h2, w2, c2), dtype=torch.bfloat16, device="cuda")
        dst2 = torch.empty((n2, c2, d2, h2, w2), dtype=torch.bfloat16, device="cuda")
        tcase2 = lambda: cv.conv3d_transpose(src2, cv.NDHWC, dst2, n2, c2, d2, h2, w2)
        tms, twarm, tcold, _ = time_layer(tcase2, max(5, args.steps), 3, torch, scrub)
        moved = 2 * src2.numel() * 2
        per_layer["transpose_ndhwc_to_ncdhw_" + L.name] = {
            "us": round(tms * 1e3, 2), "gbs": round(moved / (tms * 1e-3) / 1e9, 1),
            "pct_hbm": round(100 * moved / (tms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
            "us_warm_median": round(twarm * 1e3, 2), "us_cold": round(tcold * 1e3, 2),
            "gbs_cold": round(moved / (tcold * 1e-3) / 1e9, 1)}
        del src2, dst2
        del src, dst
        # channels-last GroupNorm (+ SiLU) between the convs
        from convolution_video_vae_amd.layer import GroupNorm
        for name, N in workloads.NORM_LAYERS.items():
            if wanted is not None and name not in wanted:
                continue
            x, gamma, beta = workloads.norm_tensors(N)
            x = x.cuda()
            y = torch.empty_like(x)
            gn = GroupNorm(N.x_shape, N.groups, gamma.cuda(), beta.cuda(), eps=N.eps,
                           silu=N.silu, t_isolated=N.t_isolated)
            gms, gwarm, gcold, _ = time_layer(lambda: gn(x, y=y), max(5, args.steps), 3, torch,
                                              scrub)
            assert torch.isfinite(y.float()).all().item()
            per_layer[name] = {
                "us": round(gms * 1e3, 2), "algorithmic_gbs": round(N.bytes / (gms * 1e-3) / 1e9, 1),
                "pct_hbm": round(100 * N.bytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                "us_warm_median": round(gwarm * 1e3, 2), "us_cold": round(gcold * 1e3, 2),
                "algorithmic_mb": round(N.bytes / 1e6, 1),
                "config": f"x NDHWC {list(N.x_shape)} bf16, {N.groups} groups, "
                          f"{'per-frame' if N.t_isolated else 'per-sample'} statistics"
                          f"{', SiLU' if N.silu else ''}"}
            del x, y, gn
            torch.cuda.empty_cache()
        # a conv and the GroupNorm of its output: statistics in a separate
        # pass over y against statistics summed in the conv's epilogue
        for name, (lname, nname) in CONV_GN_PAIRS.items():
            if wanted is not None and name not in wanted:
                continue
            L, N = workloads.LAYERS[lname], workloads.NORM_LAYERS[nname]
            case = Case(L, torch, cv)
            _, gamma, beta = workloads.norm_tensors(N)
            gn = GroupNorm(N.x_shape, N.groups, gamma.cuda(), beta.cuda(), eps=N.eps,
                           silu=N.silu, t_isolated=N.t_isolated)
            assert tuple(case.y.shape) == tuple(N.x_shape)
            part = torch.empty(cv.conv3d_gn_partials_bytes(case.layer.desc) // 4,
                               dtype=torch.float32, device="cuda")
            out = torch.empty_like(case.y)

            def two_pass():
                case()
                gn(case.y, y=out)

            def fused():
                cv.conv3d_fwd_gn_stats(case.layer.desc, case.x, case.layer.w_packed, case.y,
                                       part, case.layer.workspace)
                cv.conv3d_group_norm_from_partials(gn.desc, case.layer.desc, part, case.y,
                                                   gn.gamma, gn.beta, out, gn.workspace)
            steps = max(5, args.steps)
            tms, _ = time_case(two_pass, steps, 3, torch, LAYER_WARM_MS)
            fms, _ = time_case(fused, steps, 3, torch, LAYER_WARM_MS)
            assert torch.isfinite(out.float()).all().item()
            flops = L.flops()
            per_layer[name] = {
                "us_two_pass": round(tms * 1e3, 2), "us_fused_stats": round(fms * 1e3, 2),
                "saved_us": round((tms - fms) * 1e3, 2),
                "tflops_fused_stats": round(flops / (fms * 1e-3) / 1e12, 2),
                "config": f"{lname} conv, then {nname} ({N.groups} groups, "
                          f"{'per-frame' if N.t_isolated else 'per-sample'} statistics"
                          f"{', SiLU' if N.silu else ''}) of its output; "
                          "two_pass = conv3d_fwd + conv3d_group_norm, fused_stats = "
                          "conv3d_fwd_gn_stats + conv3d_group_norm_from_partials"}
            del case, gn, part, out
            torch.cuda.empty_cache()

    if not args.no_layers:
        stream_cases(args, per_layer, wanted, torch, cv, workloads)

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"calibrate-copy: torch.neg over {src.numel() * 2} bytes read and written, "
              "3 launches", file=sys.stderr, flush=True)
        del src, dst

    traffic = None
    if TRAFFIC is not None and TRAFFIC.get("kernel_hash") == kernel_hash() \
            and TRAFFIC.get("workload") == head.name:
        traffic = TRAFFIC["bytes"]

    enqueue = host_enqueue_us(torch, cv, workloads)
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head, args.cpu_seconds)

    out = {
        "metric": "conv3d bf16 TFLOP/s per layer shape and % of MI355X bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(head), "gflop_per_step": round(flops / 1e9, 2),
                   "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                   "parallelism": "single GPU"},
        "headline_timing": {
            "ms_back_to_back_mean": round(ms, 4),
            "ms_warm_median": round(head_warm, 4),
            "ms_cold_median": round(head_cold, 4),
            "tflops_cold": round(flops / (head_cold * 1e-3) / 1e12, 2),
            "cold": "512 MB written between calls, each call between its own events"},
        "host_enqueue": enqueue,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_hash": kernel_hash(),
                     "kernel": "conv3d igemm main kernel (one launch per step)"},
        "cpu_baseline": cpu,
        "per_layer": per_layer,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic workloads for the Conv3D layers the pages describe.

This module holds shapes and random-number recipes only: none of the
convolution's arithmetic. The GPU tests, the benchmark, the smoke entry point
and the oracle checks all draw their inputs here, so both sides of every
comparison see identical tensors.

Recipe (every draw: numpy PCG64, fp32, then converted to bf16 by PyTorch's
round-to-nearest-even cast; the second parameter of N(.,.) is the variance):
  x         ~ N(0, 1)
  w         ~ N(0, 1/(27*Cin))       (OIDHW, the checkpoint layout)
  bias      ~ N(0, 0.1), kept fp32
  residual  ~ N(0, 1)
  gamma     ~ U(0.5, 1.5)
Seed: SeedSequence([1000 + family, stream]) with stream x=0, w=1, bias=2,
residual=3, gamma=4, so each tensor is reproducible on its own.

Layer shapes come from the pages' tables: the MiniMax H3 encoder (FlyDSL
issue page, "Shapes"), the Wan 2.2 encoder's dominant shapes (same page,
"Why"), the Qwen-Image T2I 96->96 layer at 1024^2 (FlyDSL PR page, "Test
shapes") and WAN's base_dim=160 family (cuDNN page, "Overview",
"Requirements").
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

CAUSAL = dict(pad_lo=(2, 1, 1), pad_hi=(0, 1, 1))
VALID = dict(pad_lo=(0, 0, 0), pad_hi=(0, 0, 0))


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    family: int                 # seed family 1..5
    x_shape: Tuple[int, int, int, int, int]   # NDHWC
    cout: int
    stride: Tuple[int, int, int] = (1, 1, 1)
    pad_lo: Tuple[int, int, int] = (0, 0, 0)
    pad_hi: Tuple[int, int, int] = (0, 0, 0)
    bias: bool = False
    residual: bool = False
    norm_silu: bool = False
    live_taps: int = 27         # taps that can see real pixels (T=1 causal: 9)
    reflect: bool = False       # reflect spatial padding (the H3 encoder's own)
    fp8: bool = False           # e4m3fn activations and weights (bf16 output)

    @property
    def cin(self) -> int:
        return self.x_shape[4]

    def out_dhw(self):
        _, D, H, W, _ = self.x_shape
        k = 3
        return tuple((i + lo + hi - k) // s + 1 for i, lo, hi, s in
                     zip((D, H, W), self.pad_lo, self.pad_hi, self.stride))

    def out_shape(self):
        return (self.x_shape[0],) + self.out_dhw() + (self.cout,)

    @property
    def m(self) -> int:
        n = self.x_shape[0]
        d, h, w = self.out_dhw()
        return n * d * h * w

    def flops(self, live: bool = True) -> float:
        """2*M*N*K with K = 27*Cin (only the live taps when live=True)."""
        taps = self.live_taps if live else 27
        return 2.0 * self.m * self.cout * taps * self.cin


LAYERS = {
    # Tiny causal 64->64.
    "tiny_causal_64": Layer("tiny_causal_64", 1, (1, 5, 16, 16, 64), 64, bias=True, **CAUSAL),
    # H3 L5: wide channels on 16x16 frames.
    "h3_l5_1024": Layer("h3_l5_1024", 2, (1, 5, 16, 16, 1024), 1024, bias=True, **CAUSAL),
    "h3_l5_512to1024": Layer("h3_l5_512to1024", 2, (1, 5, 16, 16, 512), 1024, bias=True, **CAUSAL),
    # H3 L0: full-resolution 128->128, and its stride-(1,2,2) downsample.
    "h3_l0_128": Layer("h3_l0_128", 3, (1, 17, 256, 256, 128), 128, **CAUSAL),
    # the same layer with H3's own spatial padding: reflect instead of zeros
    "h3_l0_128_reflect": Layer("h3_l0_128_reflect", 3, (1, 17, 256, 256, 128), 128, reflect=True,
                               **CAUSAL),
    # the same layer with e4m3fn operands (the FP8 variant of the conv)
    "h3_l0_128_fp8": Layer("h3_l0_128_fp8", 3, (1, 17, 256, 256, 128), 128, fp8=True, **CAUSAL),
    "h3_l0_128_s122": Layer("h3_l0_128_s122", 3, (1, 17, 256, 256, 128), 128, stride=(1, 2, 2),
                            pad_lo=(2, 0, 0), pad_hi=(0, 1, 1)),
    # Wan encoder's pre-padded valid convs.
    "wan_valid_96": Layer("wan_valid_96", 4, (1, 6, 354, 642, 96), 96, **VALID),
    "wan_valid_384": Layer("wan_valid_384", 4, (1, 3, 46, 82, 384), 384, **VALID),
    # Qwen-Image 96->96 at 1024^2, T=1 causal: only the last temporal slice is live.
    "qwen_t1_96": Layer("qwen_t1_96", 4, (1, 1, 1024, 1024, 96), 96, live_taps=9, **CAUSAL),
    # WAN base_dim=160 family, 160->320 with the fused post-operations.
    "wan_fused_160to320": Layer("wan_fused_160to320", 5, (1, 7, 66, 122, 160), 320, bias=True,
                                residual=True, norm_silu=True, **VALID),
}

# The layer the headline throughput is quoted on (H3 L0, ~1 TFLOP per call).
HEADLINE = "h3_l0_128"


def _rng(family: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([1000 + family, stream]))


def _to_bf16(a32: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t) -> np.ndarray:
    """numpy uint16 view of a CPU bf16 tensor's bit patterns."""
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class Tensors:
    x: "object"                 # torch bf16 CPU, NDHWC
    w: "object"                 # torch bf16 CPU, OIDHW
    bias: Optional["object"]    # torch fp32 CPU [Co]
    residual: Optional["object"]  # torch bf16 CPU, NDHWC output shape
    gamma: Optional["object"]   # torch bf16 CPU [Co]


def make_tensors(layer: Layer, x_shape=None, cout=None, family=None) -> Tensors:
    """Seeded inputs for `layer` (shape overrides allow small parity cases)."""
    import torch
    fam = layer.family if family is None else family
    xs = tuple(layer.x_shape if x_shape is None else x_shape)
    co = layer.cout if cout is None else cout
    ci = xs[4]
    x = _to_bf16(_rng(fam, 0).standard_normal(xs, dtype=np.float32))
    w = _to_bf16(_rng(fam, 1).standard_normal((co, ci, 3, 3, 3), dtype=np.float32)
                 * np.float32(np.sqrt(1.0 / (27.0 * ci))))
    bias = residual = gamma = None
    if layer.bias:
        bias = torch.from_numpy(_rng(fam, 2).standard_normal((co,), dtype=np.float32)
                                * np.float32(np.sqrt(0.1)))
    if layer.residual or layer.norm_silu:
        d = tuple((i + lo + hi - 3) // s + 1 for i, lo, hi, s in
                  zip(xs[1:4], layer.pad_lo, layer.pad_hi, layer.stride))
        if layer.residual:
            residual = _to_bf16(_rng(fam, 3).standard_normal((xs[0],) + d + (co,), dtype=np.float32))
        if layer.norm_silu:
            gamma = _to_bf16(_rng(fam, 4).uniform(0.5, 1.5, size=(co,)).astype(np.float32))
    return Tensors(x, w, bias, residual, gamma)


def integer_tensors(x_shape, cout, seed=7, bias=False):
    """Integer-valued inputs: x in {-2..2}, w in {-1,0,1}, integer bias.

    Every partial sum of such a convolution is an integer below 2^24 in
    magnitude for K <= 27648, so any fp32 summation order gives the same exact
    result; only the final bf16 rounding remains.
    """
    import torch
    rng = np.random.default_rng(np.random.SeedSequence([2000, seed]))
    ci = x_shape[4]
    x = torch.from_numpy(rng.integers(-2, 3, size=x_shape).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.integers(-1, 2, size=(cout, ci, 3, 3, 3)).astype(np.float32)).to(torch.bfloat16)
    b = None
    if bias:
        b = torch.from_numpy(rng.integers(-8, 9, size=(cout,)).astype(np.float32))
    return x, w, b


# ---------------------------------------------------------------- GroupNorm

@dataclasses.dataclass(frozen=True)
class NormLayer:
    """A GroupNorm (+ SiLU) between the H3 encoder's convs: the activation
    each ResnetBlock normalises at one level (FlyDSL issue page, H3 comment:
    "Shapes" for the activations, the GroupNorm argument for the norm)."""
    name: str
    family: int
    x_shape: Tuple[int, int, int, int, int]   # NDHWC
    groups: int = 32
    silu: bool = True
    t_isolated: bool = True
    eps: float = 1e-5

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: x read once, y written once (bf16)."""
        return 2 * 2 * int(np.prod(self.x_shape))


NORM_LAYERS = {
    "gn_h3_l0_128": NormLayer("gn_h3_l0_128", 6, (1, 17, 256, 256, 128)),
    "gn_h3_l1_256": NormLayer("gn_h3_l1_256", 6, (1, 17, 128, 128, 256)),
    "gn_h3_l3_512": NormLayer("gn_h3_l3_512", 6, (1, 5, 32, 32, 512)),
    "gn_h3_l5_1024": NormLayer("gn_h3_l5_1024", 6, (1, 5, 16, 16, 1024)),
}


def norm_tensors(layer: NormLayer, x_shape=None, seed_stream: int = 0):
    """Seeded GroupNorm inputs: x bf16 NDHWC, gamma and beta fp32 [C].

    x ~ N(0, 1) + o_c with a per-channel offset o_c ~ N(0, 0.25) (a conv
    output with bias, so group means are not zero); gamma ~ U(0.5, 1.5);
    beta ~ N(0, 0.01). Seed: SeedSequence([1000 + family, s]) with s = 10 for
    x (10 + 10 k for draw k of seed_stream), 11 offsets, 12 gamma, 13 beta."""
    import torch
    xs = tuple(layer.x_shape if x_shape is None else x_shape)
    c = xs[4]
    fam = layer.family
    off = _rng(fam, 11).standard_normal(c, dtype=np.float32) * np.float32(0.5)
    x = _rng(fam, 10 + 10 * seed_stream).standard_normal(xs, dtype=np.float32)
    x += off
    gamma = torch.from_numpy(_rng(fam, 12).uniform(0.5, 1.5, size=c).astype(np.float32))
    beta = torch.from_numpy(_rng(fam, 13).standard_normal(c, dtype=np.float32) * np.float32(0.1))
    return _to_bf16(x), gamma, beta


# ---------------------------------------------------------------- streaming

# Streaming variants at the Wan 160-channel level (cuDNN page, "Causal Conv3D
# with Cache", "Normalization and Padding Variant", "Spatial Padding
# Variant"): chunks of 5 frames of 64 x 120 with two history frames, so a
# padded buffer is [1, 7, 66, 122, C] like the fused layer's input.
STREAM_LAYERS = {
    # first layer: 12-channel chunk (frames 5..9 of a 17-frame clip, a
    # strided view), two raw history frames, packed to 32 channels, then a
    # valid 32 -> 160 conv without bias
    "wan_stream_in_12to160": dict(video=(1, 12, 17, 64, 120), t0=5, t=5, history=2, c_pad=32,
                                  cout=160),
    # fused 160 -> 320 written padded for the next causal conv, two history
    # frames, two-frame cache
    "wan_fused_pad_160to320": dict(layer="wan_fused_160to320", pad_lo=(2, 1, 1),
                                   pad_hi=(0, 1, 1), history=2, cache=2),
    # bias + residual with a zero bottom row and right column (feeds a
    # stride-2 conv)
    "wan_bias_res_pad_160to160": dict(x=(1, 7, 66, 122, 160), cout=160, pad_lo=(0, 0, 0),
                                      pad_hi=(0, 1, 1)),
    # standalone post-operations above the fused tile (640 channels, a
    # quarter of the 64 x 120 level): bias, residual, L2 norm, SiLU, written
    # padded with two history frames copied in and a two-frame cache
    "wan_norm_silu_pad_640": dict(norm=(1, 5, 16, 30, 640), pad_lo=(2, 1, 1), pad_hi=(0, 1, 1),
                                  history=2, cache=2),
}

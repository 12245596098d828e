"""Channels-last GroupNorm (+ SiLU) oracle — TEST INFRASTRUCTURE ONLY.

What it computes. The MiniMax H3 comment on the FlyDSL issue page
"conv3d_implicit — accept and emit NDHWC so chained convs skip the layout
round-trip" (the GroupNorm argument) describes the norm between the encoder's
convs: a GroupNorm whose statistics are taken per frame ("time-isolated": the
encoder folds time into the batch before normalising), optionally fused with
the SiLU that follows it, and points out that in NDHWC a group's channels are
contiguous at every pixel and the fold is a free view. This module is the
plain definition, on an NDHWC bf16 tensor x [N, D, H, W, C] with G groups of
C/G consecutive channels:

  unit      one frame (n, d) when time-isolated, else one sample n (all d)
  mean, var over the unit's pixels and the group's channels; var is the
            population variance (divide by the count), as GroupNorm uses
  a         = B(((x - mean) / sqrt(var + eps)) * gamma_c + beta_c)
  out       = B(a / (1 + exp(-a)))  with SiLU, else a

B() is fp32 -> bf16 rounding to nearest, ties to even. Readings where the
page is silent: 32 groups in the workloads, eps 1e-5 (PyTorch's GroupNorm
default), fp32 gamma and beta, and two rounding points (the norm's bf16
output, then the SiLU's), as a bf16 network running GroupNorm then SiLU
produces. Everything is computed in float64 (two-pass statistics with numpy's
pairwise sums) and rounded once to fp32 before each B().

Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
import this module; it shares no code with the GPU library.
"""
from __future__ import annotations

import numpy as np


def bf16_rne(values) -> np.ndarray:
    """B(x) for each value (rounded to fp32 first): bf16 bit patterns, round
    to nearest, ties to even. Finite inputs only."""
    u = np.ascontiguousarray(np.asarray(values, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def group_norm(x, groups, gamma, beta, *, eps=1e-5, silu=False, t_isolated=True,
               intermediates=False):
    """GroupNorm of x (NDHWC bf16 bit patterns) with `groups` groups of
    consecutive channels; gamma, beta fp32 [C].

    Returns the output bits [N, D, H, W, C], or with intermediates=True a dict
    with y, a (the norm's bf16 output), mean and rstd ([units, groups],
    float64)."""
    xv = bf16_value(x)
    N, D, H, W, C = xv.shape
    if C % groups:
        raise ValueError("channels not divisible by groups")
    cpg = C // groups
    units = N * D if t_isolated else N
    xs = xv.reshape(units, -1, groups, cpg)
    mean = xs.mean(axis=(1, 3), keepdims=True)
    var = ((xs - mean) ** 2).mean(axis=(1, 3), keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    g = np.asarray(gamma, dtype=np.float64).reshape(1, 1, groups, cpg)
    b = np.asarray(beta, dtype=np.float64).reshape(1, 1, groups, cpg)
    aff = (xs - mean) * rstd * g + b
    a = bf16_rne(aff)
    if silu:
        av = bf16_value(a)
        y = bf16_rne(av / (1.0 + np.exp(-av)))
    else:
        y = a
    y = y.reshape(N, D, H, W, C)
    if not intermediates:
        return y
    return {"y": y, "a": a.reshape(N, D, H, W, C), "mean": mean.reshape(units, groups),
            "rstd": rstd.reshape(units, groups), "affine": aff.reshape(N, D, H, W, C)}

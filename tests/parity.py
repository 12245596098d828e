"""Parity rule between the GPU output and the oracle (test helper).

Several results are correct: the pages fix an fp32 accumulator and the bf16
rounding points, not the order of the fp32 sum. Two correct orders can land
on opposite sides of a bf16 rounding boundary (one ulp), and near zero — or
after a bias or residual cancels most of the conv value — one ulp of the
larger intermediate is many ulps of the small result. The rule therefore
measures the allowed error in bf16 ulps of the largest magnitude the error
can have been made at:

  ulp(s) = 2^(floor(log2 s) - 7)                       (bf16: 8 significant bits)
  raw:    |y - r| <= 2 ulp(max(|r|, |conv|, 2^-8 RMS(r)))
  fused:  |y - r| <= 4 ulp(max(|r|, |affine|, k*max(|conv|,|main|,|value|), 2^-8 RMS(r)))
          with k = sqrt(C) |gamma_c| / den, which carries a pre-norm error to
          the output's scale.

2 and 4 ulps are the bounds stated for the raw and the fused path. The
2^-8 RMS floor covers results within 1/256 of the layer's RMS of zero,
where a correct fp32 sum of tens of thousands of terms has an absolute
error comparable to the value itself.
"""
from __future__ import annotations

import numpy as np


def b2f(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def ulp_bf16(s: np.ndarray) -> np.ndarray:
    s = np.maximum(np.abs(s).astype(np.float64), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(s)) - 7)


def check(y_bits, ref, *, fused=False, gamma_bits=None, cout=None, what=""):
    """Assert the rule; return diagnostics. ref: oracle dict (intermediates=True)."""
    y = b2f(y_bits).astype(np.float64)
    r = b2f(ref["y"]).astype(np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    floor = 2.0 ** -8 * rms
    conv = np.abs(b2f(ref["conv"]).astype(np.float64))
    if fused:
        C = cout if cout is not None else r.shape[-1]
        g = np.abs(b2f(gamma_bits).astype(np.float64))
        den = ref["den"].astype(np.float64).reshape(r.shape[:-1] + (1,))
        k = np.sqrt(C) * g / den
        pre = np.maximum(np.maximum(conv, np.abs(b2f(ref["main"]))), np.abs(b2f(ref["value"])))
        scale = np.maximum.reduce([np.abs(r), np.abs(b2f(ref["affine"]).astype(np.float64)),
                                   k * pre, np.full_like(r, floor)])
        nulp = 4.0
    else:
        scale = np.maximum.reduce([np.abs(r), conv, np.full_like(r, floor)])
        nulp = 2.0
    err = np.abs(y - r)
    allowed = nulp * ulp_bf16(scale)
    bad = err > allowed
    at_r = err / ulp_bf16(np.abs(r))
    diag = {
        "n": int(r.size),
        "bit_identical": float(np.mean(y_bits == ref["y"])) if r.size else 1.0,
        "max_ulp_rule": float(np.max(err / ulp_bf16(scale))) if r.size else 0.0,
        "max_ulp_at_r": float(np.max(at_r)) if r.size else 0.0,
        "mean_signed_ulp": float(np.mean((y - r) / ulp_bf16(np.abs(r)))) if r.size else 0.0,
    }
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(r[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside the rule; "
                             f"first {detail}; diag {diag}")
    return diag


def check_group_norm(y_bits, ref, *, what=""):
    """GroupNorm (+ SiLU) rule. The GPU forms the affine as an fp32 fma on
    fp32 statistics (mean and 1/sqrt(var + eps) from fp32 per-thread sums
    combined in fp64), the oracle in fp64; either side's value can land on
    the other side of a bf16 rounding boundary, which moves a by one ulp, and
    the SiLU (slope below 1.1) carries that ulp plus its own rounding:

      |y - r| <= 2 ulp(max(|r|, |a|, 2^-8 RMS(r)))

    with a the oracle's rounded norm output. The RMS floor covers outputs
    within 1/256 of the tensor's RMS of zero (and the SiLU's far negative
    tail, where the exact value is below fp32's normal range)."""
    y = b2f(y_bits).astype(np.float64)
    r = b2f(ref["y"]).astype(np.float64)
    a = b2f(ref["a"]).astype(np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    scale = np.maximum.reduce([np.abs(r), np.abs(a), np.full_like(r, 2.0 ** -8 * rms)])
    err = np.abs(y - r)
    allowed = 2.0 * ulp_bf16(scale)
    diag = {
        "n": int(r.size),
        "bit_identical": float(np.mean(y_bits == ref["y"])) if r.size else 1.0,
        "max_ulp_rule": float(np.max(err / ulp_bf16(scale))) if r.size else 0.0,
    }
    bad = err > allowed
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(r[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside the rule; "
                             f"first {detail}; diag {diag}")
    return diag


def check_fp8(y_bits, ref, sum_abs, *, what=""):
    """e4m3 operands: the raw rule plus an accumulation term. The gfx950 fp8
    MFMA (32x32x64) does not sum its 64 products exactly: measured on N(0,1)
    operands its error stays below 2^-18.9 of the sum of the products'
    magnitudes (it behaves like aligning a group to its largest product and
    keeping about 20 bits), while bf16 products are summed exactly. So

      |y - r| <= 2 ulp(max(|r|, |conv|, 2^-8 RMS(r))) + 2^-16 * sum_k |x_k w_k|

    (8x the largest measured ratio); sum_abs is that sum per output."""
    y = b2f(y_bits).astype(np.float64)
    r = b2f(ref["y"]).astype(np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    conv = np.abs(b2f(ref["conv"]).astype(np.float64))
    scale = np.maximum.reduce([np.abs(r), conv, np.full_like(r, 2.0 ** -8 * rms)])
    allowed = 2.0 * ulp_bf16(scale) + 2.0 ** -16 * np.asarray(sum_abs, dtype=np.float64)
    err = np.abs(y - r)
    diag = {"n": int(r.size), "bit_identical": float(np.mean(y_bits == ref["y"])),
            "max_err_over_sum_abs": float(np.max(err / np.maximum(sum_abs, 1e-30)))}
    bad = err > allowed
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(r[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside the rule; "
                             f"first {detail}; diag {diag}")
    return diag
